/*
 * ha.h -- head-wise hybrid attention prefill for AMD Instinct MI355X (gfx950).
 *
 * One attention layer's prefill over a long context, head by head:
 *   - streaming heads: causal sliding-window attention (SWA);
 *   - retrieval heads: a rank-16 low-rank indexer scores key blocks (or k-means
 *     clusters of the low-rank keys), keeps the top-k per query block, and exact
 *     softmax attention runs over the selected keys plus the local window;
 *   - TriangleMix heads: sink keys + local band, dense attention for the last rows;
 *   - dense heads: plain causal attention;
 *   - Orthros output positions: full cross-attention of a scale-offset query
 *     (one output row in prefill, many in SFT / pre-training).
 *
 * Sources (page title, passage):
 *   "RTPurbo" post (tchannels.org, Анализ данных): most heads work locally, a
 *     few retrieval heads reach far; a cheap 16-dim indexer scouts candidates
 *     and exact attention runs on them in full dimension.
 *   "RTPurboV2" article (th-motor.com): ~15% retrieval heads, the rest SWA
 *     (window 8192 in deployment); projector D -> r = 16; K clustering in the
 *     low-rank space; all-sparse mode when most heads are retrieval heads.
 *   36kr interview "Agent 的注意力系统" (TriangleMix introduction): streaming
 *     region + last Q-K region in deep layers; top-k over key blocks.
 *   Same interview, GQA answer: queries of one GQA group share their keys, so
 *     one selection can serve the group (group_select); top-k matching answer:
 *     block representatives, mean or per-dimension extremes (block_score).
 *   Baidu developer article "深度解析：超长上下文注意力架构的分层优化策略",
 *     mixed-precision index section: an 8-bit quantized indexer (index_bits).
 *   "一个 Attention,两种工作模式" (Orthros), "Prefilling" and design sections:
 *     SWA for all tokens, full cross-attention for output positions, a light
 *     scale-offset separating the two query roles.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  All device buffers
 *     are allocated and owned by the caller; the library never allocates,
 *     frees or keeps a pointer past the call.
 *   - Arguments are checked on the host before any HIP call; a call that
 *     returns an error has enqueued nothing.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and is asynchronous: outputs are valid once the stream has completed.
 *     No entry point synchronises.
 *   - The library holds no global mutable state apart from the scratch of
 *     ha_prefill_static; concurrent calls of the other entry points are safe
 *     as long as they do not share output or workspace buffers.
 *   - Layouts are token-major and contiguous:
 *       Q  bf16 [N, Hq, D]       K, V  bf16 [N, Hkv, D]
 *       O  fp32 [N, Hq, D]       O_out fp32 [n_out, Hq, D]
 *     Query head h reads KV head h / (Hq / Hkv).
 *   - Supported now: head_dim 128, rank 16, q_block = k_block = 64.
 *     Other values return HA_ERR_UNSUPPORTED.
 */
#ifndef HA_H_
#define HA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HA_VERSION 6

/* Size of the device scratch array ha_prefill_static uses on each GPU. */
#define HA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum {
  HA_SWA = 0,        /* causal sliding window: keys i-w < j <= i */
  HA_RETRIEVAL = 1,  /* indexer-selected blocks or clusters + window */
  HA_TRIANGLE = 2,   /* j <= i and (j < sink or i-j < w or i >= N-last_q) */
  HA_DENSE = 3       /* j <= i */
} ha_head_kind;

typedef enum {
  HA_OK = 0,
  HA_ERR_ARG = 1,          /* null pointer, inconsistent sizes, bad head kind */
  HA_ERR_UNSUPPORTED = 2,  /* valid but not built: D != 128, r != 16, blocks != 64,
                            * Hq > 255, topk > 255, more than 16384 candidate blocks
                            * or clusters, force_block0 with clusters, index_bits 8
                            * outside block mode with block_score 0 */
  HA_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than ha_workspace_bytes() */
  HA_ERR_DEVICE = 4,       /* a HIP launch or query failed */
  HA_ERR_SCRATCH = 5       /* ha_prefill_static: the layer needs more scratch than
                            * HA_STATIC_SCRATCH_BYTES */
} ha_status;

typedef struct {
  int32_t n_tokens;      /* N >= 1 */
  int32_t n_q_heads;     /* Hq, a multiple of Hkv */
  int32_t n_kv_heads;    /* Hkv >= 1 */
  int32_t head_dim;      /* D: 128 */
  float softmax_scale;   /* <= 0 selects 1/sqrt(D) */
  int32_t window;        /* w >= 1 for SWA / RETRIEVAL / TRIANGLE heads */
  int32_t rank;          /* indexer rank r: 16 */
  int32_t q_block;       /* query rows per selection: 64 */
  int32_t k_block;       /* keys per selectable block: 64 */
  int32_t topk;          /* blocks or clusters kept per query block, >= 0 */
  int32_t force_block0;  /* 1: retrieval heads always see key block 0 */
  int32_t n_clusters;    /* 0: block selection; M > 0: k-means cluster selection */
  int32_t kmeans_iters;  /* Lloyd iterations (>= 1 when n_clusters > 0) */
  int32_t kmeans_stride; /* initial centroid m = low-rank key m*stride; M*stride <= N */
  int32_t sink;          /* TriangleMix: keys [0, sink) always visible */
  int32_t last_q;        /* TriangleMix: rows >= N - last_q attend densely */
  int32_t n_out;         /* Orthros: the last n_out rows also run cross-attention */
  int32_t group_select;  /* 0: one selection per retrieval head and query block;
                          * 1: one per KV head and query block, scored by the max
                          *    over the group's retrieval heads and shared by them
                          *    (36kr interview, GQA answer: the queries of one GQA
                          *    group share their keys); every retrieval head's row
                          *    of `sel` then holds its group's selection */
  int32_t block_score;   /* block mode only (0 when n_clusters > 0): the score of
                          * candidate key block c for query block b
                          * 0: max over causal (i, j) of qlow_i . klow_j
                          * 1: max_i qlow_i . (mean of the block's klow)
                          * 2: max_i sum_d max(q_id kmax_cd, q_id kmin_cd), kmax /
                          *    kmin the block's per-dimension key extremes (an
                          *    upper bound on every key's dot product)
                          *    (36kr interview, top-k matching answer: a block is
                          *    represented by its mean key or by a point built
                          *    from per-dimension extremes; both representatives
                          *    ignore causality inside the block) */
  int32_t index_bits;    /* 0 or 32: fp32 low-rank keys; 8: the block scores read
                          * the keys as int8 codes with one fp32 scale per key
                          * (scale = max |k| / 127, code = k / scale rounded to
                          * nearest, ties to even; Baidu developer article on
                          * long-context attention, mixed-precision index
                          * section: an 8-bit indexer).  8 is built for block
                          * mode with block_score = 0 only. */
  float topk_mass;       /* adaptive budget ("RTPurboV2" article, fixed-top-k
                          * passage: heads, sequence lengths and queries need
                          * very different numbers of context tokens; the page's
                          * own method is missing, so this rule is a proposal):
                          * 0 (or >= 1) keeps the fixed top-k; in (0, 1) the topk
                          * best candidates of a query block are the budget and
                          * only the shortest prefix of them, by (score desc, id
                          * asc), whose share of sum exp(mass_scale * score)
                          * over the budget reaches topk_mass is kept (rows of
                          * sel then hold fewer ids, -1 padded) */
  float mass_scale;      /* scale of the indexer scores in that softmax; <= 0
                          * selects 1/sqrt(rank) */
} ha_layer_desc;

/* Optional copies of the indexer's intermediate results (caller-owned device
 * buffers; any field may be NULL).  Retrieval heads are numbered in
 * increasing query-head order (Hret of them).  n_qb = ceil(N / q_block). */
typedef struct {
  int32_t* sel;        /* [Hret, n_qb, topk] ascending block/cluster ids, -1 padded */
  float* qlow;         /* [Hret, N, r] low-rank queries */
  float* klow;         /* [Hkv, N, r] low-rank keys */
  float* centroids;    /* [Hkv, M, r] */
  int32_t* assign;     /* [Hkv, N] cluster of each key */
  int32_t* csr_off;    /* [Hkv, M+1] member offsets */
  int32_t* csr_mem;    /* [Hkv, N] key positions grouped by cluster, ascending inside */
} ha_aux;

/* Human-readable name of a status code (static storage). */
const char* ha_status_string(int status);

/* HA_VERSION of the built library. */
int ha_version(void);

/* Bytes of device workspace any entry point below needs for this layer
 * (the maximum over them).  Returns 0 when the descriptor is invalid.
 * head_kind (host) [Hq]. */
size_t ha_workspace_bytes(const ha_layer_desc* desc, const int32_t* head_kind);

/* Whole-layer prefill.
 * Sources: "RTPurbo" post (most heads attend locally and run SWA; retrieval
 * heads use a cheap 16-dim indexer to pick candidates and then exact
 * attention over them in full dimension); "RTPurboV2" article (~15% retrieval
 * heads, the rest SWA; all heads sparse when most are retrieval heads);
 * TriangleMix introduction in the 36kr interview (streaming region + last Q-K
 * region); Orthros page, "Prefilling" (all tokens SWA, output positions add
 * full cross-attention).
 * Runs, on `stream`: the indexer projection and
 * selection for retrieval heads (k-means first in cluster mode), the banded /
 * dense / triangle kernels for the other heads, the gather kernel for the
 * retrieval heads, and Orthros cross-attention for the last n_out rows.
 *   head_kind  (host) [Hq] ha_head_kind values
 *   P_idx      fp32 [Hkv, D, r] indexer projection; NULL iff no retrieval head
 *   xa_scale, xa_offset  fp32 [Hq, D]; NULL iff n_out == 0
 *   O          fp32 [N, Hq, D], every row of every head written
 *   O_out      fp32 [n_out, Hq, D]; NULL iff n_out == 0
 *   aux        optional (may be NULL), see ha_aux
 *   workspace  >= ha_workspace_bytes(desc, head_kind) bytes, 256-byte aligned */
int ha_prefill(const ha_layer_desc* desc, const int32_t* head_kind,
               const void* Q, const void* K, const void* V, const float* P_idx,
               const float* xa_scale, const float* xa_offset,
               float* O, float* O_out, ha_aux* aux,
               void* workspace, size_t ws_bytes, void* stream);

/* Whole-layer prefill that allocates nothing, for callers that cannot call
 * hipMalloc or bring a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Arguments and results as
 * ha_prefill, without the workspace: the kernels use a device array of
 * HA_STATIC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends (its address is looked up once per device, on
 * the first call made with that device current).
 *   Returns HA_ERR_SCRATCH, before any HIP call, when
 *   ha_workspace_bytes(desc, head_kind) > HA_STATIC_SCRATCH_BYTES (the 1M
 *   cluster-mode layer, for one, needs about 2.4 GB).
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap on one GPU (several streams or threads) race,
 * so the caller serialises them.  No entry point ever calls hipMalloc,
 * hipFree or an allocating library routine. */
int ha_prefill_static(const ha_layer_desc* desc, const int32_t* head_kind,
                      const void* Q, const void* K, const void* V, const float* P_idx,
                      const float* xa_scale, const float* xa_offset,
                      float* O, float* O_out, ha_aux* aux, void* stream);

/* Stage: low-rank projection (RTPurboV2, low-rank projector passage).
 *   qlow[t] = Q[:, h_t, :] P[g(h_t)] for the t-th retrieval head h_t, [Hret, N, r]
 *   klow[g] = K[:, g, :] P[g] for every KV head g, [Hkv, N, r]
 * Accumulates in fp32 from bf16 inputs.  qlow may be NULL (keys only). */
int ha_index_project(const ha_layer_desc* desc, const int32_t* head_kind,
                     const void* Q, const void* K, const float* P_idx,
                     float* qlow, float* klow, void* stream);

/* Stage: block scoring + top-k (RTPurbo scout; TriangleMix interview top-k).
 * For retrieval head t and query block b: eligible blocks c >= force_block0
 * with c*k_block <= qe_b - window; score as desc->block_score says (with
 * index_bits = 8 the keys are first quantized as ha_quantize_keys does);
 * keeps the topk best by (score desc, block asc).
 *   sel  int32 [Hret, n_qb, topk], ascending, -1 padded.
 *   workspace  block_score 1 or 2, or index_bits 8: >= ha_workspace_bytes(desc,
 *              head_kind) bytes, 256-byte aligned (block representatives, 8-bit
 *              keys); may be NULL with ws_bytes 0 otherwise. */
int ha_select_blocks(const ha_layer_desc* desc, const int32_t* head_kind,
                     const float* qlow, const float* klow, int32_t* sel,
                     void* workspace, size_t ws_bytes, void* stream);

/* Stage: 8-bit indexer keys (Baidu developer article on long-context
 * attention, mixed-precision index section).
 * For every row of klow [Hkv, N, r]: scale = max_d |k_d| / 127 (IEEE fp32
 * division), code_d = k_d / scale rounded to nearest with ties to even; an
 * all-zero row gets scale 0 and zero codes.
 *   codes int8 [Hkv, N, r]; scales fp32 [Hkv, N]. */
int ha_quantize_keys(const ha_layer_desc* desc, const float* klow, int8_t* codes, float* scales, void* stream);

/* Stage: Lloyd k-means of klow per KV head (RTPurboV2 clustering passage).
 * M = n_clusters, kmeans_iters iterations, C0_m = klow_{m*stride}; ties go to
 * the lower centroid; an empty cluster keeps its centroid.  Deterministic:
 * running with iters = t reproduces the state after t iterations.
 *   klow [Hkv, N, r]; centroids [Hkv, M, r]; assign [Hkv, N];
 *   csr_off [Hkv, M+1]; csr_mem [Hkv, N] (members of cluster m at
 *   csr_mem[off[m] .. off[m+1]), ascending key position).
 * Input range: any finite klow.  The distance pass runs on fp16 matrix
 * products of two-part splits; each KV head's keys and centroids enter it
 * multiplied by one power of two (largest |component| brought into
 * [2^9, 2^10)), which is exact and leaves the argmin unchanged.  Centroid
 * sums are fp32, so max |klow| * N must stay below the fp32 range. */
int ha_kmeans(const ha_layer_desc* desc, const float* klow, float* centroids,
              int32_t* assign, int32_t* csr_off, int32_t* csr_mem,
              void* workspace, size_t ws_bytes, void* stream);

/* Stage: cluster scoring + top-k ("RTPurboV2" article, clustering passage:
 * whole clusters of semantically unrelated keys are skipped; 36kr interview,
 * top-k matching answer: candidates are scored through a representative and
 * the top-k kept).  Eligible clusters have a member j <= qe_b - window;
 * score = max over the block's rows of qlow_i . C_m; keeps the topk best by
 * (score desc, cluster asc), written ascending, -1 padded.
 *   centroids [Hkv, M, r]; csr_off, csr_mem as ha_kmeans writes them;
 *   sel [Hret, n_qb, topk];
 *   workspace >= ha_workspace_bytes(desc, head_kind) bytes, 256-byte aligned
 *             (split centroids and each cluster's first member). */
int ha_select_clusters(const ha_layer_desc* desc, const int32_t* head_kind,
                       const float* qlow, const float* centroids,
                       const int32_t* csr_off, const int32_t* csr_mem,
                       int32_t* sel, void* workspace, size_t ws_bytes, void* stream);

/* Stage: SWA, dense and TriangleMix heads of head_kind (others untouched).
 * Sources: "RTPurboV2" article (streaming heads use a sliding window, 8192 in
 * deployment); Orthros page, "Prefilling" (every prompt token runs SWA);
 * TriangleMix introduction in the 36kr interview (sink keys + local band,
 * and the last query rows attend to every earlier key).  Key sets as in
 * ha_head_kind; exact softmax, bf16 products, fp32 statistics and output.
 *   workspace  >= 256 bytes, 256-byte aligned (ha_workspace_bytes() covers it):
 *              the work counters of the persistent kernel, cleared on the
 *              stream by the call itself. */
int ha_attn_band(const ha_layer_desc* desc, const int32_t* head_kind,
                 const void* Q, const void* K, const void* V, float* O,
                 void* workspace, size_t ws_bytes, void* stream);

/* Stage: retrieval heads: window U selected keys (U key block 0 when forced).
 * Sources: "RTPurbo" post (after the indexer's scouting, exact softmax
 * attention over the candidate keys in full dimension); "RTPurboV2" article,
 * clustering passage (a selected cluster brings all its member keys); 36kr
 * interview, GQA answer (one selection can serve a GQA group).
 * Block mode reads sel only; cluster mode also reads assign/csr.
 *   csr_off, csr_mem: NULL in block mode; in cluster mode a valid CSR (each
 *              cluster's members ascending, positions in [0, N)).
 *   workspace  >= ha_workspace_bytes(desc, head_kind) bytes, 256-byte aligned:
 *              the window part's log2-sum-exp per retrieval row, in cluster
 *              mode K and V copied into CSR order (2 * Hkv * N * D bf16), so
 *              that a selected cluster's visible members are read as one
 *              contiguous range of rows, and the window pass's work counters.
 * With group_select = 1 every retrieval head of a KV group reads the sel row
 * of the group's first retrieval head (the rows ha_select_* writes are equal). */
int ha_attn_gather(const ha_layer_desc* desc, const int32_t* head_kind,
                   const void* Q, const void* K, const void* V, const int32_t* sel,
                   const int32_t* csr_off, const int32_t* csr_mem, float* O,
                   void* workspace, size_t ws_bytes, void* stream);

/* Stage: Orthros cross-attention for rows p in [N-n_out, N):
 *   q' = q_p * xa_scale[h] + xa_offset[h] (fp32), attention over keys 0..p.
 * Orthros page, "Training, SFT and inference share one mechanism": the
 * number of output positions is 1 when prefilling, the response length in
 * SFT and N in pre-training.  Flash attention on the matrix cores with q'
 * held as two bf16 parts (hi + lo, ~2^-16 relative).
 *   workspace  >= ha_workspace_bytes(desc, head_kind) bytes, 256-byte aligned
 *              (split-key partials; none when the rows fill the chip) */
int ha_attn_cross(const ha_layer_desc* desc, const void* Q, const void* K, const void* V,
                  const float* xa_scale, const float* xa_offset, float* O_out,
                  void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HA_H_ */
