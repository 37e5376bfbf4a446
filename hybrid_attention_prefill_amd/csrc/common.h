// Internal declarations shared by the host library and the HIP kernels.
// Not part of the public interface (that is include/ha.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ha {

constexpr int kHeadDim = 128;   // D
constexpr int kRank = 16;       // r
constexpr int kBlock = 64;      // q_block = k_block
constexpr int kMaxHeads = 256;  // table size; Hq <= 255 (0xFF marks an empty pack slot)
constexpr int kMaxTopk = 255;   // topk limit (the selected-key kernel keeps topk + 1 entries)
constexpr int kMaxSelCand = 16384;  // eligible blocks/clusters scored per query block in LDS

enum Kind { SWA = 0, RETRIEVAL = 1, TRIANGLE = 2, DENSE = 3 };

// A pack is up to 4 query heads of one KV head and one role that share their
// key tiles; the 4 waves of a workgroup take one head each.  Head ids are
// stored in bytes (0xFF = empty slot).
struct PackTable {
  int32_t n;
  uint32_t heads[kMaxHeads];  // 4 head ids per pack, byte w = wave w's head
  uint32_t slots[kMaxHeads];  // retrieval slot (row of sel) of each head, same packing
  int32_t sel_row[kMaxHeads]; // group-shared selection: slot of the KV group's first retrieval head
};

struct AttnParams {
  const uint16_t* Q;   // bf16 [N, Hq, D]
  const uint16_t* K;   // bf16 [N, Hkv, D]
  const uint16_t* V;
  float* O;            // fp32 [N, Hq, D]
  int N, Hq, Hkv, G;   // G = Hq / Hkv
  float c;             // softmax scale * log2(e)
  int window, sink, dense_from;   // dense_from = N - last_q (TRIANGLE)
  int kind;            // SWA, DENSE, TRIANGLE (band kernel) or RETRIEVAL (gather)
  int n_qt;            // query tiles of 64 rows
  // band kernel: the pack table holds band_np[0] packs of 4 heads (a
  // workgroup takes 64 query rows of each), then band_np[1] packs of 2 heads
  // (128 rows each), then band_np[2] single heads (256 rows): the 8 waves of
  // a workgroup always have rows to compute
  int band_np[3];
  // gather only
  const int32_t* sel;      // [Hret, n_qb, topk]
  int topk, force_block0;
  const int32_t* csr_off;  // cluster mode: [Hkv, M+1]
  const int32_t* csr_mem;  // cluster mode: [Hkv, N]
  int M;                   // 0 = block mode
  uint16_t* Kc;            // cluster mode: K and V rows in CSR order, [Hkv, N, D]
  uint16_t* Vc;            //   (row e of KV head g = key csr_mem[g][e])
  float* lse;              // [Hret, N] log2-sum-exp of the window part (retrieval heads)
  // Orthros cross-attention on the matrix cores (rows row0 .. N-1)
  const float* xs;         // [Hq, D] scale s_h
  const float* xo;         // [Hq, D] offset o_h
  float* O_out;            // [n_out, Hq, D]
  float* part;             // split-K partials [n_kc, n_out, Hq, D] (n_kc > 1)
  float* part_lse;         // [n_kc, n_out, Hq] log2-sum-exp of each partial
  int row0, n_out, n_kc, kc_tiles;   // key range split into n_kc chunks of kc_tiles 64-key tiles
};

// Retrieval heads handled by the selected-key kernel (slot t = row of sel / lse).
struct SelList {
  int32_t n_ret;
  int32_t head[kMaxHeads];
};

// Host launchers (each returns a hipError_t from the launch).
// The banded kernel is persistent: its workgroups take work items from
// per-XCD counters (kBandCounters words of device memory, cleared by the
// launcher on the stream before the kernel).
constexpr int kBandCounters = 8;
hipError_t launch_attn_band(const AttnParams& p, const PackTable& packs, uint32_t* ctr, hipStream_t s);
hipError_t launch_attn_selected(const AttnParams& p, const SelList& sl, hipStream_t s);
// Group-shared selection: every retrieval head of a KV group has the same key
// set (window + the selection row of the group's first retrieval head), so
// one workgroup computes a pack of up to 4 of them, window and selected keys
// together, and writes O (no log2-sum-exp).
hipError_t launch_attn_retrieval_group(const AttnParams& p, const PackTable& packs, hipStream_t s);
// Cluster mode: copies K and V rows into CSR order (Kc, Vc) so that the
// visible members of a cluster are one contiguous range of rows.
hipError_t launch_permute_kv(const AttnParams& p, hipStream_t s);

struct ProjParams {
  const uint16_t* X;   // bf16 [N, H, D]
  int N, H;            // H = heads in X
  const float* P;      // fp32 [Hkv, D, r]
  float* out;          // [n_entries, N, r]
  int n_entries;
  int32_t head[kMaxHeads];   // head of X for each entry
  int32_t group[kMaxHeads];  // projection group for each entry
};
hipError_t launch_project(const ProjParams& p, hipStream_t s);

struct SelectParams {
  const float* qlow;   // [Hret, N, r]
  const float* klow;   // [Hkv, N, r]   (block mode)
  const float* cent;   // [Hkv, M, r]   (cluster mode)
  const int32_t* csr_off;  // [Hkv, M+1]
  const int32_t* csr_mem;  // [Hkv, N]
  int32_t* sel;        // [Hret, n_qb, topk]
  __bf16* c_hi;        // scratch: [Hkv, M, parts * r] split centroids / block representatives
  __bf16* c_lo;
  _Float16* c_f16;     // scratch: (hi + lo) times the KV head's power-of-two scale, in fp16
  int32_t* first_mem;  // [Hkv, M] smallest member position (INT_MAX if empty or not a candidate)
  uint32_t* cnorm;     // [Hkv] largest candidate-vector norm (fp32 bits), for the scoring error bound
  const int8_t* kcodes;  // 8-bit indexer keys [Hkv, N, r] (nullptr: fp32 klow)
  const float* kscale;   // [Hkv, N] their scales
  int N, n_qb, window, topk, force_block0, M;
  float mass;            // adaptive budget: share of the top-k's softmax mass to keep (0: fixed top-k)
  float mass_scale_log2; // softmax scale of the indexer scores, times log2(e)
  int n_ret;
  int32_t group_of_ret[kMaxHeads];
  // A selection unit is a run of retrieval slots that share one top-k: one
  // slot per unit, or all slots of a KV group (group-shared selection).
  // unit[u] = first slot | slot count << 16.  Scores of a unit are the max
  // over its slots; its top-k row is written to every slot.
  int n_units;
  uint32_t unit[kMaxHeads];
};
hipError_t launch_select_blocks(const SelectParams& p, hipStream_t s);
// 8-bit indexer keys from fp32 low-rank keys (n_rows rows of r values).
hipError_t launch_quantize_keys(const float* klow, int8_t* codes, float* scales, size_t n_rows, hipStream_t s);

struct KmeansParams {
  const float* klow;   // [Hkv, N, r]
  float* cent;         // [Hkv, M, r]
  int32_t* assign;     // [Hkv, N]
  int32_t* csr_off;    // [Hkv, M+1]
  int32_t* csr_mem;    // [Hkv, N]
  int32_t* hist;       // scratch [Hkv, n_chunks, M]
  int32_t* count;      // scratch [Hkv, M]
  _Float16* c_hi;      // scratch [Hkv, M, r]: centroids split in two fp16 parts
  _Float16* c_lo;
  float* c_norm;       // scratch [Hkv, M]
  uint32_t* amax;      // scratch [Hkv]: largest |klow| component per KV head (fp32 bits)
  uint32_t* cmax;      // scratch [Hkv]: largest scaled squared centroid norm of the iteration (fp32 bits)
  uint32_t* almax;     // scratch [Hkv]: largest squared norm of the centroids' fp16 lo parts (fp32 bits)
  uint32_t* n_amb;     // scratch [Hkv]: keys the approximate assignment left undecided
  int32_t* amb;        // scratch [Hkv, N]: their positions
  uint64_t* best;      // scratch [Hkv, N]: per undecided key, min over centroid ranges of (ordered distance, index)
  int N, M, stride, n_chunks;
};
size_t kmeans_scratch_bytes(int N, int M, int Hkv);
hipError_t launch_kmeans(KmeansParams p, int Hkv, int iters, hipStream_t s);
hipError_t launch_select_clusters(const SelectParams& p, int Hkv, hipStream_t s);
size_t select_clusters_scratch_bytes(int M, int Hkv);
// Block mode with a representative score (mode 1 mean key, 2 per-dimension
// extremes): representatives of the M = n_kb key blocks into c_hi / c_lo /
// first_mem, then the cluster-scoring kernel over them.
hipError_t launch_select_block_reps(const SelectParams& p, int Hkv, int mode, hipStream_t s);
size_t select_block_reps_scratch_bytes(int n_kb, int Hkv, int mode);

// Orthros cross-attention rows: flash attention of q' = q * s + o over keys
// 0..p on the matrix cores (q' split into two bf16 parts), packs of 4 heads
// of one KV head, key range optionally split (then merged by a second kernel).
hipError_t launch_attn_cross(const AttnParams& p, const PackTable& packs, hipStream_t s);

// XCD-aware remap of a linear workgroup id: workgroups are dealt round-robin
// to the 8 XCDs; this makes consecutive logical ids land on the same XCD (and
// so share its L2).  A bijection on [0, n).
__device__ inline int xcd_remap(int bid, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = bid & 7, slot = bid >> 3;
  return (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
}

}  // namespace ha
