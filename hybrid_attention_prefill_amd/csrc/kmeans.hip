// k-means of the low-rank keys on gfx950 and cluster-level top-k selection.
//
// RTPurboV2 article, clustering passage: with the high-frequency positional
// noise filtered out by the low-rank projector, similar keys gather in the
// low-rank space; clustering them compresses the sequence dimension so whole
// clusters of unrelated keys are skipped.  Read here as plain Lloyd iteration:
//   C0_m = klow_{m*stride};  per iteration
//   a_j  = argmin_m ||klow_j - C_m||^2   (lowest m on equal fp32 distances)
//   C_m  = mean of the keys assigned to m (unchanged when none is).
//
// Every step is deterministic, so a run of t iterations reproduces the state
// after t iterations of a longer run:
//   assign   one lane per key, centroid tiles in LDS, d = |C|^2 - 2 k.C on MFMA
//   CSR      stable counting sort of key positions by cluster: per-chunk
//            histograms, a column scan, then an in-order scatter (ranks among
//            equal clusters inside a 256-key batch come from an LDS scan)
//   update   per cluster, the members' sum in CSR (position) order / count
#include "common.h"
#include "device_util.h"

#include <limits.h>

#include <type_traits>

namespace ha {
namespace {

constexpr int R = kRank;
constexpr int NT = 256;
constexpr int kChunk = 8192;      // keys per histogram chunk
constexpr int kCTile = 512;       // centroids per LDS tile in the assign step

__global__ __launch_bounds__(NT) void km_init_kernel(KmeansParams p) {
  const int g = blockIdx.y;
  const int x = blockIdx.x * NT + threadIdx.x;   // (m, r) flat
  if (x >= p.M * R) return;
  const int m = x / R, r = x % R;
  p.cent[((size_t)g * p.M + m) * R + r] = p.klow[((size_t)g * p.N + (size_t)m * p.stride) * R + r];
}

// Per iteration: centroids split into two fp16 parts and their squared
// norms, for the MFMA distance pass.
__global__ __launch_bounds__(NT) void km_prep_kernel(KmeansParams p) {
  const int g = blockIdx.y;
  const int m = blockIdx.x * NT + threadIdx.x;
  if (m >= p.M) return;
  const size_t o = ((size_t)g * p.M + m) * R;
  const float* c = p.cent + o;
  float nrm = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float v = c[r];
    nrm = fmaf(v, v, nrm);
    dev::split2_f16(v, p.c_hi[o + r], p.c_lo[o + r]);
  }
  p.c_norm[(size_t)g * p.M + m] = nrm;
}

// Assignment: each wave owns 32*KT keys (KT column blocks of 32), the
// workgroup 4 waves.  Centroids are staged in LDS 256 at a time: the two fp16
// parts of C_m as 16-bit rows, and |C_m|^2 in fp32.  For every tile of 32
// centroids and key block, one chain of three MFMAs gives
//   d^T[m][j] = |C_m|^2 - 2 C_m . k_j
// directly: the chain's accumulator starts at the norms (a lane's 16 rows,
// shared by the KT chains), and three fp16 passes over the split operands add
// -2 C_m . k_j (keys pre-scaled by -2, exact; ~2^-21 relative to |C||k|).
// The |k_j|^2 term does not change the argmin.  A lane holds one key
// and 16 of the tile's centroids in increasing order; the tile minimum is a
// min3 chain; only when some lane of a key block improves on its best does
// the wave look up the index (the lowest element equal to the tile minimum;
// tiles are scanned in increasing order and replace the best only when
// strictly smaller, so the lowest index wins on equal distances).  The two
// lane halves are merged with the same rule at the end.  Keys and centroids
// must stay well inside the fp16 range (|component| < 16384).
constexpr int kCChunk = 256;      // centroids per LDS chunk
constexpr int kCStr = 24;         // 16-bit row stride of a staged part (48 B: conflict-free 16-B reads)
constexpr int KT = 4;             // 32-key blocks per wave
constexpr float kPadNorm = 1e30f; // norm of the padding rows of a partial tile

__global__ __launch_bounds__(NT) void km_assign_kernel(KmeansParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t cs[2][kCChunk * kCStr];
  __shared__ __attribute__((aligned(16))) float cns[kCChunk];   // |C_m|^2 of the staged centroids
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int j0 = (blockIdx.x * 4 + wave) * (32 * KT);
  dev::f16x8 kh[KT], kl[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int j = min(p.N - 1, j0 + kt * 32 + lr);
    const float* kp = p.klow + ((size_t)g * p.N + j) * R + lh * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      _Float16 h, l;
      dev::split2_f16(-2.f * kp[e], h, l);
      kh[kt][e] = h;
      kl[kt][e] = l;
    }
  }
  float best[KT];
  int arg[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    best[kt] = __builtin_inff();
    arg[kt] = 0;
  }
  const _Float16* parts[2] = {p.c_hi + (size_t)g * p.M * R, p.c_lo + (size_t)g * p.M * R};
  const float* cn = p.c_norm + (size_t)g * p.M;
  for (int c0 = 0; c0 < p.M; c0 += kCChunk) {
    const int nc = min(kCChunk, p.M - c0);
    __syncthreads();
    {
      // thread t stages centroid c0 + t: two 32-B parts and the norm row
      const int m = c0 + tid;
      const bool ok = tid < nc;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4* src = reinterpret_cast<const uint4*>(parts[q] + (size_t)(ok ? m : c0) * R);
        const uint4 v0 = src[0], v1 = src[1];
        uint4* dst = reinterpret_cast<uint4*>(&cs[q][tid * kCStr]);
        dst[0] = v0;
        dst[1] = v1;
      }
      cns[tid] = ok ? cn[m] : kPadNorm;
    }
    __syncthreads();
    const int n_tiles = (nc + 31) / 32;
    for (int x = 0; x < n_tiles; ++x) {
      const int r0 = x * 32;
      const dev::f16x8 ah = *reinterpret_cast<const dev::f16x8*>(&cs[0][(r0 + lr) * kCStr + lh * 8]);
      const dev::f16x8 al = *reinterpret_cast<const dev::f16x8*>(&cs[1][(r0 + lr) * kCStr + lh * 8]);
      // the lane's 16 centroid rows lh*4 + 8q + (0..3): their norms seed
      // every chain's accumulator
      dev::f32x16 nv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(&cns[r0 + lh * 4 + 8 * q]);
        nv[4 * q + 0] = v.x;
        nv[4 * q + 1] = v.y;
        nv[4 * q + 2] = v.z;
        nv[4 * q + 3] = v.w;
      }
      const int m0 = c0 + r0;
      // KT independent MFMA chains, interleaved pass by pass
      dev::f32x16 acc[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) acc[kt] = dev::mfma32_f16(al, kh[kt], nv);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) acc[kt] = dev::mfma32_f16(ah, kl[kt], acc[kt]);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) acc[kt] = dev::mfma32_f16(ah, kh[kt], acc[kt]);
      float tmin[KT];
      bool imp = false;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        float tm = __builtin_inff();
#pragma unroll
        for (int e = 0; e < 16; e += 2) tm = __builtin_fminf(__builtin_fminf(tm, acc[kt][e]), acc[kt][e + 1]);
        tmin[kt] = tm;
        imp |= tmin[kt] < best[kt];
      }
      // rare once the scan is under way: some lane improves in some key
      // block; its index is the lowest e holding the tile minimum
      if (__any(imp)) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          int idx = 15;
#pragma unroll
          for (int e = 14; e >= 0; --e) idx = acc[kt][e] == tmin[kt] ? e : idx;
          if (tmin[kt] < best[kt]) {
            best[kt] = tmin[kt];
            arg[kt] = m0 + lh * 4 + (idx >> 2) * 8 + (idx & 3);
          }
        }
      }
    }
  }
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const float ob = __shfl_xor(best[kt], 32);
    const int oa = __shfl_xor(arg[kt], 32);
    if (ob < best[kt] || (ob == best[kt] && oa < arg[kt])) arg[kt] = oa;
    const int j = j0 + kt * 32 + lr;
    if (lh == 0 && j < p.N) p.assign[(size_t)g * p.N + j] = arg[kt];
  }
}

// per-chunk cluster histogram -> hist[g][chunk][m]
__global__ __launch_bounds__(NT) void km_hist_kernel(KmeansParams p) {
  __shared__ int h[kMaxSelCand];
  const int g = blockIdx.y, ch = blockIdx.x;
  for (int m = threadIdx.x; m < p.M; m += NT) h[m] = 0;
  __syncthreads();
  const int a = ch * kChunk, b = min(p.N, a + kChunk);
  const int32_t* as = p.assign + (size_t)g * p.N;
  for (int j = a + threadIdx.x; j < b; j += NT) atomicAdd(&h[as[j]], 1);
  __syncthreads();
  int32_t* dst = p.hist + ((size_t)g * p.n_chunks + ch) * p.M;
  for (int m = threadIdx.x; m < p.M; m += NT) dst[m] = h[m];
}

// per cluster: exclusive prefix over chunks (in place) and the total count
__global__ __launch_bounds__(NT) void km_colscan_kernel(KmeansParams p) {
  const int g = blockIdx.y;
  const int m = blockIdx.x * NT + threadIdx.x;
  if (m >= p.M) return;
  int32_t* col = p.hist + (size_t)g * p.n_chunks * p.M + m;
  int run = 0;
  for (int c = 0; c < p.n_chunks; ++c) {
    const int v = col[(size_t)c * p.M];
    col[(size_t)c * p.M] = run;
    run += v;
  }
  p.count[(size_t)g * p.M + m] = run;
}

// offsets: exclusive scan of the counts over clusters (one workgroup per KV head)
__global__ __launch_bounds__(NT) void km_offsets_kernel(KmeansParams p) {
  __shared__ int part[NT];
  const int g = blockIdx.x, tid = threadIdx.x;
  const int per = (p.M + NT - 1) / NT;
  const int a = min(p.M, tid * per), b = min(p.M, a + per);
  const int32_t* cnt = p.count + (size_t)g * p.M;
  int s = 0;
  for (int m = a; m < b; ++m) s += cnt[m];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < NT; ++t) {
      const int v = part[t];
      part[t] = run;
      run += v;
    }
  }
  __syncthreads();
  int32_t* off = p.csr_off + (size_t)g * (p.M + 1);
  int run = part[tid];
  for (int m = a; m < b; ++m) {
    off[m] = run;
    run += cnt[m];
  }
  if (tid == NT - 1) off[p.M] = run;
}

// stable scatter of key positions into CSR order, one workgroup per chunk
__global__ __launch_bounds__(NT) void km_scatter_kernel(KmeansParams p) {
  __shared__ int base[kMaxSelCand];       // [M] next free slot per cluster
  __shared__ int owner[kMaxSelCand];      // [M] lowest thread still to place a key of the cluster
  const int g = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
  const int32_t* pre = p.hist + ((size_t)g * p.n_chunks + ch) * p.M;
  const int32_t* off = p.csr_off + (size_t)g * (p.M + 1);
  for (int m = tid; m < p.M; m += NT) {
    base[m] = off[m] + pre[m];
    owner[m] = INT_MAX;
  }
  __syncthreads();
  const int a = ch * kChunk, b = min(p.N, a + kChunk);
  const int32_t* as = p.assign + (size_t)g * p.N;
  int32_t* mem = p.csr_mem + (size_t)g * p.N;
  // Keys in position order, NT at a time.  In each round the lowest thread
  // still holding a key of cluster c (the earliest position) takes c's next
  // slot, so every cluster's members stay in ascending position; a round
  // places one key per distinct cluster, and a batch rarely holds the same
  // cluster twice.
  for (int j0 = a; j0 < b; j0 += NT) {
    const int j = j0 + tid;
    const int c = j < b ? as[j] : -1;
    bool left = c >= 0;
    while (__syncthreads_or(left)) {
      if (left) atomicMin(&owner[c], tid);
      __syncthreads();
      const bool win = left && owner[c] == tid;
      if (win) {
        mem[base[c]] = j;
        base[c] += 1;
        left = false;
      }
      __syncthreads();
      if (c >= 0) owner[c] = INT_MAX;
    }
  }
}

__global__ __launch_bounds__(NT) void km_update_kernel(KmeansParams p) {
  const int g = blockIdx.y;
  const int m = blockIdx.x * (NT / R) + threadIdx.x / R;
  const int r = threadIdx.x % R;
  if (m >= p.M) return;
  const int32_t* off = p.csr_off + (size_t)g * (p.M + 1);
  const int32_t* mem = p.csr_mem + (size_t)g * p.N;
  const int lo = off[m], hi = off[m + 1];
  if (hi <= lo) return;
  const float* kl = p.klow + (size_t)g * p.N * R;
  float s = 0.f;
  for (int x = lo; x < hi; ++x) s += kl[(size_t)mem[x] * R + r];
  p.cent[((size_t)g * p.M + m) * R + r] = s / (float)(hi - lo);
}

// ---------------------------------------------------------------------------
// cluster selection: eligible clusters have a member j <= qe - window (the
// first CSR member is the smallest position); score = max over the query
// block's rows of qlow_i . C_m; the topk best by (score desc, cluster asc).

// Per layer, once: centroids split into bf16 hi/lo parts and the first
// (smallest) member position of every cluster (INT_MAX when empty).
__global__ __launch_bounds__(NT) void cluster_prep_kernel(SelectParams p) {
  const int g = blockIdx.y;
  const int m = blockIdx.x * NT + threadIdx.x;
  if (m >= p.M) return;
  const float* c = p.cent + ((size_t)g * p.M + m) * R;
  __bf16* hi = p.c_hi + ((size_t)g * p.M + m) * R;
  __bf16* lo = p.c_lo + ((size_t)g * p.M + m) * R;
#pragma unroll
  for (int r = 0; r < R; ++r) dev::split2(c[r], hi[r], lo[r]);
  const int32_t* off = p.csr_off + (size_t)g * (p.M + 1);
  const int lo_i = off[m], hi_i = off[m + 1];
  p.first_mem[(size_t)g * p.M + m] = hi_i > lo_i ? p.csr_mem[(size_t)g * p.N + lo_i] : INT_MAX;
}

// Per layer, once, for block mode with a representative score: each key
// block's representative (NPART 1: the mean of its low-rank keys; NPART 2:
// the per-dimension maxima as part 0 and minima as part 1) split into bf16
// hi/lo parts, and its first key as the "first member" (INT_MAX for block 0
// when it is attended anyway).  One thread per (block, dimension).
template <int NPART>
__global__ __launch_bounds__(NT) void block_prep_kernel(SelectParams p) {
  const int g = blockIdx.y;
  const int t = blockIdx.x * NT + threadIdx.x;
  const int c = t / R, d = t % R;
  if (c >= p.M) return;
  const int j0 = c * kBlock, j1 = min(p.N, j0 + kBlock);
  const float* kl = p.klow + (size_t)g * p.N * R + d;
  __bf16* hi = p.c_hi + ((size_t)g * p.M + c) * R * NPART;
  __bf16* lo = p.c_lo + ((size_t)g * p.M + c) * R * NPART;
  if (NPART == 1) {
    float s = 0.f;
    for (int j = j0; j < j1; ++j) s += kl[(size_t)j * R];
    dev::split2(s / (float)(j1 - j0), hi[d], lo[d]);
  } else {
    float a = -__builtin_inff(), b = __builtin_inff();
    for (int j = j0; j < j1; ++j) {
      const float v = kl[(size_t)j * R];
      a = fmaxf(a, v);
      b = fminf(b, v);
    }
    dev::split2(a, hi[d], lo[d]);
    dev::split2(b, hi[R + d], lo[R + d]);
  }
  if (d == 0) p.first_mem[(size_t)g * p.M + c] = (p.force_block0 && c == 0) ? INT_MAX : j0;
}

// One workgroup per (retrieval head, query block).  S[i][m] = qlow_i . C_m on
// MFMA (32 rows x 32 centroids per instruction, k = r = 16), split operands;
// a lane ends with 16 rows of one centroid, so the row max is a lane-local
// reduction plus one exchange with lane ^ 32.  Wave w takes centroid tiles
// w, w+4, ...  The scores stay in LDS for the exact top-k.
//
// Exact prefilter for the top-k: each of the 128 scoring lanes keeps the
// largest key it wrote.  If tau is the k-th largest of these lane maxima, at
// least k keys are >= tau, so the k-th largest key is >= tau and every key
// of the answer (ties at the k-th value included) is >= tau.  One pass
// collects the keys >= tau in index order (each wave a contiguous quarter of
// the clusters, into its own region of kCapW slots, the rest of the region
// zero-filled), and the radix select runs on those 4 * kCapW slots.  A wave
// that finds more than kCapW candidates sends the block to the full select.
//
// A unit of several slots (group-shared selection) repeats the scoring for
// each slot and keeps the max key per cluster (the order key is monotone);
// a lane owns the same clusters for every slot, so the lane maxima and the
// prefilter hold for the max scores as they do for one slot.
//
// The same kernel scores key-block representatives (block mode with a
// representative score): candidate m = key block m, "first member" = its
// first key.  NPART = 2 scores the per-dimension extremes bound as a 32-dim
// dot product: sum_d max(q_d a_d, q_d b_d) with a >= b equals
// max(q, 0) . a + min(q, 0) . b, so part 0 pairs max(q, 0) with the block
// maxima and part 1 pairs min(q, 0) with the minima.
constexpr int kSelBlocks = 1;
constexpr int kGroups = 128;      // scoring lanes (4 waves x 32)
constexpr int kCapW = 192;        // candidate slots per wave

template <int NPART>
__global__ __launch_bounds__(NT) void select_clusters_kernel(SelectParams p) {
  static_assert(kSelBlocks == 1, "the prefilter handles one query block per workgroup");
  __shared__ uint32_t keys[kSelBlocks][kMaxSelCand];
  __shared__ int hist[dev::kHistWords];
  __shared__ int tmp4[8];
  __shared__ int bcast[2];
  __shared__ uint32_t ckeys[4 * kCapW];
  __shared__ uint16_t cidx[4 * kCapW];
  __shared__ uint32_t gmax[kGroups];
  __shared__ uint32_t tau_s;
  __shared__ int ovf;
  __shared__ uint32_t sink_word;                  // store target of padding lanes
  const int t0 = (int)(p.unit[blockIdx.y] & 0xFFFFu), ns = (int)(p.unit[blockIdx.y] >> 16);
  const int tid = threadIdx.x;
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop control
  const int g = p.group_of_ret[t0];
  const int b0 = blockIdx.x * kSelBlocks;
  const int nb = min(kSelBlocks, p.n_qb - b0);
  if (p.topk == 0) return;

  int nrow[kSelBlocks], lim[kSelBlocks];
#pragma unroll
  for (int bi = 0; bi < kSelBlocks; ++bi) {
    const int qs0 = (b0 + bi) * kBlock;
    nrow[bi] = bi < nb ? min(kBlock, p.N - qs0) : 0;
    lim[bi] = bi < nb ? qs0 + nrow[bi] - 1 - p.window : -1;
  }
  // split query rows of slot t (parts as above); rows past the end of a
  // ragged last block repeat the block's first row, so the row max needs no
  // mask
  dev::bf16x8 qh[NPART][2], ql[NPART][2];
  auto load_q = [&](int t) {
    const int qs0 = b0 * kBlock;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int i = rt * 32 + lr;
      const int row = nb > 0 ? qs0 + (i < nrow[0] ? i : 0) : 0;
      const float* qp = p.qlow + ((size_t)t * p.N + row) * R + lh * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = qp[e];
#pragma unroll
        for (int part = 0; part < NPART; ++part) {
          const float vp = NPART == 1 ? v : (part == 0 ? fmaxf(v, 0.f) : fminf(v, 0.f));
          __bf16 hh, ll;
          dev::split2(vp, hh, ll);
          qh[part][rt][e] = hh;
          ql[part][rt][e] = ll;
        }
      }
    }
  };
  const __bf16* chi = p.c_hi + (size_t)g * p.M * R * NPART;
  const __bf16* clo = p.c_lo + (size_t)g * p.M * R * NPART;
  const int32_t* fm = p.first_mem + (size_t)g * p.M;
  int n_el[kSelBlocks] = {};
  uint32_t gmx = 0;                 // largest key this lane wrote
  const int n_tiles = (p.M + 31) / 32;
  // A wave's tiles are x = wave + 4 i.  Operands are loaded kPre tiles ahead
  // (register ring, static slots: the loop is unrolled by kPre).
  constexpr int kPre = 4;
  // A ring slot holds a tile's split centroids and, per lane, the first
  // member of its cluster (eligibility: a member <= lim).
  // Buffer loads: the lane's offset inside a tile is fixed and the tile's
  // offset is wave-uniform (scalar), so a load needs no vector address
  // arithmetic.  Lanes of the last tile past cluster M-1 fall outside the
  // resource's range and read zeros; their keys go to the dummy word.
  const __amdgpu_buffer_rsrc_t rs_hi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(chi), 0, p.M * NPART * R * 2, dev::kBufWord3);
  const __amdgpu_buffer_rsrc_t rs_lo = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(clo), 0, p.M * NPART * R * 2, dev::kBufWord3);
  const __amdgpu_buffer_rsrc_t rs_fm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(fm), 0, p.M * 4, dev::kBufWord3);
  auto ld = [&](int x, dev::bf16x8 (&bh)[NPART], dev::bf16x8 (&bl)[NPART], int& f) {
#pragma unroll
    for (int part = 0; part < NPART; ++part) {
      const int vo = (lr * NPART + part) * R * 2 + lh * 16;
      const int so = x * 32 * NPART * R * 2;
      bh[part] = __builtin_bit_cast(dev::bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs_hi, vo, so, 0));
      bl[part] = __builtin_bit_cast(dev::bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs_lo, vo, so, 0));
    }
    f = (int)__builtin_amdgcn_raw_buffer_load_b32(rs_fm, lr * 4, x * 32 * 4, 0);
  };
  dev::bf16x8 rbh[kPre][NPART], rbl[kPre][NPART];
  int rfm[kPre];
  const int lim0 = lim[0];
  for (int s = 0; s < ns; ++s) {
    load_q(t0 + s);
    // slot order, as in the loop body, so the first group waits only for its own slot
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      ld(min(n_tiles - 1, wave + 4 * u), rbh[u], rbl[u], rfm[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // The keys of tile x are finished one tile later, after the products of
    // the next tile are issued, so the matrix-result reads never wait on the
    // products just issued.  Key of a cluster: order key of the row max, 0 if
    // ineligible (no member <= lim); padding lanes store to a dummy word.
    dev::f32x16 pacc[2] = {dev::f32x16{}, dev::f32x16{}};
    int pm = INT_MAX;                 // the first finish stores 0 to the dummy word
    bool pel = false;
    // The loop is instantiated once for the first slot of a unit (plain
    // store) and once for later slots (max with the stored key), so its body
    // is one basic block and the previous tile's vector work can be placed
    // between the current tile's matrix products.
    auto run = [&](auto later_slot) {
      constexpr bool kLater = decltype(later_slot)::value;
      auto finish = [&]() {
        float mx = -__builtin_inff();
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, pacc[rt][e]);
        mx = dev::pair32_max(mx);
        const bool mok = pm < p.M;
        const bool el = mok & pel;
        const uint32_t key = el ? dev::order_key(mx) : 0u;
        uint32_t* dst = mok ? &keys[0][pm] : &sink_word;
        if constexpr (kLater) {
          *dst = max(*dst, key);
        } else {
          *dst = key;
          n_el[0] += (int)(el & (lh == 0));
        }
        gmx = max(gmx, key);
      };
      // Groups of kPre tiles run whole (tiles past the end compute on the
      // last tile and store nothing: their centroid index is >= M), so the
      // body has no branches around loads.
      for (int x0 = wave; x0 < n_tiles; x0 += 4 * kPre) {
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
          const int x = x0 + 4 * u;
          // the two row tiles' chains alternate, so no product waits on the
          // one just issued
          dev::f32x16 acc[2] = {dev::f32x16{}, dev::f32x16{}};
#pragma unroll
          for (int part = 0; part < NPART; ++part) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) acc[rt] = dev::mfma32(ql[part][rt], rbh[u][part], acc[rt]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) acc[rt] = dev::mfma32(qh[part][rt], rbl[u][part], acc[rt]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) acc[rt] = dev::mfma32(qh[part][rt], rbh[u][part], acc[rt]);
          }
          // eligibility of the slot's cluster, taken before the slot's refill
          // is issued (the empty asm orders the two), so the refill lands in
          // the slot's own registers: no ring rotation copies, which would
          // wait for the newest loads
          const bool fel = (lim0 >= 0) & (rfm[u] <= lim0);
          { const int fi = fel; asm volatile("" ::"v"(fi) : "memory"); }
          ld(min(x + 4 * kPre, n_tiles - 1), rbh[u], rbl[u], rfm[u]);
          finish();
          pacc[0] = acc[0];
          pacc[1] = acc[1];
          pm = x * 32 + lr;
          pel = fel;
          // products of this tile, the previous tile's vector work between
          // them, then the slot's refill
#pragma unroll
          for (int i = 0; i < 6 * NPART; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x020, 2 * NPART + 1, 0);
        }
      }
      finish();
    };
    if (s == 0) run(std::integral_constant<bool, false>{});
    else run(std::integral_constant<bool, true>{});
  }
  if (lh == 0) gmax[wave * 32 + lr] = gmx;
  if (tid == 0) {
    tau_s = 1u;
    ovf = 0;
  }
  int nE;
  dev::block_excl_scan(n_el[0], tmp4, &nE);     // (synchronizes)
  const int k = min(p.topk, nE);
  const size_t row_stride = (size_t)p.n_qb * p.topk;   // between slots' sel rows
  int32_t* out = p.sel + ((size_t)t0 * p.n_qb + b0) * p.topk;
  // a unit of several slots selects into LDS (the histogram is free once the
  // last radix pass is done) and copies the row to every slot
  int32_t* dst_row = ns == 1 ? out : reinterpret_cast<int32_t*>(hist);
  auto copy_row = [&]() {
    if (ns == 1) return;
    __syncthreads();
    for (int x = tid; x < ns * p.topk; x += NT) {
      const int s = x / p.topk, e = x - s * p.topk;
      out[s * row_stride + e] = dst_row[e];
    }
  };
  if (k > kGroups) {
    dev::topk_select(keys[0], p.M, k, p.topk, 0, dst_row, hist, tmp4, bcast);
    copy_row();
    return;
  }
  // tau = k-th largest lane maximum (the one with #{>} < k <= #{>=});
  // eligible keys are >= 1, so tau >= 1 also drops the ineligible ones
  if (k > 0 && tid < kGroups) {
    const uint32_t gv = gmax[tid];
    int gt = 0, ge = 0;
    for (int j = 0; j < kGroups; ++j) {
      const uint32_t v = gmax[j];
      gt += v > gv;
      ge += v >= gv;
    }
    if (gt < k && k <= ge && gv > 1u) tau_s = gv;
  }
  __syncthreads();
  const uint32_t tau = tau_s;
  {
    const int per = ((p.M + 4 * 64 - 1) / (4 * 64)) * 64;
    const int wa = min(p.M, wave * per), wb = min(p.M, wa + per);
    uint32_t* ck = ckeys + wave * kCapW;
    uint16_t* ci = cidx + wave * kCapW;
    int cnt = 0;
    for (int x0 = wa; x0 < wb; x0 += 64) {
      const int x = x0 + lane;
      const uint32_t u = x < wb ? keys[0][x] : 0u;
      const bool take = u >= tau;
      const uint64_t b = __ballot(take);
      const int pos = cnt + (int)__popcll(b & ((1ull << lane) - 1ull));
      if (take && pos < kCapW) {
        ck[pos] = u;
        ci[pos] = (uint16_t)x;
      }
      cnt += (int)__popcll(b);
    }
    for (int pos = cnt + lane; pos < kCapW; pos += 64) ck[pos] = 0u;
    if (cnt > kCapW && lane == 0) ovf = 1;
  }
  __syncthreads();
  if (ovf == 0) {
    dev::topk_select(ckeys, 4 * kCapW, k, p.topk, 0, dst_row, hist, tmp4, bcast, cidx);
  } else {
    dev::topk_select(keys[0], p.M, k, p.topk, 0, dst_row, hist, tmp4, bcast);
  }
  copy_row();
}

}  // namespace

size_t kmeans_scratch_bytes(int N, int M, int Hkv) {
  const size_t n_chunks = (size_t)(N + kChunk - 1) / kChunk;
  return (size_t)Hkv * n_chunks * M * sizeof(int32_t) + (size_t)Hkv * M * sizeof(int32_t) +
         (size_t)Hkv * M * (2 * R * sizeof(_Float16) + sizeof(float)) + 256;
}

hipError_t launch_kmeans(KmeansParams p, int Hkv, int iters, hipStream_t s) {
  p.n_chunks = (p.N + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(km_init_kernel, dim3((p.M * R + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
  hipError_t e = hipGetLastError();
  for (int it = 0; it < iters && e == hipSuccess; ++it) {
    hipLaunchKernelGGL(km_prep_kernel, dim3((p.M + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_assign_kernel, dim3((p.N + 4 * 32 * KT - 1) / (4 * 32 * KT), Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_hist_kernel, dim3(p.n_chunks, Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_colscan_kernel, dim3((p.M + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_offsets_kernel, dim3(Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_scatter_kernel, dim3(p.n_chunks, Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_update_kernel, dim3((p.M + (NT / R) - 1) / (NT / R), Hkv), dim3(NT), 0, s, p);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_select_clusters(const SelectParams& p, int Hkv, hipStream_t s) {
  if (p.n_ret == 0 || p.n_qb == 0) return hipSuccess;
  hipLaunchKernelGGL(cluster_prep_kernel, dim3((p.M + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
  hipLaunchKernelGGL(select_clusters_kernel<1>, dim3((p.n_qb + kSelBlocks - 1) / kSelBlocks, p.n_units), dim3(NT),
                     0, s, p);
  return hipGetLastError();
}

size_t select_clusters_scratch_bytes(int M, int Hkv) {
  return (size_t)Hkv * M * (2 * R * sizeof(__bf16) + sizeof(int32_t));
}

hipError_t launch_select_block_reps(const SelectParams& p, int Hkv, int mode, hipStream_t s) {
  if (p.n_units == 0 || p.n_qb == 0) return hipSuccess;
  const dim3 prep((p.M * R + NT - 1) / NT, Hkv), grid((p.n_qb + kSelBlocks - 1) / kSelBlocks, p.n_units);
  if (mode == 2) {
    hipLaunchKernelGGL(block_prep_kernel<2>, prep, dim3(NT), 0, s, p);
    hipLaunchKernelGGL(select_clusters_kernel<2>, grid, dim3(NT), 0, s, p);
  } else {
    hipLaunchKernelGGL(block_prep_kernel<1>, prep, dim3(NT), 0, s, p);
    hipLaunchKernelGGL(select_clusters_kernel<1>, grid, dim3(NT), 0, s, p);
  }
  return hipGetLastError();
}

size_t select_block_reps_scratch_bytes(int n_kb, int Hkv, int mode) {
  const size_t npart = mode == 2 ? 2 : 1;
  return (size_t)Hkv * n_kb * (2 * R * npart * sizeof(__bf16) + sizeof(int32_t));
}

}  // namespace ha
