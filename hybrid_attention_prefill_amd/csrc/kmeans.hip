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
//   assign   one thread per key, centroid tiles in LDS, d = |C|^2 - 2 k.C
//   CSR      stable counting sort of key positions by cluster: per-chunk
//            histograms, a column scan, then an in-order scatter (ranks among
//            equal clusters inside a 256-key batch come from an LDS scan)
//   update   per cluster, the members' sum in CSR (position) order / count
#include "common.h"
#include "device_util.h"

#include <limits.h>

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

__global__ __launch_bounds__(NT) void km_assign_kernel(KmeansParams p) {
  __shared__ float cs[kCTile * R];
  __shared__ float cn[kCTile];
  const int g = blockIdx.y;
  const int j = blockIdx.x * NT + threadIdx.x;
  const bool ok = j < p.N;
  float k[R];
  {
    const float* kp = p.klow + ((size_t)g * p.N + (ok ? j : 0)) * R;
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      const float4 v = *reinterpret_cast<const float4*>(kp + r);
      k[r] = v.x; k[r + 1] = v.y; k[r + 2] = v.z; k[r + 3] = v.w;
    }
  }
  float best = __builtin_inff();
  int arg = 0;
  const float* C = p.cent + (size_t)g * p.M * R;
  for (int m0 = 0; m0 < p.M; m0 += kCTile) {
    const int nm = min(kCTile, p.M - m0);
    __syncthreads();
    for (int x = threadIdx.x; x < nm * R; x += NT) cs[x] = C[(size_t)m0 * R + x];
    __syncthreads();
    for (int x = threadIdx.x; x < nm; x += NT) {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) s = fmaf(cs[x * R + r], cs[x * R + r], s);
      cn[x] = s;
    }
    __syncthreads();
    for (int mm = 0; mm < nm; ++mm) {
      const float* c = cs + mm * R;
      float dot = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) dot = fmaf(k[r], c[r], dot);
      const float d = fmaf(-2.f, dot, cn[mm]);
      if (d < best) {
        best = d;
        arg = m0 + mm;
      }
    }
  }
  if (ok) p.assign[(size_t)g * p.N + j] = arg;
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
  __shared__ int batch[NT];
  const int g = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
  const int32_t* pre = p.hist + ((size_t)g * p.n_chunks + ch) * p.M;
  const int32_t* off = p.csr_off + (size_t)g * (p.M + 1);
  for (int m = tid; m < p.M; m += NT) base[m] = off[m] + pre[m];
  __syncthreads();
  const int a = ch * kChunk, b = min(p.N, a + kChunk);
  const int32_t* as = p.assign + (size_t)g * p.N;
  int32_t* mem = p.csr_mem + (size_t)g * p.N;
  for (int j0 = a; j0 < b; j0 += NT) {
    const int j = j0 + tid;
    const int c = j < b ? as[j] : -1;
    batch[tid] = c;
    __syncthreads();
    int rank = 0, after = 0;
    const int nb = min(NT, b - j0);
    for (int t = 0; t < nb; ++t) {
      const int ct = batch[t];
      rank += (t < tid) & (ct == c);
      after += (t > tid) & (ct == c);
    }
    if (c >= 0) mem[base[c] + rank] = j;
    __syncthreads();
    if (c >= 0 && after == 0) base[c] += rank + 1;
    __syncthreads();
  }
}

// centroid = mean of members in CSR order; 16 lanes per cluster, lane = dim
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

__global__ __launch_bounds__(NT) void select_clusters_kernel(SelectParams p) {
  __shared__ uint32_t keys[kMaxSelCand];
  __shared__ float qs[kBlock * R];
  __shared__ int hist[256];
  __shared__ int tmp4[4];
  __shared__ int bcast[2];
  const int b = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int g = p.group_of_ret[t];
  const int qs0 = b * kBlock;
  const int nrow = min(kBlock, p.N - qs0);
  const int lim = qs0 + nrow - 1 - p.window;
  int32_t* out = p.sel + ((size_t)t * p.n_qb + b) * p.topk;
  if (p.topk == 0) return;
  for (int x = tid; x < nrow * R; x += NT) qs[x] = p.qlow[((size_t)t * p.N + qs0) * R + x];
  __syncthreads();
  const int32_t* off = p.csr_off + (size_t)g * (p.M + 1);
  const int32_t* mem = p.csr_mem + (size_t)g * p.N;
  const float* C = p.cent + (size_t)g * p.M * R;
  int n_el = 0;
  for (int m = tid; m < p.M; m += NT) {
    const int lo = off[m], hi = off[m + 1];
    const bool el = lim >= 0 && hi > lo && mem[lo] <= lim;
    uint32_t key = 0u;
    if (el) {
      float c[R];
#pragma unroll
      for (int r = 0; r < R; r += 4) {
        const float4 v = *reinterpret_cast<const float4*>(C + (size_t)m * R + r);
        c[r] = v.x; c[r + 1] = v.y; c[r + 2] = v.z; c[r + 3] = v.w;
      }
      float mx = -__builtin_inff();
      for (int i = 0; i < nrow; ++i) {
        float dot = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) dot = fmaf(qs[i * R + r], c[r], dot);
        mx = fmaxf(mx, dot);
      }
      key = dev::order_key(mx);
      ++n_el;
    }
    keys[m] = key;
  }
  int nE;
  dev::block_excl_scan(n_el, tmp4, &nE);
  __syncthreads();
  // ineligible clusters hold key 0, below every real score's key, so the
  // k = min(topk, nE) largest keys are eligible clusters only.
  dev::topk_select(keys, p.M, min(p.topk, nE), p.topk, 0, out, hist, tmp4, bcast);
}

}  // namespace

size_t kmeans_scratch_bytes(int N, int M, int Hkv) {
  const size_t n_chunks = (size_t)(N + kChunk - 1) / kChunk;
  return (size_t)Hkv * n_chunks * M * sizeof(int32_t) + (size_t)Hkv * M * sizeof(int32_t);
}

hipError_t launch_kmeans(KmeansParams p, int Hkv, int iters, hipStream_t s) {
  p.n_chunks = (p.N + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(km_init_kernel, dim3((p.M * R + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
  hipError_t e = hipGetLastError();
  for (int it = 0; it < iters && e == hipSuccess; ++it) {
    hipLaunchKernelGGL(km_assign_kernel, dim3((p.N + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_hist_kernel, dim3(p.n_chunks, Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_colscan_kernel, dim3((p.M + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_offsets_kernel, dim3(Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_scatter_kernel, dim3(p.n_chunks, Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_update_kernel, dim3((p.M + (NT / R) - 1) / (NT / R), Hkv), dim3(NT), 0, s, p);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_select_clusters(const SelectParams& p, hipStream_t s) {
  if (p.n_ret == 0 || p.n_qb == 0) return hipSuccess;
  hipLaunchKernelGGL(select_clusters_kernel, dim3(p.n_qb, p.n_ret), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace ha
