// Low-rank indexer on gfx950: projection to r = 16 and per-query-block top-k
// selection of key blocks.
//
// RTPurboV2 article, low-rank projector passage: query and key are mapped
// from D to r = 16 by a projector that keeps the low-frequency components.
// RTPurbo post: the 16-dim indexer scouts candidate keys; exact attention then
// runs on them.  TriangleMix interview (top-k matching): keys are grouped in
// blocks, scored, and the top-k blocks kept.
//
// Block score: s_{b,c} = max over causal pairs (i in query block b, j in key
// block c, j <= i) of qlow_i . klow_j, over the eligible blocks
// c >= force_block0 with c*64 <= qe_b - window.  Selection keeps the topk best
// by (score desc, block asc): an exact radix select on the order-preserving
// integer image of the fp32 score, ties resolved by block index.
#include "common.h"
#include "device_util.h"

#include <limits.h>

namespace ha {
namespace {

constexpr int D = kHeadDim;
constexpr int R = kRank;
constexpr int NT = 256;

// ---------------------------------------------------------------------------
// Projection: one 16-lane group per row; lane part p holds d in [8p, 8p+8),
// computes 16 partial outputs, then a 4-step reduce-scatter leaves output r
// in lane r of the group.  HBM-bound: 256 B read, 64 B written per row.
__global__ __launch_bounds__(NT) void project_kernel(ProjParams p) {
  __shared__ float Ps[D * R];
  const int e = blockIdx.y;
  const int grp = p.group[e], head = p.head[e];
  for (int x = threadIdx.x; x < D * R; x += NT) Ps[x] = p.P[(size_t)grp * D * R + x];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = lane & 15;
  const int i = blockIdx.x * 16 + wave * 4 + (lane >> 4);
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  if (i < p.N) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p.X + ((size_t)i * p.H + head) * D + part * 8);
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const uint32_t bits = (dd & 1) ? (w4[dd >> 1] & 0xFFFF0000u) : (w4[dd >> 1] << 16);
      const float x = __uint_as_float(bits);
      const float* prow = Ps + (part * 8 + dd) * R;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = fmaf(x, prow[r], acc[r]);
    }
  }
#pragma unroll
  for (int step = 8; step >= 1; step >>= 1) {
    const bool hi = (lane & step) != 0;
#pragma unroll
    for (int j = 0; j < step; ++j) {
      const float keep = hi ? acc[step + j] : acc[j];
      const float give = hi ? acc[j] : acc[step + j];
      acc[j] = keep + __shfl_xor(give, step);
    }
  }
  if (i < p.N) p.out[((size_t)e * p.N + i) * R + part] = acc[0];
}

// One workgroup per (retrieval head, query block).  Wave w scores the
// eligible blocks c = c_lo + w, c_lo + w + 4, ...; each lane holds one query
// row's low-rank vector, keys are read wave-uniformly.
__global__ __launch_bounds__(NT) void select_blocks_kernel(SelectParams p) {
  __shared__ uint32_t keys[kMaxSelCand];
  __shared__ int hist[256];
  __shared__ int tmp4[4];
  __shared__ int bcast[2];
  const int b = blockIdx.x, t = blockIdx.y;
  const int g = p.group_of_ret[t];
  const int qs = b * kBlock;
  const int qe = min(p.N, qs + kBlock) - 1;
  const int c_lo = p.force_block0 ? 1 : 0;
  const int c_hi = (qe - p.window >= 0) ? (qe - p.window) / kBlock : -1;
  const int nE = max(0, c_hi - c_lo + 1);
  int32_t* out = p.sel + ((size_t)t * p.n_qb + b) * p.topk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (p.topk == 0) return;
  if (nE <= p.topk) {
    for (int x = tid; x < p.topk; x += NT) out[x] = x < nE ? c_lo + x : -1;
    return;
  }
  const int i = qs + lane;
  const bool row_ok = i < p.N;
  float q[R];
  {
    const float* qp = p.qlow + ((size_t)t * p.N + (row_ok ? i : qs)) * R;
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      const float4 v = *reinterpret_cast<const float4*>(qp + r);
      q[r] = v.x; q[r + 1] = v.y; q[r + 2] = v.z; q[r + 3] = v.w;
    }
  }
  const float* kbase = p.klow + (size_t)g * p.N * R;
  for (int x = wave; x < nE; x += 4) {
    const int c = c_lo + x;
    const int j0 = c * kBlock;
    const int nj = min(kBlock, p.N - j0);
    float mx = -__builtin_inff();
    for (int jj = 0; jj < nj; ++jj) {
      const float* kp = kbase + (size_t)(j0 + jj) * R;
      float dot = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) dot = fmaf(q[r], kp[r], dot);
      if (row_ok && j0 + jj <= i) mx = fmaxf(mx, dot);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) keys[x] = dev::order_key(mx);
  }
  __syncthreads();
  dev::topk_select(keys, nE, p.topk, p.topk, c_lo, out, hist, tmp4, bcast);
}

}  // namespace

hipError_t launch_project(const ProjParams& p, hipStream_t s) {
  if (p.n_entries == 0 || p.N == 0) return hipSuccess;
  hipLaunchKernelGGL(project_kernel, dim3((p.N + 15) / 16, p.n_entries), dim3(NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_select_blocks(const SelectParams& p, hipStream_t s) {
  if (p.n_ret == 0 || p.n_qb == 0) return hipSuccess;
  hipLaunchKernelGGL(select_blocks_kernel, dim3(p.n_qb, p.n_ret), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace ha
