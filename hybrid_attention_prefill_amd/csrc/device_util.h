// Device helpers shared by the selection kernels (256-thread workgroups).
#pragma once

#include "common.h"

namespace ha {
namespace dev {

constexpr int kNT = 256;

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over the 256 threads in thread order; *total = sum.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp4, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) tmp4[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) base += tmp4[w];
    tot += tmp4[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exact top-k over keys[0..n) (order-preserving uint32 images of the scores),
// larger key first, lower index first among equal keys.  Writes the chosen
// indices + id_base in ascending order to out[0..k), -1 in out[k..topk).
__device__ inline void topk_select(const uint32_t* keys, int n, int k, int topk, int id_base, int32_t* out,
                            int* hist, int* tmp4, int* bcast) {
  const int tid = threadIdx.x;
  if (k > n) k = n;
  if (k <= 0) {
    for (int x = tid; x < topk; x += kNT) out[x] = -1;
    return;
  }
  uint32_t prefix = 0, pmask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int x = tid; x < n; x += kNT) {
      const uint32_t u = keys[x];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, dstar = 0;
      for (int d = 255; d >= 0; --d) {
        if (cum + hist[d] >= need) {
          dstar = d;
          break;
        }
        cum += hist[d];
      }
      bcast[0] = dstar;
      bcast[1] = need - cum;
    }
    __syncthreads();
    prefix |= (uint32_t)bcast[0] << shift;
    pmask |= 255u << shift;
    need = bcast[1];
    __syncthreads();
  }
  // prefix is the k-th largest key; take every key above it and the first
  // `need` keys equal to it in index order.
  const int chunk = (n + kNT - 1) / kNT;
  const int a = min(n, tid * chunk), b = min(n, a + chunk);
  int ties = 0;
  for (int x = a; x < b; ++x) ties += keys[x] == prefix;
  int tot;
  int tie_base = block_excl_scan(ties, tmp4, &tot);
  int chosen = 0;
  {
    int tr = tie_base;
    for (int x = a; x < b; ++x) {
      const uint32_t u = keys[x];
      if (u > prefix) ++chosen;
      else if (u == prefix) { if (tr < need) ++chosen; ++tr; }
    }
  }
  int pos = block_excl_scan(chosen, tmp4, &tot);
  {
    int tr = tie_base;
    for (int x = a; x < b; ++x) {
      const uint32_t u = keys[x];
      bool take = false;
      if (u > prefix) take = true;
      else if (u == prefix) { take = tr < need; ++tr; }
      if (take) out[pos++] = id_base + x;
    }
  }
  for (int x = k + tid; x < topk; x += kNT) out[x] = -1;
}

}  // namespace dev
}  // namespace ha
