// Device helpers shared by the selection kernels (256-thread workgroups).
#pragma once

#include "common.h"

namespace ha {
namespace dev {

constexpr int kNT = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp32 x = hi + lo (+ rest) with hi, lo bf16: hi = rn(x), lo = rn(x - hi).
// Products of split operands reproduce fp32 dot products to ~1e-5 relative
// with three MFMA passes (hi*hi + hi*lo + lo*hi).
__device__ __forceinline__ void split2(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// Three bf16 parts: x = hi + mid + lo to ~2^-24 relative; six MFMA passes
// (hi*hi, hi*mid, mid*hi, mid*mid, hi*lo, lo*hi) give fp32-accurate dots.
__device__ __forceinline__ void split3(float x, __bf16& hi, __bf16& mid, __bf16& lo) {
  hi = (__bf16)x;
  const float r = x - (float)hi;
  mid = (__bf16)r;
  lo = (__bf16)(r - (float)mid);
}

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
