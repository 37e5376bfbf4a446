// Device helpers shared by the selection kernels (256-thread workgroups).
#pragma once

#include "common.h"

namespace ha {
namespace dev {

constexpr int kNT = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
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

// Reductions over a lane pair (l, l ^ 32) or (l, l ^ 16) with the gfx950
// lane-swap instructions: VALU only, no LDS round trip.  With both operands
// equal, permlane32_swap returns (v[l % 32], v[32 + l % 32]) in lane l and
// permlane16_swap returns (v[l & ~16], v[l | 16]), so both lanes of a pair
// combine the same two values in the same order.
// The value lane l ^ 32 holds: the swap returns the pair's two values, and
// one of them is this lane's own.
__device__ __forceinline__ uint32_t pair32_other(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return r[0] ^ r[1] ^ v;
}
__device__ __forceinline__ float pair32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp16 parts: x = hi + lo to ~2^-22 relative (11 + 11 mantissa bits) for
// |x| well inside the fp16 range; three MFMA passes (hi*hi, hi*lo, lo*hi)
// give dots to ~2^-21 of |a||b|.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void split2_f16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}
__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over the workgroup's threads in thread order;
// *total = sum.  NW = waves in the workgroup; tmp holds NW ints.
template <int NW = 4>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) base += tmp[w];
    tot += tmp[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Word 3 of a raw buffer resource on gfx9 parts (gfx950 included): 32-bit
// data format, no swizzle.  Offsets at or past num_records read zeros.
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The float an order key was made from.
__device__ __forceinline__ float key_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

constexpr int kHistCopies = 8;            // histogram replicas (cuts same-bin atomic conflicts)
constexpr int kHistStride = 257;          // words between replicas (different banks)
constexpr int kHistWords = kHistCopies * kHistStride;

// Exact top-k over keys[0..n) (order-preserving uint32 images of the scores),
// larger key first, lower index first among equal keys.  Writes the chosen
// indices + id_base in ascending order to out[0..k), -1 in out[k..topk)
// (with idmap, idmap[x] replaces x + id_base; idmap must be increasing).
// Radix select on 8-bit digits: per pass, a histogram of the keys that match
// the digits found so far (8 lane-strided replicas, so lanes with equal
// digits mostly hit different words), then one wave finds the digit where
// the count from the top reaches k.  hist needs kHistWords ints.
// The radix passes of topk_select alone: the k-th largest of keys[0..n)
// (1 <= k <= n); *need_out = how many keys equal to it are among the k.
__device__ inline uint32_t radix_kth(const uint32_t* keys, int n, int k, int* hist, int* bcast, int* need_out) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0, pmask = 0;
  int need = k;
  int* myhist = hist + (lane & (kHistCopies - 1)) * kHistStride;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int x = tid; x < kHistWords; x += kNT) hist[x] = 0;
    __syncthreads();
    for (int x = tid; x < n; x += kNT) {
      const uint32_t u = keys[x];
      if ((u & pmask) == prefix) atomicAdd(&myhist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 4l .. 4l+3; merge the replicas, then a suffix scan
      // over lanes (from digit 255 down) finds the digit d* where the count of
      // keys with digit > d* is < need <= count with digit >= d*
      int c[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int v = 0;
#pragma unroll
        for (int r = 0; r < kHistCopies; ++r) v += hist[r * kHistStride + lane * 4 + q];
        c[q] = v;
      }
      const int tot = c[0] + c[1] + c[2] + c[3];
      // inclusive suffix sum over lanes >= lane
      int suf = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_down(suf, o);
        if (lane + o < 64) suf += t;
      }
      const int above = suf - tot;            // keys with digits in lanes > lane
      // the owning lane: above < need <= suf
      if (above < need && need <= suf) {
        int cum = above, dstar = lane * 4;
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (cum + c[q] >= need) {
            dstar = lane * 4 + q;
            break;
          }
          cum += c[q];
        }
        bcast[0] = dstar;
        bcast[1] = need - cum;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)bcast[0] << shift;
    pmask |= 255u << shift;
    need = bcast[1];
    __syncthreads();
  }
  *need_out = need;
  return prefix;
}

__device__ inline void topk_select(const uint32_t* keys, int n, int k, int topk, int id_base, int32_t* out,
                                   int* hist, int* tmp4, int* bcast, const uint16_t* idmap = nullptr,
                                   uint32_t* out_keys = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (k > n) k = n;
  if (k <= 0) {
    for (int x = tid; x < topk; x += kNT) out[x] = -1;
    return;
  }
  int need;
  const uint32_t prefix = radix_kth(keys, n, k, hist, bcast, &need);
  // prefix is the k-th largest key; take every key above it and the first
  // `need` keys equal to it in index order.  Wave w scans a contiguous quarter
  // of the index range in rounds of 64 consecutive keys (lane = offset);
  // ranks among ties and output positions come from ballots.
  const int wave = tid >> 6;
  const int per_wave = ((n + 4 * 64 - 1) / (4 * 64)) * 64;
  const int wa = min(n, wave * per_wave), wb = min(n, wa + per_wave);
  int gt = 0, eq = 0;
  for (int x0 = wa; x0 < wb; x0 += 64) {
    const int x = x0 + lane;
    const uint32_t u = x < wb ? keys[x] : 0u;
    gt += (int)__popcll(__ballot(x < wb && u > prefix));
    eq += (int)__popcll(__ballot(x < wb && u == prefix));
  }
  if (lane == 0) {
    tmp4[wave] = eq;
    tmp4[4 + wave] = gt;
  }
  __syncthreads();
  int tie_run = 0, pos_run = 0;
  for (int w = 0; w < wave; ++w) {
    const int eqw = tmp4[w], gtw = tmp4[4 + w];
    pos_run += gtw + max(0, min(need - tie_run, eqw));
    tie_run += eqw;
  }
  for (int x0 = wa; x0 < wb; x0 += 64) {
    const int x = x0 + lane;
    const uint32_t u = x < wb ? keys[x] : 0u;
    const bool is_tie = x < wb && u == prefix;
    const uint64_t tb = __ballot(is_tie);
    const int tie_rank = tie_run + (int)__popcll(tb & ((1ull << lane) - 1ull));
    const bool take = x < wb && (u > prefix || (is_tie && tie_rank < need));
    const uint64_t kb = __ballot(take);
    if (take) {
      const int pos = pos_run + (int)__popcll(kb & ((1ull << lane) - 1ull));
      out[pos] = idmap ? (int)idmap[x] : id_base + x;
      if (out_keys) out_keys[pos] = u;
    }
    tie_run += (int)__popcll(tb);
    pos_run += (int)__popcll(kb);
  }
  __syncthreads();
  for (int x = k + tid; x < topk; x += kNT) out[x] = -1;
}

// Adaptive budget (a proposal for the RTPurboV2 article's point that heads,
// lengths and queries need different numbers of tokens): row[0..k) holds the
// top-k ids in ascending order and rkeys[0..k) their order keys (k <= kNT).
// Keeps the shortest prefix, in (score desc, id asc) order, whose share of
// sum exp(scale * s) over the k reaches `mass`, and rewrites row[0..topk)
// ascending with -1 padding.  scale_log2 = scale * log2(e).  wrank needs kNT
// floats, tmp 8 ints, bcast 2 ints; called by all kNT threads.
__device__ inline void adaptive_cut(int32_t* row, const uint32_t* rkeys, int k, int topk, float scale_log2,
                                    float mass, float* wrank, int* tmp, int* bcast) {
  const int tid = threadIdx.x, lane = tid & 63;
  int rank = 0, id = -1;
  uint32_t key = 0u;
  if (tid < k) {
    key = rkeys[tid];
    id = row[tid];
    for (int j = 0; j < k; ++j) {
      const uint32_t kj = rkeys[j];
      rank += (kj > key) | ((kj == key) & (j < tid));   // ids ascend with j
    }
    if (rank == 0) bcast[0] = (int)key;
  }
  __syncthreads();
  const float s0 = key_value((uint32_t)bcast[0]);
  if (tid < k) wrank[rank] = exp2f((key_value(key) - s0) * scale_log2);
  __syncthreads();
  // inclusive prefix sums in rank order: one wave, four ranks per lane
  if (tid < 64) {
    float v[4];
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * lane + e;
      run += r < k ? wrank[r] : 0.f;
      v[e] = run;
    }
    float inc = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    const float base = inc - run;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * lane + e < k) wrank[4 * lane + e] = base + v[e];
  }
  __syncthreads();
  const float thr = mass * wrank[k - 1];
  if (tid < k) {
    const bool hit = wrank[tid] >= thr && (tid == 0 || wrank[tid - 1] < thr);
    if (hit) bcast[1] = tid + 1;
  }
  __syncthreads();
  const int n = bcast[1];
  const bool keep = tid < k && rank < n;
  int kept;
  const int pos = block_excl_scan((int)keep, tmp, &kept);   // (synchronizes)
  __syncthreads();
  if (keep) row[pos] = id;
  for (int x = kept + tid; x < topk; x += kNT) row[x] = -1;
  __syncthreads();
}

}  // namespace dev
}  // namespace ha
