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
//   assign   one lane per key, centroid tiles in LDS, d = |C|^2 - 2 k.C on MFMA:
//            one fp16 product pass decides every key whose two best
//            distances lie further apart than the pass's error bound; the
//            others get the exact three-product pass
//   CSR      stable counting sort of key positions by cluster: per-chunk
//            histograms, a column scan, then an in-order scatter (ranks among
//            equal clusters inside a 256-key batch come from an LDS scan)
//   update   per cluster, the members' sum in CSR (position) order / count
#include "common.h"
#include "device_util.h"

#include <limits.h>

#include <algorithm>
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
  if (blockIdx.x == 0 && threadIdx.x == 0) p.amax[g] = 0u;
  if (x >= p.M * R) return;
  const int m = x / R, r = x % R;
  p.cent[((size_t)g * p.M + m) * R + r] = p.klow[((size_t)g * p.N + (size_t)m * p.stride) * R + r];
}

// Largest |component| of each KV head's low-rank keys, as fp32 bits (for a
// non-negative float the bit pattern orders as the value): grid-stride
// float4 reads, a wave maximum, one atomic per wave.
constexpr int kAmaxBlocks = 512;
__global__ __launch_bounds__(NT) void km_amax_kernel(KmeansParams p) {
  const int g = blockIdx.y;
  const float4* src = reinterpret_cast<const float4*>(p.klow + (size_t)g * p.N * R);
  const size_t n4 = (size_t)p.N * R / 4;
  uint32_t m = 0u;
  for (size_t x = (size_t)blockIdx.x * NT + threadIdx.x; x < n4; x += (size_t)gridDim.x * NT) {
    const float4 v = src[x];
    m = max(m, max(max(__float_as_uint(fabsf(v.x)), __float_as_uint(fabsf(v.y))),
                   max(__float_as_uint(fabsf(v.z)), __float_as_uint(fabsf(v.w)))));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if ((threadIdx.x & 63) == 0) atomicMax(&p.amax[g], m);
}

// Power of two that brings the KV head's largest key component into
// [2^9, 2^10): keys and centroids are multiplied by it before the fp16
// split, so the split neither overflows (fp16 max 65504) nor falls into the
// fp16 subnormals, whatever the keys' range.  Multiplying by a power of two
// is exact and scales every distance by the same factor, so the argmin is
// unchanged.  The exponent is clamped to fp32's normal range.
__device__ __forceinline__ float key_scale(uint32_t amax_bits) {
  const int e_max = (int)((amax_bits >> 23) & 0xFFu) - 127;
  const int e = min(127, max(-126, 9 - e_max));
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

// Per iteration: centroids (times the KV head's key scale) split into two
// fp16 parts and their squared norms, for the MFMA distance pass.
// The largest scaled squared norm goes to cmax and the largest squared norm
// of the lo parts to almax (wave maxima, one atomic per wave; both start at
// zero, km_clear_kernel).
__global__ __launch_bounds__(NT) void km_prep_kernel(KmeansParams p) {
  const int g = blockIdx.y;
  const int m = blockIdx.x * NT + threadIdx.x;
  float nrm = 0.f, lnrm = 0.f;
  if (m < p.M) {
    const float sc = key_scale(p.amax[g]);
    const size_t o = ((size_t)g * p.M + m) * R;
    const float* c = p.cent + o;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = c[r] * sc;
      nrm = fmaf(v, v, nrm);
      _Float16 h, l;
      dev::split2_f16(v, h, l);
      p.c_hi[o + r] = h;
      p.c_lo[o + r] = l;
      lnrm = fmaf((float)l, (float)l, lnrm);
    }
    p.c_norm[(size_t)g * p.M + m] = nrm;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    nrm = fmaxf(nrm, __shfl_xor(nrm, o));
    lnrm = fmaxf(lnrm, __shfl_xor(lnrm, o));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMax(&p.cmax[g], __float_as_uint(nrm));
    atomicMax(&p.almax[g], __float_as_uint(lnrm));
  }
}

// Per iteration, before km_prep: the per-head maximum and the count of
// undecided keys start at zero.
__global__ void km_clear_kernel(KmeansParams p, int Hkv) {
  if ((int)threadIdx.x < Hkv) {
    p.cmax[threadIdx.x] = 0u;
    p.almax[threadIdx.x] = 0u;
    p.n_amb[threadIdx.x] = 0u;
  }
}

// Exact assignment: each wave owns 32*KT keys (KT column blocks of 32), the
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
// enter the split multiplied by the KV head's power-of-two key scale
// (key_scale), so every component lies below 2^10 in magnitude.
constexpr int kCChunk = 256;      // centroids per LDS chunk
constexpr int kCStr = 24;         // 16-bit row stride of a staged part (48 B: conflict-free 16-B reads)
constexpr int KT = 4;             // 32-key blocks per wave
constexpr float kPadNorm = 1e30f; // norm of the padding rows of a partial tile

// It scores the keys the approximate pass (km_assign_approx_kernel) left
// undecided, p.amb[g][0 .. p.n_amb[g]), against one of kExactSplit ranges of
// centroids (blockIdx.z; few keys are undecided, so the ranges spread them
// over the chip): per key the range's minimum and its index, lowest index on
// equal distances, go into p.best[g][slot] by a 64-bit atomic minimum of
// (order key of the distance, index), which keeps the lowest index of the
// overall minimum whatever the ranges' order; km_assign_commit_kernel writes
// them out.  Workgroups step over the key blocks, so the grid needs no
// count of them.
constexpr int kExactSplit = 8;
constexpr int kExactBlocks = 128;  // workgroups per KV head and range (at most)
__device__ __forceinline__ uint32_t order_key(float d) {
  const uint32_t u = __float_as_uint(d);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__global__ __launch_bounds__(NT) void km_assign_exact_kernel(KmeansParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t cs[2][kCChunk * kCStr];
  __shared__ __attribute__((aligned(16))) float cns[kCChunk];   // |C_m|^2 of the staged centroids
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int n_keys = (int)p.n_amb[g];
  const int span = ((p.M + kExactSplit - 1) / kExactSplit + 31) / 32 * 32;
  const int c_lo = (int)blockIdx.z * span, c_hi = min(p.M, c_lo + span);
  if (c_lo >= c_hi) return;
  const float ksc = -2.f * key_scale(p.amax[g]);
  for (int kb = blockIdx.x; kb * 4 * 32 * KT < n_keys; kb += gridDim.x) {
  const int j0 = (kb * 4 + wave) * (32 * KT);
  // key of slot i (slots past the count repeat the last key and write nothing)
  auto key_of = [&](int i) { return (int)p.amb[(size_t)g * p.N + min(n_keys - 1, i)]; };
  dev::f16x8 kh[KT], kl[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int j = key_of(j0 + kt * 32 + lr);
    const float* kp = p.klow + ((size_t)g * p.N + j) * R + lh * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      _Float16 h, l;
      dev::split2_f16(ksc * kp[e], h, l);
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
  for (int c0 = c_lo; c0 < c_hi; c0 += kCChunk) {
    const int nc = min(kCChunk, c_hi - c0);
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
    const bool take = ob < best[kt] || (ob == best[kt] && oa < arg[kt]);
    const float b = take ? ob : best[kt];
    const int a = take ? oa : arg[kt];
    const int i = j0 + kt * 32 + lr;
    if (lh == 0 && i < n_keys)
      atomicMin(reinterpret_cast<unsigned long long*>(p.best + (size_t)g * p.N + i),
                ((unsigned long long)order_key(b) << 32) | (uint32_t)a);
  }
  }
}

// The undecided keys' assignments: the index half of p.best.
__global__ __launch_bounds__(NT) void km_assign_commit_kernel(KmeansParams p) {
  const int g = blockIdx.y;
  const int n_keys = (int)p.n_amb[g];
  for (int i = blockIdx.x * NT + threadIdx.x; i < n_keys; i += gridDim.x * NT)
    p.assign[(size_t)g * p.N + p.amb[(size_t)g * p.N + i]] = (int32_t)(uint32_t)p.best[(size_t)g * p.N + i];
}

// Approximate assignment with certification; the exact kernel above defines
// the result.  One fp16 product per (key, centroid), ah * kh, gives
//   d~ = |C'|^2 + k' . C'      (C' = s C, k' = -2 s k, s the key scale)
// within eps of the three-product value the exact kernel compares, where
//   eps = 1.002 (max|al| |k'| + max|C'| |kl|) + 2^-17 (max|C'|^2 + |k'| max|C'|)
//         + 2^-10 (|k'| + max|C'|)
// (al, kl: the lo parts the exact kernel uses; by Cauchy-Schwarz the dropped
// al . kh + ah . kl are at most |al| |kh| + |ah| |kl|, and |kh| <= |k'|
// (1 + 2^-11), |ah| <= |C'| (1 + 2^-11); fp32 accumulation of up to 64
// terms plus the recompute below, 2^-17 of the magnitudes; fp16 subnormals
// and flushes cost at most 2^-14 per component, under the last term).  Per key and lane
// half the pass keeps the smallest d~ (b1, in tile x1) and the second
// smallest tile minimum (b2: med3 of b1, b2 and the tile's minimum).  Then
// the lane recomputes its 16 values of tile x1 with fp32 dot products of the
// same fp16 operands (only the accumulation order differs) for the index of
// b1 (lowest on equal values) and the tile's second smallest value w2.  The
// halves merge into the winner I1 and the second smallest value B2 over all
// other centroids.  The winner's own three-product value dw (hi.hi + hi.lo +
// lo.hi over the exact kernel's fp16 parts, fp32 dot products) lies within
// tw = 2^-17 (max|C'|^2 + |k'| max|C'|) + 2^-10 (|k'| + max|C'|) of the
// exact kernel's value (another summation order, fp16 subnormal handling),
// and every other centroid's exact value is at least its approximate value
// minus eps; so when B2 - eps > dw + tw, I1 is the exact kernel's unique
// minimum and is written.  Otherwise the key is appended to p.amb (its
// p.best entry set to all ones) for the exact kernel (the list order
// varies; each key's result does not).
//
// The accumulator seed |C'_m|^2 comes from one more MFMA instead of 16 LDS
// floats per lane: the norm split into three bf16 parts (exact: 24 bits) in
// row m, k = 0..2 of a bf16 operand, times a column of ones, summed exactly
// in fp32, so the seed is the fp32 norm itself.
__global__ __launch_bounds__(NT, 4) void km_assign_approx_kernel(KmeansParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t cs[kCChunk * kCStr];
  __shared__ __attribute__((aligned(16))) uint16_t cs3[kCChunk * kCStr];   // norm parts, then zeros
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int j0 = (blockIdx.x * 4 + wave) * (32 * KT);
  const float ksc = -2.f * key_scale(p.amax[g]);
  // per key: the fp16 key and the certification bound eps (both lane halves)
  const float cmx = sqrtf(__uint_as_float(p.cmax[g])), alx = sqrtf(__uint_as_float(p.almax[g]));
  dev::f16x8 kh[KT];
  float eps[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int j = min(p.N - 1, j0 + kt * 32 + lr);
    const float* kp = p.klow + ((size_t)g * p.N + j) * R + lh * 8;
    float ss = 0.f, sl = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = ksc * kp[e];
      ss = fmaf(v, v, ss);
      _Float16 h, l;
      dev::split2_f16(v, h, l);
      kh[kt][e] = h;
      sl = fmaf((float)l, (float)l, sl);
    }
    const float kn = sqrtf(dev::pair32_sum(ss)), kln = sqrtf(dev::pair32_sum(sl));
    eps[kt] = 1.002f * (alx * kn + cmx * kln) + 0x1p-17f * (cmx * cmx + kn * cmx) + 0x1p-10f * (kn + cmx);
  }
  const __bf16 one = (__bf16)1.f, zero = (__bf16)0.f;
  const dev::bf16x8 ones3 = {one, one, one, zero, zero, zero, zero, zero};
  float b1[KT], b2[KT];
  int x1[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    b1[kt] = __builtin_inff();
    b2[kt] = __builtin_inff();
    x1[kt] = 0;
  }
  const _Float16* chi = p.c_hi + (size_t)g * p.M * R;
  const _Float16* clo = p.c_lo + (size_t)g * p.M * R;
  const float* cn = p.c_norm + (size_t)g * p.M;
  for (int c0 = 0; c0 < p.M; c0 += kCChunk) {
    const int nc = min(kCChunk, p.M - c0);
    __syncthreads();
    {
      // thread t stages centroid c0 + t: its hi part and its norm
      const int m = c0 + tid;
      const bool ok = tid < nc;
      const uint4* src = reinterpret_cast<const uint4*>(chi + (size_t)(ok ? m : c0) * R);
      const uint4 v0 = src[0], v1 = src[1];
      uint4* dst = reinterpret_cast<uint4*>(&cs[tid * kCStr]);
      dst[0] = v0;
      dst[1] = v1;
      __bf16 nh, nm, nl;
      dev::split3(ok ? cn[m] : kPadNorm, nh, nm, nl);
      const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, nh) | ((uint32_t)__builtin_bit_cast(uint16_t, nm) << 16);
      uint4* dn = reinterpret_cast<uint4*>(&cs3[tid * kCStr]);
      dn[0] = make_uint4(w0, (uint32_t)__builtin_bit_cast(uint16_t, nl), 0u, 0u);
      dn[1] = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    const int n_tiles = (nc + 31) / 32;
    for (int x = 0; x < n_tiles; ++x) {
      const int r0 = x * 32;
      const dev::f16x8 ah = *reinterpret_cast<const dev::f16x8*>(&cs[(r0 + lr) * kCStr + lh * 8]);
      const dev::bf16x8 a3 = *reinterpret_cast<const dev::bf16x8*>(&cs3[(r0 + lr) * kCStr + lh * 8]);
      const dev::f32x16 nv = dev::mfma32(a3, ones3, dev::f32x16{});
      dev::f32x16 acc[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) acc[kt] = dev::mfma32_f16(ah, kh[kt], nv);
      const int tile = (c0 + r0) >> 5;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        float tm = __builtin_inff();
#pragma unroll
        for (int e = 0; e < 16; e += 2) tm = __builtin_fminf(__builtin_fminf(tm, acc[kt][e]), acc[kt][e + 1]);
        const bool lt = tm < b1[kt];
        b2[kt] = __builtin_amdgcn_fmed3f(b1[kt], b2[kt], tm);
        x1[kt] = lt ? tile : x1[kt];
        b1[kt] = lt ? tm : b1[kt];
      }
      // the products first (separate accumulators), then their minima
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, KT + 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
    }
  }
  uint32_t* list = reinterpret_cast<uint32_t*>(p.amb) + (size_t)g * p.N;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    // the key's 16 components: this lane's 8 and the other half's
    const auto kw = __builtin_bit_cast(dev::u32x4, kh[kt]);
    dev::u32x4 ko;
#pragma unroll
    for (int q = 0; q < 4; ++q) ko[q] = dev::pair32_other(kw[q]);
    const dev::u32x4 klo = lh ? ko : kw, khi = lh ? kw : ko;
    // tile x1's 16 values of this lane, recomputed
    float w1 = __builtin_inff(), w2 = __builtin_inff();
    int i1 = 0;
    const int mb = x1[kt] * 32 + lh * 4;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = mb + (e >> 2) * 8 + (e & 3);
      if (m < p.M) {
        const dev::u32x4* cp = reinterpret_cast<const dev::u32x4*>(chi + (size_t)m * R);
        const dev::u32x4 c0v = cp[0], c1v = cp[1];
        float d = cn[m];
        // (vector elements are copied to scalars before the bit casts: a bit
        // cast of an element access reads element 0 with this compiler)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t ca = c0v[q], cb = c1v[q], ka = klo[q], kb = khi[q];
          d = __builtin_amdgcn_fdot2(__builtin_bit_cast(dev::f16x2, ca), __builtin_bit_cast(dev::f16x2, ka), d, false);
          d = __builtin_amdgcn_fdot2(__builtin_bit_cast(dev::f16x2, cb), __builtin_bit_cast(dev::f16x2, kb), d, false);
        }
        if (d < w1) {
          w2 = w1;
          w1 = d;
          i1 = m;
        } else {
          w2 = fminf(w2, d);
        }
      }
    }
    // merge the halves (lane lr and lr + 32 hold the same key)
    const float sb1 = b1[kt], sb2 = fminf(b2[kt], w2);
    const float ob1 = __uint_as_float(dev::pair32_other(__float_as_uint(sb1)));
    const float ob2 = __uint_as_float(dev::pair32_other(__float_as_uint(sb2)));
    const int oi1 = (int)dev::pair32_other((uint32_t)i1);
    const float B2 = fminf(fmaxf(sb1, ob1), fminf(sb2, ob2));
    const int I1 = (sb1 < ob1 || (sb1 == ob1 && i1 < oi1)) ? i1 : oi1;
    // the winner's three-product value (hi.hi + hi.lo + lo.hi over the same
    // fp16 parts as the exact kernel, fp32 dot products), each lane half
    // taking its 8 components
    const int j = j0 + kt * 32 + lr;
    float dw, kn;
    {
      const float* kp = p.klow + ((size_t)g * p.N + min(p.N - 1, j)) * R + lh * 8;
      dev::f16x8 kl8;
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = ksc * kp[e];
        ss = fmaf(v, v, ss);
        _Float16 h, l;
        dev::split2_f16(v, h, l);
        kl8[e] = l;
      }
      kn = sqrtf(dev::pair32_sum(ss));
      const dev::u32x4 klw = __builtin_bit_cast(dev::u32x4, kl8);
      const dev::u32x4 chw = *reinterpret_cast<const dev::u32x4*>(chi + (size_t)I1 * R + lh * 8);
      const dev::u32x4 clw = *reinterpret_cast<const dev::u32x4*>(clo + (size_t)I1 * R + lh * 8);
      float part = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t a = chw[q], b = clw[q], x = kw[q], y = klw[q];
        part = __builtin_amdgcn_fdot2(__builtin_bit_cast(dev::f16x2, a), __builtin_bit_cast(dev::f16x2, x), part, false);
        part = __builtin_amdgcn_fdot2(__builtin_bit_cast(dev::f16x2, a), __builtin_bit_cast(dev::f16x2, y), part, false);
        part = __builtin_amdgcn_fdot2(__builtin_bit_cast(dev::f16x2, b), __builtin_bit_cast(dev::f16x2, x), part, false);
      }
      const float other = __uint_as_float(dev::pair32_other(__float_as_uint(part)));
      dw = cn[I1] + (lh ? other + part : part + other);
    }
    // every other centroid's approximate value is within eps of its exact
    // one, and dw within tw of the winner's exact value (the same terms in
    // another fp32 order, and fp16 subnormal handling): if the second
    // smallest approximate value, lowered by eps, still exceeds dw + tw,
    // the winner is the exact kernel's unique minimum
    const float tw = 0x1p-17f * (cmx * cmx + kn * cmx) + 0x1p-10f * (kn + cmx);
    const bool cert = B2 - eps[kt] > dw + tw;
    const bool mine = lh == 0 && j < p.N;
    if (mine && cert) p.assign[(size_t)g * p.N + j] = I1;
    // undecided keys: one atomic per wave, slots in lane order
    const bool amb = mine && !cert;
    const uint64_t bal = __ballot(amb);
    if (bal != 0ull) {
      uint32_t base = 0u;
      if (lane == 0) base = atomicAdd(&p.n_amb[g], (uint32_t)__popcll(bal));
      base = __shfl(base, 0);
      if (amb) {
        const uint32_t slot = base + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
        list[slot] = (uint32_t)j;
        p.best[(size_t)g * p.N + slot] = ~0ull;
      }
    }
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
  int c = 0;
  // eight chunks' counts in flight at a time
  for (; c + 8 <= p.n_chunks; c += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = col[(size_t)(c + u) * p.M];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      col[(size_t)(c + u) * p.M] = run;
      run += v[u];
    }
  }
  for (; c < p.n_chunks; ++c) {
    const int v = col[(size_t)c * p.M];
    col[(size_t)c * p.M] = run;
    run += v;
  }
  p.count[(size_t)g * p.M + m] = run;
}

// offsets: exclusive scan of the counts over clusters (one workgroup per KV
// head): each thread sums a contiguous run of counts, a workgroup scan of
// the sums gives every run's start, and the run is written out
__global__ __launch_bounds__(NT) void km_offsets_kernel(KmeansParams p) {
  __shared__ int tmp[NT / 64];
  const int g = blockIdx.x, tid = threadIdx.x;
  const int per = (p.M + NT - 1) / NT;
  const int a = min(p.M, tid * per), b = min(p.M, a + per);
  const int32_t* cnt = p.count + (size_t)g * p.M;
  int s = 0;
  int m = a;
  for (; m + 8 <= b; m += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = cnt[m + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; m < b; ++m) s += cnt[m];
  int total;
  const int base = dev::block_excl_scan<NT / 64>(s, tmp, &total);
  int32_t* off = p.csr_off + (size_t)g * (p.M + 1);
  int run = base;
  m = a;
  for (; m + 8 <= b; m += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = cnt[m + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      off[m + u] = run;
      run += v[u];
    }
  }
  for (; m < b; ++m) {
    off[m] = run;
    run += cnt[m];
  }
  if (tid == 0) off[p.M] = total;
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
  // the chunk's assignments, all loads in flight at once (thread t holds
  // positions a + t + NT i)
  constexpr int kPer = kChunk / NT;
  int cl[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = a + tid + NT * i;
    cl[i] = j < b ? as[j] : -1;
  }
  // Keys in position order, NT at a time.  In each round the lowest thread
  // still holding a key of cluster c (the earliest position) takes c's next
  // slot, so every cluster's members stay in ascending position; a round
  // places one key per distinct cluster, and a batch rarely holds the same
  // cluster twice.
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = a + tid + NT * i;
    const int c = cl[i];
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
  int x = lo;
  // eight members' loads in flight, added in member order
  for (; x + 8 <= hi; x += 8) {
    int j[8];
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) j[u] = mem[x + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = kl[(size_t)j[u] * R + r];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; x < hi; ++x) s += kl[(size_t)mem[x] * R + r];
  p.cent[((size_t)g * p.M + m) * R + r] = s / (float)(hi - lo);
}

// ---------------------------------------------------------------------------
// cluster selection: eligible clusters have a member j <= qe - window (the
// first CSR member is the smallest position); score = max over the query
// block's rows of qlow_i . C_m; the topk best by (score desc, cluster asc).

// Largest candidate-vector norm of a KV head (fp32 bits; a non-negative
// float orders as its bits): per wave the max of the lanes' squared norms,
// one atomic per wave (a NaN norm counts as +inf).  The counters start at
// zero (sel_clear_kernel).
__device__ __forceinline__ void cnorm_max(uint32_t* cnorm, float n2) {
  if (n2 != n2) n2 = __builtin_inff();   // a NaN component makes the bound infinite
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) n2 = fmaxf(n2, __shfl_xor(n2, o));
  if ((threadIdx.x & 63) == 0) atomicMax(cnorm, __float_as_uint(sqrtf(n2)));
}

__global__ void sel_clear_kernel(uint32_t* w, int n) {
  if ((int)threadIdx.x < n) w[threadIdx.x] = 0u;
}

// Per layer, once: centroids split into bf16 hi/lo parts, the first
// (smallest) member position of every cluster (INT_MAX when empty) and the
// largest centroid norm.
__global__ __launch_bounds__(NT) void cluster_prep_kernel(SelectParams p) {
  const int g = blockIdx.y;
  const int m = blockIdx.x * NT + threadIdx.x;
  float n2 = 0.f;
  if (m < p.M) {
    const float* c = p.cent + ((size_t)g * p.M + m) * R;
    __bf16* hi = p.c_hi + ((size_t)g * p.M + m) * R;
    __bf16* lo = p.c_lo + ((size_t)g * p.M + m) * R;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = c[r];
      n2 = fmaf(v, v, n2);
      dev::split2(v, hi[r], lo[r]);
    }
    const int32_t* off = p.csr_off + (size_t)g * (p.M + 1);
    const int lo_i = off[m], hi_i = off[m + 1];
    p.first_mem[(size_t)g * p.M + m] = hi_i > lo_i ? p.csr_mem[(size_t)g * p.N + lo_i] : INT_MAX;
  }
  cnorm_max(p.cnorm + g, n2);
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
  float n2 = 0.f;
  if (c < p.M) {
    const int j0 = c * kBlock, j1 = min(p.N, j0 + kBlock);
    const float* kl = p.klow + (size_t)g * p.N * R + d;
    __bf16* hi = p.c_hi + ((size_t)g * p.M + c) * R * NPART;
    __bf16* lo = p.c_lo + ((size_t)g * p.M + c) * R * NPART;
    if (NPART == 1) {
      float s = 0.f;
      for (int j = j0; j < j1; ++j) s += kl[(size_t)j * R];
      const float v = s / (float)(j1 - j0);
      n2 = v * v;
      dev::split2(v, hi[d], lo[d]);
    } else {
      float a = -__builtin_inff(), b = __builtin_inff();
      for (int j = j0; j < j1; ++j) {
        const float v = kl[(size_t)j * R];
        a = fmaxf(a, v);
        b = fminf(b, v);
      }
      n2 = fmaf(a, a, b * b);
      dev::split2(a, hi[d], lo[d]);
      dev::split2(b, hi[R + d], lo[R + d]);
    }
    if (d == 0) p.first_mem[(size_t)g * p.M + c] = (p.force_block0 && c == 0) ? INT_MAX : j0;
  }
  // the R threads of a block are consecutive lanes: their sum is the block's
  // squared norm (NPART 2: of the 2R-vector of maxima and minima)
#pragma unroll
  for (int o = 1; o < R; o <<= 1) n2 += __shfl_xor(n2, o);
  cnorm_max(p.cnorm + g, n2);
}

// Power of two that brings a norm into [2^8, 2^9): the approximate pass
// scores fp16 copies of the queries and the candidate table, scaled by it
// (scaling by a power of two is exact and scales every score alike); norms
// outside [2^-60, 2^60] are not scaled and take the exact pass instead.
__device__ __forceinline__ float norm_scale(float nrm) {
  const int e = (int)((__float_as_uint(nrm) >> 23) & 0xFFu) - 127;
  return __uint_as_float((uint32_t)(min(127, max(-126, 8 - e)) + 127) << 23);
}
__device__ __forceinline__ bool norm_in_range(float nrm) { return nrm >= 0x1p-60f && nrm <= 0x1p60f; }

// Per layer, once, after the prep kernels: the candidate table (hi + lo, the
// value the exact products see) times the KV head's norm_scale, in fp16.
template <int NPART>
__global__ __launch_bounds__(NT) void table_f16_kernel(SelectParams p) {
  const int g = blockIdx.y;
  const size_t x = (size_t)blockIdx.x * NT + threadIdx.x, n = (size_t)p.M * R * NPART;
  if (x >= n) return;
  const float sc = norm_scale(__uint_as_float(p.cnorm[g]));
  const size_t o = (size_t)g * n + x;
  p.c_f16[o] = (_Float16)(((float)p.c_hi[o] + (float)p.c_lo[o]) * sc);
}

// One workgroup per (retrieval head, query block).  S[i][m] = qlow_i . C_m on
// MFMA (32 rows x 32 centroids per instruction, k = r = 16); a lane ends with
// 16 rows of one centroid, so the row max is a lane-local reduction plus one
// exchange with lane ^ 32.  Wave w takes centroid tiles w, w+4, ...  Only
// clusters with a member at or before the block's last row minus the window
// are eligible.
//
// Exact scores (the selection's definition): split operands, three bf16
// passes ql.ch + qh.cl + qh.ch, fp32-accurate; the order key of the row max
// ranks the clusters (larger first, lower index first among equal keys).
// They are computed only where they decide something:
//   1. approximate pass: one fp16 product per (row, cluster), on copies of
//      the query rows and of the table scaled by powers of two (norm_scale of
//      the largest row norm over the unit's slots, and of the largest table
//      norm), gives a scaled approximate row max a_m for every cluster (-inf
//      when ineligible) in LDS; each of the 128 scoring lanes keeps the
//      largest it wrote.
//   2. error bound, in the scaled units: with Q = max_i |q_i| and
//      C = max_m |C_m| after scaling (both in [2^8, 2^9)),
//        eps = 1.1 * 2^-10 * Q * C + 2^-10 (Q + C) + 2^-20 + a denormal floor
//      bounds |a_m - three-pass score| (fp16 rounding of both operands,
//      2^-11 relative each, against the three-pass products' own 2^-15
//      from the dropped lo*lo terms, Cauchy-Schwarz over the components,
//      fp32 accumulation of up to 48 products; the absolute terms cover fp16
//      subnormals).  The row max moves by at most eps as well.
//   3. prefilter: tau = the topk-th largest lane maximum.  At least topk
//      eligible clusters have a >= tau, hence exact score >= tau - eps, so
//      the k-th exact score is >= tau - eps and every cluster of the exact
//      top-k (ties included) has a >= tau - 2 eps.  Those candidates are
//      collected in index order (each wave a contiguous quarter of the
//      clusters, into its own region of kCapW slots).  Fewer than topk valid
//      lane maxima: every eligible cluster is a candidate.
//   4. the candidates are re-scored with the three passes (the same
//      operands and the same product order as a full exact pass, so the
//      keys are bit-identical to it), packed with their index as
//      (key << 32 | 0xFFFF - m), and a candidate is chosen when fewer than k
//      packed keys exceed its own; the chosen ones keep index order.
// More than kCapW candidates in a wave or 2 * NT in all, a bound that is not
// finite, or a budget above 128 (k > kGroups) sends the block through the
// exact pass over every cluster and a radix select over all of them.
//
// A unit of several slots (group-shared selection) repeats the scoring for
// each slot and keeps the max per cluster (the order key is monotone); a
// lane owns the same clusters for every slot, so the lane maxima and the
// prefilter hold for the max scores as they do for one slot, and the bound
// uses the largest row norm over the slots.
//
// The same kernel scores key-block representatives (block mode with a
// representative score): candidate m = key block m, "first member" = its
// first key.  NPART = 2 scores the per-dimension extremes bound as a 32-dim
// dot product: sum_d max(q_d a_d, q_d b_d) with a >= b equals
// max(q, 0) . a + min(q, 0) . b, so part 0 pairs max(q, 0) with the block
// maxima and part 1 pairs min(q, 0) with the minima; |(max(q,0), min(q,0))|
// = |q| and the candidate norm is |(a, b)|.
constexpr int kSelBlocks = 1;
// Padding after the selection tables: the last tile's lanes past the end
// read up to 31 rows of 64 B (split parts) and 31 first members beyond M.
constexpr size_t kTablePad = 4096;
constexpr int kGroups = 128;      // scoring lanes (4 waves x 32)
constexpr int kCapW = 192;        // candidate slots per wave
constexpr float kEpsRel = 1.1f * 0x1p-10f;

template <int NPART>
__global__ __launch_bounds__(NT, 2) void select_clusters_kernel(SelectParams p) {
  static_assert(kSelBlocks == 1, "the prefilter handles one query block per workgroup");
  // scores (approximate pass: fp32 values; exact pass: order keys); after
  // the candidates are collected, scratch for their packed keys and the
  // budget's weights
  __shared__ __attribute__((aligned(16))) uint32_t keys[kMaxSelCand + 32];   // + 32: approximate-pass sink
  __shared__ int hist[dev::kHistWords];
  __shared__ int tmp4[8];
  __shared__ int bcast[2];
  __shared__ uint16_t cidx[4 * kCapW];
  __shared__ uint32_t gmax[kGroups];
  __shared__ uint32_t tau_s;
  __shared__ int cnt_s[4], nel_s[4];
  __shared__ uint32_t sink_word;                  // store target of padding lanes (exact pass)
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
  // query rows of slot t: lane (lr, lh) holds dimensions lh*8 .. lh*8+7 of
  // rows lr and 32 + lr; rows past the end of a ragged last block repeat the
  // block's first row, so the row max needs no mask
  auto load_rows = [&](int t, float (&v)[2][8]) {
    const int qs0 = b0 * kBlock;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int i = rt * 32 + lr;
      const int row = nb > 0 ? qs0 + (i < nrow[0] ? i : 0) : 0;
      const float* qp = p.qlow + ((size_t)t * p.N + row) * R + lh * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[rt][e] = qp[e];
    }
  };
  // largest squared row norm over the unit's slots (every lane ends with
  // the block's value; all waves compute the same), and whether some row
  // norm is not finite
  float qn2 = 0.f;
  bool qbad = false;
  for (int s = 0; s < ns; ++s) {
    float v[2][8];
    load_rows(t0 + s, v);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[rt][e], v[rt][e], ss);
      const float rn2 = dev::pair32_sum(ss);
      qbad |= !(rn2 <= __FLT_MAX__);
      qn2 = fmaxf(qn2, rn2);
    }
  }
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) qn2 = fmaxf(qn2, __shfl_xor(qn2, o));
  const float qn = sqrtf(qn2), cn = __uint_as_float(p.cnorm[g]);
  const bool approx = p.topk <= kGroups && !__any(qbad) && norm_in_range(qn) && norm_in_range(cn);
  const float sq = norm_scale(qn);
  // the split rows (parts as above) and, for the approximate pass, their
  // scaled fp16 copies
  dev::bf16x8 qh[NPART][2], ql[NPART][2];
  dev::f16x8 qf[NPART][2];
  auto load_q = [&](int t) {
    float v[2][8];
    load_rows(t, v);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int part = 0; part < NPART; ++part) {
          const float x = v[rt][e];
          const float vp = NPART == 1 ? x : (part == 0 ? fmaxf(x, 0.f) : fminf(x, 0.f));
          __bf16 hh, ll;
          dev::split2(vp, hh, ll);
          qh[part][rt][e] = hh;
          ql[part][rt][e] = ll;
          qf[part][rt][e] = (_Float16)(vp * sq);
        }
  };
  const __bf16* chi = p.c_hi + (size_t)g * p.M * R * NPART;
  const __bf16* clo = p.c_lo + (size_t)g * p.M * R * NPART;
  const int32_t* fm = p.first_mem + (size_t)g * p.M;
  int n_el = 0;                     // exact pass: eligible clusters counted by this lane
  uint32_t gmx = 0;                 // exact pass: largest key this lane wrote
  float gmxf = -__builtin_inff();   // approximate pass: largest value this lane wrote
  const int n_tiles = (p.M + 31) / 32;
  // Buffer loads: the lane's offset inside a tile is fixed and the tile's
  // offset is wave-uniform (scalar), so a load needs no vector address
  // arithmetic.  Lanes of the last tile past cluster M-1 may read past the
  // end of a table (the scalar offset is not part of the range check): the
  // scratch is padded by kTablePad bytes so those reads stay inside it, and
  // whatever they return is discarded.
  const __amdgpu_buffer_rsrc_t rs_hi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(chi), 0, p.M * NPART * R * 2, dev::kBufWord3);
  const __amdgpu_buffer_rsrc_t rs_lo = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(clo), 0, p.M * NPART * R * 2, dev::kBufWord3);
  const __amdgpu_buffer_rsrc_t rs_f16 = __builtin_amdgcn_make_buffer_rsrc(
      p.c_f16 + (size_t)g * p.M * R * NPART, 0, p.M * NPART * R * 2, dev::kBufWord3);
  const __amdgpu_buffer_rsrc_t rs_fm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(fm), 0, p.M * 4, dev::kBufWord3);
  const int lim0 = lim[0];
  float* keysf = reinterpret_cast<float*>(keys);

  // Scoring pass over every cluster tile: approximate (one product, hi
  // parts only) or exact (three products).
  auto scan = [&](auto exact_c) {
    constexpr bool kExact = decltype(exact_c)::value;
    // operands are loaded kPre tiles ahead (register ring, static slots: the
    // loop is unrolled by kPre); a slot holds a tile's split centroids and,
    // per lane, the first member of its cluster (eligibility: a member <= lim)
    constexpr int kPre = (kExact || NPART == 2) ? 4 : 8;
    constexpr int kProd = kExact ? 3 : 1;
    auto ld = [&](int x, dev::bf16x8 (&bh)[NPART], dev::bf16x8 (&bl)[NPART], int& f) {
#pragma unroll
      for (int part = 0; part < NPART; ++part) {
        const int vo = (lr * NPART + part) * R * 2 + lh * 16;
        const int so = x * 32 * NPART * R * 2;
        if constexpr (kExact) {
          bh[part] = __builtin_bit_cast(dev::bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs_hi, vo, so, 0));
          bl[part] = __builtin_bit_cast(dev::bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs_lo, vo, so, 0));
        } else {
          // the fp16 copy, carried in the hi slot's registers
          bh[part] = __builtin_bit_cast(dev::bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs_f16, vo, so, 0));
        }
      }
      f = (int)__builtin_amdgcn_raw_buffer_load_b32(rs_fm, lr * 4, x * 32 * 4, 0);
    };
    dev::bf16x8 rbh[kPre][NPART], rbl[kPre][NPART];
    int rfm[kPre];
    gmx = 0;
    gmxf = -__builtin_inff();
    n_el = 0;
    for (int s = 0; s < ns; ++s) {
      load_q(t0 + s);
      // slot order, as in the loop body, so the first group waits only for its own slot
#pragma unroll
      for (int u = 0; u < kPre; ++u) {
        ld(min(n_tiles - 1, wave + 4 * u), rbh[u], rbl[u], rfm[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // The scores of tile x are finished one tile later, after the products
      // of the next tile are issued, so the matrix-result reads never wait on
      // the products just issued.
      dev::f32x16 pacc[2] = {dev::f32x16{}, dev::f32x16{}};
      bool pel = false;
      // the first finish stores 0 (exact) or -inf (approximate) to a sink;
      // so do tiles past the end, which would otherwise add a second copy of
      // the last tile's values to the lane maxima
      int pm = kExact ? INT_MAX : kMaxSelCand + lr;
      // The loop is instantiated once for the first slot of a unit (plain
      // store) and once for later slots (max with the stored value), so its
      // body is one basic block and the previous tile's vector work can be
      // placed between the current tile's matrix products.
      auto run = [&](auto later_slot) {
        constexpr bool kLater = decltype(later_slot)::value;
        auto finish = [&]() {
          float mx = -__builtin_inff();
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, pacc[rt][e]);
          mx = dev::pair32_max(mx);
          if constexpr (kExact) {
            const bool mok = pm < p.M;
            const bool el = mok & pel;
            const uint32_t key = el ? dev::order_key(mx) : 0u;
            uint32_t* dst = mok ? &keys[pm] : &sink_word;
            if constexpr (kLater) {
              *dst = max(*dst, key);
            } else {
              *dst = key;
              n_el += (int)(el & (lh == 0));
            }
            gmx = max(gmx, key);
          } else {
            const float v = pel ? mx : -__builtin_inff();
            if constexpr (kLater) keysf[pm] = fmaxf(keysf[pm], v);
            else keysf[pm] = v;
            gmxf = fmaxf(gmxf, v);
          }
        };
        // Groups of kPre tiles run whole (tiles past the end compute on the
        // last tile), so the body has no branches around loads.
        for (int x0 = wave; x0 < n_tiles; x0 += 4 * kPre) {
#pragma unroll
          for (int u = 0; u < kPre; ++u) {
            const int x = x0 + 4 * u;
            // the two row tiles' chains alternate, so no product waits on the
            // one just issued
            dev::f32x16 acc[2] = {dev::f32x16{}, dev::f32x16{}};
#pragma unroll
            for (int part = 0; part < NPART; ++part) {
              if constexpr (kExact) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) acc[rt] = dev::mfma32(ql[part][rt], rbh[u][part], acc[rt]);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) acc[rt] = dev::mfma32(qh[part][rt], rbl[u][part], acc[rt]);
              }
              if constexpr (kExact) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) acc[rt] = dev::mfma32(qh[part][rt], rbh[u][part], acc[rt]);
              } else {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                  acc[rt] = dev::mfma32_f16(qf[part][rt], __builtin_bit_cast(dev::f16x8, rbh[u][part]), acc[rt]);
              }
            }
            // eligibility of the slot's cluster, taken before the slot's refill
            // is issued (the empty asm orders the two), so the refill lands in
            // the slot's own registers: no ring rotation copies, which would
            // wait for the newest loads
            // (approximate pass: lanes past cluster M-1 and tiles past the
            // end are ineligible)
            const bool real = x < n_tiles;
            const bool fel = (lim0 >= 0) & (rfm[u] <= lim0) & (kExact || (real & (lr < p.M - x * 32)));
            { const int fi = fel; asm volatile("" ::"v"(fi) : "memory"); }
            ld(min(x + 4 * kPre, n_tiles - 1), rbh[u], rbl[u], rfm[u]);
            finish();
            pacc[0] = acc[0];
            pacc[1] = acc[1];
            pm = (kExact || real ? x * 32 : kMaxSelCand) + lr;
            pel = fel;
            // products of this tile, the previous tile's vector work between
            // them, then the slot's refill
#pragma unroll
            for (int i = 0; i < 2 * kProd * NPART; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, kExact ? 5 : 10, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x020, (kExact ? 2 : 1) * NPART + 1, 0);
          }
        }
        finish();
      };
      // a wave without tiles stores nothing
      if (wave < n_tiles) {
        if (s == 0) run(std::integral_constant<bool, false>{});
        else run(std::integral_constant<bool, true>{});
      }
    }
  };

  const size_t row_stride = (size_t)p.n_qb * p.topk;   // between slots' sel rows
  int32_t* out = p.sel + ((size_t)t0 * p.n_qb + b0) * p.topk;
  // a unit of several slots, or the adaptive budget, selects into LDS (the
  // histogram is free once the last radix pass is done), cuts the row to the
  // budget and copies it to every slot; the chosen keys go behind the row
  const bool adaptive = p.mass > 0.f;
  int32_t* dst_row = (ns == 1 && !adaptive) ? out : reinterpret_cast<int32_t*>(hist);
  uint32_t* rkeys = adaptive ? reinterpret_cast<uint32_t*>(hist) + 1024 : nullptr;
  auto copy_row = [&](int k) {
    if (dst_row == out) return;
    __syncthreads();
    // the scores are dead once the select is done: they hold the budget's weights
    if (adaptive && k > 0)
      dev::adaptive_cut(dst_row, rkeys, k, p.topk, p.mass_scale_log2, p.mass, keysf, tmp4, bcast);
    for (int x = tid; x < ns * p.topk; x += NT) {
      const int s = x / p.topk, e = x - s * p.topk;
      out[s * row_stride + e] = dst_row[e];
    }
  };
  // exact keys of every cluster, then the radix select over all of them
  auto select_all_exact = [&]() {
    scan(std::integral_constant<bool, true>{});
    int nE;
    dev::block_excl_scan(n_el, tmp4, &nE);     // (synchronizes)
    const int k = min(p.topk, nE);
    dev::topk_select(keys, p.M, k, p.topk, 0, dst_row, hist, tmp4, bcast, nullptr, rkeys);
    copy_row(k);
  };
  if (!approx) {
    select_all_exact();
    return;
  }
  scan(std::integral_constant<bool, false>{});
  if (lh == 0) gmax[wave * 32 + lr] = dev::order_key(gmxf);
  __syncthreads();
  // tau = the topk-th largest lane maximum: the largest T with at least topk
  // maxima >= T, found bit by bit from the top with wave ballots
  if (wave == 0) {
    const uint32_t a = gmax[lane], b = gmax[64 + lane];
    uint32_t pre = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = pre | (1u << bit);
      const int n = (int)__popcll(__ballot(a >= c)) + (int)__popcll(__ballot(b >= c));
      if (n >= p.topk) pre = c;
    }
    if (lane == 0) tau_s = pre;
  }
  __syncthreads();
  // candidate threshold; -FLT_MAX (every eligible cluster) when fewer than
  // topk lane maxima are finite
  const float tv = dev::key_value(tau_s);
  const float sc = norm_scale(cn), qs = qn * sq, cs = cn * sc;
  const float eps = kEpsRel * qs * cs + 0x1p-10f * (qs + cs) + 0x1p-20f +
                    0x1p-120f * sq * sc * (8.f * (qn + cn) + 1.f);
  const bool bound_ok = eps < 1e36f && !(tv > 1e36f) && !(tv != tv);
  const float thr = tv >= -1e36f ? fmaxf(tv - 2.f * eps, -__FLT_MAX__) : -__FLT_MAX__;
  // collect: all of the wave's values first (latency), then in index order
  const int per = ((p.M + 4 * 64 - 1) / (4 * 64)) * 64;
  const int wa = min(p.M, wave * per), wb = min(p.M, wa + per);
  uint16_t* ci = cidx + wave * kCapW;
  int cnt = 0, nel = 0;
  constexpr int kColl = 16;
  for (int x0 = wa; x0 < wb; x0 += 64 * kColl) {
    float v[kColl];
#pragma unroll
    for (int i = 0; i < kColl; ++i) {
      const int x = x0 + 64 * i + lane;
      v[i] = x < wb ? keysf[x] : -__builtin_inff();
    }
#pragma unroll
    for (int i = 0; i < kColl; ++i) {
      nel += (int)__popcll(__ballot(v[i] >= -__FLT_MAX__));
      const bool take = v[i] >= thr;
      const uint64_t bt = __ballot(take);
      const int pos = cnt + (int)__popcll(bt & ((1ull << lane) - 1ull));
      if (take && pos < kCapW) ci[pos] = (uint16_t)(x0 + 64 * i + lane);
      cnt += (int)__popcll(bt);
    }
  }
  if (lane == 0) {
    cnt_s[wave] = cnt;
    nel_s[wave] = nel;
  }
  __syncthreads();
  int n = 0, base = 0, nE = 0;
  bool ovf = !bound_ok;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int c = cnt_s[w];
    base += w < wave ? c : 0;
    n += c;
    nE += nel_s[w];
    ovf |= c > kCapW;
  }
  ovf |= n > 2 * NT;
  if (ovf) {
    __syncthreads();    // the scores are rewritten
    select_all_exact();
    return;
  }
  const int k = min(p.topk, nE);
  // exact keys of the wave's candidates, 32 at a time: lane (lr, lh) loads
  // candidate lr's parts for dimensions lh*8 .. lh*8+7, as in the scan;
  // packed keys go to pk[base + pos] (index order across the waves)
  // (every tile's operands are loaded before the first product: the rows
  // are gathered from L2, and their latency would otherwise add up per tile)
  uint64_t* pk = reinterpret_cast<uint64_t*>(keys);
  constexpr int kMaxCT = kCapW / 32;
  const int n_ct = (cnt + 31) / 32;
  dev::bf16x8 cbh[kMaxCT][NPART], cbl[kMaxCT][NPART];
  int cm[kMaxCT];
#pragma unroll
  for (int x = 0; x < kMaxCT; ++x) {
    const int pos = x * 32 + lr;
    cm[x] = pos < cnt ? (int)ci[pos] : 0;
    if (x < n_ct) {
#pragma unroll
      for (int part = 0; part < NPART; ++part) {
        const int vo = (cm[x] * NPART + part) * R * 2 + lh * 16;
        cbh[x][part] = __builtin_bit_cast(dev::bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs_hi, vo, 0, 0));
        cbl[x][part] = __builtin_bit_cast(dev::bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs_lo, vo, 0, 0));
      }
    }
  }
  for (int s = 0; s < ns; ++s) {
    if (ns > 1) load_q(t0 + s);
#pragma unroll
    for (int x = 0; x < kMaxCT; ++x) {
      if (x < n_ct) {
        const int pos = x * 32 + lr;
        dev::f32x16 acc[2] = {dev::f32x16{}, dev::f32x16{}};
#pragma unroll
        for (int part = 0; part < NPART; ++part) {
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) acc[rt] = dev::mfma32(ql[part][rt], cbh[x][part], acc[rt]);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) acc[rt] = dev::mfma32(qh[part][rt], cbl[x][part], acc[rt]);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) acc[rt] = dev::mfma32(qh[part][rt], cbh[x][part], acc[rt]);
        }
        float mx = -__builtin_inff();
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[rt][e]);
        mx = dev::pair32_max(mx);
        const uint64_t kk = ((uint64_t)dev::order_key(mx) << 32) | (uint32_t)(0xFFFF - cm[x]);
        if (pos < cnt && lh == 0) pk[base + pos] = s == 0 ? kk : max(pk[base + pos], kk);
      }
    }
  }
  // pads the reads below to whole groups of kRankU; ranks below every key
  constexpr int kRankU = 16;
  if (tid < kRankU) pk[n + tid] = 0ull;
  __syncthreads();
  // rank = number of packed keys above one's own (all distinct); chosen when
  // rank < k, so exactly k are chosen.  Candidate t and t + NT per thread;
  // kRankU broadcast reads in flight per step.
  const uint64_t ka = tid < n ? pk[tid] : 0ull, kb = tid + NT < n ? pk[tid + NT] : 0ull;
  int ra = 0, rb = 0;
  const bool two = n > NT;
  for (int j = 0; j < n; j += kRankU) {
    uint64_t u[kRankU];
#pragma unroll
    for (int e = 0; e < kRankU; ++e) u[e] = pk[j + e];
#pragma unroll
    for (int e = 0; e < kRankU; ++e) ra += (int)(u[e] > ka);
    if (two) {
#pragma unroll
      for (int e = 0; e < kRankU; ++e) rb += (int)(u[e] > kb);
    }
  }
  const bool ca = tid < n && ra < k, cb = tid + NT < n && rb < k;
  int na;
  const int pa = dev::block_excl_scan((int)ca, tmp4, &na);   // (synchronizes)
  int nbb;
  const int pb = na + dev::block_excl_scan((int)cb, tmp4, &nbb);
  if (ca) {
    dst_row[pa] = 0xFFFF - (int)(uint32_t)(ka & 0xFFFFu);
    if (rkeys) rkeys[pa] = (uint32_t)(ka >> 32);
  }
  if (cb) {
    dst_row[pb] = 0xFFFF - (int)(uint32_t)(kb & 0xFFFFu);
    if (rkeys) rkeys[pb] = (uint32_t)(kb >> 32);
  }
  for (int x = k + tid; x < p.topk; x += NT) dst_row[x] = -1;
  copy_row(k);
}

}  // namespace

size_t kmeans_scratch_bytes(int N, int M, int Hkv) {
  const size_t n_chunks = (size_t)(N + kChunk - 1) / kChunk;
  return (size_t)Hkv * n_chunks * M * sizeof(int32_t) + (size_t)Hkv * M * sizeof(int32_t) +
         (size_t)Hkv * M * (2 * R * sizeof(_Float16) + sizeof(float)) + 4 * (size_t)Hkv * sizeof(uint32_t) +
         (size_t)Hkv * N * sizeof(int32_t) + (size_t)Hkv * N * sizeof(uint64_t) + 768;
}

hipError_t launch_kmeans(KmeansParams p, int Hkv, int iters, hipStream_t s) {
  p.n_chunks = (p.N + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(km_init_kernel, dim3((p.M * R + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
  const int amax_blocks = (int)std::min<size_t>(kAmaxBlocks, ((size_t)p.N * R / 4 + NT - 1) / NT);
  hipLaunchKernelGGL(km_amax_kernel, dim3(amax_blocks, Hkv), dim3(NT), 0, s, p);
  hipError_t e = hipGetLastError();
  const dim3 assign_grid((p.N + 4 * 32 * KT - 1) / (4 * 32 * KT), Hkv);
  const dim3 exact_grid(std::min<int>(kExactBlocks, assign_grid.x), Hkv, kExactSplit);
  const dim3 commit_grid(std::min<int>(256, (p.N + NT - 1) / NT), Hkv);
  for (int it = 0; it < iters && e == hipSuccess; ++it) {
    hipLaunchKernelGGL(km_clear_kernel, dim3(1), dim3(kMaxHeads), 0, s, p, Hkv);
    hipLaunchKernelGGL(km_prep_kernel, dim3((p.M + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_assign_approx_kernel, assign_grid, dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_assign_exact_kernel, exact_grid, dim3(NT), 0, s, p);
    hipLaunchKernelGGL(km_assign_commit_kernel, commit_grid, dim3(NT), 0, s, p);
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
  hipLaunchKernelGGL(sel_clear_kernel, dim3(1), dim3(kMaxHeads), 0, s, p.cnorm, Hkv);
  hipLaunchKernelGGL(cluster_prep_kernel, dim3((p.M + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
  hipLaunchKernelGGL(table_f16_kernel<1>, dim3((p.M * R + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
  hipLaunchKernelGGL(select_clusters_kernel<1>, dim3((p.n_qb + kSelBlocks - 1) / kSelBlocks, p.n_units), dim3(NT),
                     0, s, p);
  return hipGetLastError();
}

size_t select_clusters_scratch_bytes(int M, int Hkv) {
  return (size_t)Hkv * M * (3 * R * sizeof(__bf16) + sizeof(int32_t)) + (size_t)Hkv * sizeof(uint32_t) + kTablePad;
}

hipError_t launch_select_block_reps(const SelectParams& p, int Hkv, int mode, hipStream_t s) {
  if (p.n_units == 0 || p.n_qb == 0) return hipSuccess;
  const dim3 prep((p.M * R + NT - 1) / NT, Hkv), grid((p.n_qb + kSelBlocks - 1) / kSelBlocks, p.n_units);
  hipLaunchKernelGGL(sel_clear_kernel, dim3(1), dim3(kMaxHeads), 0, s, p.cnorm, Hkv);
  if (mode == 2) {
    hipLaunchKernelGGL(block_prep_kernel<2>, prep, dim3(NT), 0, s, p);
    hipLaunchKernelGGL(table_f16_kernel<2>, dim3((p.M * R * 2 + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(select_clusters_kernel<2>, grid, dim3(NT), 0, s, p);
  } else {
    hipLaunchKernelGGL(block_prep_kernel<1>, prep, dim3(NT), 0, s, p);
    hipLaunchKernelGGL(table_f16_kernel<1>, dim3((p.M * R + NT - 1) / NT, Hkv), dim3(NT), 0, s, p);
    hipLaunchKernelGGL(select_clusters_kernel<1>, grid, dim3(NT), 0, s, p);
  }
  return hipGetLastError();
}

size_t select_block_reps_scratch_bytes(int n_kb, int Hkv, int mode) {
  const size_t npart = mode == 2 ? 2 : 1;
  return (size_t)Hkv * n_kb * (3 * R * npart * sizeof(__bf16) + sizeof(int32_t)) + (size_t)Hkv * sizeof(uint32_t) +
         kTablePad;
}

}  // namespace ha
