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
// Projection on MFMA: a wave takes 16 rows at a time; X[16 x 128] (bf16,
// exact) times P[128 x 16] with P split into three bf16 parts, so the three
// products per k-step reproduce the fp32 result (v_mfma_f32_16x16x32_bf16,
// A = X rows, B = P slice).  Lane l feeds row l%16 / column l%16 with
// k = 8 (l/16) .. +8 of each 32-wide k-step and ends with rows 4 (l/16) + e
// of output column l%16.  A workgroup walks a contiguous range of rows of
// one entry; two row groups are in flight per iteration.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(dev::bf16x8 a, dev::bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(NT) void project_kernel(ProjParams p, int rows_per_wg) {
  const int e = blockIdx.y;
  const int grp = p.group[e], head = p.head[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lq = lane & 15, lg = lane >> 4;
  dev::bf16x8 ph[4], pm[4], pl[4];
  {
    const float* src = p.P + (size_t)grp * D * R;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        __bf16 h, m, l;
        dev::split3(src[(ks * 32 + lg * 8 + x) * R + lq], h, m, l);
        ph[ks][x] = h;
        pm[ks][x] = m;
        pl[ks][x] = l;
      }
  }
  const int r0 = blockIdx.x * rows_per_wg, r1 = min(p.N, r0 + rows_per_wg);
  for (int base = r0 + wave * 32; base < r1; base += 128) {
    dev::bf16x8 xa[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = base + u * 16 + lq;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (i < r1) {
          xa[u][ks] = *reinterpret_cast<const dev::bf16x8*>(p.X + ((size_t)i * p.H + head) * D + ks * 32 + lg * 8);
        } else {
#pragma unroll
          for (int x = 0; x < 8; ++x) xa[u][ks][x] = (__bf16)0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        acc = mfma16(xa[u][ks], pl[ks], acc);
        acc = mfma16(xa[u][ks], pm[ks], acc);
        acc = mfma16(xa[u][ks], ph[ks], acc);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = base + u * 16 + lg * 4 + q;
        if (i < r1) p.out[((size_t)e * p.N + i) * R + lq] = acc[q];
      }
    }
  }
}

// One workgroup per (retrieval head, query block).  Wave w scores the
// eligible blocks c = c_lo + w, c_lo + w + 4, ... on MFMA: S[i][j] =
// qlow_i . klow_j for the 64 x 64 pairs as 2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 (k = r = 16) over hi/lo bf16 splits of both
// operands (three passes, ~1e-5 relative), then the block's max: 32 max3
// per lane and a reduction over the wave.  Rows past the end of a ragged
// block repeat its first row (no mask); pairs with j > i or j >= N are
// masked only in the tiles that reach past the block's first row.
__device__ __forceinline__ void split_row8(const float* __restrict__ src, dev::bf16x8& hi, dev::bf16x8& lo) {
  const float4 a = *reinterpret_cast<const float4*>(src);
  const float4 b = *reinterpret_cast<const float4*>(src + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h, l;
    dev::split2(v[e], h, l);
    hi[e] = h;
    lo[e] = l;
  }
}

__device__ __forceinline__ float wave_max(float v) {
  v = dev::pair32_max(dev::pair16_max(v));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// A unit of several slots (group-shared selection) scores every block once
// per slot and keeps the max (the order key is monotone, so the max of keys
// is the key of the max); a wave owns the same blocks for every slot.
//
// kInt8 (8-bit indexer keys): the keys are int8 codes (exact in bf16) with one
// scale per key; S = Q K^T is formed with the queries as the A operand, so a
// lane holds one key column and applies its scale once to the max of its
// column (scale >= 0): two passes (hi, lo parts of q) instead of three.
//
// keys: dynamic LDS of n_qb words (the eligible blocks of one query block)
template <bool kInt8>
__global__ __launch_bounds__(NT) void select_blocks_kernel(SelectParams p) {
  extern __shared__ uint32_t keys[];
  __shared__ int hist[dev::kHistWords];
  __shared__ int tmp4[8];
  __shared__ int bcast[2];
  __shared__ uint32_t sel_keys[dev::kNT];   // adaptive budget: keys of the top-k
  __shared__ float wrank[dev::kNT];
  const int b = blockIdx.x;
  const int t0 = (int)(p.unit[blockIdx.y] & 0xFFFFu), ns = (int)(p.unit[blockIdx.y] >> 16);
  const int g = p.group_of_ret[t0];
  const int qs = b * kBlock;
  const int nrow = min(kBlock, p.N - qs);
  const int qe = qs + nrow - 1;
  const int c_lo = p.force_block0 ? 1 : 0;
  const int c_hi = (qe - p.window >= 0) ? (qe - p.window) / kBlock : -1;
  const int nE = max(0, c_hi - c_lo + 1);
  const size_t row_stride = (size_t)p.n_qb * p.topk;   // between slots' sel rows
  int32_t* out = p.sel + ((size_t)t0 * p.n_qb + b) * p.topk;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (p.topk == 0) return;
  const bool adaptive = p.mass > 0.f;
  if (nE <= p.topk && !adaptive) {
    for (int s = 0; s < ns; ++s)
      for (int x = tid; x < p.topk; x += NT) out[s * row_stride + x] = x < nE ? c_lo + x : -1;
    return;
  }
  for (int s = 0; s < ns; ++s) {
    const int t = t0 + s;
    // A operands: query rows qs + 32 rt + lr, k-half lh
    dev::bf16x8 qh[2], ql[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int i = rt * 32 + lr;
      const int row = qs + (i < nrow ? i : 0);
      split_row8(p.qlow + ((size_t)t * p.N + row) * R + lh * 8, qh[rt], ql[rt]);
    }
    if constexpr (kInt8) {
      const int8_t* cbase = p.kcodes + (size_t)g * p.N * R;
      const float* sbase = p.kscale + (size_t)g * p.N;
      // keys j0 + 32 kt + lr of block c as B operands (8 codes per lane) and
      // their scales; rows past N read key N-1 (masked below); the next
      // block is loaded one iteration ahead
      auto kload8 = [&](int c, uint2 (&v)[2], float (&sc)[2]) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int j = min(c * kBlock + kt * 32 + lr, p.N - 1);
          v[kt] = *reinterpret_cast<const uint2*>(cbase + (size_t)j * R + lh * 8);
          sc[kt] = sbase[j];
        }
      };
      uint2 nk[2];
      float ns[2];
      kload8(c_lo + min(wave, nE - 1), nk, ns);
      for (int x = wave; x < nE; x += 4) {
        const int c = c_lo + x;
        const int j0 = c * kBlock;
        dev::bf16x8 kq[2];
        float ks[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const uint32_t w2[2] = {nk[kt].x, nk[kt].y};
#pragma unroll
          for (int e = 0; e < 8; ++e) kq[kt][e] = (__bf16)(float)(int8_t)(w2[e >> 2] >> (8 * (e & 3)));
          ks[kt] = ns[kt];
        }
        kload8(c_lo + min(x + 4, nE - 1), nk, ns);
        const bool edge = j0 + kBlock - 1 > qs;     // some pair may have j > i or j >= N
        float mx = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          // column j = j0 + 32 kt + lr; element e: row qs + 32 rt + 4 lh + 8 (e/4) + e%4
          const int j = j0 + kt * 32 + lr;
          float m = -__builtin_inff();
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            dev::f32x16 acc = {};
            acc = dev::mfma32(ql[rt], kq[kt], acc);
            acc = dev::mfma32(qh[rt], kq[kt], acc);
            if (edge) {
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int ii = rt * 32 + lh * 4 + (e >> 2) * 8 + (e & 3);
                const bool vis = (ii < nrow) & (j <= qs + ii) & (j < p.N);
                m = fmaxf(m, vis ? acc[e] : -__builtin_inff());
              }
            } else {
#pragma unroll
              for (int e = 0; e < 16; ++e) m = fmaxf(m, acc[e]);
            }
          }
          mx = fmaxf(mx, m == -__builtin_inff() ? m : m * ks[kt]);
        }
        mx = wave_max(mx);
        if (lane == 0) keys[x] = s == 0 ? dev::order_key(mx) : max(keys[x], dev::order_key(mx));
      }
      continue;
    }
    const float* kbase = p.klow + (size_t)g * p.N * R;
    // B operands: keys j0 + 32 kt + lr of block c (rows past N read key N-1,
    // masked below); the next block's rows are loaded one iteration ahead
    auto kload = [&](int c, float4 (&v)[2][2]) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const float* src = kbase + (size_t)min(c * kBlock + kt * 32 + lr, p.N - 1) * R + lh * 8;
        v[kt][0] = *reinterpret_cast<const float4*>(src);
        v[kt][1] = *reinterpret_cast<const float4*>(src + 4);
      }
    };
    float4 nk[2][2];
    kload(c_lo + min(wave, nE - 1), nk);
    for (int x = wave; x < nE; x += 4) {
      const int c = c_lo + x;
      const int j0 = c * kBlock;
      dev::bf16x8 kh[2], kl[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const float v[8] = {nk[kt][0].x, nk[kt][0].y, nk[kt][0].z, nk[kt][0].w,
                            nk[kt][1].x, nk[kt][1].y, nk[kt][1].z, nk[kt][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 h, l;
          dev::split2(v[e], h, l);
          kh[kt][e] = h;
          kl[kt][e] = l;
        }
      }
      kload(c_lo + min(x + 4, nE - 1), nk);
      const bool edge = j0 + kBlock - 1 > qs;     // some pair may have j > i or j >= N
      float mx = -__builtin_inff();
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          // S^T tile: rows = keys (A = k), columns = queries (B = q)
          dev::f32x16 acc = {};
          acc = dev::mfma32(kl[kt], qh[rt], acc);
          acc = dev::mfma32(kh[kt], ql[rt], acc);
          acc = dev::mfma32(kh[kt], qh[rt], acc);
          if (edge) {
            // lane: query column qs + 32 rt + lr; element e: key j0 + 32 kt + 4 lh + 8 (e/4) + e%4
            const int i = qs + rt * 32 + lr;
            const bool row_ok = rt * 32 + lr < nrow;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int j = j0 + kt * 32 + lh * 4 + (e >> 2) * 8 + (e & 3);
              const bool vis = row_ok & (j <= i) & (j < p.N);
              mx = fmaxf(mx, vis ? acc[e] : -__builtin_inff());
            }
          } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[e]);
          }
        }
      mx = wave_max(mx);
      if (lane == 0) keys[x] = s == 0 ? dev::order_key(mx) : max(keys[x], dev::order_key(mx));
    }
  }
  __syncthreads();
  if (ns == 1 && !adaptive) {
    dev::topk_select(keys, nE, p.topk, p.topk, c_lo, out, hist, tmp4, bcast);
    return;
  }
  // shared row: select into LDS (the histogram is free once the last radix
  // pass is done), cut it to the adaptive budget, then write it to every
  // slot of the unit
  int32_t* shared_row = reinterpret_cast<int32_t*>(hist);
  dev::topk_select(keys, nE, p.topk, p.topk, c_lo, shared_row, hist, tmp4, bcast, nullptr,
                   adaptive ? sel_keys : nullptr);
  __syncthreads();
  if (adaptive && min(p.topk, nE) > 0)
    dev::adaptive_cut(shared_row, sel_keys, min(p.topk, nE), p.topk, p.mass_scale_log2, p.mass, wrank, tmp4, bcast);
  for (int x = tid; x < ns * p.topk; x += NT) {
    const int s = x / p.topk, e = x - s * p.topk;
    out[s * row_stride + e] = shared_row[e];
  }
}

// 8-bit indexer keys: one thread per key row; scale = max |k| / 127 (IEEE
// fp32 division), code = k / scale rounded to nearest, ties to even; an
// all-zero key gets scale 0 and zero codes.
__global__ __launch_bounds__(NT) void quantize_keys_kernel(const float* __restrict__ klow, int8_t* __restrict__ codes,
                                                           float* __restrict__ scales, size_t n_rows) {
  const size_t row = (size_t)blockIdx.x * NT + threadIdx.x;
  if (row >= n_rows) return;
  const float4* src = reinterpret_cast<const float4*>(klow + row * R);
  float v[R];
#pragma unroll
  for (int q = 0; q < R / 4; ++q) {
    const float4 a = src[q];
    v[4 * q] = a.x;
    v[4 * q + 1] = a.y;
    v[4 * q + 2] = a.z;
    v[4 * q + 3] = a.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int d = 0; d < R; ++d) amax = fmaxf(amax, fabsf(v[d]));
  const float sc = amax / 127.0f;
  uint32_t w[R / 4];
#pragma unroll
  for (int q = 0; q < R / 4; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = sc > 0.f ? (int)__builtin_rintf(v[4 * q + e] / sc) : 0;
      word |= (uint32_t)(uint8_t)(int8_t)c << (8 * e);
    }
    w[q] = word;
  }
  *reinterpret_cast<uint4*>(codes + row * R) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[row] = sc;
}

}  // namespace

hipError_t launch_quantize_keys(const float* klow, int8_t* codes, float* scales, size_t n_rows, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_keys_kernel, dim3((unsigned)((n_rows + NT - 1) / NT)), dim3(NT), 0, s, klow, codes,
                     scales, n_rows);
  return hipGetLastError();
}

hipError_t launch_project(const ProjParams& p, hipStream_t s) {
  if (p.n_entries == 0 || p.N == 0) return hipSuccess;
  // about 2048 workgroups in total, each over a multiple of 16 rows
  const int target = max(1, 2048 / p.n_entries);
  int per = (p.N + target - 1) / target;
  per = max(16, (per + 15) / 16 * 16);
  hipLaunchKernelGGL(project_kernel, dim3((p.N + per - 1) / per, p.n_entries), dim3(NT), 0, s, p, per);
  return hipGetLastError();
}

hipError_t launch_select_blocks(const SelectParams& p, hipStream_t s) {
  if (p.n_ret == 0 || p.n_qb == 0) return hipSuccess;
  const size_t lds = (size_t)p.n_qb * sizeof(uint32_t);
  const void* fn = p.kcodes ? reinterpret_cast<const void*>(select_blocks_kernel<true>)
                            : reinterpret_cast<const void*>(select_blocks_kernel<false>);
  if (lds > 32 * 1024) {   // large tables: allow the dynamic size explicitly
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (p.kcodes) hipLaunchKernelGGL(select_blocks_kernel<true>, dim3(p.n_qb, p.n_units), dim3(NT), lds, s, p);
  else hipLaunchKernelGGL(select_blocks_kernel<false>, dim3(p.n_qb, p.n_units), dim3(NT), lds, s, p);
  return hipGetLastError();
}

}  // namespace ha
