// Orthros cross-attention for output positions (Orthros page, "Prefilling"
// section: only the last prompt token runs full cross-attention over the
// whole KV; design section: SWA and cross-attention share the projections and
// a light scale-offset separates the two query roles).
//
//   q'_h = q_{p,h} * s_h + o_h   (fp32, not re-rounded)
//   O_out[p, h] = softmax over keys 0..p of (scale q'_h . k_j) applied to v_j
//
// A memory-bound GEMV: every key/value row of the KV head is read once per
// output position.  Split over 1024-key chunks: each workgroup produces, for
// the G query heads of one KV head, a partial (max, sum, weighted V); a
// second kernel merges the chunks.
#include "common.h"

namespace ha {
namespace {

constexpr int D = kHeadDim;
constexpr int NT = 256;
constexpr int CH = kCrossChunk;
constexpr int kMaxG = 16;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ __launch_bounds__(NT) void cross_partial_kernel(CrossParams p) {
  __shared__ float qs[kMaxG][D];
  __shared__ float sc[kMaxG][CH];
  __shared__ float ms[kMaxG];
  const int c = blockIdx.x, g = blockIdx.y, oi = blockIdx.z;
  const int prow = p.N - p.n_out + oi;
  const int j0 = c * CH;
  const int nj = max(0, min(CH, prow + 1 - j0));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  for (int x = tid; x < G * D; x += NT) {
    const int hh = x / D, d = x % D;
    const int h = g * G + hh;
    const uint16_t qb = p.Q[((size_t)prow * p.Hq + h) * D + d];
    const float q = __uint_as_float((uint32_t)qb << 16);
    qs[hh][d] = fmaf(q, p.xs[h * D + d], p.xo[h * D + d]);
  }
  __syncthreads();
  const size_t rs = (size_t)p.Hkv * D;
  // scores (log2 domain): s = c * q' . k
  for (int jj = tid; jj < nj; jj += NT) {
    const uint4* kr = reinterpret_cast<const uint4*>(p.K + (size_t)(j0 + jj) * rs + g * D);
    for (int h4 = 0; h4 < G; h4 += 4) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int v = 0; v < D / 8; ++v) {
        const uint4 w = kr[v];
        const float k8[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                             bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int hh = min(h4 + u, G - 1);
          float a = acc[u];
#pragma unroll
          for (int e = 0; e < 8; ++e) a = fmaf(qs[hh][v * 8 + e], k8[e], a);
          acc[u] = a;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (h4 + u < G) sc[h4 + u][jj] = acc[u] * p.c;
    }
  }
  __syncthreads();
  // per head: chunk max and exp2
  for (int hh = wave; hh < G; hh += 4) {
    float mx = -__builtin_inff();
    for (int jj = lane; jj < nj; jj += 64) mx = fmaxf(mx, sc[hh][jj]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    for (int jj = lane; jj < nj; jj += 64) sc[hh][jj] = exp2f(sc[hh][jj] - mx);
    if (lane == 0) ms[hh] = mx;
  }
  __syncthreads();
  // weighted V: lane -> 2 consecutive d, wave -> heads wave, wave+4, ...
  for (int hh = wave; hh < G; hh += 4) {
    const int h = g * G + hh;
    float a0 = 0.f, a1 = 0.f, l = 0.f;
    for (int jj = 0; jj < nj; ++jj) {
      const float pw = sc[hh][jj];
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p.V + (size_t)(j0 + jj) * rs + g * D + lane * 2);
      a0 = fmaf(pw, bf16_lo(w), a0);
      a1 = fmaf(pw, bf16_hi(w), a1);
      l += pw;
    }
    float* dst = p.part + (((size_t)oi * p.Hq + h) * p.n_chunks + c) * (D + 2);
    dst[lane * 2] = a0;
    dst[lane * 2 + 1] = a1;
    if (lane == 0) {
      dst[D] = nj > 0 ? ms[hh] : -__builtin_inff();
      dst[D + 1] = nj > 0 ? l : 0.f;
    }
  }
}

__global__ __launch_bounds__(D) void cross_combine_kernel(CrossParams p) {
  const int h = blockIdx.x, oi = blockIdx.y, d = threadIdx.x;
  const float* base = p.part + ((size_t)oi * p.Hq + h) * p.n_chunks * (D + 2);
  float M = -__builtin_inff();
  for (int c = 0; c < p.n_chunks; ++c) M = fmaxf(M, base[c * (D + 2) + D]);
  float L = 0.f, acc = 0.f;
  for (int c = 0; c < p.n_chunks; ++c) {
    const float m = base[c * (D + 2) + D];
    if (m == -__builtin_inff()) continue;
    const float wgt = exp2f(m - M);
    L += wgt * base[c * (D + 2) + D + 1];
    acc += wgt * base[c * (D + 2) + d];
  }
  p.O_out[((size_t)oi * p.Hq + h) * D + d] = L > 0.f ? acc / L : 0.f;
}

}  // namespace

hipError_t launch_cross(const CrossParams& p, hipStream_t s) {
  if (p.n_out == 0) return hipSuccess;
  if (p.G > kMaxG) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cross_partial_kernel, dim3(p.n_chunks, p.Hkv, p.n_out), dim3(NT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cross_combine_kernel, dim3(p.Hq, p.n_out), dim3(D), 0, s, p);
  return hipGetLastError();
}

}  // namespace ha
