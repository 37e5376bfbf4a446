// Flash attention for gfx950: banded / dense / TriangleMix heads, and the
// local-window part of retrieval heads (with a per-row log2-sum-exp so the
// selected-key part can be merged in afterwards).
//
// The attention itself is exact softmax over each query's key set (RTPurbo
// post: exact attention on the selected candidates in full dimension; the
// SWA and TriangleMix masks are static key sets).  Arithmetic: bf16 inputs,
// QK^T and PV on v_mfma_f32_32x32x16_bf16, softmax statistics and the output
// accumulator in fp32, P rounded to bf16 for the PV product.
//
// Workgroup = 4 waves.  Each wave owns 64 query rows of one head; the 4 heads
// of a "pack" share one KV head and the same rows, so every 64-key K/V tile
// staged in LDS serves 256 query rows.  Tiles are double-buffered: global
// loads of tile t+1 are in flight (in registers) while tile t is computed.
//
// Per wave and 64-key tile the contraction is laid out transposed,
//   S^T[key][query] = K Q^T     (A = K rows from LDS, B = Q^T held in registers)
//   O^T[d][query]  += V^T P^T   (A = V^T rows from LDS, B = P^T from registers)
// so that each lane owns whole query columns: the row max / row sum of a
// query live in one lane pair (lane, lane^32), and P never leaves registers.
#include "common.h"

#include <limits.h>

namespace ha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
constexpr int BK = 64;
constexpr int KSTR = D + 8;          // K row stride in LDS (bf16): 272 B, conflict-free 16-B reads
constexpr int VSTR = BK + 8;         // V^T row stride in LDS (bf16): 144 B
constexpr int K_ELEMS = BK * KSTR;
constexpr int V_ELEMS = D * VSTR;
constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;   // 35840 B per buffer
constexpr int Q_ELEMS = 64 * KSTR;             // one wave's 64 query rows (17408 B)
constexpr int SMEM_ELEMS = 2 * BUF_ELEMS + 4 * Q_ELEMS;
constexpr int NT = 256;
constexpr float kNegInf = -__builtin_inff();
constexpr float kMInit = -1e30f;     // finite start for the running max
constexpr float kSlack = 8.f;        // log2 headroom before the reference max moves

// visible(i, j) = j <= i - a  &&  (i - j < b  ||  j < sink  ||  i >= dense_from)
struct MaskSpec {
  int a, b, sink, dense_from;
};

struct TileRegs {
  u32x4 k[4];
  u32x4 v[4];
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Global -> registers for one 64-key tile of K and V (KV head g).
// K: 1024 chunks of 16 B, chunk id = c*256 + tid -> (key slot c*16 + tid/16,
// d = (tid%16)*8): coalesced rows.  V: thread -> key slots 4*(tid%16) + x,
// d = 8*(tid/16) .. +8 (transposed on the LDS store).  rows[0..3] are the key
// rows of the K slots, rows[4..7] those of the V slots; -1 = zero fill.
__device__ __forceinline__ void tile_load(TileRegs& r, const uint16_t* __restrict__ K,
                                          const uint16_t* __restrict__ V, const int (&rows)[8],
                                          size_t rs, int g, int tid) {
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int key = rows[c];
    r.k[c] = (key >= 0) ? *reinterpret_cast<const u32x4*>(K + (size_t)key * rs + g * D + (tid & 15) * 8) : z;
  }
  const int dc = tid >> 4;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int key = rows[4 + x];
    r.v[x] = (key >= 0) ? *reinterpret_cast<const u32x4*>(V + (size_t)key * rs + g * D + dc * 8) : z;
  }
}

// Key slots this thread loads: K slots c*16 + tid/16, V slots 4*(tid%16) + x.
__device__ __forceinline__ int k_slot(int c, int tid) { return c * 16 + (tid >> 4); }
__device__ __forceinline__ int v_slot(int x, int tid) { return (tid & 15) * 4 + x; }

__device__ __forceinline__ void contiguous_rows(int (&rows)[8], int k0, int N, int tid) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int key = k0 + k_slot(c, tid);
    rows[c] = key < N ? key : -1;
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int key = k0 + v_slot(x, tid);
    rows[4 + x] = key < N ? key : -1;
  }
}

// Position of key u (0..15) of a 16-key PV k-step inside an LDS V^T row, so
// that the 8 keys one MFMA lane consumes are contiguous.  A lane of half
// g = lane/32 holds, for C-layout element e, key g*4 + (e/4)*8 + e%4; the
// slot it feeds at k-step element e' (0..7) is 8g + e'.
__device__ __forceinline__ int vt_pos(int u) {
  return 8 * ((u >> 2) & 1) + 4 * (u >> 3) + (u & 3);
}

__device__ __forceinline__ void tile_store(const TileRegs& r, uint16_t* buf, int tid) {
  uint16_t* Ks = buf;
  uint16_t* Vt = buf + K_ELEMS;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int id = c * NT + tid;
    *reinterpret_cast<u32x4*>(Ks + (id >> 4) * KSTR + (id & 15) * 8) = r.k[c];
  }
  const int kg = tid & 15, dc = tid >> 4;
  const int pos = 16 * (kg >> 2) + vt_pos((kg * 4) & 15);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t a0 = r.v[0][w], a1 = r.v[1][w], a2 = r.v[2][w], a3 = r.v[3][w];
    u32x2 ev, od;
    ev[0] = (a0 & 0xFFFFu) | (a1 << 16);
    ev[1] = (a2 & 0xFFFFu) | (a3 << 16);
    od[0] = (a0 >> 16) | (a1 & 0xFFFF0000u);
    od[1] = (a2 >> 16) | (a3 & 0xFFFF0000u);
    *reinterpret_cast<u32x2*>(Vt + (dc * 8 + 2 * w) * VSTR + pos) = ev;
    *reinterpret_cast<u32x2*>(Vt + (dc * 8 + 2 * w + 1) * VSTR + pos) = od;
  }
}

struct WaveAcc {
  f32x16 o[2][4];   // O^T: [query half][d block]
  float m[2];       // running max (raw score units) per query half
  float l[2];       // running sum, partial over this lane's keys
};

__device__ __forceinline__ bool tile_full(const MaskSpec& ms, int q0, int k0) {
  if (k0 + 63 > q0 - ms.a) return false;
  if ((q0 + 63) - k0 < ms.b) return true;
  if (k0 + 63 < ms.sink) return true;
  if (q0 >= ms.dense_from) return true;
  return false;
}

// One 64-key tile against the wave's 64 query rows, as two 32-key halves
// (each half is one online-softmax step; this keeps 32 score registers live).
// The tile's keys are k0 .. k0+63.
__device__ __forceinline__ void tile_compute(const uint16_t* __restrict__ buf, const uint16_t* __restrict__ Qs,
                                             WaveAcc& acc, int lane, int q0, int k0, const MaskSpec& ms,
                                             float c) {
  const uint16_t* Ks = buf;
  const uint16_t* Vt = buf + K_ELEMS;
  const int lr = lane & 31, lh = lane >> 5;
  const bool full = tile_full(ms, q0, k0);

  // S^T = K Q^T for the 64 x 64 tile: [key half][query half]
  f32x16 s[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][qb][e] = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const bf16x8 q0f = *reinterpret_cast<const bf16x8*>(Qs + lr * KSTR + t * 16 + lh * 8);
    const bf16x8 q1f = *reinterpret_cast<const bf16x8*>(Qs + (32 + lr) * KSTR + t * 16 + lh * 8);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + lr) * KSTR + t * 16 + lh * 8);
      s[kb][0] = mfma(kf, q0f, s[kb][0]);
      s[kb][1] = mfma(kf, q1f, s[kb][1]);
    }
  }

  // each 32-key half is one online-softmax step followed by its PV k-steps
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if (!full) {
      const int jb = k0 + kb * 32 + lh * 4;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int i = q0 + qb * 32 + lr;
        const bool dense_row = i >= ms.dense_from;
        const int dd = i - jb;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = (e >> 2) * 8 + (e & 3);
          const int d = dd - off;
          const bool vis = (d >= ms.a) & ((d < ms.b) | (jb + off < ms.sink) | dense_row);
          s[kb][qb][e] = vis ? s[kb][qb][e] : kNegInf;
        }
      }
    }

    // Online softmax with a lazily moved reference max: the exponent base m
    // only changes when a row max exceeds it by more than kSlack (log2
    // units), so P <= 2^kSlack and the accumulator rescale is rare.
    bf16x8 pf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = kNegInf;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][qb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (__any((mx - acc.m[qb]) * c > kSlack)) {
        const float mnew = fmaxf(acc.m[qb], mx);
        const float alpha = __builtin_amdgcn_exp2f((acc.m[qb] - mnew) * c);
        acc.m[qb] = mnew;
        acc.l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc.o[qb][db] *= alpha;
      }
      const float nb = -acc.m[qb] * c;
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][e], c, nb));
        s[kb][qb][e] = pv;
        sum += pv;
      }
      acc.l[qb] += sum;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[qb][h2][e] = (__bf16)s[kb][qb][h2 * 8 + e];
    }

#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int t4 = kb * 2 + h2;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vt + (db * 32 + lr) * VSTR + t4 * 16 + lh * 8);
        acc.o[0][db] = mfma(vf, pf[0][h2], acc.o[0][db]);
        acc.o[1][db] = mfma(vf, pf[1][h2], acc.o[1][db]);
      }
    }
  }
}

// The wave's 64 query rows -> LDS (rows >= N are zero).
__device__ __forceinline__ void load_q_lds(uint16_t* Qs, const uint16_t* __restrict__ Q, int N, int Hq, int h,
                                           int q0, int lane) {
#pragma unroll 4
  for (int c = 0; c < 16; ++c) {
    const int id = c * 64 + lane;        // 1024 chunks of 16 B
    const int row = id >> 4, dc = id & 15;
    const int i = q0 + row;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (i < N) v = *reinterpret_cast<const u32x4*>(Q + ((size_t)i * Hq + h) * D + dc * 8);
    *reinterpret_cast<u32x4*>(Qs + row * KSTR + dc * 8) = v;
  }
}

__device__ __forceinline__ void acc_init(WaveAcc& acc) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    acc.m[qb] = kMInit;
    acc.l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.o[qb][db][e] = 0.f;
  }
}

__device__ __forceinline__ void store_o(const WaveAcc& acc, float* __restrict__ O, float* __restrict__ lse,
                                        int slot, int N, int Hq, int h, int q0, int lane, float c) {
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = acc.l[qb] + __shfl_xor(acc.l[qb], 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int i = q0 + qb * 32 + lr;
    if (i >= N) continue;
    if (lse != nullptr && lh == 0) lse[(size_t)slot * N + i] = acc.m[qb] * c + __log2f(lt);
    float* row = O + ((size_t)i * Hq + h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 v;
        v.x = acc.o[qb][db][r4 * 4 + 0] * inv;
        v.y = acc.o[qb][db][r4 * 4 + 1] * inv;
        v.z = acc.o[qb][db][r4 * 4 + 2] * inv;
        v.w = acc.o[qb][db][r4 * 4 + 3] * inv;
        *reinterpret_cast<float4*>(row + db * 32 + lh * 4 + r4 * 8) = v;
      }
  }
}

// Shared pipeline over T tiles; k0_of(idx) is the first key of tile idx.
// Tile t+1 is in flight (registers) while tile t is computed from LDS.
template <class K0Of>
__device__ __forceinline__ void run_tiles(const AttnParams& p, uint16_t* smem, int T, int g, int h, int slot,
                                          bool active, int q0, const MaskSpec& ms, K0Of&& k0_of) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t rs = (size_t)p.Hkv * D;
  uint16_t* Qs = smem + 2 * BUF_ELEMS + wave * Q_ELEMS;
  WaveAcc acc;
  acc_init(acc);
  if (active) load_q_lds(Qs, p.Q, p.N, p.Hq, h, q0, lane);

  TileRegs r;
  int rows[8];
  int k0 = k0_of(0);
  contiguous_rows(rows, k0, p.N, tid);
  tile_load(r, p.K, p.V, rows, rs, g, tid);
  tile_store(r, smem, tid);
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    const int cur = k0;
    if (t + 1 < T) {
      k0 = k0_of(t + 1);
      contiguous_rows(rows, k0, p.N, tid);
      tile_load(r, p.K, p.V, rows, rs, g, tid);
    }
    if (active) tile_compute(smem + (t & 1) * BUF_ELEMS, Qs, acc, lane, q0, cur, ms, p.c);
    if (t + 1 < T) tile_store(r, smem + ((t + 1) & 1) * BUF_ELEMS, tid);
    __syncthreads();
  }
  if (active) store_o(acc, p.O, p.lse, slot, p.N, p.Hq, h, q0, lane, p.c);
}

__global__ __launch_bounds__(NT, 1) void attn_band_kernel(AttnParams p, PackTable packs) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];
  const int wave = threadIdx.x >> 6;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int pk = lid / p.n_qt;
  int qt = lid % p.n_qt;
  if (p.kind != SWA) qt = p.n_qt - 1 - qt;   // long causal rows first
  const uint32_t pw = packs.heads[pk];
  const int h = (pw >> (8 * wave)) & 0xFF;
  const bool active = h != 0xFF;
  const int g = (int)(pw & 0xFF) / p.G;
  const int q0 = qt * BK;
  const int hi_t = min(p.N - 1, q0 + 63) >> 6;

  MaskSpec ms;
  int bl = 0, st = 0;
  if (p.kind == DENSE) {
    ms = {0, INT_MAX, 0, INT_MAX};
  } else if (p.kind == SWA) {
    ms = {0, p.window, 0, INT_MAX};
    bl = max(0, q0 - p.window + 1) >> 6;
  } else {  // TRIANGLE
    ms = {0, p.window, p.sink, p.dense_from};
    if (q0 + 63 < p.dense_from) {
      bl = max(0, q0 - p.window + 1) >> 6;
      st = min((p.sink + 63) >> 6, bl);
    }
  }
  const int T = st + (hi_t - bl + 1);
  const int slot = (packs.slots[pk] >> (8 * wave)) & 0xFF;
  run_tiles(p, smem, T, g, h, slot, active, q0, ms,
            [&](int idx) { return (idx < st ? idx : bl + idx - st) * BK; });
}

}  // namespace

hipError_t launch_attn_band(const AttnParams& p, const PackTable& packs, hipStream_t s) {
  const int nwg = packs.n * p.n_qt;
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_band_kernel, dim3(nwg), dim3(NT), 0, s, p, packs);
  return hipGetLastError();
}

}  // namespace ha
