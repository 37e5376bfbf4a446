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
// Workgroup = 8 waves, two per SIMD.  A workgroup serves a "pack" of heads of
// one KV head: 64 query rows of 4 heads, 128 rows of 2 heads or 256 rows of
// one head, so every 64-key K/V tile staged in LDS serves 256 query rows;
// wave w takes head slot w % n and query rows 32 * (w / n) .. +31 of the
// workgroup's rows (n = heads in the pack).  A wave needs about 200
// registers (Q fragments, a 64 x 32 score tile and a 128 x 32 output
// accumulator), so two waves share each SIMD and the hardware overlaps one
// wave's softmax with the other's matrix products and LDS reads.  Tiles are
// double-buffered in LDS: a step stages tile t+1 from registers, starts the
// loads of tile t+2 and computes tile t; waves 0-3 stage V (transposed),
// waves 4-7 stage K.
//
// Per wave and 64-key tile the contraction is laid out transposed,
//   S^T[key][query] = K Q^T     (A = K rows from LDS, B = Q^T held in registers)
//   O^T[d][query]  += V^T P^T   (A = V^T rows from LDS, B = P^T from registers)
// so that each lane owns one query column: the row max / row sum of a query
// live in one lane pair (lane, lane^32), and P never leaves registers.
#include "common.h"
#include "device_util.h"

#include <limits.h>

#include <algorithm>

namespace ha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
constexpr int SMEM_ELEMS = 2 * BUF_ELEMS;
constexpr int NT = 512;
constexpr int QW = 32;               // query rows per wave
constexpr float kNegInf = -__builtin_inff();
constexpr float kMInit = -1e30f;     // finite start for the running max
constexpr float kSlack = 8.f;        // log2 headroom before the reference max moves

// visible(i, j) = j <= i - a  &&  (i - j < b  ||  j < sink  ||  i >= dense_from)
struct MaskSpec {
  int a, b, sink, dense_from;
};

// One thread's share of a 64-key K/V tile: threads 0-255 hold 4 keys x 8 d
// of V, threads 256-511 four 16-byte chunks of K rows.
struct TileRegs {
  u32x4 x[4];
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Per-thread source of its share of a tile: V threads read key slots
// 4*(t%16) + x at d = 8*(t/16) .. +8; K threads read chunk id = c*256 + t ->
// key slot id/16, d = (id%16)*8 (coalesced rows).  Slot x of the tile is key
// k0 + kbase + x*kstep.  The tensor base is uniform per wave (waves 0-3 read
// V, 4-7 K), so a load is that scalar base plus a 32-bit per-lane offset.
struct TileSrc {
  const char* base;       // tensor + KV head offset (wave-uniform)
  uint32_t off[4];        // byte offsets of the thread's slots for k0 = 0
  int kbase, kstep, dbyte;
};

__device__ __forceinline__ TileSrc tile_src(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                            int g, int rs, int tid, bool v_wave) {
  TileSrc s;
  const uint16_t* t = v_wave ? V : K;
  s.base = reinterpret_cast<const char*>(t + g * D);
  if (v_wave) {
    s.kbase = (tid & 15) * 4;
    s.kstep = 1;
    s.dbyte = (tid >> 4) * 16;
  } else {
    const int u = tid - 256;
    s.kbase = u >> 4;
    s.kstep = 16;
    s.dbyte = (u & 15) * 16;
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) s.off[x] = (uint32_t)((s.kbase + x * s.kstep) * rs * 2 + s.dbyte);
  return s;
}

// Global -> registers for the 64-key tile starting at k0.  Keys past the end
// of the sequence are read as key N-1: they lie after every query row, so
// the causal mask removes them (P = 0) and the finite stand-in values leave
// the products exact.  No per-lane branches, so the loads stay in flight
// until the LDS store needs them.
__device__ __forceinline__ void tile_load(TileRegs& r, const TileSrc& src, int k0, int N, int rs) {
  const char* p = src.base + (size_t)k0 * rs * 2;
  if (k0 + BK <= N) {
#pragma unroll
    for (int x = 0; x < 4; ++x) r.x[x] = *reinterpret_cast<const u32x4*>(p + src.off[x]);
  } else {
    const int lim = N - 1 - k0;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int kr = min(src.kbase + x * src.kstep, lim);
      r.x[x] = *reinterpret_cast<const u32x4*>(p + (uint32_t)(kr * rs * 2 + src.dbyte));
    }
  }
}

// Position of key u (0..15) of a 16-key PV k-step inside an LDS V^T row, so
// that the 8 keys one MFMA lane consumes are contiguous.  A lane of half
// g = lane/32 holds, for C-layout element e, key g*4 + (e/4)*8 + e%4; the
// slot it feeds at k-step element e' (0..7) is 8g + e'.
__device__ __forceinline__ int vt_pos(int u) {
  return 8 * ((u >> 2) & 1) + 4 * (u >> 3) + (u & 3);
}

__device__ __forceinline__ void tile_store(const TileRegs& r, uint16_t* buf, int tid, bool v_wave) {
  if (v_wave) {
    uint16_t* Vt = buf + K_ELEMS;
    const int kg = tid & 15, dc = tid >> 4;
    const int pos = 16 * (kg >> 2) + vt_pos((kg * 4) & 15);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // keys x = 0..3 of d = dc*8 + 2w (low halves) and dc*8 + 2w + 1 (high)
      const uint32_t a0 = r.x[0][w], a1 = r.x[1][w], a2 = r.x[2][w], a3 = r.x[3][w];
      u32x2 ev, od;
      ev[0] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
      ev[1] = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
      od[0] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
      od[1] = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
      *reinterpret_cast<u32x2*>(Vt + (dc * 8 + 2 * w) * VSTR + pos) = ev;
      *reinterpret_cast<u32x2*>(Vt + (dc * 8 + 2 * w + 1) * VSTR + pos) = od;
    }
  } else {
    uint16_t* Ks = buf;
    const int t = tid - 256;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int id = c * 256 + t;
      *reinterpret_cast<u32x4*>(Ks + (id >> 4) * KSTR + (id & 15) * 8) = r.x[c];
    }
  }
}

// Instruction-scheduler pins for a block of 16 MFMAs fed by 16 LDS fragment
// reads: the first kAhead reads, then (MFMA, read) pairs, then the last
// MFMAs, so each read has about kAhead MFMA issue slots (32 cycles each) to
// land.  Other instructions are placed freely around them.
constexpr int kAhead = 4;
template <int Id>
__device__ __forceinline__ void schedule_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, kAhead, Id);   // DS reads
#pragma unroll
  for (int n = 0; n < 16 - kAhead; ++n) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, Id);      // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, Id);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kAhead, Id);
}


struct WaveAcc {
  f32x16 o[4];   // O^T: [d block]
  float m;       // running max (raw score units) of this lane's query
  float l;       // running sum, partial over this lane's keys
};

// Every key of the tile visible to every one of the wave's 32 rows.
__device__ __forceinline__ bool tile_full(const MaskSpec& ms, int q0, int k0) {
  if (k0 + 63 > q0 - ms.a) return false;
  if ((q0 + QW - 1) - k0 < ms.b) return true;
  if (k0 + 63 < ms.sink) return true;
  if (q0 >= ms.dense_from) return true;
  return false;
}

// No key of the tile visible to any of the wave's rows.
__device__ __forceinline__ bool tile_empty(const MaskSpec& ms, int q0, int k0) {
  if (k0 > q0 + QW - 1 - ms.a) return true;                     // all keys after every row
  if (q0 + QW - 1 >= ms.dense_from) return false;
  if (k0 < ms.sink) return false;
  return q0 - (k0 + 63) >= ms.b;                                // all keys behind every window
}

// One 64-key tile (keys k0 .. k0+63) against the wave's 32 query rows: one
// online-softmax step.  kSplitQ: the query is the sum of two bf16 parts,
// qf in registers and the low part in LDS (qlo: this wave's 8 fragments x
// 64 lanes), so S takes two products per k-step.
template <bool kSplitQ>
__device__ __forceinline__ void tile_compute(const uint16_t* __restrict__ buf, const bf16x8 (&qf)[8],
                                             const uint16_t* __restrict__ qlo, WaveAcc& acc, int lane, int q0,
                                             int k0, const MaskSpec& ms, float c) {
  const uint16_t* Ks = buf;
  const uint16_t* Vt = buf + K_ELEMS;
  const int lr = lane & 31, lh = lane >> 5;
  const bool full = tile_full(ms, q0, k0);

  // S^T = K Q^T: [key half] x 32 queries
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    bf16x8 qlt;
    if constexpr (kSplitQ) qlt = *reinterpret_cast<const bf16x8*>(qlo + (t * 64 + lane) * 8);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + lr) * KSTR + t * 16 + lh * 8);
      s[kb] = mfma(kf, qf[t], s[kb]);
      if constexpr (kSplitQ) s[kb] = mfma(kf, qlt, s[kb]);
    }
  }
  // issue order: fragment reads run kAhead MFMAs ahead of their use
  if constexpr (!kSplitQ) schedule_reads_ahead<0>();

  if (!full) {
    const int i = q0 + lr;
    const bool dense_row = i >= ms.dense_from;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int jb = k0 + kb * 32 + lh * 4;
      const int dd = i - jb;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int off = (e >> 2) * 8 + (e & 3);
        const int d = dd - off;
        const bool vis = (d >= ms.a) & ((d < ms.b) | (jb + off < ms.sink) | dense_row);
        s[kb][e] = vis ? s[kb][e] : kNegInf;
      }
    }
  }

  // Online softmax with a lazily moved reference max: the exponent base m
  // only changes when a row max exceeds it by more than kSlack (log2
  // units), so P <= 2^kSlack and the accumulator rescale is rare.
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
  mx = dev::pair32_max(mx);
  if (__any((mx - acc.m) * c > kSlack)) {
    const float mnew = fmaxf(acc.m, mx);
    const float alpha = __builtin_amdgcn_exp2f((acc.m - mnew) * c);
    acc.m = mnew;
    acc.l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) acc.o[db] *= alpha;
  }
  // P in bf16 feeds the PV product; the row sum adds the same bf16 values
  // (v_dot2 against (1, 1)), so numerator and denominator use equal weights
  const float nb = -acc.m * c;
  float sum = 0.f;
  bf16x8 pf[2][2];
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[kb][h2][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][h2 * 8 + e], c, nb));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 pr = {pf[kb][h2][2 * q], pf[kb][h2][2 * q + 1]};
        sum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum, false);
      }
    }
  }
  acc.l += sum;

#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int t4 = kb * 2 + h2;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vt + (db * 32 + lr) * VSTR + t4 * 16 + lh * 8);
        acc.o[db] = mfma(vf, pf[kb][h2], acc.o[db]);
      }
    }
  schedule_reads_ahead<1>();
}

// Q^T fragments (B operands) of the wave's 32 query rows; rows >= N are zero.
__device__ __forceinline__ void load_q(bf16x8 (&qf)[8], const uint16_t* __restrict__ Q, int N, int Hq, int h,
                                       int q0, int lane) {
  const int i = q0 + (lane & 31), lh = lane >> 5;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (i < N) {
      qf[t] = *reinterpret_cast<const bf16x8*>(Q + ((size_t)i * Hq + h) * D + t * 16 + lh * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[t][e] = (__bf16)0.f;
    }
  }
}

__device__ __forceinline__ void acc_init(WaveAcc& acc) {
  acc.m = kMInit;
  acc.l = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc.o[db][e] = 0.f;
}

__device__ __forceinline__ void store_o(const WaveAcc& acc, float* __restrict__ O, float* __restrict__ lse,
                                        int slot, int N, int Hq, int h, int q0, int lane, float c) {
  const int lr = lane & 31, lh = lane >> 5;
  const float lt = dev::pair32_sum(acc.l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int i = q0 + lr;
  if (i >= N) return;
  if (lse != nullptr && lh == 0) lse[(size_t)slot * N + i] = acc.m * c + __log2f(lt);
  float* row = O + ((size_t)i * Hq + h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 v;
      v.x = acc.o[db][r4 * 4 + 0] * inv;
      v.y = acc.o[db][r4 * 4 + 1] * inv;
      v.z = acc.o[db][r4 * 4 + 2] * inv;
      v.w = acc.o[db][r4 * 4 + 3] * inv;
      *reinterpret_cast<float4*>(row + db * 32 + lh * 4 + r4 * 8) = v;
    }
}

// Orthros cross-attention query of the wave's rows: q' = q * s_h + o_h in
// fp32 (Orthros page, design section: a scale-offset separates the cross-
// attention query from the SWA query), held as two bf16 parts hi + lo
// (relative error ~2^-16): hi in registers, lo in the wave's LDS region
// (written and read back by the same lane); rows >= N are zero.
__device__ __forceinline__ void load_q_cross(bf16x8 (&qh)[8], uint16_t* qlo, const AttnParams& p, int h, int q0,
                                             int lane) {
  const int i = q0 + (lane & 31), lh = lane >> 5;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int d0 = t * 16 + lh * 8;
    if (i < p.N) {
      const bf16x8 q = *reinterpret_cast<const bf16x8*>(p.Q + ((size_t)i * p.Hq + h) * D + d0);
      const float* sp = p.xs + (size_t)h * D + d0;
      const float* op = p.xo + (size_t)h * D + d0;
      bf16x8 lo8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 hi, lo;
        dev::split2(fmaf((float)q[e], sp[e], op[e]), hi, lo);
        qh[t][e] = hi;
        lo8[e] = lo;
      }
      *reinterpret_cast<bf16x8*>(qlo + (t * 64 + lane) * 8) = lo8;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qh[t][e] = (__bf16)0.f;
      *reinterpret_cast<bf16x8*>(qlo + (t * 64 + lane) * 8) = qh[t];
    }
  }
}

// Cross-attention rows: normalised output to O_out (one key chunk), or the
// chunk's normalised partial and log2-sum-exp (split key range).
__device__ __forceinline__ void store_cross(const WaveAcc& acc, const AttnParams& p, int kc, int h, int q0,
                                            int lane) {
  const int lr = lane & 31, lh = lane >> 5;
  const float lt = dev::pair32_sum(acc.l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int i = q0 + lr;
  if (i >= p.N) return;
  const size_t r = (size_t)(i - p.row0);
  float* row;
  if (p.n_kc == 1) {
    row = p.O_out + (r * p.Hq + h) * D;
  } else {
    const size_t pr = ((size_t)kc * p.n_out + r) * p.Hq + h;
    row = p.part + pr * D;
    if (lh == 0) p.part_lse[pr] = lt > 0.f ? acc.m * p.c + __log2f(lt) : -__builtin_inff();
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 v;
      v.x = acc.o[db][r4 * 4 + 0] * inv;
      v.y = acc.o[db][r4 * 4 + 1] * inv;
      v.z = acc.o[db][r4 * 4 + 2] * inv;
      v.w = acc.o[db][r4 * 4 + 3] * inv;
      *reinterpret_cast<float4*>(row + db * 32 + lh * 4 + r4 * 8) = v;
    }
}

// Shared pipeline over T tiles; k0_of(idx) is the first key of tile idx.
// Step t first stages tile t+1 (registers loaded during step t-1) into the
// other LDS buffer, which tile t-1 left before the last barrier, and starts
// the global loads of tile t+2 into the same registers; then it computes
// tile t.  The LDS writes drain under the compute; one barrier per step.
// kCross: Orthros cross-attention rows (split query, low parts in LDS after
// the two tile buffers; output to O_out or the partials of key chunk `slot`).
template <bool kCross, class K0Of>
__device__ __forceinline__ void run_tiles(const AttnParams& p, uint16_t* smem, int T, int g, int h, int slot,
                                          bool active, int q0, const MaskSpec& ms, K0Of&& k0_of) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int rs = p.Hkv * D;   // elements between consecutive keys
  bf16x8 qf[8];
  uint16_t* qlo = kCross ? smem + SMEM_ELEMS + (tid >> 6) * (8 * 64 * 8) : nullptr;
  WaveAcc acc;
  acc_init(acc);
  if (active) {
    if constexpr (kCross) load_q_cross(qf, qlo, p, h, q0, lane);
    else load_q(qf, p.Q, p.N, p.Hq, h, q0, lane);
  }

  TileRegs r;
  const bool v_wave = __builtin_amdgcn_readfirstlane(tid >> 6) < 4;
  const TileSrc src = tile_src(p.K, p.V, g, rs, tid, v_wave);
  tile_load(r, src, k0_of(0), p.N, rs);
  tile_store(r, smem, tid, v_wave);
  if (T > 1) tile_load(r, src, k0_of(1), p.N, rs);
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    if (t + 1 < T) {
      tile_store(r, smem + ((t + 1) & 1) * BUF_ELEMS, tid, v_wave);
      if (t + 2 < T) tile_load(r, src, k0_of(t + 2), p.N, rs);
    }
    const int cur = k0_of(t);
    if (active && !tile_empty(ms, q0, cur))
      tile_compute<kCross>(smem + (t & 1) * BUF_ELEMS, qf, qlo, acc, lane, q0, cur, ms, p.c);
    __syncthreads();
  }
  if (active) {
    if constexpr (kCross) store_cross(acc, p, slot, h, q0, lane);
    else store_o(acc, p.O, p.lse, slot, p.N, p.Hq, h, q0, lane, p.c);
  }
}

// A band work item: one pack of heads x one tile of query rows (64 rows of
// 4 heads, 128 of 2 or 256 of 1), with its closed-form key-tile schedule:
// tiles idx < st are the sink tiles idx * 64, the rest the band tiles
// bl + idx - st (no tile without a visible key for some row of the item).
struct BandItem {
  int valid;
  int pk;         // pack
  int sh;         // log2 of the heads per pack
  int qt0;        // first query row
  int g;          // KV head
  int bl, st, T;  // tile schedule
};

// Item lid in the launch's order: pack classes in turn (4-, 2-, 1-head
// packs), pack by pack, and inside a pack the row tiles from the last (the
// longest causal rows) to the first for dense and triangle heads.
__device__ __forceinline__ BandItem band_item(const AttnParams& p, const PackTable& packs, int lid) {
  BandItem it{};
  if (lid < 0) return it;
  int c = 0, rem = lid, base = 0, nq = 1;
  for (; c < 3; ++c) {
    nq = (p.N + (BK << c) - 1) / (BK << c);
    const int nwg = p.band_np[c] * nq;
    if (rem < nwg) break;
    rem -= nwg;
    base += p.band_np[c];
  }
  if (c == 3) return it;
  it.valid = 1;
  it.pk = base + rem / nq;
  int qt = rem % nq;
  if (p.kind != SWA) qt = nq - 1 - qt;
  it.sh = 2 - c;
  const int rows = BK << c;
  it.qt0 = qt * rows;
  it.g = (int)(packs.heads[it.pk] & 0xFF) / p.G;
  const int hi_t = min(p.N - 1, it.qt0 + rows - 1) >> 6;
  if (p.kind == SWA) {
    it.bl = max(0, it.qt0 - p.window + 1) >> 6;
  } else if (p.kind == TRIANGLE && it.qt0 + rows - 1 < p.dense_from) {
    it.bl = max(0, it.qt0 - p.window + 1) >> 6;
    it.st = min((p.sink + 63) >> 6, it.bl);
  }
  it.T = it.st + (hi_t - it.bl + 1);
  return it;
}

__device__ __forceinline__ int item_k0(const BandItem& it, int idx) {
  return (idx < it.st ? idx : it.bl + idx - it.st) * BK;
}

// Persistent banded / dense / triangle kernel.  Every workgroup (one per CU)
// takes items of its XCD's share of the launch order (XCD x = workgroup id
// mod nx serves a contiguous range of items, so the items resident on one XCD
// are neighbouring row tiles of one pack, whose band tiles overlap in its
// L2): first three fixed items (its rank, + the XCD's workgroup count, + twice
// that), then one item at a time from the XCD's counter, so long items (the
// dense last rows of a triangle layer come first in the order) spread over
// workgroups and the rest balance around them.  The K/V tile pipeline runs
// across item boundaries: the next item's first tiles are staged while the
// current item's last tiles compute, so a new item starts without waiting
// for its first tile.  Three items are known at any time (the one computing
// and the next two): the pipeline looks at most two tiles ahead.
__global__ __launch_bounds__(NT, 1) void attn_band_kernel(AttnParams p, PackTable packs, uint32_t* ctr,
                                                          int n_items) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];
  __shared__ int s_next;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int nx = min(8, (int)gridDim.x);
  const int x = blockIdx.x % nx, j = blockIdx.x / nx;
  const int nW = ((int)gridDim.x - x + nx - 1) / nx;      // workgroups of this XCD share
  const int per = n_items / nx, rem = n_items % nx;
  const int lo = x * per + min(x, rem), hi = lo + per + (x < rem ? 1 : 0);
  auto item_id = [&](int k) { return k < hi ? k : -1; };

  BandItem I0 = band_item(p, packs, item_id(lo + j));
  if (!I0.valid) return;
  BandItem I1 = band_item(p, packs, item_id(lo + j + nW));
  BandItem I2 = band_item(p, packs, item_id(lo + j + 2 * nW));

  MaskSpec ms;
  if (p.kind == DENSE) ms = {0, INT_MAX, 0, INT_MAX};
  else if (p.kind == SWA) ms = {0, p.window, 0, INT_MAX};
  else ms = {0, p.window, p.sink, p.dense_from};

  const int rs = p.Hkv * D;   // elements between consecutive keys
  const bool v_wave = __builtin_amdgcn_readfirstlane(tid >> 6) < 4;
  TileRegs r;
  auto src_for = [&](int g) { return tile_src(p.K, p.V, g, rs, tid, v_wave); };

  // loader cursor: the position whose tile the registers hold: tile lj of
  // item L, which is lq items after the computing one (a copy, so that no
  // item is ever selected by a run-time index, which would put the queue in
  // scratch memory); valid while has_l
  BandItem L = I0;
  int lq = 0, lj = 0;
  bool has_l;
  auto advance = [&]() -> bool {
    if (lj + 1 < L.T) {
      ++lj;
      return true;
    }
    if (lq == 0 && I1.valid) {
      L = I1;
      lq = 1;
      lj = 0;
      return true;
    }
    if (lq == 1 && I2.valid) {
      L = I2;
      lq = 2;
      lj = 0;
      return true;
    }
    return false;
  };
  // prologue: the first tile into buffer 0, the second into registers
  tile_load(r, src_for(I0.g), item_k0(I0, 0), p.N, rs);
  tile_store(r, smem, tid, v_wave);
  has_l = advance();
  if (has_l) tile_load(r, src_for(L.g), item_k0(L, lj), p.N, rs);
  __syncthreads();

  int buf = 0;
  while (true) {
    // per-wave view of the item
    const int hs = wave & ((1 << I0.sh) - 1);
    const uint32_t pw = packs.heads[I0.pk];
    const int h = (pw >> (8 * hs)) & 0xFF;
    const int q0 = I0.qt0 + QW * (wave >> I0.sh);
    const bool active = h != 0xFF && q0 < p.N;
    const int slot = (packs.slots[I0.pk] >> (8 * hs)) & 0xFF;
    bf16x8 qf[8];
    WaveAcc acc;
    acc_init(acc);
    if (active) load_q(qf, p.Q, p.N, p.Hq, h, q0, lane);
    // the item's query fragments are complete before its tile loop, so the
    // loop's waits on them cannot also drain the tile loads in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    for (int t = 0; t < I0.T; ++t) {
      const bool last = t + 1 == I0.T;
      if (last && tid == 0) s_next = item_id(lo + 3 * nW + (int)atomicAdd(&ctr[x], 1u));
      if (has_l) {
        // stage the loaded tile into the other buffer, load the next one
        tile_store(r, smem + (buf ^ 1) * BUF_ELEMS, tid, v_wave);
        has_l = advance();
        if (has_l) tile_load(r, src_for(L.g), item_k0(L, lj), p.N, rs);
      }
      const int cur = item_k0(I0, t);
      if (active && !tile_empty(ms, q0, cur))
        tile_compute<false>(smem + buf * BUF_ELEMS, qf, nullptr, acc, lane, q0, cur, ms, p.c);
      __syncthreads();
      buf ^= 1;
    }
    if (active) store_o(acc, p.O, p.lse, slot, p.N, p.Hq, h, q0, lane, p.c);
    // next item: the queue moves up by one and takes the fetched item
    I0 = I1;
    I1 = I2;
    I2 = band_item(p, packs, __builtin_amdgcn_readfirstlane(s_next));
    if (has_l) --lq;
    if (!I0.valid) break;
    __syncthreads();   // every wave has read s_next before it is written again
  }
}

// Orthros cross-attention for many output positions (Orthros page: in
// pre-training every position predicts, in SFT the response positions do, so
// the cross-attention rows form a causal flash attention over all keys).
// Workgroup = (pack, 64-row tile of the rows row0 .. N-1, key chunk kc);
// chunks of kc_tiles key tiles spread short row ranges over the chip.
__global__ __launch_bounds__(NT, 1) void attn_cross_mfma_kernel(AttnParams p, PackTable packs) {
  // two tile buffers + the low query parts of the 8 waves (8 KB each)
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS + 8 * 8 * 64 * 8];
  const int wave = threadIdx.x >> 6;
  const int hs = wave & 3;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_pack = p.n_qt * p.n_kc;
  const int pk = lid / per_pack;
  const int rem = lid % per_pack;
  const int qt = p.n_qt - 1 - rem / p.n_kc;   // long causal rows first
  const int kc = rem % p.n_kc;
  const uint32_t pw = packs.heads[pk];
  const int h = (pw >> (8 * hs)) & 0xFF;
  const int g = (int)(pw & 0xFF) / p.G;
  const int qt0 = p.row0 + qt * BK;
  const int q0 = qt0 + QW * (wave >> 2);
  const bool active = h != 0xFF && q0 < p.N;
  const int n_tiles = (min(p.N - 1, qt0 + 63) >> 6) + 1;
  const int kt0 = kc * p.kc_tiles;
  const int T = min(n_tiles, kt0 + p.kc_tiles) - kt0;
  if (T <= 0) {   // chunk past the tile's last key: an empty partial
    if (active) {
      WaveAcc acc;
      acc_init(acc);
      store_cross(acc, p, kc, h, q0, threadIdx.x & 63);
    }
    return;
  }
  const MaskSpec ms = {0, INT_MAX, 0, INT_MAX};
  run_tiles<true>(p, smem, T, g, h, kc, active, q0, ms, [&](int idx) { return (kt0 + idx) * BK; });
}

// Merge of the key-chunk partials of one (output row, head): weights
// 2^(lse_c - max) on the normalised partials.
__global__ __launch_bounds__(D) void cross_merge_kernel(AttnParams p) {
  const int r = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  float M = -__builtin_inff();
  for (int kc = 0; kc < p.n_kc; ++kc) M = fmaxf(M, p.part_lse[((size_t)kc * p.n_out + r) * p.Hq + h]);
  float wsum = 0.f, acc = 0.f;
  if (M > -__builtin_inff()) {
    for (int kc = 0; kc < p.n_kc; ++kc) {
      const size_t pr = ((size_t)kc * p.n_out + r) * p.Hq + h;
      const float wgt = exp2f(p.part_lse[pr] - M);
      wsum += wgt;
      acc = fmaf(wgt, p.part[pr * D + d], acc);
    }
  }
  p.O_out[((size_t)r * p.Hq + h) * D + d] = wsum > 0.f ? acc / wsum : 0.f;
}

}  // namespace

// Clears the per-XCD item counters of a persistent launch.
__global__ void clear_counters_kernel(uint32_t* ctr) {
  if (threadIdx.x < kBandCounters) ctr[threadIdx.x] = 0u;
}

hipError_t launch_attn_band(const AttnParams& p, const PackTable& packs, uint32_t* ctr, hipStream_t s) {
  if (p.band_np[0] + p.band_np[1] + p.band_np[2] != packs.n) return hipErrorInvalidValue;
  int n_items = 0;
  for (int c = 0; c < 3; ++c) n_items += p.band_np[c] * ((p.N + (BK << c) - 1) / (BK << c));
  if (n_items == 0) return hipSuccess;
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(clear_counters_kernel, dim3(1), dim3(64), 0, s, ctr);
  // one workgroup per CU (the kernel's registers and LDS allow one)
  const int grid = std::max(1, std::min(n_items, n_cu));
  hipLaunchKernelGGL(attn_band_kernel, dim3(grid), dim3(NT), 0, s, p, packs, ctr, n_items);
  return hipGetLastError();
}

hipError_t launch_attn_cross(const AttnParams& p, const PackTable& packs, hipStream_t s) {
  const int nwg = packs.n * p.n_qt * p.n_kc;
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_cross_mfma_kernel, dim3(nwg), dim3(NT), 0, s, p, packs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_kc == 1) return e;
  hipLaunchKernelGGL(cross_merge_kernel, dim3(p.n_out, p.Hq), dim3(D), 0, s, p);
  return hipGetLastError();
}

}  // namespace ha
