// Retrieval heads: attention over the indexer-selected keys outside the local
// window, merged into the window result.
//
// RTPurbo post: the 16-dim indexer picks candidate keys from the past
// context, then exact softmax attention runs on that small set in full head
// dimension, next to the head's local window.  The key set of row i is
//   window(i) U {j <= i - w : j in a selected key block / selected cluster}
// (U key block 0 when forced).  The window part is computed by the banded
// kernel, which also leaves the row's log2-sum-exp; this kernel computes the
// selected part for one (retrieval head, 64-row query block) and merges:
//   O = (O_win 2^lse_win + O_sel 2^lse_sel) / (2^lse_win + 2^lse_sel).
//
// The selected part reads K/V rows by position.  In cluster mode the members
// of a cluster lie anywhere in the sequence; a copy of K and V in CSR order
// (made once per layer after k-means, one pass over K/V) turns the visible
// members of a selected cluster (a prefix of its ascending member list) into
// one contiguous range of rows, so tiles are read as runs of rows rather
// than as 64 rows from 64 places.  Each tile slot carries two numbers: the
// row it loads (CSR index or key position; looked up from LDS, no memory
// read) and the key position that the causal / window mask tests (read from
// the CSR together with the tile's K/V rows and staged in LDS with them).
//
// A workgroup takes one (head, 64-row query block); each 64-key gathered
// tile is staged in LDS (K rows, V transposed) and split between the waves:
// wave w owns query rows
// 32 (w % 2) .. +31 and key half w / 2 (keys 32 (w / 2) .. +31 of every
// tile), so a wave reads half a tile per step.  S^T = K Q^T and O^T += V^T P^T
// on v_mfma_f32_32x32x16_bf16 (a lane owns one query column), fp32 online
// softmax per key half; the two halves' (max, sum, O) are merged through LDS
// at the end.  Rows of tile t+2 are looked up while tile t is computed and
// tile t+1 is in flight; two workgroups fit on a CU.
#include "common.h"
#include "device_util.h"

#include <limits.h>

namespace ha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int KSTR = D + 8;
constexpr int VSTR = BK + 8;
constexpr int K_ELEMS = BK * KSTR;
constexpr int V_ELEMS = D * VSTR;
constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
constexpr float kNegInf = -__builtin_inff();
constexpr float kMInit = -1e30f;
constexpr float kSlack = 8.f;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of key u (0..15) of a 16-key PV k-step inside an LDS V^T row, so
// that the 8 keys one MFMA lane consumes are contiguous.  A lane of half
// g = lane/32 holds, for C-layout element e, key g*4 + (e/4)*8 + e%4; the
// slot it feeds at k-step element e' (0..7) is 8g + e'.
__device__ __forceinline__ int vt_pos(int u) { return 8 * ((u >> 2) & 1) + 4 * (u >> 3) + (u & 3); }

struct TileRegs {
  u32x4 k[4];
  u32x4 v[4];
  int row, pos;   // row of slot `lane` and the word read for its key position
};

// Key position of a tile slot: the CSR member at that index in cluster mode,
// else the row itself; -1 for an empty slot.  Every wave issues the read
// (block mode reads a word of `any`, a valid address, and ignores it): no
// branch around it, and it is not used until the tile is staged (pos_of),
// so it stays in flight with the tile's rows.
__device__ __forceinline__ void slot_position(const int32_t* __restrict__ mem, const int32_t* __restrict__ any,
                                              int row, int& r_row, int& r_pos) {
  r_row = row;
  r_pos = mem ? mem[max(row, 0)] : *any;
}
__device__ __forceinline__ int pos_of(int row, int pos, bool clus) { return row < 0 ? -1 : (clus ? pos : row); }

// K slots c*16 + tid/16 (16-B chunk tid%16); V slots 4*(tid%16) + x (d chunk
// tid/16).  Kb / Vb point at the KV head's first row, rs = elements between
// rows.  Empty slots (row -1) read row 0: the mask drops them (P = 0) and
// the finite stand-in values leave the products exact; no per-lane
// branches, so the loads stay in flight until the LDS store.
__device__ __forceinline__ void tile_load(TileRegs& r, const uint16_t* __restrict__ Kb,
                                          const uint16_t* __restrict__ Vb, const int* kidx, size_t rs, int tid,
                                          const int32_t* __restrict__ mem) {
  slot_position(mem, reinterpret_cast<const int32_t*>(Kb), kidx[tid & 63], r.row, r.pos);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int row = max(0, kidx[c * 16 + (tid >> 4)]);
    r.k[c] = *reinterpret_cast<const u32x4*>(Kb + (size_t)row * rs + (tid & 15) * 8);
  }
  const int dc = tid >> 4;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int row = max(0, kidx[(tid & 15) * 4 + x]);
    r.v[x] = *reinterpret_cast<const u32x4*>(Vb + (size_t)row * rs + dc * 8);
  }
}

__device__ __forceinline__ void tile_store(const TileRegs& r, uint16_t* buf, int* kposb, int tid, bool pos_wave,
                                           bool clus) {
  uint16_t* Ks = buf;
  uint16_t* Vt = buf + K_ELEMS;
  if (pos_wave) kposb[tid & 63] = pos_of(r.row, r.pos, clus);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int id = c * NT + tid;
    *reinterpret_cast<u32x4*>(Ks + (id >> 4) * KSTR + (id & 15) * 8) = r.k[c];
  }
  const int kg = tid & 15, dc = tid >> 4;
  const int pos = 16 * (kg >> 2) + vt_pos((kg * 4) & 15);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // keys x = 0..3 of d = dc*8 + 2w (low halves) and dc*8 + 2w + 1 (high)
    const uint32_t a0 = r.v[0][w], a1 = r.v[1][w], a2 = r.v[2][w], a3 = r.v[3][w];
    u32x2 ev, od;
    ev[0] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
    ev[1] = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
    od[0] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
    od[1] = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
    *reinterpret_cast<u32x2*>(Vt + (dc * 8 + 2 * w) * VSTR + pos) = ev;
    *reinterpret_cast<u32x2*>(Vt + (dc * 8 + 2 * w + 1) * VSTR + pos) = od;
  }
}

// Entries of one query block: key block 0 when forced, then the selected
// blocks / clusters (sel = the block's selection row).  For entry e:
// ent[e] = its first row (block id, or CSR start of the cluster) and
// cntv[e] = its keys at positions <= lim (a prefix of the block, or a prefix
// of the cluster's ascending member list).  Cluster counts: wave w takes
// entries w, w + NW, ... and counts members <= lim 64 at a time with a
// ballot; the first 64 members of 8 entries are read at once (independent
// loads, clamped into the member range), longer prefixes go on 64 at a
// time.  Every thread takes part; the results are visible on return.
template <int NW>
__device__ __forceinline__ void entry_table(const AttnParams& p, const int32_t* __restrict__ sel, int g, int lim,
                                            int ne, int* ent, int* ehi, int* cntv) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int f0 = p.force_block0 ? 1 : 0;
  const int n_kb = (p.N + BK - 1) / BK;
  const bool clus = p.M > 0;
  if (tid < ne) {
    int start = 0, cnt = 0, hi = 0;
    if (lim >= 0) {
      if (f0 && tid == 0) {
        cnt = min(BK, lim + 1);
      } else {
        const int v = sel[tid - f0];
        if (clus) {
          if (v >= 0 && v < p.M) {
            const int32_t* off = p.csr_off + (size_t)g * (p.M + 1);
            start = off[v];
            hi = off[v + 1];
          }
        } else if (v >= 0 && v < n_kb && !(f0 && v == 0)) {
          start = v;
          cnt = max(0, min(BK, lim - v * BK + 1));
        }
      }
    }
    ent[tid] = start;
    ehi[tid] = hi;
    cntv[tid] = cnt;
  }
  __syncthreads();
  if (!clus || lim < 0) return;
  const int32_t* mem = p.csr_mem + (size_t)g * p.N;
  for (int e0 = wave; e0 < ne; e0 += 8 * NW) {
    int lo[8], hi[8], m[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * NW;
      lo[u] = e < ne ? ent[e] : 0;
      hi[u] = e < ne ? ehi[e] : 0;
      m[u] = mem[min(lo[u] + lane, max(hi[u] - 1, 0))];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * NW;
      int c = (int)__popcll(__ballot(lo[u] + lane < hi[u] && m[u] <= lim));
      if (c == 64) {   // a full round: the prefix may go on
        for (int x0 = lo[u] + 64; x0 < hi[u]; x0 += 64) {
          const int x = x0 + lane;
          const int cc = (int)__popcll(__ballot(x < hi[u] && mem[min(x, hi[u] - 1)] <= lim));
          c += cc;
          if (cc < 64) break;
        }
      }
      if (e < ne && lane == 0) cntv[e] = c;
    }
  }
  __syncthreads();
}

struct Acc {
  f32x16 o[4];  // O^T: d block db -> rows d = 32 db + 4 (lane/32) + 8 (e/4) + e%4, column = the lane's query
  float m, l;   // running max (raw scores) and this lane's partial sum
};

// The wave's key half (keys 32 kh .. +31) of one tile against its 32 query
// rows.  Key j of slot s is visible to row i iff j >= 0 and j <= i - w
// (outside the window).
__device__ __forceinline__ void tile_compute(const uint16_t* __restrict__ buf, const int* __restrict__ kpos,
                                             const bf16x8 (&qf)[8], Acc& acc, int lane, int kh, int i, int w,
                                             float c) {
  const uint16_t* Ks = buf;
  const uint16_t* Vt = buf + K_ELEMS;
  const int lr = lane & 31, lh = lane >> 5;
  f32x16 s;
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kh * 32 + lr) * KSTR + t * 16 + lh * 8);
    s = mfma(kf, qf[t], s);
  }
  float mx = kNegInf;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int4 jv = *reinterpret_cast<const int4*>(kpos + kh * 32 + lh * 4 + q * 8);
    const int js[4] = {jv.x, jv.y, jv.z, jv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool vis = (js[e] >= 0) & (i - js[e] >= w);
      s[q * 4 + e] = vis ? s[q * 4 + e] : kNegInf;
      mx = fmaxf(mx, s[q * 4 + e]);
    }
  }
  mx = dev::pair32_max(mx);
  // lazily moved reference max (see the banded kernel): rescale only when a
  // row max exceeds it by more than kSlack in log2 units
  if (__any((mx - acc.m) * c > kSlack)) {
    const float mnew = fmaxf(acc.m, mx);
    const float alpha = __builtin_amdgcn_exp2f((acc.m - mnew) * c);
    acc.m = mnew;
    acc.l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) acc.o[db] *= alpha;
  }
  // P in bf16 feeds the PV product; the row sum adds the same bf16 values
  const float nb = -acc.m * c;
  float sum = 0.f;
  bf16x8 pf[2];
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int e = 0; e < 16; ++e) pf[e >> 3][e & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[e], c, nb));
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const bf16x2 pr = {pf[q >> 2][2 * (q & 3)], pf[q >> 2][2 * (q & 3) + 1]};
    sum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum, false);
  }
  acc.l += sum;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int t4 = kh * 2 + h2;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vt + (db * 32 + lr) * VSTR + t4 * 16 + lh * 8);
      acc.o[db] = mfma(vf, pf[h2], acc.o[db]);
    }
  }
}

__global__ __launch_bounds__(NT, 2) void attn_selected_kernel(AttnParams p, SelList sl) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BUF_ELEMS];
  __shared__ __attribute__((aligned(16))) int kidx[3][BK];    // row each slot loads
  __shared__ __attribute__((aligned(16))) int kposb[2][BK];   // key positions of the staged tiles
  __shared__ int ent[kMaxTopk + 1];     // block id (block mode) or CSR start (cluster mode)
  __shared__ int ehi[kMaxTopk + 1];     // cluster mode: end of the member range
  __shared__ int pre[kMaxTopk + 2];     // prefix of visible key counts per entry
  __shared__ int tmp4[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // XCD k (workgroup id mod 8) takes the query blocks b = k mod 8 of every
  // head, head after head, long blocks first: the workgroups resident on an
  // XCD are blocks of one head (which select mostly the same clusters /
  // blocks, so the rows they share come from that XCD's L2), and every XCD
  // gets a share of short and long blocks of every head
  const int xcd = blockIdx.x & 7, wg_slot = blockIdx.x >> 3;
  const int nq8 = (p.n_qt + 7) / 8;
  const int t = wg_slot / nq8;
  const int b = p.n_qt - 1 - ((wg_slot % nq8) * 8 + xcd);
  if (b < 0) return;   // padding of n_qt to a multiple of 8
  const int h = sl.head[t];
  const int g = h / p.G;
  const int q0 = b * BK;
  const int lim = min(p.N, q0 + BK) - 1 - p.window;   // keys j <= lim can be visible
  const int32_t* mem = p.csr_mem ? p.csr_mem + (size_t)g * p.N : nullptr;

  // entries: forced block 0 + the selection; count of keys j <= lim in each
  const int ne = p.topk + (p.force_block0 ? 1 : 0);
  entry_table<4>(p, p.sel + ((size_t)t * p.n_qt + b) * p.topk, g, lim, ne, ent, ehi, pre);
  const int cnt = tid < ne ? pre[tid] : 0;
  int total;
  const int excl = dev::block_excl_scan<4>(cnt, tmp4, &total);
  if (tid < ne) pre[tid] = excl;
  if (tid == 0) pre[ne] = total;
  __syncthreads();
  const int T = (total + BK - 1) / BK;
  if (T == 0) return;

  // row of slot s of tile idx (flat index f = 64 idx + s over the entries):
  // the key position (block mode) or the CSR index (cluster mode).  Slot s
  // of every tile is looked up by thread 4 s, so all waves share the work;
  // that thread's entry index (the largest e with pre[e] <= f) only moves
  // forward from tile to tile.
  const bool owner = (tid & 3) == 0;
  const int slot = tid >> 2;
  int cur_e = 0;
  auto lookup = [&](int idx, int s) -> int {
    const int f = idx * BK + s;
    if (f >= total) return -1;
    while (cur_e + 1 < ne && pre[cur_e + 1] <= f) ++cur_e;
    const int r = f - pre[cur_e];
    return p.M > 0 ? ent[cur_e] + r : ent[cur_e] * BK + r;
  };
  const int lr = lane & 31, lh = lane >> 5;
  const int kh = wave >> 1;                   // key half of every tile
  const int i = q0 + (wave & 1) * 32 + lr;    // this lane's query row
  bf16x8 qf[8];
#pragma unroll
  for (int t8 = 0; t8 < 8; ++t8) {
    if (i < p.N) {
      qf[t8] = *reinterpret_cast<const bf16x8*>(p.Q + ((size_t)i * p.Hq + h) * D + t8 * 16 + lh * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[t8][e] = (__bf16)0.f;
    }
  }
  Acc acc;
  acc.m = kMInit;
  acc.l = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc.o[db][e] = 0.f;

  const bool clus = p.M > 0;
  const size_t rs = clus ? (size_t)D : (size_t)p.Hkv * D;
  const uint16_t* Kb = clus ? p.Kc + (size_t)g * p.N * D : p.K + g * D;
  const uint16_t* Vb = clus ? p.Vc + (size_t)g * p.N * D : p.V + g * D;
  const int32_t* cmem = clus ? mem : nullptr;
  const bool pos_wave = __builtin_amdgcn_readfirstlane(wave) == 0;
  // every earlier global read (Q fragments, entry table) is complete here, so
  // the waits inside the loop count only the tile loads
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  if (owner) {
    kidx[0][slot] = lookup(0, slot);
    kidx[1][slot] = T > 1 ? lookup(1, slot) : -1;
  }
  __syncthreads();
  TileRegs r;
  tile_load(r, Kb, Vb, kidx[0], rs, tid, cmem);
  tile_store(r, smem, kposb[0], tid, pos_wave, clus);
  __syncthreads();
  for (int tt = 0; tt < T; ++tt) {
    if (tt + 1 < T) tile_load(r, Kb, Vb, kidx[(tt + 1) % 3], rs, tid, cmem);
    const bool prep = tt + 2 < T && owner;
    const int nrow = prep ? lookup(tt + 2, slot) : -1;
    tile_compute(smem + (tt & 1) * BUF_ELEMS, kposb[tt & 1], qf, acc, lane, kh, i, p.window, p.c);
    if (tt + 1 < T) tile_store(r, smem + ((tt + 1) & 1) * BUF_ELEMS, kposb[(tt + 1) & 1], tid, pos_wave, clus);
    if (prep) kidx[(tt + 2) % 3][slot] = nrow;
    __syncthreads();
  }

  // merge the key halves: waves 2, 3 hand (m, l, O) to waves 0, 1 through
  // LDS (the tile buffers are free after the loop's last barrier)
  float* xch = reinterpret_cast<float*>(smem) + (wave & 1) * (64 * 67);
  if (kh == 1) {
    float* x = xch + lane * 67;
    x[0] = acc.m;
    x[1] = acc.l;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) x[2 + db * 16 + e] = acc.o[db][e];
  }
  __syncthreads();
  if (kh == 1) return;
  {
    const float* x = xch + lane * 67;
    const float m1 = x[0], l1 = x[1];
    const float mm = fmaxf(acc.m, m1);
    const float a0 = __builtin_amdgcn_exp2f((acc.m - mm) * p.c), a1 = __builtin_amdgcn_exp2f((m1 - mm) * p.c);
    acc.m = mm;
    acc.l = acc.l * a0 + l1 * a1;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.o[db][e] = acc.o[db][e] * a0 + x[2 + db * 16 + e] * a1;
  }

  // merge with the window result of the row
  const float lt = dev::pair32_sum(acc.l);
  if (i >= p.N || !(lt > 0.f)) return;
  const float lse_s = acc.m * p.c + __log2f(lt);
  const float lse_w = p.lse[(size_t)t * p.N + i];
  const float M = fmaxf(lse_s, lse_w);
  const float ws = exp2f(lse_s - M), ww = exp2f(lse_w - M);
  const float inv = 1.f / (ws + ww);
  const float fs = ws * inv / lt, fw = ww * inv;
  float* row = p.O + ((size_t)i * p.Hq + h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4* dst = reinterpret_cast<float4*>(row + db * 32 + lh * 4 + r4 * 8);
      float4 v = *dst;
      v.x = fmaf(v.x, fw, acc.o[db][r4 * 4 + 0] * fs);
      v.y = fmaf(v.y, fw, acc.o[db][r4 * 4 + 1] * fs);
      v.z = fmaf(v.z, fw, acc.o[db][r4 * 4 + 2] * fs);
      v.w = fmaf(v.w, fw, acc.o[db][r4 * 4 + 3] * fs);
      *dst = v;
    }
}

// ---------------------------------------------------------------------------
// Group-shared selection (36kr interview, GQA answer: the query heads of one
// GQA group share their keys, so one selection serves the group).  Every
// retrieval head of a KV group then has the same key set per query block,
// window included, so one workgroup computes a pack of up to 4 of them
// completely: the window tiles (contiguous keys) and the gathered tiles go
// through one online softmax and O is written once (no separate window pass,
// no log2-sum-exp, no read-back of O).  8 waves: wave w takes head slot
// w % 4 and query rows 32 (w / 4) .. +31 and computes the whole tile, so a
// tile read from HBM serves 256 rows; waves 0-3 stage V (transposed), waves
// 4-7 K, wave 0 also the gathered slots' key positions.  Step t stages tile
// t+1 from registers, starts the loads of tile t+2, looks up the rows of
// gathered tile t+3 (from LDS only) and computes tile t; one barrier per
// step, and no wait inside a step covers the loads that step starts.
namespace grp {

constexpr int NT8 = 512;
constexpr int QW = 32;     // query rows per wave
constexpr int kRing = 4;   // looked-up rows of gathered tiles

struct Regs {
  u32x4 x[4];
  int row, pos;   // row of slot `lane` and the word read for its key position
};

// Thread's share of a tile: V threads (waves 0-3) read slots 4 (tid % 16) + x
// at d = 8 (tid / 16) .. +8; K threads read 16-byte chunk (u % 16) of slot
// 16 x + u / 16 (u = tid - 256).
__device__ __forceinline__ int slot_of(int tid, int x, bool v_wave) {
  return v_wave ? (tid & 15) * 4 + x : x * 16 + ((tid - 256) >> 4);
}
__device__ __forceinline__ int dbyte_of(int tid, bool v_wave) {
  return v_wave ? (tid >> 4) * 16 : ((tid - 256) & 15) * 16;
}

// Gathered tile: base = the KV head's first row (V or K, original or in CSR
// order), rs2 = bytes between rows; empty slots (row -1) read row 0.
__device__ __forceinline__ void load_gathered(Regs& r, const char* __restrict__ base, const int* kidx, int rs2,
                                              int tid, bool v_wave, const int32_t* __restrict__ mem) {
  slot_position(mem, reinterpret_cast<const int32_t*>(base), kidx[tid & 63], r.row, r.pos);
  const int db = dbyte_of(tid, v_wave);
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int row = max(0, kidx[slot_of(tid, x, v_wave)]);
    r.x[x] = *reinterpret_cast<const u32x4*>(base + (size_t)row * rs2 + db);
  }
}

// Window tile: keys k0 .. k0+63 (keys past N read key N-1; masked).
__device__ __forceinline__ void load_window(Regs& r, const char* __restrict__ base, int k0, int N, int rs2, int tid,
                                            bool v_wave) {
  const int db = dbyte_of(tid, v_wave);
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int row = min(k0 + slot_of(tid, x, v_wave), N - 1);
    r.x[x] = *reinterpret_cast<const u32x4*>(base + (size_t)row * rs2 + db);
  }
}

__device__ __forceinline__ void store(const Regs& r, uint16_t* buf, int* kposb, int tid, bool v_wave,
                                      bool pos_wave, bool clus) {
  if (pos_wave) kposb[tid & 63] = pos_of(r.row, r.pos, clus);
  if (v_wave) {
    uint16_t* Vt = buf + K_ELEMS;
    const int kg = tid & 15, dc = tid >> 4;
    const int pos = 16 * (kg >> 2) + vt_pos((kg * 4) & 15);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
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
    const int u = tid - 256;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int id = x * 256 + u;
      *reinterpret_cast<u32x4*>(Ks + (id >> 4) * KSTR + (id & 15) * 8) = r.x[x];
    }
  }
}

// The whole tile (both key halves) against the wave's 32 rows (this lane's
// row i).  Gathered tile: key of slot s is kpos[s], visible iff j >= 0 and
// i - j >= w.  Window tile (keys k0 + s): visible iff 0 <= i - j < w; the
// mask is skipped when every key is visible to every row of the wave.
__device__ __forceinline__ void compute(const uint16_t* __restrict__ buf, const int* __restrict__ kpos,
                                        bool gathered, int k0, bool full, const bf16x8 (&qf)[8], Acc& acc,
                                        int lane, int i, int w, float c) {
  const uint16_t* Ks = buf;
  const uint16_t* Vt = buf + K_ELEMS;
  const int lr = lane & 31, lh = lane >> 5;
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + lr) * KSTR + t * 16 + lh * 8);
      s[kb] = mfma(kf, qf[t], s[kb]);
    }
  if (gathered) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int4 jv = *reinterpret_cast<const int4*>(kpos + kb * 32 + lh * 4 + q * 8);
        const int js[4] = {jv.x, jv.y, jv.z, jv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vis = (js[e] >= 0) & (i - js[e] >= w);
          s[kb][q * 4 + e] = vis ? s[kb][q * 4 + e] : kNegInf;
        }
      }
  } else if (!full) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int dd = i - (k0 + kb * 32 + lh * 4);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int d = dd - ((e >> 2) * 8 + (e & 3));
        const bool vis = (d >= 0) & (d < w);
        s[kb][e] = vis ? s[kb][e] : kNegInf;
      }
    }
  }
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
  const float nb = -acc.m * c;
  float sum = 0.f;
  bf16x8 pf[2][2];
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
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
}

}  // namespace grp

__global__ __launch_bounds__(grp::NT8, 1) void attn_retrieval_group_kernel(AttnParams p, PackTable packs) {
  using namespace grp;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BUF_ELEMS];
  __shared__ __attribute__((aligned(16))) int kidx[kRing][BK];   // rows of gathered tiles
  __shared__ __attribute__((aligned(16))) int kposb[2][BK];      // key positions of the staged tiles
  __shared__ int ent[kMaxTopk + 1];     // block id (block mode) or CSR start (cluster mode)
  __shared__ int ehi[kMaxTopk + 1];     // cluster mode: end of the member range
  __shared__ int pre[kMaxTopk + 2];     // prefix of visible key counts per entry
  __shared__ int tmp8[8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD k (workgroup id mod 8) takes the query blocks b = k mod 8, long key
  // lists first, and the packs of a query block side by side: every XCD gets
  // a share of short and long blocks, and its resident workgroups are nearby
  // query blocks (similar selections) of the same packs, sharing rows in L2
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int pk = slot % packs.n;
  const int b = p.n_qt - 1 - ((slot / packs.n) * 8 + xcd);
  if (b < 0) return;   // padding of n_qt to a multiple of 8
  const uint32_t pw = packs.heads[pk];
  const int hs = wave & 3;
  const int h = (pw >> (8 * hs)) & 0xFF;
  const int g = (int)(pw & 0xFF) / p.G;
  const int srow = packs.sel_row[pk];
  const int q0 = b * BK;
  const int lim = min(p.N, q0 + BK) - 1 - p.window;   // keys j <= lim can be selected
  const int32_t* mem = p.csr_mem ? p.csr_mem + (size_t)g * p.N : nullptr;

  // window tiles: keys max(0, q0 - w + 1) .. min(N - 1, q0 + 63)
  const int wlo = max(0, q0 - p.window + 1) >> 6;
  const int T_win = (min(p.N - 1, q0 + 63) >> 6) - wlo + 1;

  // entries: forced block 0 + the selection; count of keys j <= lim in each
  const int ne = p.topk + (p.force_block0 ? 1 : 0);
  entry_table<8>(p, p.sel + ((size_t)srow * p.n_qt + b) * p.topk, g, lim, ne, ent, ehi, pre);
  const int cnt = tid < ne ? pre[tid] : 0;
  int total;
  const int excl = dev::block_excl_scan<8>(cnt, tmp8, &total);
  if (tid < ne) pre[tid] = excl;
  if (tid == 0) pre[ne] = total;
  __syncthreads();
  const int T_sel = (total + BK - 1) / BK;
  const int T = T_win + T_sel;

  // row of slot s of gathered tile idx (flat index f = 64 idx + s): key
  // position (block mode) or CSR index (cluster mode); slot s of every tile
  // is looked up by thread 8 s, whose entry index only moves forward
  const bool owner = (tid & 7) == 0;
  const int kslot = tid >> 3;
  int cur_e = 0;
  auto lookup = [&](int idx) -> int {
    const int f = idx * BK + kslot;
    if (f >= total) return -1;
    while (cur_e + 1 < ne && pre[cur_e + 1] <= f) ++cur_e;
    const int r = f - pre[cur_e];
    return p.M > 0 ? ent[cur_e] + r : ent[cur_e] * BK + r;
  };

  const int lr = lane & 31, lh = lane >> 5;
  const int qw = q0 + QW * (wave >> 2);
  const int i = qw + lr;
  const bool active = h != 0xFF && qw < p.N;
  bf16x8 qf[8];
  if (active) {
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) {
      if (i < p.N) {
        qf[t8] = *reinterpret_cast<const bf16x8*>(p.Q + ((size_t)i * p.Hq + h) * D + t8 * 16 + lh * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[t8][e] = (__bf16)0.f;
      }
    }
  }
  Acc acc;
  acc.m = kMInit;
  acc.l = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc.o[db][e] = 0.f;

  const bool v_wave = wave < 4;
  const bool clus = p.M > 0;
  const int rs2w = p.Hkv * D * 2;                       // bytes between keys of K / V
  const int rs2 = clus ? D * 2 : rs2w;                  // ... of the gathered rows
  const char* wbase = reinterpret_cast<const char*>((v_wave ? p.V : p.K) + g * D);
  const char* gbase = clus ? reinterpret_cast<const char*>((v_wave ? p.Vc : p.Kc) + (size_t)g * p.N * D) : wbase;
  const int32_t* cmem = clus ? mem : nullptr;
  const bool pos_wave = wave == 0;
  auto load_tile = [&](Regs& r, int u) {
    if (u < T_win) load_window(r, wbase, (wlo + u) * BK, p.N, rs2w, tid, v_wave);
    else load_gathered(r, gbase, kidx[(u - T_win) % kRing], rs2, tid, v_wave, cmem);
  };
  // every earlier global read (Q fragments, entry table) is complete here, so
  // the waits inside the loop count only the tile loads
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  if (owner) {
#pragma unroll
    for (int x = 0; x < 3; ++x) kidx[x][kslot] = x < T_sel ? lookup(x) : -1;
  }
  __syncthreads();
  Regs r;
  load_tile(r, 0);
  store(r, smem, kposb[0], tid, v_wave, pos_wave, clus);
  if (T > 1) load_tile(r, 1);
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    if (t + 1 < T) {
      store(r, smem + ((t + 1) & 1) * BUF_ELEMS, kposb[(t + 1) & 1], tid, v_wave, pos_wave, clus);
      if (t + 2 < T) load_tile(r, t + 2);
    }
    const int gt = t + 3 - T_win;   // gathered tile looked up in this step
    const bool prep = owner && gt >= 3 && gt < T_sel;
    const int nrow = prep ? lookup(gt) : -1;
    if (active) {
      const bool gathered = t >= T_win;
      const int k0 = (wlo + t) * BK;
      // window tile: all keys visible to every row of the wave / to none
      const bool full = !gathered && k0 + 63 <= qw && qw + QW - 1 - k0 < p.window;
      const bool empty = !gathered && (k0 > qw + QW - 1 || qw - (k0 + 63) >= p.window);
      if (!empty) compute(smem + (t & 1) * BUF_ELEMS, kposb[t & 1], gathered, k0, full, qf, acc, lane, i, p.window,
                          p.c);
    }
    if (prep) kidx[gt % kRing][kslot] = nrow;
    __syncthreads();
  }

  if (!active || i >= p.N) return;
  const float lt = dev::pair32_sum(acc.l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  float* row = p.O + ((size_t)i * p.Hq + h) * D;
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

// Cluster mode: row e of KV head g in Kc / Vc is key csr_mem[g][e] of K / V
// (16 threads per row, 16 bytes each; positions are clamped into [0, N)).
// Memory-bound: K and V are read once and written once.
__global__ __launch_bounds__(256) void permute_kv_kernel(AttnParams p) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = t >> 4;   // g * N + e
  const int c = (int)(t & 15);
  if (row >= (size_t)p.Hkv * p.N) return;
  const int g = (int)(row / (size_t)p.N);
  const int j = min(max((int)p.csr_mem[row], 0), p.N - 1);
  const size_t src = ((size_t)j * p.Hkv + g) * D + c * 8;
  const size_t dst = row * D + c * 8;
  *reinterpret_cast<u32x4*>(p.Kc + dst) = *reinterpret_cast<const u32x4*>(p.K + src);
  *reinterpret_cast<u32x4*>(p.Vc + dst) = *reinterpret_cast<const u32x4*>(p.V + src);
}

}  // namespace

hipError_t launch_permute_kv(const AttnParams& p, hipStream_t s) {
  const size_t threads = (size_t)p.Hkv * p.N * 16;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_kv_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_selected(const AttnParams& p, const SelList& sl, hipStream_t s) {
  const int nwg = sl.n_ret * ((p.n_qt + 7) / 8 * 8);
  if (nwg == 0 || (p.topk == 0 && !p.force_block0)) return hipSuccess;
  hipLaunchKernelGGL(attn_selected_kernel, dim3(nwg), dim3(NT), 0, s, p, sl);
  return hipGetLastError();
}

hipError_t launch_attn_retrieval_group(const AttnParams& p, const PackTable& packs, hipStream_t s) {
  const int nwg = packs.n * ((p.n_qt + 7) / 8 * 8);
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_retrieval_group_kernel, dim3(nwg), dim3(grp::NT8), 0, s, p, packs);
  return hipGetLastError();
}

}  // namespace ha
