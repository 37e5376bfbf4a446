// Host side of the C ABI declared in include/ha.h: argument checks (before
// any HIP call), workspace layout, head packing and launch order.
#include "ha.h"

#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "common.h"

namespace ha {
namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Heads {
  std::vector<int> ret;       // retrieval heads, ascending
  std::vector<int> ret_slot;  // [Hq] slot in ret or -1
  bool any_band = false;
};

int check_desc(const ha_layer_desc* d, const int32_t* kinds, Heads* out) {
  if (!d) return HA_ERR_ARG;
  if (d->n_tokens < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1) return HA_ERR_ARG;
  if (d->n_q_heads % d->n_kv_heads != 0) return HA_ERR_ARG;
  if (d->head_dim < 1 || d->q_block < 1 || d->k_block < 1) return HA_ERR_ARG;
  // head ids travel as bytes in the pack tables, 0xFF marking an empty slot
  if (d->n_q_heads > kMaxHeads - 1) return HA_ERR_UNSUPPORTED;
  if (d->head_dim != kHeadDim) return HA_ERR_UNSUPPORTED;
  if (d->q_block != kBlock || d->k_block != kBlock) return HA_ERR_UNSUPPORTED;
  if (d->n_out < 0 || d->n_out > d->n_tokens) return HA_ERR_ARG;
  if (!kinds) return HA_ERR_ARG;
  if (d->group_select != 0 && d->group_select != 1) return HA_ERR_ARG;
  if (d->block_score < 0 || d->block_score > 2) return HA_ERR_ARG;
  if (d->block_score != 0 && d->n_clusters > 0) return HA_ERR_ARG;   // a block-mode option
  if (d->index_bits != 0 && d->index_bits != 8 && d->index_bits != 32) return HA_ERR_ARG;
  // 8-bit keys are built for the max-pair block scores
  if (d->index_bits == 8 && (d->n_clusters > 0 || d->block_score != 0)) return HA_ERR_UNSUPPORTED;
  if (!(d->topk_mass >= 0.f) || !std::isfinite(d->topk_mass) || !std::isfinite(d->mass_scale)) return HA_ERR_ARG;
  Heads h;
  h.ret_slot.assign(d->n_q_heads, -1);
  bool need_window = false, any_tri = false;
  for (int i = 0; i < d->n_q_heads; ++i) {
    const int k = kinds[i];
    if (k < HA_SWA || k > HA_DENSE) return HA_ERR_ARG;
    if (k == HA_RETRIEVAL) {
      h.ret_slot[i] = (int)h.ret.size();
      h.ret.push_back(i);
    } else {
      h.any_band = true;
    }
    if (k != HA_DENSE) need_window = true;
    if (k == HA_TRIANGLE) any_tri = true;
  }
  if (need_window && d->window < 1) return HA_ERR_ARG;
  if (any_tri && (d->sink < 0 || d->last_q < 0)) return HA_ERR_ARG;
  if (!h.ret.empty()) {
    if (d->rank < 1 || d->topk < 0) return HA_ERR_ARG;
    if (d->force_block0 != 0 && d->force_block0 != 1) return HA_ERR_ARG;
    if (d->rank != kRank) return HA_ERR_UNSUPPORTED;
    if (d->topk > kMaxTopk) return HA_ERR_UNSUPPORTED;
    if (d->n_clusters < 0) return HA_ERR_ARG;
    if (d->n_clusters > 0) {
      if (d->kmeans_iters < 1 || d->kmeans_stride < 1) return HA_ERR_ARG;
      if ((int64_t)d->n_clusters * d->kmeans_stride > d->n_tokens) return HA_ERR_ARG;
      if (d->n_clusters > kMaxSelCand) return HA_ERR_UNSUPPORTED;
      if (d->force_block0) return HA_ERR_UNSUPPORTED;   // block 0 is a block-mode rule
    } else {
      const int n_kb = (d->n_tokens + kBlock - 1) / kBlock;
      if (n_kb > kMaxSelCand) return HA_ERR_UNSUPPORTED;
    }
  }
  if (out) *out = std::move(h);
  return HA_OK;
}

inline int n_qb_of(const ha_layer_desc* d) { return (d->n_tokens + kBlock - 1) / kBlock; }

// Orthros cross-attention runs on the matrix cores: workgroups = packs x row
// tiles x key chunks.  Few row tiles split the key range so that about 1024
// workgroups run; chunks hold >= 8 tiles.
struct CrossPlan {
  int n_packs, n_qt, n_kc, kc_tiles;
};

CrossPlan cross_plan(const ha_layer_desc* d) {
  CrossPlan c{};
  const int G = d->n_q_heads / d->n_kv_heads;
  c.n_packs = d->n_kv_heads * ((G + 3) / 4);
  c.n_qt = (d->n_out + kBlock - 1) / kBlock;
  const int n_kt = (d->n_tokens + kBlock - 1) / kBlock;
  const int base = c.n_packs * c.n_qt;
  int n_kc = base >= 512 ? 1 : (1024 + base - 1) / base;
  n_kc = std::max(1, std::min(n_kc, n_kt / 8));
  c.kc_tiles = (n_kt + n_kc - 1) / n_kc;
  c.n_kc = (n_kt + c.kc_tiles - 1) / c.kc_tiles;
  return c;
}

// Workspace of the cross-attention stage (split-key partials).
size_t cross_ws_bytes(const ha_layer_desc* d) {
  if (d->n_out <= 0) return 0;
  const size_t n_out = (size_t)d->n_out, Hq = (size_t)d->n_q_heads;
  const CrossPlan c = cross_plan(d);
  if (c.n_kc == 1) return 0;
  return align_up((size_t)c.n_kc * n_out * Hq * kHeadDim * sizeof(float)) +
         align_up((size_t)c.n_kc * n_out * Hq * sizeof(float));
}

struct Layout {
  size_t qlow, klow, sel, lse, cent, assign, csr_off, csr_mem, km_scratch, kvc, rep, kq, cross, band, total;
};

// 8-bit indexer keys: int8 codes [Hkv, N, r] then fp32 scales [Hkv, N].
size_t kq_bytes(const ha_layer_desc* d) {
  if (d->index_bits != 8) return 0;
  const size_t rows = (size_t)d->n_kv_heads * d->n_tokens;
  return align_up(rows * kRank) + align_up(rows * sizeof(float));
}

// Block mode with a representative score: the key blocks' representatives.
size_t rep_bytes(const ha_layer_desc* d) {
  if (d->n_clusters > 0 || d->block_score == 0) return 0;
  return align_up(select_block_reps_scratch_bytes(n_qb_of(d), d->n_kv_heads, d->block_score));
}

// Cluster mode: K and V copied into CSR order for the selected-key kernels.
size_t kvc_bytes(const ha_layer_desc* d) {
  return d->n_clusters > 0 ? align_up(2 * (size_t)d->n_kv_heads * d->n_tokens * kHeadDim * sizeof(uint16_t)) : 0;
}

Layout layout_of(const ha_layer_desc* d, const Heads& h) {
  Layout L{};
  size_t off = 0;
  const size_t N = (size_t)d->n_tokens, Hret = h.ret.size();
  L.qlow = off;
  off += align_up(Hret * N * kRank * sizeof(float));
  L.klow = off;
  off += Hret ? align_up((size_t)d->n_kv_heads * N * kRank * sizeof(float)) : 0;
  L.sel = off;
  off += align_up(Hret * (size_t)n_qb_of(d) * (size_t)std::max(0, d->topk) * sizeof(int32_t));
  L.lse = off;
  off += align_up(Hret * N * sizeof(float));
  const size_t M = (Hret && d->n_clusters > 0) ? (size_t)d->n_clusters : 0, Hkv = (size_t)d->n_kv_heads;
  L.cent = off;
  off += align_up(Hkv * M * kRank * sizeof(float));
  L.assign = off;
  off += M ? align_up(Hkv * N * sizeof(int32_t)) : 0;
  L.csr_off = off;
  off += M ? align_up(Hkv * (M + 1) * sizeof(int32_t)) : 0;
  L.csr_mem = off;
  off += M ? align_up(Hkv * N * sizeof(int32_t)) : 0;
  L.km_scratch = off;
  off += M ? align_up(std::max(kmeans_scratch_bytes(d->n_tokens, (int)M, d->n_kv_heads),
                               select_clusters_scratch_bytes((int)M, d->n_kv_heads)))
           : 0;
  L.kvc = off;
  off += Hret ? kvc_bytes(d) : 0;
  L.rep = off;
  off += Hret ? rep_bytes(d) : 0;
  L.kq = off;
  off += Hret ? kq_bytes(d) : 0;
  L.cross = off;
  off += cross_ws_bytes(d);
  L.band = off;              // item counters of the persistent banded kernel
  off += kAlign;
  L.total = off;
  return L;
}

inline float scale_c(const ha_layer_desc* d) {
  const float sc = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
  return sc * 1.4426950408889634f;
}

inline int dev_status(hipError_t e) { return e == hipSuccess ? HA_OK : HA_ERR_DEVICE; }

// Packs of up to 4 heads with one role and one KV head.
void build_packs(const ha_layer_desc* d, const int32_t* kinds, int kind, const std::vector<int>& slot,
                 PackTable* pt) {
  const int G = d->n_q_heads / d->n_kv_heads;
  pt->n = 0;
  for (int g = 0; g < d->n_kv_heads; ++g) {
    uint32_t w = 0, s = 0;
    int cnt = 0, row = -1;
    for (int hh = 0; hh < G; ++hh) {
      const int h = g * G + hh;
      if (kind >= 0 && kinds[h] != kind) continue;   // kind < 0: every head
      const int sl = slot.empty() ? 0 : std::max(0, slot[h]);
      if (row < 0) row = sl;
      w |= (uint32_t)h << (8 * cnt);
      s |= (uint32_t)sl << (8 * cnt);
      if (++cnt == 4) {
        pt->heads[pt->n] = w;
        pt->slots[pt->n] = s;
        pt->sel_row[pt->n] = row;
        ++pt->n;
        w = s = 0;
        cnt = 0;
      }
    }
    if (cnt) {
      for (int x = cnt; x < 4; ++x) w |= 0xFFu << (8 * x);
      pt->heads[pt->n] = w;
      pt->slots[pt->n] = s;
      pt->sel_row[pt->n] = row;
      ++pt->n;
    }
  }
}

// Band kernel packs by head count: 4-head packs, then 2-head, then 1-head
// (a 3-head pack becomes a 2-head and a 1-head pack), with the class sizes
// in p->band_np.
void order_band_packs(PackTable* pt, AttnParams* p) {
  uint32_t h[3][kMaxHeads], sl[3][kMaxHeads];
  int32_t row[3][kMaxHeads];
  int n[3] = {0, 0, 0};
  auto put = [&](int c, uint32_t w, uint32_t s, int32_t r) {
    h[c][n[c]] = w;
    sl[c][n[c]] = s;
    row[c][n[c]] = r;
    ++n[c];
  };
  for (int i = 0; i < pt->n; ++i) {
    const uint32_t w = pt->heads[i], s = pt->slots[i];
    int cnt = 0;
    while (cnt < 4 && ((w >> (8 * cnt)) & 0xFFu) != 0xFFu) ++cnt;
    if (cnt == 4) {
      put(0, w, s, pt->sel_row[i]);
    } else if (cnt == 3) {
      put(1, w | 0xFFFF0000u, s & 0xFFFFu, pt->sel_row[i]);
      put(2, ((w >> 16) & 0xFFu) | 0xFFFFFF00u, (s >> 16) & 0xFFu, pt->sel_row[i]);
    } else if (cnt == 2) {
      put(1, w, s, pt->sel_row[i]);
    } else if (cnt == 1) {
      put(2, w, s, pt->sel_row[i]);
    }
  }
  int k = 0;
  for (int c = 0; c < 3; ++c) {
    for (int i = 0; i < n[c]; ++i, ++k) {
      pt->heads[k] = h[c][i];
      pt->slots[k] = sl[c][i];
      pt->sel_row[k] = row[c][i];
    }
    p->band_np[c] = n[c];
  }
  pt->n = k;
}

AttnParams attn_params(const ha_layer_desc* d, const void* Q, const void* K, const void* V, float* O) {
  AttnParams p{};
  p.Q = static_cast<const uint16_t*>(Q);
  p.K = static_cast<const uint16_t*>(K);
  p.V = static_cast<const uint16_t*>(V);
  p.O = O;
  p.N = d->n_tokens;
  p.Hq = d->n_q_heads;
  p.Hkv = d->n_kv_heads;
  p.G = d->n_q_heads / d->n_kv_heads;
  p.c = scale_c(d);
  p.window = d->window;
  p.sink = d->sink;
  p.dense_from = d->n_tokens - d->last_q;
  p.n_qt = n_qb_of(d);
  p.topk = d->topk;
  p.force_block0 = d->force_block0;
  return p;
}

int run_band(const ha_layer_desc* d, const int32_t* kinds, const void* Q, const void* K, const void* V,
             float* O, uint32_t* ctr, hipStream_t s) {
  AttnParams p = attn_params(d, Q, K, V, O);
  static const int band_kinds[3] = {TRIANGLE, DENSE, SWA};
  for (int kind : band_kinds) {
    PackTable pt;
    build_packs(d, kinds, kind, {}, &pt);
    if (pt.n == 0) continue;
    order_band_packs(&pt, &p);
    p.kind = kind;
    const int st = dev_status(launch_attn_band(p, pt, ctr, s));
    if (st != HA_OK) return st;
  }
  return HA_OK;
}

int run_project(const ha_layer_desc* d, const Heads& h, const void* Q, const void* K, const float* P,
                float* qlow, float* klow, hipStream_t s) {
  const int G = d->n_q_heads / d->n_kv_heads;
  ProjParams pp{};
  pp.N = d->n_tokens;
  pp.P = P;
  if (qlow && !h.ret.empty()) {
    pp.X = static_cast<const uint16_t*>(Q);
    pp.H = d->n_q_heads;
    pp.out = qlow;
    pp.n_entries = (int)h.ret.size();
    for (int t = 0; t < pp.n_entries; ++t) {
      pp.head[t] = h.ret[t];
      pp.group[t] = h.ret[t] / G;
    }
    const int st = dev_status(launch_project(pp, s));
    if (st != HA_OK) return st;
  }
  if (klow) {
    pp.X = static_cast<const uint16_t*>(K);
    pp.H = d->n_kv_heads;
    pp.out = klow;
    pp.n_entries = d->n_kv_heads;
    for (int g = 0; g < pp.n_entries; ++g) {
      pp.head[g] = g;
      pp.group[g] = g;
    }
    const int st = dev_status(launch_project(pp, s));
    if (st != HA_OK) return st;
  }
  return HA_OK;
}

// Adaptive budget of the selection kernels (off unless 0 < topk_mass < 1).
void fill_mass(const ha_layer_desc* d, SelectParams* sp) {
  const bool on = d->topk_mass > 0.f && d->topk_mass < 1.f;
  sp->mass = on ? d->topk_mass : 0.f;
  const float sc = d->mass_scale > 0.f ? d->mass_scale : 1.0f / sqrtf((float)kRank);
  sp->mass_scale_log2 = sc * 1.4426950408889634f;
}

// Selection units: one per retrieval slot, or one per KV group in
// group-shared mode (slots are numbered in head order, so a group's slots
// are consecutive).
void fill_units(const ha_layer_desc* d, const Heads& h, SelectParams* sp) {
  const int G = d->n_q_heads / d->n_kv_heads;
  sp->n_units = 0;
  for (int t = 0; t < (int)h.ret.size(); ++t) {
    if (d->group_select && t > 0 && h.ret[t] / G == h.ret[t - 1] / G) {
      sp->unit[sp->n_units - 1] += 1u << 16;
    } else {
      sp->unit[sp->n_units++] = (uint32_t)t | (1u << 16);
    }
  }
}

int run_select_blocks(const ha_layer_desc* d, const Heads& h, const float* qlow, const float* klow,
                      int32_t* sel, void* rep, void* kq, hipStream_t s) {
  const int G = d->n_q_heads / d->n_kv_heads;
  SelectParams sp{};
  sp.qlow = qlow;
  sp.klow = klow;
  sp.sel = sel;
  sp.N = d->n_tokens;
  sp.n_qb = n_qb_of(d);
  sp.window = d->window;
  sp.topk = d->topk;
  sp.force_block0 = d->force_block0;
  sp.n_ret = (int)h.ret.size();
  for (int t = 0; t < sp.n_ret; ++t) sp.group_of_ret[t] = h.ret[t] / G;
  fill_units(d, h, &sp);
  fill_mass(d, &sp);
  if (d->index_bits == 8) {
    const size_t rows = (size_t)d->n_kv_heads * d->n_tokens;
    int8_t* codes = static_cast<int8_t*>(kq);
    float* scales = reinterpret_cast<float*>(static_cast<char*>(kq) + align_up(rows * kRank));
    const int st = dev_status(launch_quantize_keys(klow, codes, scales, rows, s));
    if (st != HA_OK) return st;
    sp.kcodes = codes;
    sp.kscale = scales;
  }
  if (d->block_score == 0) return dev_status(launch_select_blocks(sp, s));
  // representatives: scored like centroids, candidate m = key block m
  const size_t nparts = (size_t)d->n_kv_heads * sp.n_qb * kRank * (d->block_score == 2 ? 2 : 1);
  sp.M = sp.n_qb;
  sp.c_hi = static_cast<__bf16*>(rep);
  sp.c_lo = sp.c_hi + nparts;
  sp.c_f16 = reinterpret_cast<_Float16*>(sp.c_lo + nparts);
  sp.first_mem = reinterpret_cast<int32_t*>(sp.c_f16 + nparts);
  sp.cnorm = reinterpret_cast<uint32_t*>(sp.first_mem + (size_t)d->n_kv_heads * sp.M);
  return dev_status(launch_select_block_reps(sp, d->n_kv_heads, d->block_score, s));
}

// Retrieval heads: the window part through the banded kernel (which also
// leaves each row's log2-sum-exp), then the selected keys, merged in; with
// group-shared selection one kernel computes both parts.
int run_gather(const ha_layer_desc* d, const int32_t* kinds, const Heads& h, const void* Q, const void* K,
               const void* V, const int32_t* sel, const int32_t* csr_off, const int32_t* csr_mem, float* O,
               float* lse, void* kvc, uint32_t* ctr, hipStream_t s) {
  if (h.ret.empty()) return HA_OK;
  AttnParams p = attn_params(d, Q, K, V, O);
  PackTable pt;
  build_packs(d, kinds, RETRIEVAL, h.ret_slot, &pt);
  p.sel = sel;
  int st = HA_OK;
  if (d->n_clusters > 0) {
    p.csr_off = csr_off;
    p.csr_mem = csr_mem;
    p.M = d->n_clusters;
    p.Kc = static_cast<uint16_t*>(kvc);
    p.Vc = p.Kc + (size_t)d->n_kv_heads * d->n_tokens * kHeadDim;
    st = dev_status(launch_permute_kv(p, s));
    if (st != HA_OK) return st;
  }
  // group-shared selection: window and selected keys of a pack in one kernel
  p.kind = RETRIEVAL;
  if (d->group_select) return dev_status(launch_attn_retrieval_group(p, pt, s));
  p.kind = SWA;
  p.lse = lse;
  PackTable bt = pt;
  order_band_packs(&bt, &p);
  st = dev_status(launch_attn_band(p, bt, ctr, s));
  if (st != HA_OK) return st;
  p.kind = RETRIEVAL;
  SelList sl;
  sl.n_ret = (int)h.ret.size();
  for (int t = 0; t < sl.n_ret; ++t) sl.head[t] = h.ret[t];
  return dev_status(launch_attn_selected(p, sl, s));
}

int run_kmeans(const ha_layer_desc* d, const float* klow, float* cent, int32_t* assign, int32_t* csr_off,
               int32_t* csr_mem, void* scratch, hipStream_t s) {
  KmeansParams kp{};
  kp.klow = klow;
  kp.cent = cent;
  kp.assign = assign;
  kp.csr_off = csr_off;
  kp.csr_mem = csr_mem;
  kp.N = d->n_tokens;
  kp.M = d->n_clusters;
  kp.stride = d->kmeans_stride;
  const size_t Hkv = (size_t)d->n_kv_heads, M = (size_t)d->n_clusters;
  const size_t n_chunks = ((size_t)d->n_tokens + 8191) / 8192;
  kp.hist = static_cast<int32_t*>(scratch);
  kp.count = kp.hist + Hkv * n_chunks * M;
  kp.c_norm = reinterpret_cast<float*>(kp.count + Hkv * M);
  // 16-byte vector loads read the split centroids: start them on an aligned address
  kp.c_hi = reinterpret_cast<_Float16*>(align_up(reinterpret_cast<uintptr_t>(kp.c_norm + Hkv * M)));
  kp.c_lo = kp.c_hi + Hkv * M * kRank;
  kp.amax = reinterpret_cast<uint32_t*>(kp.c_lo + Hkv * M * kRank);
  kp.cmax = kp.amax + Hkv;
  kp.almax = kp.cmax + Hkv;
  kp.n_amb = kp.almax + Hkv;
  kp.amb = reinterpret_cast<int32_t*>(align_up(reinterpret_cast<uintptr_t>(kp.n_amb + Hkv)));
  kp.best = reinterpret_cast<uint64_t*>(align_up(reinterpret_cast<uintptr_t>(kp.amb + Hkv * (size_t)d->n_tokens)));
  return dev_status(launch_kmeans(kp, d->n_kv_heads, d->kmeans_iters, s));
}

int run_select_clusters(const ha_layer_desc* d, const Heads& h, const float* qlow, const float* cent,
                        const int32_t* csr_off, const int32_t* csr_mem, int32_t* sel, void* scratch,
                        hipStream_t s) {
  const int G = d->n_q_heads / d->n_kv_heads;
  SelectParams sp{};
  sp.qlow = qlow;
  sp.cent = cent;
  sp.csr_off = csr_off;
  sp.csr_mem = csr_mem;
  sp.sel = sel;
  sp.N = d->n_tokens;
  sp.n_qb = n_qb_of(d);
  sp.window = d->window;
  sp.topk = d->topk;
  sp.M = d->n_clusters;
  sp.n_ret = (int)h.ret.size();
  for (int t = 0; t < sp.n_ret; ++t) sp.group_of_ret[t] = h.ret[t] / G;
  fill_units(d, h, &sp);
  fill_mass(d, &sp);
  const size_t nparts = (size_t)d->n_kv_heads * d->n_clusters * kRank;
  sp.c_hi = static_cast<__bf16*>(scratch);
  sp.c_lo = sp.c_hi + nparts;
  sp.c_f16 = reinterpret_cast<_Float16*>(sp.c_lo + nparts);
  sp.first_mem = reinterpret_cast<int32_t*>(sp.c_f16 + nparts);
  sp.cnorm = reinterpret_cast<uint32_t*>(sp.first_mem + (size_t)d->n_kv_heads * d->n_clusters);
  return dev_status(launch_select_clusters(sp, d->n_kv_heads, s));
}

int run_cross(const ha_layer_desc* d, const void* Q, const void* K, const void* V, const float* xs,
              const float* xo, float* O_out, float* part, hipStream_t s) {
  if (d->n_out == 0) return HA_OK;
  AttnParams p = attn_params(d, Q, K, V, nullptr);
  const CrossPlan c = cross_plan(d);
  p.kind = DENSE;
  p.xs = xs;
  p.xo = xo;
  p.O_out = O_out;
  p.row0 = d->n_tokens - d->n_out;
  p.n_out = d->n_out;
  p.n_qt = c.n_qt;
  p.n_kc = c.n_kc;
  p.kc_tiles = c.kc_tiles;
  if (c.n_kc > 1) {
    p.part = part;
    p.part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(part) +
                                          align_up((size_t)c.n_kc * d->n_out * d->n_q_heads * kHeadDim * sizeof(float)));
  }
  PackTable pt;
  build_packs(d, nullptr, -1, {}, &pt);
  return dev_status(launch_attn_cross(p, pt, s));
}

inline char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// Scratch of ha_prefill_static.  In host code `scratch` is only a handle for
// the symbol lookup; its device address (one copy per GPU) comes from
// hipGetSymbolAddress, taken once per device with that device current.
__device__ __attribute__((aligned(256))) unsigned char scratch[HA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HA_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return HA_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HA_OK;
}

bool ws_ok(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return true;
  if (!ws || ws_bytes < need) return false;
  return (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) == 0;
}

}  // namespace
}  // namespace ha

using namespace ha;

extern "C" {

const char* ha_status_string(int status) {
  switch (status) {
    case HA_OK: return "HA_OK";
    case HA_ERR_ARG: return "HA_ERR_ARG: invalid argument";
    case HA_ERR_UNSUPPORTED: return "HA_ERR_UNSUPPORTED: configuration not supported by this library";
    case HA_ERR_WORKSPACE: return "HA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case HA_ERR_DEVICE: return "HA_ERR_DEVICE: HIP launch failed";
    case HA_ERR_SCRATCH: return "HA_ERR_SCRATCH: the layer needs more scratch than the static array holds";
    default: return "unknown ha_status";
  }
}

int ha_version(void) { return HA_VERSION; }

size_t ha_workspace_bytes(const ha_layer_desc* desc, const int32_t* head_kind) {
  Heads h;
  if (check_desc(desc, head_kind, &h) != HA_OK) return 0;
  return layout_of(desc, h).total;
}

int ha_prefill(const ha_layer_desc* desc, const int32_t* head_kind, const void* Q, const void* K,
               const void* V, const float* P_idx, const float* xa_scale, const float* xa_offset, float* O,
               float* O_out, ha_aux* aux, void* workspace, size_t ws_bytes, void* stream) {
  Heads h;
  int st = check_desc(desc, head_kind, &h);
  if (st != HA_OK) return st;
  if (!Q || !K || !V || !O) return HA_ERR_ARG;
  if (!h.ret.empty() && !P_idx) return HA_ERR_ARG;
  if (desc->n_out > 0 && (!xa_scale || !xa_offset || !O_out)) return HA_ERR_ARG;
  const Layout L = layout_of(desc, h);
  if (!ws_ok(workspace, ws_bytes, L.total)) return HA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (!h.ret.empty()) {
    float* qlow = (aux && aux->qlow) ? aux->qlow : reinterpret_cast<float*>(ws_at(workspace, L.qlow));
    float* klow = (aux && aux->klow) ? aux->klow : reinterpret_cast<float*>(ws_at(workspace, L.klow));
    int32_t* sel = (aux && aux->sel) ? aux->sel : reinterpret_cast<int32_t*>(ws_at(workspace, L.sel));
    st = run_project(desc, h, Q, K, P_idx, qlow, klow, s);
    if (st != HA_OK) return st;
    const int32_t* off = nullptr;
    const int32_t* mem = nullptr;
    if (desc->n_clusters > 0) {
      float* cent = (aux && aux->centroids) ? aux->centroids : reinterpret_cast<float*>(ws_at(workspace, L.cent));
      int32_t* asg = (aux && aux->assign) ? aux->assign : reinterpret_cast<int32_t*>(ws_at(workspace, L.assign));
      int32_t* co = (aux && aux->csr_off) ? aux->csr_off : reinterpret_cast<int32_t*>(ws_at(workspace, L.csr_off));
      int32_t* cm = (aux && aux->csr_mem) ? aux->csr_mem : reinterpret_cast<int32_t*>(ws_at(workspace, L.csr_mem));
      st = run_kmeans(desc, klow, cent, asg, co, cm, ws_at(workspace, L.km_scratch), s);
      if (st != HA_OK) return st;
      st = run_select_clusters(desc, h, qlow, cent, co, cm, sel, ws_at(workspace, L.km_scratch), s);
      if (st != HA_OK) return st;
      off = co;
      mem = cm;
    } else {
      st = run_select_blocks(desc, h, qlow, klow, sel, ws_at(workspace, L.rep), ws_at(workspace, L.kq), s);
      if (st != HA_OK) return st;
    }
    st = run_gather(desc, head_kind, h, Q, K, V, sel, off, mem, O, reinterpret_cast<float*>(ws_at(workspace, L.lse)),
                    ws_at(workspace, L.kvc), reinterpret_cast<uint32_t*>(ws_at(workspace, L.band)), s);
    if (st != HA_OK) return st;
  }
  if (h.any_band) {
    st = run_band(desc, head_kind, Q, K, V, O, reinterpret_cast<uint32_t*>(ws_at(workspace, L.band)), s);
    if (st != HA_OK) return st;
  }
  if (desc->n_out > 0) {
    st = run_cross(desc, Q, K, V, xa_scale, xa_offset, O_out, reinterpret_cast<float*>(ws_at(workspace, L.cross)), s);
    if (st != HA_OK) return st;
  }
  return HA_OK;
}

int ha_prefill_static(const ha_layer_desc* desc, const int32_t* head_kind, const void* Q, const void* K,
                      const void* V, const float* P_idx, const float* xa_scale, const float* xa_offset, float* O,
                      float* O_out, ha_aux* aux, void* stream) {
  Heads h;
  int st = check_desc(desc, head_kind, &h);
  if (st != HA_OK) return st;
  if (!Q || !K || !V || !O) return HA_ERR_ARG;
  if (!h.ret.empty() && !P_idx) return HA_ERR_ARG;
  if (desc->n_out > 0 && (!xa_scale || !xa_offset || !O_out)) return HA_ERR_ARG;
  if (layout_of(desc, h).total > HA_STATIC_SCRATCH_BYTES) return HA_ERR_SCRATCH;
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != HA_OK) return st;
  return ha_prefill(desc, head_kind, Q, K, V, P_idx, xa_scale, xa_offset, O, O_out, aux, ws,
                    HA_STATIC_SCRATCH_BYTES, stream);
}

int ha_index_project(const ha_layer_desc* desc, const int32_t* head_kind, const void* Q, const void* K,
                     const float* P_idx, float* qlow, float* klow, void* stream) {
  Heads h;
  int st = check_desc(desc, head_kind, &h);
  if (st != HA_OK) return st;
  if (h.ret.empty()) return HA_ERR_ARG;
  if (!P_idx || !K || !klow || (qlow && !Q)) return HA_ERR_ARG;
  return run_project(desc, h, Q, K, P_idx, qlow, klow, static_cast<hipStream_t>(stream));
}

int ha_select_blocks(const ha_layer_desc* desc, const int32_t* head_kind, const float* qlow, const float* klow,
                     int32_t* sel, void* workspace, size_t ws_bytes, void* stream) {
  Heads h;
  int st = check_desc(desc, head_kind, &h);
  if (st != HA_OK) return st;
  if (h.ret.empty() || desc->n_clusters != 0) return HA_ERR_ARG;
  if (!qlow || !klow || !sel) return HA_ERR_ARG;
  // representatives first, then the 8-bit keys
  const size_t rb = rep_bytes(desc);
  if (!ws_ok(workspace, ws_bytes, rb + kq_bytes(desc))) return HA_ERR_WORKSPACE;
  return run_select_blocks(desc, h, qlow, klow, sel, workspace, ws_at(workspace, rb),
                           static_cast<hipStream_t>(stream));
}

int ha_quantize_keys(const ha_layer_desc* desc, const float* klow, int8_t* codes, float* scales, void* stream) {
  if (!desc) return HA_ERR_ARG;
  if (desc->n_tokens < 1 || desc->n_kv_heads < 1) return HA_ERR_ARG;
  if (desc->rank != kRank) return desc->rank < 1 ? HA_ERR_ARG : HA_ERR_UNSUPPORTED;
  if (!klow || !codes || !scales) return HA_ERR_ARG;
  return dev_status(launch_quantize_keys(klow, codes, scales, (size_t)desc->n_kv_heads * desc->n_tokens,
                                         static_cast<hipStream_t>(stream)));
}

int ha_kmeans(const ha_layer_desc* desc, const float* klow, float* centroids, int32_t* assign, int32_t* csr_off,
              int32_t* csr_mem, void* workspace, size_t ws_bytes, void* stream) {
  if (!desc) return HA_ERR_ARG;
  const ha_layer_desc* d = desc;
  if (d->n_tokens < 1 || d->n_kv_heads < 1 || d->n_clusters < 1 || d->kmeans_iters < 1 || d->kmeans_stride < 1)
    return HA_ERR_ARG;
  if ((int64_t)d->n_clusters * d->kmeans_stride > d->n_tokens) return HA_ERR_ARG;
  if (d->rank != kRank) return d->rank < 1 ? HA_ERR_ARG : HA_ERR_UNSUPPORTED;
  if (d->n_clusters > kMaxSelCand) return HA_ERR_UNSUPPORTED;
  if (!klow || !centroids || !assign || !csr_off || !csr_mem) return HA_ERR_ARG;
  if (!ws_ok(workspace, ws_bytes, align_up(kmeans_scratch_bytes(d->n_tokens, d->n_clusters, d->n_kv_heads))))
    return HA_ERR_WORKSPACE;
  return run_kmeans(d, klow, centroids, assign, csr_off, csr_mem, workspace, static_cast<hipStream_t>(stream));
}

int ha_select_clusters(const ha_layer_desc* desc, const int32_t* head_kind, const float* qlow,
                       const float* centroids, const int32_t* csr_off, const int32_t* csr_mem, int32_t* sel,
                       void* workspace, size_t ws_bytes, void* stream) {
  Heads h;
  int st = check_desc(desc, head_kind, &h);
  if (st != HA_OK) return st;
  if (h.ret.empty() || desc->n_clusters < 1) return HA_ERR_ARG;
  if (!qlow || !centroids || !csr_off || !csr_mem || !sel) return HA_ERR_ARG;
  if (!ws_ok(workspace, ws_bytes, align_up(select_clusters_scratch_bytes(desc->n_clusters, desc->n_kv_heads))))
    return HA_ERR_WORKSPACE;
  return run_select_clusters(desc, h, qlow, centroids, csr_off, csr_mem, sel, workspace,
                             static_cast<hipStream_t>(stream));
}

int ha_attn_band(const ha_layer_desc* desc, const int32_t* head_kind, const void* Q, const void* K, const void* V,
                 float* O, void* workspace, size_t ws_bytes, void* stream) {
  Heads h;
  int st = check_desc(desc, head_kind, &h);
  if (st != HA_OK) return st;
  if (!Q || !K || !V || !O) return HA_ERR_ARG;
  if (!ws_ok(workspace, ws_bytes, kAlign)) return HA_ERR_WORKSPACE;
  return run_band(desc, head_kind, Q, K, V, O, static_cast<uint32_t*>(workspace), static_cast<hipStream_t>(stream));
}

int ha_attn_gather(const ha_layer_desc* desc, const int32_t* head_kind, const void* Q, const void* K,
                   const void* V, const int32_t* sel, const int32_t* csr_off, const int32_t* csr_mem, float* O,
                   void* workspace, size_t ws_bytes, void* stream) {
  Heads h;
  int st = check_desc(desc, head_kind, &h);
  if (st != HA_OK) return st;
  if (h.ret.empty()) return HA_ERR_ARG;
  if (!Q || !K || !V || !O || (desc->topk > 0 && !sel)) return HA_ERR_ARG;
  if (desc->n_clusters > 0 && (!csr_off || !csr_mem)) return HA_ERR_ARG;
  const size_t lse_bytes = align_up(h.ret.size() * (size_t)desc->n_tokens * sizeof(float));
  const size_t kvc = kvc_bytes(desc);
  if (!ws_ok(workspace, ws_bytes, lse_bytes + kvc + kAlign)) return HA_ERR_WORKSPACE;
  return run_gather(desc, head_kind, h, Q, K, V, sel, csr_off, csr_mem, O, static_cast<float*>(workspace),
                    ws_at(workspace, lse_bytes), reinterpret_cast<uint32_t*>(ws_at(workspace, lse_bytes + kvc)),
                    static_cast<hipStream_t>(stream));
}

int ha_attn_cross(const ha_layer_desc* desc, const void* Q, const void* K, const void* V, const float* xa_scale,
                  const float* xa_offset, float* O_out, void* workspace, size_t ws_bytes, void* stream) {
  if (!desc) return HA_ERR_ARG;
  if (desc->n_tokens < 1 || desc->n_q_heads < 1 || desc->n_kv_heads < 1 ||
      desc->n_q_heads % desc->n_kv_heads != 0 || desc->n_out < 1 || desc->n_out > desc->n_tokens)
    return HA_ERR_ARG;
  if (desc->head_dim != kHeadDim) return desc->head_dim < 1 ? HA_ERR_ARG : HA_ERR_UNSUPPORTED;
  if (desc->n_q_heads > kMaxHeads - 1) return HA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !xa_scale || !xa_offset || !O_out) return HA_ERR_ARG;
  if (!ws_ok(workspace, ws_bytes, cross_ws_bytes(desc))) return HA_ERR_WORKSPACE;
  return run_cross(desc, Q, K, V, xa_scale, xa_offset, O_out, static_cast<float*>(workspace),
                   static_cast<hipStream_t>(stream));
}

}  // extern "C"
