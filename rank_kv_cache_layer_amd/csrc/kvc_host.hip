// Host side of libkvc: argument validation, per-hop rotation tables, anchor-set logic,
// workspace planning and kernel launches behind the C ABI of include/kvc.h.
//
// Anchor sets follow KVCMAS (arXiv 2609.34060) App. A.3 "Variable Segment Lengths":
//   gate set A_k   = anchors whose stored length >= k (k = gate_len, 0 -> S)
//   coverage S_cov = min(S, longest stored length)
//   correction set = anchors whose stored length >= S_cov
// Rows >= S_cov keep the re-aligned source.  Rotation angles are evaluated in double
// precision here and handed to the kernels as float cos/sin tables.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "kvc_internal.h"
#include "kvc_peaks.h"

using namespace kvc;

namespace {

thread_local char g_err[512] = "";

kvc_status fail(kvc_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}
kvc_status ok() {
  g_err[0] = 0;
  return KVC_OK;
}

size_t esize(kvc_dtype t) { return t == KVC_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

kvc_status check_shape(const kvc_shape& s) {
  if (s.n_layers < 1 || s.seq_len < 1 || s.n_kv_heads < 1)
    return fail(KVC_E_SHAPE, "shape: n_layers, seq_len and n_kv_heads must be >= 1 (got %d, %d, %d)", s.n_layers,
                s.seq_len, s.n_kv_heads);
  if (s.head_dim < 2 || (s.head_dim & 1) || s.head_dim > KVC_MAX_HEAD_DIM)
    return fail(KVC_E_SHAPE, "shape: head_dim must be even and in [2, %d] (got %d)", KVC_MAX_HEAD_DIM, s.head_dim);
  if ((int64_t)s.n_kv_heads * s.head_dim > 65536)
    return fail(KVC_E_SHAPE, "shape: n_kv_heads * head_dim > 65536");
  if ((int64_t)s.n_layers > 256) return fail(KVC_E_SHAPE, "shape: n_layers > 256");
  return KVC_OK;
}

kvc_status check_dtype(kvc_dtype t, const char* what) {
  if (t != KVC_F32 && t != KVC_BF16) return fail(KVC_E_DTYPE, "%s: unknown dtype %d", what, (int)t);
  return KVC_OK;
}

kvc_status make_tab(RopeTab& tab, int64_t dp, int head_dim, const kvc_rope* rope) {
  memset(&tab, 0, sizeof tab);
  tab.active = dp != 0;
  const int h = head_dim / 2;
  for (int c = 0; c < h; ++c) {
    double w;
    if (rope->inv_freq) {
      w = rope->inv_freq[c];
    } else {
      w = pow(rope->theta, -2.0 * (double)c / (double)head_dim);
    }
    if (!std::isfinite(w)) return fail(KVC_E_PARAM, "rope: non-finite frequency at pair %d", c);
    const double phi = (double)dp * w;
    tab.cs[c] = (float)cos(phi);
    tab.sn[c] = (float)sin(phi);
  }
  return KVC_OK;
}

kvc_status check_rope(const kvc_rope* rope) {
  if (!rope) return fail(KVC_E_NULL, "rope descriptor is NULL");
  if (!rope->inv_freq && !(rope->theta > 0.0 && std::isfinite(rope->theta)))
    return fail(KVC_E_PARAM, "rope: theta must be positive and finite when inv_freq is NULL");
  return KVC_OK;
}

struct Sets {
  int k = 0, s_cov = 0;
  uint64_t gate = 0, corr = 0;
  int n_gate = 0;
  std::vector<int> corr_list, use_list;
};

bool is_live(const kvc_pool& p, int a) { return !p.live || p.live[a] != 0; }

// A-row offset and length of every anchor, and rows per layer of the A arrays
int64_t anchor_rows(const kvc_pool& p, int32_t* off, int32_t* len) {
  int64_t tot = 0;
  for (int a = 0; a < p.n_anchors; ++a) {
    off[a] = p.slot_rows > 0 ? a * p.slot_rows : (int32_t)tot;
    len[a] = is_live(p, a) ? p.anchor_len[a] : 0;
    tot += p.slot_rows > 0 ? p.slot_rows : p.anchor_len[a];
  }
  return tot;
}

Sets anchor_sets(const kvc_pool& p, int S, int gate_len) {
  Sets s;
  s.k = gate_len == 0 ? S : gate_len;
  int maxlen = 0, n_live = 0;
  for (int a = 0; a < p.n_anchors; ++a)
    if (is_live(p, a)) {
      maxlen = std::max(maxlen, (int)p.anchor_len[a]);
      ++n_live;
    }
  s.s_cov = n_live ? std::min(S, maxlen) : 0;
  for (int a = 0; a < p.n_anchors; ++a) {
    if (!is_live(p, a)) continue;
    const int len = p.anchor_len[a];
    if (len >= s.k) { s.gate |= 1ull << a; ++s.n_gate; }
    if (len >= s.s_cov) { s.corr |= 1ull << a; s.corr_list.push_back(a); }
    if ((s.gate | s.corr) >> a & 1) s.use_list.push_back(a);
  }
  return s;
}

kvc_status check_pool(const kvc_pool* p, const kvc_shape& sh, kvc_dtype cache_t, bool need_base, bool need_delta) {
  if (!p) return fail(KVC_E_NULL, "pool descriptor is NULL");
  if (p->n_anchors < 0 || p->n_anchors > KVC_MAX_ANCHORS)
    return fail(KVC_E_SHAPE, "pool: n_anchors must be in [0, %d] (got %d)", KVC_MAX_ANCHORS, p->n_anchors);
  if (p->rank_base < 1 || p->rank_base > 1024 || p->rank_delta < 1 || p->rank_delta > 1024)
    return fail(KVC_E_SHAPE, "pool: ranks must be in [1, 1024] (got %d, %d)", p->rank_base, p->rank_delta);
  if (p->capacity < 0 || (p->capacity > 0 && p->capacity < p->n_anchors))
    return fail(KVC_E_PARAM, "pool: capacity must be 0 or >= n_anchors");
  if (p->dtype != cache_t) return fail(KVC_E_DTYPE, "pool dtype %d differs from cache dtype %d", p->dtype, cache_t);
  if (p->n_anchors == 0) return KVC_OK;
  if (!p->anchor_len) return fail(KVC_E_NULL, "pool: anchor_len is NULL");
  if (p->slot_rows < 0) return fail(KVC_E_SHAPE, "pool: slot_rows = %d < 0", p->slot_rows);
  int64_t tot = 0;
  for (int a = 0; a < p->n_anchors; ++a) {
    if (!is_live(*p, a) && p->slot_rows > 0) {   // an empty or foreign slot: its length is not read
      tot += p->slot_rows;
      continue;
    }
    if (p->anchor_len[a] < 1) return fail(KVC_E_SHAPE, "pool: anchor_len[%d] = %d < 1", a, p->anchor_len[a]);
    if (p->slot_rows > 0 && p->anchor_len[a] > p->slot_rows)
      return fail(KVC_E_SHAPE, "pool: anchor_len[%d] = %d exceeds slot_rows = %d", a, p->anchor_len[a], p->slot_rows);
    tot += p->slot_rows > 0 ? p->slot_rows : p->anchor_len[a];
  }
  if (tot * std::max(p->rank_base, p->rank_delta) >= (1ll << 40)) return fail(KVC_E_SHAPE, "pool: too many rows");
  const void* ptrs[8] = {p->baseA_k, p->baseB_k, p->baseA_v, p->baseB_v,
                         p->deltaA_k, p->deltaB_k, p->deltaA_v, p->deltaB_v};
  static const char* names[8] = {"baseA_k", "baseB_k", "baseA_v", "baseB_v",
                                 "deltaA_k", "deltaB_k", "deltaA_v", "deltaB_v"};
  for (int i = 0; i < 8; ++i) {
    if ((i < 4 && !need_base) || (i >= 4 && !need_delta)) continue;
    if (!ptrs[i]) return fail(KVC_E_NULL, "pool: %s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(KVC_E_ALIGN, "pool: %s is not 16-byte aligned", names[i]);
  }
  (void)sh;
  return KVC_OK;
}

kvc_status check_params(const kvc_params* prm, int S) {
  if (!prm) return fail(KVC_E_NULL, "params is NULL");
  if (!std::isfinite(prm->tau)) return fail(KVC_E_PARAM, "params: tau must be finite");
  if (!(prm->temp_gate > 0.0) || !std::isfinite(prm->temp_gate))
    return fail(KVC_E_PARAM, "params: temp_gate must be > 0");
  if (!(prm->temp_weight > 0.0) || !std::isfinite(prm->temp_weight))
    return fail(KVC_E_PARAM, "params: temp_weight must be > 0");
  if (prm->gate_len < 0 || prm->gate_len > S) return fail(KVC_E_PARAM, "params: gate_len must be in [0, seq_len]");
  if (prm->mode != KVC_SCORE_PAGES && prm->mode != KVC_SCORE_COS_R)
    return fail(KVC_E_PARAM, "params: unknown mode %d", prm->mode);
  if (prm->options & ~3) return fail(KVC_E_PARAM, "params: unknown option bits 0x%x", prm->options);
  if (prm->trace) {
    const kvc_trace* t = prm->trace;
    if (t->capacity < 0 || t->capacity > KVC_TRACE_MAX || t->count < 0)
      return fail(KVC_E_PARAM, "params: trace capacity must be in [0, %d]", KVC_TRACE_MAX);
    for (int i = t->count; i < t->capacity; ++i)
      if (!t->start[i] || !t->stop[i]) return fail(KVC_E_NULL, "params: trace event %d is NULL", i);
  }
  return KVC_OK;
}

// ---------------------------------------------------------------- path selection
int32_t D_of(const kvc_shape& s) { return s.n_kv_heads * s.head_dim; }

// The fused bf16 MFMA kernel: one work-group holds 64 tokens x all D channels (D / 128 waves,
// at most 8), head_dim 64 or 128, ranks in steps of 16.
bool fused_ok(const kvc_shape& sh, const kvc_pool& p, const kvc_params& prm, bool pages_scores, bool apply) {
  if (p.dtype != KVC_BF16 || (prm.options & 1)) return false;
  const int D = D_of(sh);
  if ((sh.head_dim != 64 && sh.head_dim != 128) || D % 128 || D > 1024) return false;
  if (pages_scores) {
    const int r = p.rank_base;
    if (r != 16 && r != 32 && r != 64 && r != 128) return false;
  }
  if (apply && (p.rank_delta % 16 || p.rank_delta > 256)) return false;
  return true;
}

bool cos_mfma_ok(const kvc_shape& sh, const kvc_pool& p, const kvc_params& prm) {
  if (p.dtype != KVC_BF16 || (prm.options & 1)) return false;
  const int D = D_of(sh);
  if ((sh.head_dim != 64 && sh.head_dim != 128) || D % 128 || D > 1024) return false;
  return p.rank_base == 32 || p.rank_base == 64 || p.rank_base == 128;
}

// The second mode's GEMM scoring: ranks 32, 64 and 128, bf16, unless a single-pass kernel is
// asked for (option bit 1 keeps the older per-anchor-group kernel); a layer must fit a 32-bit
// buffer.
bool cos_gemm_ok(const kvc_shape& sh, const kvc_pool& p, const kvc_params& prm) {
  const int r = p.rank_base;
  if (p.dtype != KVC_BF16 || (prm.options & 3) || (r != 32 && r != 64 && r != 128)) return false;
  const int D = D_of(sh);
  if ((sh.head_dim != 64 && sh.head_dim != 128) || D % 32) return false;
  return (uint64_t)sh.seq_len * D * 2 < (1ull << 31);
}

// The two-pass bf16 path: 128-token x 256-channel work-groups (D a multiple of 256), scoring
// ranks 16/32 (and 64/128 in steps of 64 ranks with the result blocks held across them), apply
// ranks 8 (padded to the MFMA's 16 on chip), 16, 32 and 64/128/256 (as slices of 32), within
// the LDS budget.
constexpr size_t kLdsBudget = 160 * 1024;
bool split_ok(const kvc_shape& sh, const kvc_pool& p, const kvc_params& prm, bool pages_scores, bool apply) {
  if (p.dtype != KVC_BF16 || (prm.options & 3)) return false;
  const int D = D_of(sh);
  if ((sh.head_dim != 64 && sh.head_dim != 128) || D % kSplitWidth) return false;
  if (pages_scores) {
    const int rb = p.rank_base;
    if (rb != 16 && rb != 32 && rb != 64 && rb != 128) return false;   // 64 / 128: rank slices of 32
    if (split_score_lds(rb) + 8 * 1024 > kLdsBudget) return false;
  }
  if (apply) {
    const int rd = p.rank_delta;
    if (rd != 8 && rd != 16 && rd != 32 && split_apply_slices(rd) == 1) return false;
    if (split_apply_lds(p.rank_delta) + 2 * 1024 > kLdsBudget) return false;
  }
  return true;
}

// ------------------------------------------------------------------- workspace
struct Plan {
  bool split_match = false;   // first-mode scores in the two-pass path
  bool split_apply = false;   // apply in the two-pass path
  bool fused_match = false;   // PAGES scores inside the fused kernel
  bool fused_apply = false;   // apply inside the fused kernel
  bool fused_split = false;   // PAGES scores in the fused kernel, weights through the workspace to the two-pass apply
  bool cos_mfma = false;
  bool cos_gemm = false;        // second-mode scores as one GEMM per layer-side
  size_t off_pack_cos = 0;
  int tile = 0, n_tiles = 0, s_work = 0, generic_tt = 0;
  size_t off_scores = 0, off_w = 0, off_partials = 0, off_pack_base = 0, off_pack_delta = 0, off_mpart = 0;
  size_t off_wa = 0;            // anchor-major token weights of the two-pass path
  size_t off_gsum = 0;          // per-layer gate sums (fp64)
  size_t total = 0;
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
// packed B operands hold ranks in slices of 16 (rows past the rank are zero)
size_t rpad16(int r) { return (size_t)((r + 15) & ~15); }

Plan plan(int call, const kvc_shape& sh, const kvc_pool& p, const kvc_params* prm, const Sets& s) {
  Plan pl;
  const int S = sh.seq_len, D = D_of(sh), L = sh.n_layers, N = std::max(p.n_anchors, 1);
  kvc_params dflt = {0.3, 1.0, 1.0, 0, KVC_SCORE_PAGES, 0, 0, nullptr};
  const kvc_params& P = prm ? *prm : dflt;
  const bool do_match = call == KVC_CALL_MATCH || call == KVC_CALL_CORRECT;
  const bool do_apply = call == KVC_CALL_APPLY || call == KVC_CALL_CORRECT;
  const bool pages = P.mode == KVC_SCORE_PAGES;
  size_t off = 0;
  if (do_apply) {
    pl.split_apply = split_ok(sh, p, P, false, true);
    pl.fused_apply = !pl.split_apply && fused_ok(sh, p, P, false, true);
  }
  if (do_match) {
    const int n_use = (int)s.use_list.size();
    pl.s_work = s.n_gate ? std::max(s.s_cov, s.k) : s.s_cov;
    pl.split_match = pages && split_ok(sh, p, P, true, do_apply);
    if (pl.split_match && do_apply && !pl.split_apply) pl.split_match = false;
    if (do_apply && pages && !pl.split_match && pl.split_apply) {
      // scores from the fused kernel: the two-pass apply only where it takes the rank in slices
      // (at ranks 64 and up the fused apply is the slower half); otherwise the pair stays on
      // the fused kernel
      if (split_apply_slices(p.rank_delta) > 1 && fused_ok(sh, p, P, true, false)) {
        pl.fused_split = true;
      } else {
        pl.split_apply = false;
        pl.fused_apply = fused_ok(sh, p, P, false, true);
      }
    }
    pl.fused_match = !pl.split_match && pages && fused_ok(sh, p, P, true, false) &&
                     (!do_apply || pl.fused_apply || pl.fused_split);
    if (pl.split_match) {
      const int tt = split_score_tile(p.rank_base);
      const int ntt = (S + tt - 1) / tt, nct = D / kSplitWidth;
      pl.tile = tt;
      pl.n_tiles = ntt * nct;
      pl.off_mpart = off;
      off += up256(sizeof(float) * (size_t)nct * 2 * L * N * S);
    } else if (pl.fused_match) {
      pl.tile = kFusedTile;
      pl.n_tiles = (S + kFusedTile - 1) / kFusedTile;
      if (pl.fused_split) {
        pl.off_w = off;
        off += up256(sizeof(float) * 2 * (size_t)L * S * N);
      }
    } else {
      pl.cos_gemm = !pages && cos_gemm_ok(sh, p, P);
      pl.cos_mfma = !pages && !pl.cos_gemm && cos_mfma_ok(sh, p, P);
      if (pl.cos_gemm) {
        pl.tile = kCosTile;
        pl.off_pack_cos = off;
        off += up256(sizeof(uint16_t) * cos_gemm_packed_elems(L, std::max(n_use, 1), p.rank_base, D));
      } else if (pl.cos_mfma) {
        pl.tile = kCosTile;
      } else {
        pl.generic_tt = std::max(1, 256 / std::max(n_use, 1));
        pl.tile = pl.generic_tt;
      }
      pl.n_tiles = pl.s_work > 0 ? (pl.s_work + pl.tile - 1) / pl.tile : 0;
      pl.off_scores = off;
      off += up256(sizeof(float) * 2 * (size_t)L * S * N);
      if (!(do_apply && (pl.fused_apply || pl.split_apply) && !pages)) {   // weights materialised unless fused
        pl.off_w = off;
        off += up256(sizeof(float) * 2 * (size_t)L * S * N);
      }
    }
    pl.off_partials = off;
    off += up256(sizeof(float) * 3 * (size_t)L * std::max(pl.n_tiles, 1) * N);
    pl.off_gsum = off;
    off += up256(sizeof(double) * 3 * (size_t)(1 + L) * N);
    if (pl.fused_match || pl.split_match) {
      pl.off_pack_base = off;
      off += up256(2 * 2 * (size_t)L * N * D * rpad16(p.rank_base));
    }
  }
  if (do_apply && (pl.fused_apply || pl.split_apply)) {
    pl.off_pack_delta = off;
    off += up256(2 * 2 * (size_t)L * N * D * rpad16(p.rank_delta));
  }
  if (pl.split_match || pl.split_apply) {
    pl.off_wa = off;
    off += up256(sizeof(float) * 2 * (size_t)L * N * S);
  }
  pl.total = off;
  return pl;
}

PoolGeom geom(const kvc_pool& p, const kvc_shape& sh, int r) {
  PoolGeom g;
  memset(&g, 0, sizeof g);
  g.n = p.n_anchors;
  g.r = r;
  const int64_t tot = anchor_rows(p, g.off, g.len);
  g.a_layer_stride = tot * r;
  g.b_layer_stride = (int64_t)p.n_anchors * r * D_of(sh);
  return g;
}

// Brackets one launch with the caller's trace events (if any).
struct Tracer {
  kvc_trace* t;
  hipStream_t st;
  int slot = -1;
  void begin(int id) {
    slot = -1;
    if (!t || t->count >= t->capacity || t->count >= KVC_TRACE_MAX) return;
    slot = t->count++;
    t->kernel_id[slot] = id;
    (void)hipEventRecord((hipEvent_t)t->start[slot], st);   // best effort: a missing event reads as no time
  }
  void end() {
    if (slot >= 0) (void)hipEventRecord((hipEvent_t)t->stop[slot], st);
    slot = -1;
  }
};

kvc_status hip_fail(hipError_t e, const char* what) {
  return fail(KVC_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

kvc_status fused_tab(FusedTab& ft, int64_t dp, int head_dim, const kvc_rope* rope) {
  RopeTab t;
  kvc_status s = make_tab(t, dp, head_dim, rope);
  if (s != KVC_OK) return s;
  memset(&ft, 0, sizeof ft);
  for (int c = 0; c < head_dim / 2 && c < kFusedHalf; ++c) {
    ft.cs[c] = t.cs[c];
    ft.sn[c] = t.sn[c];
  }
  ft.active = t.active;
  return KVC_OK;
}

// Packs B factors of both sides into MFMA operand chunks.
// slices > 1: each anchor's r x D factor packs as `slices` matrices of r / slices rows (the
// rows of one slice are contiguous, so the factor array is read as slices x n_anchors matrices);
// the packed size is the same.
kvc_status pack_pair(const void* bk, const void* bv, uint16_t* dst, int r, int negate, const FusedTab* key_tab,
                     const kvc_shape& sh, const kvc_pool& p, Tracer& tr, int trace_id, hipStream_t st,
                     int slices = 1) {
  if (p.n_anchors == 0) return KVC_OK;
  const size_t per = (size_t)sh.n_layers * p.n_anchors * D_of(sh) * rpad16(r);
  const uint16_t* src[2] = {(const uint16_t*)bk, (const uint16_t*)bv};
  uint16_t* dsts[2] = {dst, dst + per};
  const int neg[2] = {negate, negate};
  const FusedTab* tabs[2] = {key_tab, nullptr};
  tr.begin(trace_id);
  hipError_t e = launch_pack_b(src, dsts, neg, tabs, 2, sh.n_layers, p.n_anchors * slices, r / slices, D_of(sh),
                               sh.head_dim, st);
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "pack factors");
  return KVC_OK;
}

// Common fields of the fused kernel's arguments.
kvc_status fused_args(FusedArgs& f, const void* k_src, const void* v_src, const kvc_shape& sh, int64_t p_src,
                      int64_t p_tgt, const kvc_rope* rope, const kvc_pool& p, const Sets& s, float inv_temp) {
  memset(&f, 0, sizeof f);
  f.z[0] = (const uint16_t*)k_src;
  f.z[1] = (const uint16_t*)v_src;
  f.n_layers = sh.n_layers;
  f.S = sh.seq_len;
  f.D = D_of(sh);
  f.n_tiles = (sh.seq_len + kFusedTile - 1) / kFusedTile;
  f.s_cov = s.corr_list.empty() ? 0 : s.s_cov;
  f.k_gate = s.k;
  f.r_b = p.rank_base;
  f.r_d = p.rank_delta;
  f.N = p.n_anchors;
  f.mask_corr = s.corr;
  f.mask_gate = s.gate;
  f.n_use = (int)s.use_list.size();
  for (int i = 0; i < f.n_use; ++i) f.use[i] = (uint8_t)s.use_list[i];
  f.n_corr = (int)s.corr_list.size();
  for (int i = 0; i < f.n_corr; ++i) f.corr[i] = (uint8_t)s.corr_list[i];
  const int64_t tot = anchor_rows(p, f.off, f.len);
  f.ab_layer = tot * p.rank_base;
  f.ad_layer = tot * p.rank_delta;
  f.inv_temp = inv_temp;
  kvc_status st;
  if ((st = fused_tab(f.can, -p_src, sh.head_dim, rope)) != KVC_OK) return st;
  if ((st = fused_tab(f.shift, p_tgt - p_src, sh.head_dim, rope)) != KVC_OK) return st;
  return KVC_OK;
}

// Common fields of the two-pass kernels' arguments.
kvc_status split_args(SplitArgs& f, const void* k_src, const void* v_src, const kvc_shape& sh, int64_t p_src,
                      int64_t p_tgt, const kvc_rope* rope, const kvc_pool& p, const Sets& s, float inv_temp) {
  memset(&f, 0, sizeof f);
  f.z[0] = (const uint16_t*)k_src;
  f.z[1] = (const uint16_t*)v_src;
  f.n_layers = sh.n_layers;
  f.layer0 = 0;
  f.n_grp = sh.n_layers;
  f.S = sh.seq_len;
  f.D = D_of(sh);
  f.ntt = (sh.seq_len + kScoreTile - 1) / kScoreTile;   // set per launch by the kernels
  f.nct = D_of(sh) / kSplitWidth;
  f.N = p.n_anchors;
  f.r_b = p.rank_base;
  f.r_d = p.rank_delta;
  f.s_cov = s.corr_list.empty() ? 0 : s.s_cov;
  f.k_gate = s.k;
  f.mask_corr = s.corr;
  f.mask_gate = s.gate;
  f.n_use = (int)s.use_list.size();
  for (int i = 0; i < f.n_use; ++i) f.use[i] = (uint8_t)s.use_list[i];
  f.n_corr = (int)s.corr_list.size();
  for (int i = 0; i < f.n_corr; ++i) f.corr[i] = (uint8_t)s.corr_list[i];
  const int64_t tot = anchor_rows(p, f.off, f.len);
  f.ab_layer = tot * p.rank_base;
  f.ad_layer = tot * p.rank_delta;
  f.inv_temp = inv_temp;
  f.inv_d = 1.f / (float)D_of(sh);
  kvc_status st;
  if ((st = fused_tab(f.can, -p_src, sh.head_dim, rope)) != KVC_OK) return st;
  if ((st = fused_tab(f.shift, p_tgt - p_src, sh.head_dim, rope)) != KVC_OK) return st;
  return KVC_OK;
}

// Packs the delta B factors (key rows turned by R(p_tgt)) and fills the apply fields.
kvc_status split_apply_fields(SplitArgs& f, void* k_out, void* v_out, const kvc_shape& sh, int64_t p_tgt,
                              const kvc_rope* rope, const kvc_pool& p, char* ws, const Plan& pl, Tracer& tr,
                              hipStream_t st) {
  FusedTab tgt;
  kvc_status r;
  if ((r = fused_tab(tgt, p_tgt, sh.head_dim, rope)) != KVC_OK) return r;
  uint16_t* pd = reinterpret_cast<uint16_t*>(ws + pl.off_pack_delta);
  if ((r = pack_pair(p.deltaB_k, p.deltaB_v, pd, p.rank_delta, 0, &tgt, sh, p, tr, KVC_K_PACK_DELTA, st,
                     split_apply_slices(p.rank_delta))) != KVC_OK)
    return r;
  const size_t per_d = (size_t)sh.n_layers * p.n_anchors * D_of(sh) * rpad16(p.rank_delta);
  f.out[0] = (uint16_t*)k_out; f.out[1] = (uint16_t*)v_out;
  f.Ad[0] = (const uint16_t*)p.deltaA_k; f.Ad[1] = (const uint16_t*)p.deltaA_v;
  f.Bd[0] = pd; f.Bd[1] = pd + per_d;
  f.apply = 1;
  return KVC_OK;
}

// Anchor-major token weights for the two-pass apply (and the caller's copy, if requested).
kvc_status run_split_weights(SplitArgs& f, int wmode, char* ws, const Plan& pl, Tracer& tr, hipStream_t st) {
  f.wa = reinterpret_cast<float*>(ws + pl.off_wa);
  if (f.n_corr < 1) {   // no correcting anchor (e.g. every arena slot empty): the caller's weights are 0
    const int64_t n = (int64_t)f.n_layers * f.S * f.N;   // [n_layers][seq_len][n_anchors]
    for (int s = 0; s < 2; ++s)
      if (f.w_out[s]) {
        hipError_t e = launch_fill(f.w_out[s], n, 0.f, st);
        if (e != hipSuccess) return hip_fail(e, "weights fill");
      }
    return KVC_OK;
  }
  tr.begin(KVC_K_WEIGHTS_SPLIT);
  hipError_t e = launch_split_weights(f, wmode, st);
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "weights kernel");
  return KVC_OK;
}

kvc_status run_split_apply(const SplitArgs& f, const kvc_shape& sh, Tracer& tr, hipStream_t st) {
  tr.begin(KVC_K_APPLY_SPLIT);
  hipError_t e = launch_split_apply(f, sh.head_dim, st);
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "apply kernel");
  return KVC_OK;
}

kvc_status run_gate(const kvc_shape& sh, const kvc_pool& p, const kvc_params& prm, const Sets& s, const float* partials,
                    double* gsum, int n_tiles, kvc_match_out* out, const int32_t* pred_flags, Tracer& tr,
                    hipStream_t st) {
  GateArgs g;
  memset(&g, 0, sizeof g);
  g.partials = partials;
  g.gsum = gsum;
  g.dist = out->dist; g.stat = out->stat; g.flags = out->flags;
  g.pred_flags = pred_flags;
  g.n_layers = sh.n_layers; g.n_tiles = n_tiles; g.N = p.n_anchors; g.mode = prm.mode;
  g.capacity = p.capacity == 0 ? p.n_anchors : p.capacity;
  g.mask_gate = s.gate; g.tau = prm.tau; g.temp_gate = prm.temp_gate;
  tr.begin(KVC_K_GATE);
  hipError_t e = launch_gate(g, st);
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "gate kernel");
  return KVC_OK;
}

// Materialised scores (second mode, or any shape through the generic kernel) + gate partials.
kvc_status run_scores(const void* k_src, const void* v_src, const kvc_shape& sh, int64_t p_src, const kvc_rope* rope,
                      const kvc_pool& p, const kvc_params& prm, const Sets& s, const Plan& pl, char* ws, Tracer& tr,
                      hipStream_t st) {
  const int n_use = (int)s.use_list.size();
  if (n_use == 0 || pl.n_tiles == 0) return KVC_OK;
  ScoreArgs a;
  memset(&a, 0, sizeof a);
  a.z[0] = k_src; a.z[1] = v_src;
  a.A[0] = p.baseA_k; a.A[1] = p.baseA_v;
  a.B[0] = p.baseB_k; a.B[1] = p.baseB_v;
  a.scores = reinterpret_cast<float*>(ws + pl.off_scores);
  a.partials = reinterpret_cast<float*>(ws + pl.off_partials);
  a.n_layers = sh.n_layers; a.S = sh.seq_len; a.D = D_of(sh); a.head_dim = sh.head_dim;
  a.s_cov = s.s_cov; a.k_gate = s.k; a.s_work = pl.s_work; a.n_tiles = pl.n_tiles;
  a.mask_corr = s.corr; a.mask_gate = s.gate;
  a.n_use = n_use;
  for (int i = 0; i < n_use; ++i) a.use[i] = s.use_list[i];
  a.g = geom(p, sh, p.rank_base);
  kvc_status s2 = make_tab(a.can, -p_src, sh.head_dim, rope);
  if (s2 != KVC_OK) return s2;
  hipError_t e;
  if (pl.cos_gemm) {
    CosGemmArgs c;
    memset(&c, 0, sizeof c);
    c.z[0] = (const uint16_t*)k_src; c.z[1] = (const uint16_t*)v_src;
    c.A[0] = (const uint16_t*)p.baseA_k; c.A[1] = (const uint16_t*)p.baseA_v;
    c.B[0] = (const uint16_t*)p.baseB_k; c.B[1] = (const uint16_t*)p.baseB_v;
    uint16_t* packed = reinterpret_cast<uint16_t*>(ws + pl.off_pack_cos);
    c.packed = packed;
    c.scores = a.scores; c.partials = a.partials;
    c.a_layer_stride = a.g.a_layer_stride; c.b_layer_stride = a.g.b_layer_stride;
    c.n_layers = a.n_layers; c.S = a.S; c.D = a.D; c.head_dim = a.head_dim; c.N = p.n_anchors;
    c.k_gate = a.k_gate; c.n_tiles = a.n_tiles; c.mask_gate = a.mask_gate;
    c.r = p.rank_base;
    c.n_use = n_use;
    for (int i = 0; i < n_use; ++i) c.use[i] = s.use_list[i];
    for (int i = 0; i < p.n_anchors; ++i) { c.off[i] = a.g.off[i]; c.len[i] = a.g.len[i]; }
    c.can = a.can;
    tr.begin(KVC_K_PACK_COS);
    e = launch_pack_cos(c, packed, st);
    tr.end();
    if (e != hipSuccess) return hip_fail(e, "pack kernel");
    tr.begin(KVC_K_SCORE_COS_GEMM);
    e = launch_score_cos_gemm(c, st);
  } else if (pl.cos_mfma) {
    tr.begin(KVC_K_SCORE_COS);
    e = launch_score_cos_mfma(a, st);
  } else {
    tr.begin(KVC_K_SCORE_GENERIC);
    e = launch_score_generic(a, p.dtype == KVC_BF16, prm.mode, pl.generic_tt, st);
  }
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "score kernel");
  return KVC_OK;
}

kvc_status run_softmax(const kvc_shape& sh, const kvc_pool& p, const kvc_params& prm, const Sets& s, const float* scores,
                       float* const w_out[2], Tracer& tr, hipStream_t st) {
  if (p.n_anchors == 0) return KVC_OK;
  SoftmaxArgs m;
  memset(&m, 0, sizeof m);
  m.scores = scores;
  m.w[0] = w_out[0]; m.w[1] = w_out[1];
  m.n_layers = sh.n_layers; m.S = sh.seq_len; m.N = p.n_anchors; m.s_cov = s.s_cov; m.mode = prm.mode;
  m.mask_corr = s.corr;
  m.inv_temp = (float)(1.0 / prm.temp_weight);
  tr.begin(KVC_K_SOFTMAX);
  hipError_t e = launch_softmax(m, st);
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "softmax kernel");
  return KVC_OK;
}

kvc_status run_apply_generic(const void* k_src, const void* v_src, void* k_out, void* v_out, const kvc_shape& sh,
                             int64_t p_src, int64_t p_tgt, const kvc_rope* rope, const kvc_pool& p, const float* w_k,
                             const float* w_v, int s_cov, const std::vector<int>& corr, Tracer& tr, hipStream_t st) {
  ApplyArgs a;
  memset(&a, 0, sizeof a);
  a.z[0] = k_src; a.z[1] = v_src;
  a.out[0] = k_out; a.out[1] = v_out;
  a.A[0] = p.deltaA_k; a.A[1] = p.deltaA_v;
  a.B[0] = p.deltaB_k; a.B[1] = p.deltaB_v;
  a.w[0] = w_k; a.w[1] = w_v;
  a.n_layers = sh.n_layers; a.S = sh.seq_len; a.D = D_of(sh); a.head_dim = sh.head_dim; a.s_cov = s_cov;
  a.n_corr = (int)corr.size();
  for (int i = 0; i < a.n_corr; ++i) a.corr[i] = corr[i];
  a.g = geom(p, sh, p.rank_delta);
  kvc_status s2 = make_tab(a.shift, p_tgt - p_src, sh.head_dim, rope);
  if (s2 != KVC_OK) return s2;
  if ((s2 = make_tab(a.tgt, p_tgt, sh.head_dim, rope)) != KVC_OK) return s2;
  tr.begin(KVC_K_APPLY_GENERIC);
  hipError_t e = launch_apply_generic(a, p.dtype == KVC_BF16, st);
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "apply kernel");
  return KVC_OK;
}

// The whole hop (or its match half when k_out == nullptr): every path of the library.
//   fused PAGES : pack base (+ delta) -> fused kernel (scores, weights, apply) -> gate
//   second mode : scores -> gate -> fused kernel (weights from scores, apply)
//   generic     : scores -> gate -> softmax -> generic apply
kvc_status run_hop(const void* k_src, const void* v_src, void* k_out, void* v_out, const kvc_shape& sh, int64_t p_src,
                   int64_t p_tgt, const kvc_rope* rope, const kvc_pool& p, const kvc_params& prm, const Sets& s,
                   const Plan& pl, char* ws, kvc_match_out* out, const int32_t* pred_flags, hipStream_t st) {
  Tracer tr{prm.trace, st};
  const bool apply = k_out != nullptr;
  float* partials = reinterpret_cast<float*>(ws + pl.off_partials);
  const float inv_temp = (float)(1.0 / prm.temp_weight);
  kvc_status r;
  if (pl.split_match) {
    uint16_t* pb = reinterpret_cast<uint16_t*>(ws + pl.off_pack_base);
    // base ranks 64 / 128 are packed as one matrix per rank slice of 32 (a scoring step takes two)
    if ((r = pack_pair(p.baseB_k, p.baseB_v, pb, p.rank_base, 1, nullptr, sh, p, tr, KVC_K_PACK_BASE, st,
                       split_apply_slices(p.rank_base))) != KVC_OK)
      return r;
    SplitArgs f;
    if ((r = split_args(f, k_src, v_src, sh, p_src, p_tgt, rope, p, s, inv_temp)) != KVC_OK) return r;
    const size_t per_b = (size_t)sh.n_layers * p.n_anchors * D_of(sh) * rpad16(p.rank_base);
    f.Ab[0] = (const uint16_t*)p.baseA_k; f.Ab[1] = (const uint16_t*)p.baseA_v;
    f.Bb[0] = pb; f.Bb[1] = pb + per_b;
    f.mpart = reinterpret_cast<float*>(ws + pl.off_mpart);
    f.partials = partials;
    f.w_out[0] = out->w_k; f.w_out[1] = out->w_v;
    if (p.n_anchors > 0) {
      tr.begin(KVC_K_SCORE_SPLIT);
      hipError_t e = launch_split_score(f, sh.head_dim, st);
      tr.end();
      if (e != hipSuccess) return hip_fail(e, "score kernel");
    }
    if ((r = run_gate(sh, p, prm, s, partials, reinterpret_cast<double*>(ws + pl.off_gsum), pl.n_tiles, out, pred_flags, tr, st)) != KVC_OK) return r;
    if (apply || out->w_k || out->w_v)
      if ((r = run_split_weights(f, SPLIT_W_PARTIALS, ws, pl, tr, st)) != KVC_OK) return r;
    if (apply) {
      if ((r = split_apply_fields(f, k_out, v_out, sh, p_tgt, rope, p, ws, pl, tr, st)) != KVC_OK) return r;
      if ((r = run_split_apply(f, sh, tr, st)) != KVC_OK) return r;
    }
    if (out->s_cov) *out->s_cov = s.s_cov;
    return KVC_OK;
  }
  if (pl.fused_match) {
    uint16_t* pb = reinterpret_cast<uint16_t*>(ws + pl.off_pack_base);
    if ((r = pack_pair(p.baseB_k, p.baseB_v, pb, p.rank_base, 1, nullptr, sh, p, tr, KVC_K_PACK_BASE, st)) != KVC_OK)
      return r;
    FusedArgs f;
    if ((r = fused_args(f, k_src, v_src, sh, p_src, p_tgt, rope, p, s, inv_temp)) != KVC_OK) return r;
    const size_t per_b = (size_t)sh.n_layers * p.n_anchors * D_of(sh) * rpad16(p.rank_base);
    f.Ab[0] = (const uint16_t*)p.baseA_k; f.Ab[1] = (const uint16_t*)p.baseA_v;
    f.Bb[0] = pb; f.Bb[1] = pb + per_b;
    f.w_out[0] = out->w_k; f.w_out[1] = out->w_v;
    f.partials = partials;
    const size_t plane = (size_t)sh.n_layers * sh.seq_len * std::max(p.n_anchors, 1);
    float* wts = reinterpret_cast<float*>(ws + pl.off_w);
    if (apply && pl.fused_split) {   // token weights to the workspace; the caller's copy comes from the apply's pass
      f.w_out[0] = wts;
      f.w_out[1] = wts + plane;
    } else if (apply) {
      FusedTab tgt;
      if ((r = fused_tab(tgt, p_tgt, sh.head_dim, rope)) != KVC_OK) return r;
      uint16_t* pd = reinterpret_cast<uint16_t*>(ws + pl.off_pack_delta);
      if ((r = pack_pair(p.deltaB_k, p.deltaB_v, pd, p.rank_delta, 0, &tgt, sh, p, tr, KVC_K_PACK_DELTA, st)) != KVC_OK)
        return r;
      const size_t per_d = (size_t)sh.n_layers * p.n_anchors * D_of(sh) * rpad16(p.rank_delta);
      f.out[0] = (uint16_t*)k_out; f.out[1] = (uint16_t*)v_out;
      f.Ad[0] = (const uint16_t*)p.deltaA_k; f.Ad[1] = (const uint16_t*)p.deltaA_v;
      f.Bd[0] = pd; f.Bd[1] = pd + per_d;
      f.apply = 1;
    }
    tr.begin(KVC_K_FUSED);
    hipError_t e = launch_fused(f, FUSED_PAGES, sh.head_dim, st);
    tr.end();
    if (e != hipSuccess) return hip_fail(e, "fused kernel");
    if ((r = run_gate(sh, p, prm, s, partials, reinterpret_cast<double*>(ws + pl.off_gsum), pl.n_tiles, out, pred_flags, tr, st)) != KVC_OK) return r;
    if (apply && pl.fused_split) {
      SplitArgs g;
      if ((r = split_args(g, k_src, v_src, sh, p_src, p_tgt, rope, p, s, inv_temp)) != KVC_OK) return r;
      if ((r = split_apply_fields(g, k_out, v_out, sh, p_tgt, rope, p, ws, pl, tr, st)) != KVC_OK) return r;
      g.w_in[0] = wts; g.w_in[1] = wts + plane;
      g.w_out[0] = out->w_k; g.w_out[1] = out->w_v;
      if ((r = run_split_weights(g, SPLIT_W_GIVEN, ws, pl, tr, st)) != KVC_OK) return r;
      if ((r = run_split_apply(g, sh, tr, st)) != KVC_OK) return r;
    }
    if (out->s_cov) *out->s_cov = s.s_cov;
    return KVC_OK;
  }
  // materialised scores
  if ((r = run_scores(k_src, v_src, sh, p_src, rope, p, prm, s, pl, ws, tr, st)) != KVC_OK) return r;
  if ((r = run_gate(sh, p, prm, s, partials, reinterpret_cast<double*>(ws + pl.off_gsum), pl.n_tiles, out, pred_flags, tr, st)) != KVC_OK) return r;
  const float* scores = reinterpret_cast<const float*>(ws + pl.off_scores);
  const size_t plane = (size_t)sh.n_layers * sh.seq_len * std::max(p.n_anchors, 1);
  if (apply && pl.split_apply) {
    // second scoring mode: weights formed from the scores inside the apply kernel
    SplitArgs f;
    if ((r = split_args(f, k_src, v_src, sh, p_src, p_tgt, rope, p, s, inv_temp)) != KVC_OK) return r;
    if ((r = split_apply_fields(f, k_out, v_out, sh, p_tgt, rope, p, ws, pl, tr, st)) != KVC_OK) return r;
    f.w_in[0] = scores; f.w_in[1] = scores + plane;
    f.w_out[0] = out->w_k; f.w_out[1] = out->w_v;
    if ((r = run_split_weights(f, SPLIT_W_SCORES, ws, pl, tr, st)) != KVC_OK) return r;
    if ((r = run_split_apply(f, sh, tr, st)) != KVC_OK) return r;
  } else if (apply && pl.fused_apply) {
    // second scoring mode: weights formed from the scores inside the fused kernel
    FusedArgs f;
    if ((r = fused_args(f, k_src, v_src, sh, p_src, p_tgt, rope, p, s, inv_temp)) != KVC_OK) return r;
    FusedTab tgt;
    if ((r = fused_tab(tgt, p_tgt, sh.head_dim, rope)) != KVC_OK) return r;
    uint16_t* pd = reinterpret_cast<uint16_t*>(ws + pl.off_pack_delta);
    if ((r = pack_pair(p.deltaB_k, p.deltaB_v, pd, p.rank_delta, 0, &tgt, sh, p, tr, KVC_K_PACK_DELTA, st)) != KVC_OK)
      return r;
    const size_t per_d = (size_t)sh.n_layers * p.n_anchors * D_of(sh) * rpad16(p.rank_delta);
    f.out[0] = (uint16_t*)k_out; f.out[1] = (uint16_t*)v_out;
    f.Ad[0] = (const uint16_t*)p.deltaA_k; f.Ad[1] = (const uint16_t*)p.deltaA_v;
    f.Bd[0] = pd; f.Bd[1] = pd + per_d;
    f.w_in[0] = scores; f.w_in[1] = scores + plane;
    f.w_out[0] = out->w_k; f.w_out[1] = out->w_v;
    f.apply = 1;
    tr.begin(KVC_K_FUSED);
    hipError_t e = launch_fused(f, FUSED_SCORES, sh.head_dim, st);
    tr.end();
    if (e != hipSuccess) return hip_fail(e, "fused kernel");
  } else {
    float* wbuf = reinterpret_cast<float*>(ws + pl.off_w);
    float* w_out[2] = {out->w_k ? out->w_k : wbuf, out->w_v ? out->w_v : wbuf + plane};
    if ((r = run_softmax(sh, p, prm, s, scores, w_out, tr, st)) != KVC_OK) return r;
    if (apply &&
        (r = run_apply_generic(k_src, v_src, k_out, v_out, sh, p_src, p_tgt, rope, p, w_out[0], w_out[1],
                               s.corr_list.empty() ? 0 : s.s_cov, s.corr_list, tr, st)) != KVC_OK)
      return r;
  }
  if (out->s_cov) *out->s_cov = s.s_cov;
  return KVC_OK;
}


kvc_status check_cache(const void* k, const void* v, const char* nk, const char* nv) {
  if (!k) return fail(KVC_E_NULL, "%s is NULL", nk);
  if (!v) return fail(KVC_E_NULL, "%s is NULL", nv);
  if (!aligned16(k)) return fail(KVC_E_ALIGN, "%s is not 16-byte aligned", nk);
  if (!aligned16(v)) return fail(KVC_E_ALIGN, "%s is not 16-byte aligned", nv);
  return KVC_OK;
}

kvc_status check_match_out(const kvc_match_out* out, const kvc_shape& sh, const kvc_pool& p) {
  if (!out) return fail(KVC_E_NULL, "match output descriptor is NULL");
  if (!out->dist || !out->stat || !out->flags) return fail(KVC_E_NULL, "match output: dist/stat/flags must be set");
  (void)sh;
  (void)p;
  return KVC_OK;
}

// Full validation of one correct-hop request (no launches).
struct HopReq {
  const void *k_src, *v_src;
  void *k_out, *v_out;
  int64_t p_src, p_tgt;
  const kvc_pool* pool;
  kvc_match_out* out;
};

kvc_status validate_hop(const HopReq& h, kvc_dtype dt, const kvc_shape& sh, const kvc_rope* rope,
                        const kvc_params* prm, bool check_src) {
  kvc_status s;
  if ((s = check_dtype(dt, "cache")) != KVC_OK) return s;
  if ((s = check_shape(sh)) != KVC_OK) return s;
  if ((s = check_rope(rope)) != KVC_OK) return s;
  if ((s = check_params(prm, sh.seq_len)) != KVC_OK) return s;
  if ((s = check_pool(h.pool, sh, dt, true, true)) != KVC_OK) return s;
  if (check_src && (s = check_cache(h.k_src, h.v_src, "k_src", "v_src")) != KVC_OK) return s;
  if ((s = check_cache(h.k_out, h.v_out, "k_out", "v_out")) != KVC_OK) return s;
  if ((s = check_match_out(h.out, sh, *h.pool)) != KVC_OK) return s;
  const size_t bytes = (size_t)sh.n_layers * sh.seq_len * D_of(sh) * esize(dt);
  if (overlaps(h.k_out, bytes, h.v_out, bytes)) return fail(KVC_E_ALIAS, "k_out overlaps v_out");
  if (check_src) {
    const void* srcs[2] = {h.k_src, h.v_src};
    const void* outs[2] = {h.k_out, h.v_out};
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 2; ++j)
        if (overlaps(outs[i], bytes, srcs[j], bytes))
          return fail(KVC_E_ALIAS, "output %s overlaps source %s", i ? "v_out" : "k_out", j ? "v_src" : "k_src");
  }
  return KVC_OK;
}

// ----------------------------------------------------------------- batched chain levels
// KVCMAS Sec. 3.2 Eq. 6 and App. A.3 "Cache Materialization": a materialised target is the next
// edge's source, so hop h of every request depends only on hop h - 1 of the same request.  The
// hops of one level (the same depth in their chains) are independent and run as one grid per
// kernel: descriptors of every hop in device memory, each hop with its own workspace region.
struct LevelHop {
  int idx;   // index in the caller's hop array
  HopReq h;
  Sets sets;
  Plan pl;
  const int32_t* pred;
};

// a hop the batched kernels take: the two-pass path end to end, with at least one anchor to apply
bool batchable(const Plan& pl, const Sets& s, const kvc_pool& p) {
  return pl.split_match && pl.split_apply && !pl.fused_split && p.n_anchors > 0 && !s.corr_list.empty() &&
         (p.rank_base == 16 || p.rank_base == 32);
}

size_t level_desc_bytes(int n) {
  return up256(sizeof(SplitArgs) * n) + up256(sizeof(GateArgs) * n) + up256(sizeof(PackArgs) * 2 * n);
}

// per-hop regions of a level run batched: one plan-sized region per hop
size_t level_region_bytes(const std::vector<LevelHop>& v) {
  size_t t = 0;
  for (const LevelHop& x : v) t += up256(x.pl.total);
  return t;
}

// Host descriptors of one batched group; `region` = its hops' workspace regions.
struct LevelArgs {
  std::vector<SplitArgs> sa;
  std::vector<GateArgs> ga;
  std::vector<PackArgs> pa;
};

kvc_status level_args(LevelArgs& la, const std::vector<LevelHop>& v, const kvc_shape& sh, const kvc_rope* rope,
                      const kvc_params& prm, char* region) {
  const int n = (int)v.size();
  la.sa.resize(n);
  la.ga.resize(n);
  la.pa.resize(2 * n);
  const float inv_temp = (float)(1.0 / prm.temp_weight);
  const int D = D_of(sh);
  for (int i = 0; i < n; ++i) {
    const LevelHop& x = v[i];
    const kvc_pool& p = *x.h.pool;
    char* w = region;
    region += up256(x.pl.total);
    kvc_status r;
    SplitArgs& f = la.sa[i];
    if ((r = split_args(f, x.h.k_src, x.h.v_src, sh, x.h.p_src, x.h.p_tgt, rope, p, x.sets, inv_temp)) != KVC_OK)
      return r;
    // operands: base B negated (scores E = Z - A B), delta B with key rows turned by R(p_tgt)
    uint16_t* pb = reinterpret_cast<uint16_t*>(w + x.pl.off_pack_base);
    uint16_t* pd = reinterpret_cast<uint16_t*>(w + x.pl.off_pack_delta);
    const size_t per_b = (size_t)sh.n_layers * p.n_anchors * D * rpad16(p.rank_base);
    const size_t per_d = (size_t)sh.n_layers * p.n_anchors * D * rpad16(p.rank_delta);
    FusedTab tgt;
    if ((r = fused_tab(tgt, x.h.p_tgt, sh.head_dim, rope)) != KVC_OK) return r;
    {
      const uint16_t* src[2] = {(const uint16_t*)p.baseB_k, (const uint16_t*)p.baseB_v};
      uint16_t* dst[2] = {pb, pb + per_b};
      const int neg[2] = {1, 1};
      const FusedTab* tabs[2] = {nullptr, nullptr};
      if (!make_pack_args(la.pa[2 * i], src, dst, neg, tabs, 2, sh.n_layers, p.n_anchors, p.rank_base, D,
                          sh.head_dim))
        return fail(KVC_E_PARAM, "batched hop: base factors cannot be packed");
    }
    {
      const int sl = split_apply_slices(p.rank_delta);
      const uint16_t* src[2] = {(const uint16_t*)p.deltaB_k, (const uint16_t*)p.deltaB_v};
      uint16_t* dst[2] = {pd, pd + per_d};
      const int neg[2] = {0, 0};
      const FusedTab* tabs[2] = {&tgt, nullptr};
      if (!make_pack_args(la.pa[2 * i + 1], src, dst, neg, tabs, 2, sh.n_layers, p.n_anchors * sl,
                          p.rank_delta / sl, D, sh.head_dim))
        return fail(KVC_E_PARAM, "batched hop: delta factors cannot be packed");
    }
    f.Ab[0] = (const uint16_t*)p.baseA_k; f.Ab[1] = (const uint16_t*)p.baseA_v;
    f.Bb[0] = pb; f.Bb[1] = pb + per_b;
    f.mpart = reinterpret_cast<float*>(w + x.pl.off_mpart);
    f.partials = reinterpret_cast<float*>(w + x.pl.off_partials);
    f.w_out[0] = x.h.out->w_k; f.w_out[1] = x.h.out->w_v;
    f.wa = reinterpret_cast<float*>(w + x.pl.off_wa);
    f.out[0] = (uint16_t*)x.h.k_out; f.out[1] = (uint16_t*)x.h.v_out;
    f.Ad[0] = (const uint16_t*)p.deltaA_k; f.Ad[1] = (const uint16_t*)p.deltaA_v;
    f.Bd[0] = pd; f.Bd[1] = pd + per_d;
    f.apply = 1;
    GateArgs& g = la.ga[i];
    memset(&g, 0, sizeof g);
    g.partials = f.partials;
    g.gsum = reinterpret_cast<double*>(w + x.pl.off_gsum);
    g.dist = x.h.out->dist; g.stat = x.h.out->stat; g.flags = x.h.out->flags;
    g.pred_flags = x.pred;
    g.n_layers = sh.n_layers; g.n_tiles = x.pl.n_tiles; g.N = p.n_anchors; g.mode = prm.mode;
    g.capacity = p.capacity == 0 ? p.n_anchors : p.capacity;
    g.mask_gate = x.sets.gate; g.tau = prm.tau; g.temp_gate = prm.temp_gate;
  }
  return KVC_OK;
}

// device copies of a group's descriptors at `d` (level_desc_bytes(n) bytes, uploaded already)
kvc_status launch_level(const LevelArgs& la, const char* d, const kvc_shape& sh, const kvc_params& prm,
                        hipStream_t st) {
  const int n = (int)la.sa.size();
  Tracer tr{prm.trace, st};
  const SplitArgs* ds = reinterpret_cast<const SplitArgs*>(d);
  const GateArgs* dg = reinterpret_cast<const GateArgs*>(d + up256(sizeof(SplitArgs) * n));
  const PackArgs* dp = reinterpret_cast<const PackArgs*>(d + up256(sizeof(SplitArgs) * n) + up256(sizeof(GateArgs) * n));
  tr.begin(KVC_K_PACK_BASE);
  hipError_t e = launch_pack_b_batch(dp, la.pa.data(), 2 * n, st);
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "batched pack kernel");
  tr.begin(KVC_K_SCORE_SPLIT);
  e = launch_split_score_batch(ds, la.sa.data(), n, sh.head_dim, st);
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "batched score kernel");
  tr.begin(KVC_K_GATE);
  e = launch_gate_batch(dg, la.ga.data(), n, st);
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "batched gate kernels");
  tr.begin(KVC_K_WEIGHTS_SPLIT);
  e = launch_split_weights_batch(ds, la.sa.data(), n, st);
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "batched weights kernel");
  tr.begin(KVC_K_APPLY_SPLIT);
  e = launch_split_apply_batch(ds, la.sa.data(), n, sh.head_dim, st);
  tr.end();
  if (e != hipSuccess) return hip_fail(e, "batched apply kernel");
  return KVC_OK;
}

// Chain depth of every hop (0 = reads a given source) and the hops of each level in index order.
std::vector<std::vector<int>> chain_levels(const kvc_hop_desc* hops, int n) {
  std::vector<int> lev(n, 0);
  int top = 0;
  for (int i = 0; i < n; ++i) {
    lev[i] = hops[i].chain_prev >= 0 ? lev[hops[i].chain_prev] + 1 : 0;
    top = std::max(top, lev[i]);
  }
  std::vector<std::vector<int>> out(n ? top + 1 : 0);
  for (int i = 0; i < n; ++i) out[lev[i]].push_back(i);
  return out;
}

HopReq hop_req(const kvc_hop_desc* hops, int i) {
  const kvc_hop_desc& d = hops[i];
  return HopReq{d.chain_prev >= 0 ? hops[d.chain_prev].k_out : d.k_src,
                d.chain_prev >= 0 ? hops[d.chain_prev].v_out : d.v_src,
                d.k_out, d.v_out, d.p_src, d.p_tgt, &d.pool, const_cast<kvc_match_out*>(&d.out)};
}

// The hops of each level: groups launched as one grid per kernel (at most kMaxBatch hops each),
// and hops that take another path, run one call at a time.
struct BatchLevel {
  std::vector<std::vector<LevelHop>> groups;
  std::vector<int> single;
};
struct BatchPlan {
  std::vector<BatchLevel> levels;
  size_t ws_desc = 0;      // descriptors of every group, uploaded once at the start
  size_t ws_region = 0;    // largest group's per-hop regions (reused level after level)
  size_t ws_batched = 0;   // ws_desc + ws_region
  size_t ws_single = 0;    // largest one-hop workspace
};

BatchPlan batch_plan(const kvc_hop_desc* hops, int n, kvc_dtype dt, const kvc_shape& sh, const kvc_params& prm) {
  BatchPlan bp;
  const bool mode_ok = dt == KVC_BF16 && prm.mode == KVC_SCORE_PAGES && prm.options == 0;
  for (const std::vector<int>& ids : chain_levels(hops, n)) {
    BatchLevel lv;
    std::vector<LevelHop> cur;
    for (int i : ids) {
      const kvc_hop_desc& d = hops[i];
      LevelHop x{i, hop_req(hops, i), anchor_sets(d.pool, sh.seq_len, prm.gate_len), Plan(), nullptr};
      x.pl = plan(KVC_CALL_CORRECT, sh, d.pool, &prm, x.sets);
      x.pred = d.chain_prev >= 0 ? hops[d.chain_prev].out.flags : nullptr;
      bp.ws_single = std::max(bp.ws_single, x.pl.total);
      if (mode_ok && batchable(x.pl, x.sets, d.pool)) {
        cur.push_back(x);
        if ((int)cur.size() == kMaxBatch) {
          lv.groups.push_back(cur);
          cur.clear();
        }
      } else {
        lv.single.push_back(i);
      }
    }
    if (!cur.empty()) lv.groups.push_back(cur);
    for (const auto& g : lv.groups) {
      bp.ws_desc += level_desc_bytes((int)g.size());
      bp.ws_region = std::max(bp.ws_region, level_region_bytes(g));
    }
    bp.levels.push_back(lv);
  }
  // one-hop calls of a batched run use the space after the descriptors too
  bp.ws_batched = bp.ws_desc ? bp.ws_desc + std::max(bp.ws_region, bp.ws_single) : 0;
  return bp;
}

}  // namespace

kvc_status kvc::report(kvc_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

// ================================================================== C ABI
extern "C" {

int32_t kvc_abi_version(void) { return KVC_ABI_VERSION; }

const char* kvc_status_str(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_E_NULL: return "null pointer";
    case KVC_E_SHAPE: return "bad shape";
    case KVC_E_DTYPE: return "bad dtype";
    case KVC_E_ALIGN: return "misaligned pointer";
    case KVC_E_ALIAS: return "output aliases input";
    case KVC_E_WORKSPACE: return "workspace too small";
    case KVC_E_HIP: return "HIP runtime error";
    case KVC_E_PARAM: return "bad parameter";
    case KVC_E_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* kvc_last_error(void) { return g_err; }

size_t kvc_workspace_size(int32_t call, kvc_shape shape, const kvc_pool* pool, const kvc_params* params) {
  if (call != KVC_CALL_MATCH && call != KVC_CALL_APPLY && call != KVC_CALL_CORRECT) return 0;
  if (check_shape(shape) != KVC_OK || !pool || pool->n_anchors < 0 || pool->n_anchors > KVC_MAX_ANCHORS) return 0;
  if (pool->n_anchors > 0 && !pool->anchor_len) return 0;
  for (int a = 0; a < pool->n_anchors; ++a)
    if (is_live(*pool, a) && pool->anchor_len[a] < 1) return 0;
  const int gl = params ? params->gate_len : 0;
  Sets s = anchor_sets(*pool, shape.seq_len, gl);
  return plan(call, shape, *pool, params, s).total;
}

kvc_status kvc_align_rope(const void* k_in, void* k_out, kvc_dtype in_t, kvc_dtype out_t, kvc_shape shape,
                          int64_t pos_from, int64_t pos_to, const kvc_rope* rope, void* stream) {
  kvc_status s;
  if ((s = check_dtype(in_t, "in_t")) != KVC_OK) return s;
  if ((s = check_dtype(out_t, "out_t")) != KVC_OK) return s;
  if ((s = check_shape(shape)) != KVC_OK) return s;
  if ((s = check_rope(rope)) != KVC_OK) return s;
  if (!k_in || !k_out) return fail(KVC_E_NULL, "k_in/k_out is NULL");
  if (!aligned16(k_in) || !aligned16(k_out)) return fail(KVC_E_ALIGN, "k_in/k_out not 16-byte aligned");
  const size_t n = (size_t)shape.n_layers * shape.seq_len * D_of(shape);
  const size_t bi = n * esize(in_t), bo = n * esize(out_t);
  if (k_in == k_out) {
    if (in_t != out_t) return fail(KVC_E_ALIAS, "in-place re-alignment needs in_t == out_t");
  } else if (overlaps(k_in, bi, k_out, bo)) {
    return fail(KVC_E_ALIAS, "k_out partially overlaps k_in");
  }
  RopeTab tab;
  if ((s = make_tab(tab, pos_to - pos_from, shape.head_dim, rope)) != KVC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if (!tab.active && k_in == k_out) return ok();
  hipError_t e = launch_align(k_in, k_out, in_t == KVC_BF16, out_t == KVC_BF16,
                              (int64_t)shape.n_layers * shape.seq_len, shape.n_kv_heads, shape.head_dim, tab, st);
  if (e != hipSuccess) return hip_fail(e, "align kernel");
  return ok();
}

kvc_status kvc_match_anchors(const void* k_src, const void* v_src, kvc_dtype dtype, kvc_shape shape, int64_t p_src,
                             const kvc_rope* rope, const kvc_pool* pool, const kvc_params* params,
                             kvc_match_out* out, void* workspace, size_t ws_bytes, void* stream) {
  kvc_status s;
  if ((s = check_dtype(dtype, "cache")) != KVC_OK) return s;
  if ((s = check_shape(shape)) != KVC_OK) return s;
  if ((s = check_rope(rope)) != KVC_OK) return s;
  if ((s = check_params(params, shape.seq_len)) != KVC_OK) return s;
  if ((s = check_pool(pool, shape, dtype, true, false)) != KVC_OK) return s;
  if ((s = check_cache(k_src, v_src, "k_src", "v_src")) != KVC_OK) return s;
  if ((s = check_match_out(out, shape, *pool)) != KVC_OK) return s;
  const size_t wbytes = sizeof(float) * (size_t)shape.n_layers * shape.seq_len * pool->n_anchors;
  if ((out->w_k && !aligned16(out->w_k)) || (out->w_v && !aligned16(out->w_v)))
    return fail(KVC_E_ALIGN, "w_k/w_v not 16-byte aligned");
  if (out->w_k && out->w_v && overlaps(out->w_k, wbytes, out->w_v, wbytes))
    return fail(KVC_E_ALIAS, "w_k overlaps w_v");
  Sets sets = anchor_sets(*pool, shape.seq_len, params->gate_len);
  Plan pl = plan(KVC_CALL_MATCH, shape, *pool, params, sets);
  if (pl.total && (!workspace || ws_bytes < pl.total))
    return fail(KVC_E_WORKSPACE, "workspace: need %zu bytes, got %zu", pl.total, workspace ? ws_bytes : (size_t)0);
  if (workspace && !aligned16(workspace)) return fail(KVC_E_ALIGN, "workspace not 16-byte aligned");
  s = run_hop(k_src, v_src, nullptr, nullptr, shape, p_src, 0, rope, *pool, *params, sets, pl, (char*)workspace, out,
              nullptr, (hipStream_t)stream);
  return s == KVC_OK ? ok() : s;
}

kvc_status kvc_apply_lowrank_delta(const void* k_src, const void* v_src, void* k_out, void* v_out, kvc_dtype dtype,
                                   kvc_shape shape, int64_t p_src, int64_t p_tgt, const kvc_rope* rope,
                                   const kvc_pool* pool, const float* w_k, const float* w_v, int32_t s_cov,
                                   void* workspace, size_t ws_bytes, void* stream) {
  kvc_status s;
  if ((s = check_dtype(dtype, "cache")) != KVC_OK) return s;
  if ((s = check_shape(shape)) != KVC_OK) return s;
  if ((s = check_rope(rope)) != KVC_OK) return s;
  if ((s = check_pool(pool, shape, dtype, false, true)) != KVC_OK) return s;
  if ((s = check_cache(k_src, v_src, "k_src", "v_src")) != KVC_OK) return s;
  if ((s = check_cache(k_out, v_out, "k_out", "v_out")) != KVC_OK) return s;
  if (s_cov < 0 || s_cov > shape.seq_len) return fail(KVC_E_PARAM, "s_cov must be in [0, seq_len]");
  if (pool->n_anchors > 0 && s_cov > 0) {
    if (!w_k || !w_v) return fail(KVC_E_NULL, "w_k/w_v is NULL");
    if (!aligned16(w_k) || !aligned16(w_v)) return fail(KVC_E_ALIGN, "w_k/w_v not 16-byte aligned");
  }
  const size_t bytes = (size_t)shape.n_layers * shape.seq_len * D_of(shape) * esize(dtype);
  const void* srcs[2] = {k_src, v_src};
  const void* outs[2] = {k_out, v_out};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j)
      if (overlaps(outs[i], bytes, srcs[j], bytes))
        return fail(KVC_E_ALIAS, "output %s overlaps source %s", i ? "v_out" : "k_out", j ? "v_src" : "k_src");
  if (overlaps(k_out, bytes, v_out, bytes)) return fail(KVC_E_ALIAS, "k_out overlaps v_out");
  // correction set of an explicit-weight apply: anchors covering the first s_cov rows
  Sets sets;
  sets.k = shape.seq_len;
  sets.s_cov = s_cov;
  if (s_cov > 0)
    for (int a = 0; a < pool->n_anchors; ++a)
      if (is_live(*pool, a) && pool->anchor_len[a] >= s_cov) {
        sets.corr |= 1ull << a;
        sets.corr_list.push_back(a);
        sets.use_list.push_back(a);
      }
  Plan pl = plan(KVC_CALL_APPLY, shape, *pool, nullptr, sets);
  if (pl.total && (!workspace || ws_bytes < pl.total))
    return fail(KVC_E_WORKSPACE, "workspace: need %zu bytes, got %zu", pl.total, workspace ? ws_bytes : (size_t)0);
  if (workspace && !aligned16(workspace)) return fail(KVC_E_ALIGN, "workspace not 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  Tracer tr{nullptr, st};
  if (pl.split_apply) {
    SplitArgs f;
    if ((s = split_args(f, k_src, v_src, shape, p_src, p_tgt, rope, *pool, sets, 1.f)) != KVC_OK) return s;
    if ((s = split_apply_fields(f, k_out, v_out, shape, p_tgt, rope, *pool, (char*)workspace, pl, tr, st)) != KVC_OK)
      return s;
    f.w_in[0] = w_k; f.w_in[1] = w_v;
    if ((s = run_split_weights(f, SPLIT_W_GIVEN, (char*)workspace, pl, tr, st)) != KVC_OK) return s;
    if ((s = run_split_apply(f, shape, tr, st)) != KVC_OK) return s;
  } else if (pl.fused_apply) {
    FusedArgs f;
    if ((s = fused_args(f, k_src, v_src, shape, p_src, p_tgt, rope, *pool, sets, 1.f)) != KVC_OK) return s;
    FusedTab tgt;
    if ((s = fused_tab(tgt, p_tgt, shape.head_dim, rope)) != KVC_OK) return s;
    uint16_t* pd = reinterpret_cast<uint16_t*>((char*)workspace + pl.off_pack_delta);
    if ((s = pack_pair(pool->deltaB_k, pool->deltaB_v, pd, pool->rank_delta, 0, &tgt, shape, *pool, tr,
                       KVC_K_PACK_DELTA, st)) != KVC_OK)
      return s;
    const size_t per_d = (size_t)shape.n_layers * pool->n_anchors * D_of(shape) * rpad16(pool->rank_delta);
    f.out[0] = (uint16_t*)k_out; f.out[1] = (uint16_t*)v_out;
    f.Ad[0] = (const uint16_t*)pool->deltaA_k; f.Ad[1] = (const uint16_t*)pool->deltaA_v;
    f.Bd[0] = pd; f.Bd[1] = pd + per_d;
    f.w_in[0] = w_k; f.w_in[1] = w_v;
    f.apply = 1;
    hipError_t e = launch_fused(f, FUSED_GIVEN, shape.head_dim, st);
    if (e != hipSuccess) return hip_fail(e, "fused kernel");
  } else {
    s = run_apply_generic(k_src, v_src, k_out, v_out, shape, p_src, p_tgt, rope, *pool, w_k, w_v,
                          sets.corr_list.empty() ? 0 : s_cov, sets.corr_list, tr, st);
    if (s != KVC_OK) return s;
  }
  return ok();
}

static kvc_status correct_one(const HopReq& h, kvc_dtype /* validated by the caller; the pool carries it */,
                              const kvc_shape& sh, const kvc_rope* rope,
                              const kvc_params* prm, char* ws, size_t ws_bytes, const int32_t* pred_flags,
                              hipStream_t st) {
  const kvc_pool& p = *h.pool;
  Sets sets = anchor_sets(p, sh.seq_len, prm->gate_len);
  Plan pl = plan(KVC_CALL_CORRECT, sh, p, prm, sets);
  if (pl.total && (!ws || ws_bytes < pl.total))
    return fail(KVC_E_WORKSPACE, "workspace: need %zu bytes, got %zu", pl.total, ws ? ws_bytes : (size_t)0);
  return run_hop(h.k_src, h.v_src, h.k_out, h.v_out, sh, h.p_src, h.p_tgt, rope, p, *prm, sets, pl, ws, h.out,
                 pred_flags, st);
}

kvc_status kvc_correct_hop(const void* k_src, const void* v_src, void* k_out, void* v_out, kvc_dtype dtype,
                           kvc_shape shape, int64_t p_src, int64_t p_tgt, const kvc_rope* rope, const kvc_pool* pool,
                           const kvc_params* params, kvc_match_out* out, void* workspace, size_t ws_bytes,
                           void* stream) {
  HopReq h{k_src, v_src, k_out, v_out, p_src, p_tgt, pool, out};
  kvc_status s = validate_hop(h, dtype, shape, rope, params, true);
  if (s != KVC_OK) return s;
  if (workspace && !aligned16(workspace)) return fail(KVC_E_ALIGN, "workspace not 16-byte aligned");
  s = correct_one(h, dtype, shape, rope, params, (char*)workspace, ws_bytes, nullptr, (hipStream_t)stream);
  return s == KVC_OK ? ok() : s;
}

size_t kvc_hops_batched_workspace_size(const kvc_hop_desc* hops, int32_t n_hops, kvc_dtype dtype, kvc_shape shape,
                                       const kvc_params* params) {
  if (!hops || n_hops < 1 || !params || check_shape(shape) != KVC_OK) return 0;
  for (int i = 0; i < n_hops; ++i) {
    const kvc_pool& p = hops[i].pool;
    if (hops[i].chain_prev >= i || p.n_anchors < 0 || p.n_anchors > KVC_MAX_ANCHORS || (p.n_anchors && !p.anchor_len))
      return 0;
    for (int a = 0; a < p.n_anchors; ++a)
      if (is_live(p, a) && p.anchor_len[a] < 1) return 0;
  }
  const BatchPlan bp = batch_plan(hops, n_hops, dtype, shape, *params);
  return std::max(bp.ws_batched, bp.ws_single);
}

kvc_status kvc_correct_hops_batched(const kvc_hop_desc* hops, int32_t n_hops, kvc_dtype dtype, kvc_shape shape,
                                    const kvc_rope* rope, const kvc_params* params, void* workspace, size_t ws_bytes,
                                    void* stream) {
  if (n_hops < 0) return fail(KVC_E_PARAM, "n_hops < 0");
  if (n_hops == 0) return ok();
  if (!hops) return fail(KVC_E_NULL, "hops is NULL");
  if (workspace && !aligned16(workspace)) return fail(KVC_E_ALIGN, "workspace not 16-byte aligned");
  // validate everything before the first launch
  for (int i = 0; i < n_hops; ++i) {
    const kvc_hop_desc& d = hops[i];
    if (d.chain_prev >= i) return fail(KVC_E_PARAM, "hop %d: chain_prev must precede the hop", i);
    kvc_status s = validate_hop(hop_req(hops, i), dtype, shape, rope, params, true);
    if (s != KVC_OK) {
      char buf[512];
      snprintf(buf, sizeof buf, "hop %d: %s", i, g_err);
      return fail(s, "%s", buf);
    }
  }
  const BatchPlan bp = batch_plan(hops, n_hops, dtype, shape, *params);
  if (bp.ws_single && (!workspace || ws_bytes < bp.ws_single))
    return fail(KVC_E_WORKSPACE, "workspace needs %zu bytes (one hop at a time) or %zu (batched), got %zu",
                bp.ws_single, std::max(bp.ws_single, bp.ws_batched), workspace ? ws_bytes : (size_t)0);
  // batched levels when the workspace holds the descriptors and the largest group; otherwise
  // every hop on its own
  const bool batched = bp.ws_desc && workspace && ws_bytes >= bp.ws_batched;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  std::vector<LevelArgs> args;
  if (batched) {
    // every group's descriptors (per-hop regions after the descriptor area), one upload
    std::vector<char> host(bp.ws_desc);
    size_t off = 0;
    for (const BatchLevel& lv : bp.levels)
      for (const auto& g : lv.groups) {
        args.emplace_back();
        kvc_status s = level_args(args.back(), g, shape, rope, *params, ws + bp.ws_desc);
        if (s != KVC_OK) return s;
        const int n = (int)g.size();
        const LevelArgs& la = args.back();
        memcpy(host.data() + off, la.sa.data(), sizeof(SplitArgs) * n);
        memcpy(host.data() + off + up256(sizeof(SplitArgs) * n), la.ga.data(), sizeof(GateArgs) * n);
        memcpy(host.data() + off + up256(sizeof(SplitArgs) * n) + up256(sizeof(GateArgs) * n), la.pa.data(),
               sizeof(PackArgs) * 2 * n);
        off += level_desc_bytes(n);
      }
    hipError_t e = hipMemcpyAsync(ws, host.data(), bp.ws_desc, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "batched hops: descriptor upload");
  }
  size_t doff = 0;
  size_t gi = 0;
  for (const BatchLevel& lv : bp.levels) {
    std::vector<int> one = lv.single;
    if (batched) {
      for (const auto& g : lv.groups) {
        kvc_status s = launch_level(args[gi++], ws + doff, shape, *params, st);
        if (s != KVC_OK) return s;
        for (const LevelHop& x : g)
          if (x.h.out->s_cov) *x.h.out->s_cov = x.sets.s_cov;
        doff += level_desc_bytes((int)g.size());
      }
    } else {
      for (const auto& g : lv.groups)
        for (const LevelHop& x : g) one.push_back(x.idx);
      std::sort(one.begin(), one.end());
    }
    // past the descriptor area when batched (later groups' descriptors are already there)
    char* ws1 = batched ? ws + bp.ws_desc : ws;
    const size_t ws1_bytes = batched ? ws_bytes - bp.ws_desc : ws_bytes;
    for (int i : one) {
      const kvc_hop_desc& d = hops[i];
      const int32_t* pred = d.chain_prev >= 0 ? hops[d.chain_prev].out.flags : nullptr;
      kvc_status s = correct_one(hop_req(hops, i), dtype, shape, rope, params, ws1, ws1_bytes, pred, st);
      if (s != KVC_OK) return s;
    }
  }
  return ok();
}

size_t kvc_svd_workspace_size(int32_t n_mats, int32_t rows, int32_t cols, int32_t rank, int32_t oversample) {
  if (n_mats < 1 || rows < 1 || cols < 1 || rank < 1 || oversample < 0) return 0;
  return svd_workspace_bytes(n_mats, rows, cols, rank, oversample);
}

kvc_status kvc_anchor_refresh_svd(const float* z, int32_t n_mats, int32_t rows, int32_t cols, int32_t rank,
                                  void* a_out, void* b_out, kvc_dtype out_t, float* sigma_out, int32_t oversample,
                                  int32_t power_iters, uint64_t seed, void* workspace, size_t ws_bytes,
                                  void* stream) {
  kvc_status s;
  if ((s = check_dtype(out_t, "out_t")) != KVC_OK) return s;
  if (!z || !a_out || !b_out || !sigma_out) return fail(KVC_E_NULL, "z/a_out/b_out/sigma_out is NULL");
  if (!aligned16(z) || !aligned16(a_out) || !aligned16(b_out) || !aligned16(sigma_out))
    return fail(KVC_E_ALIGN, "svd buffers must be 16-byte aligned");
  if (n_mats < 1 || rows < 1 || cols < 1) return fail(KVC_E_SHAPE, "svd: n_mats, rows, cols must be >= 1");
  if (rank < 1 || oversample < 0 || rank + oversample > std::min(rows, cols) || rank + oversample > 256)
    return fail(KVC_E_SHAPE, "svd: need 1 <= rank, rank + oversample <= min(rows, cols, 256)");
  if (rows % 4 || cols % 4) return fail(KVC_E_SHAPE, "svd: rows and cols must be multiples of 4");
  if (power_iters < 0 || power_iters > 16) return fail(KVC_E_PARAM, "svd: power_iters must be in [0, 16]");
  const size_t need = svd_workspace_bytes(n_mats, rows, cols, rank, oversample);
  if (!workspace || ws_bytes < need) return fail(KVC_E_WORKSPACE, "svd workspace: need %zu bytes", need);
  if (!aligned16(workspace)) return fail(KVC_E_ALIGN, "workspace not 16-byte aligned");
  const size_t zb = (size_t)n_mats * rows * cols * 4;
  if (overlaps(z, zb, a_out, (size_t)n_mats * rows * rank * esize(out_t)) ||
      overlaps(z, zb, b_out, (size_t)n_mats * rank * cols * esize(out_t)))
    return fail(KVC_E_ALIAS, "svd outputs overlap the input");
  hipError_t e = svd_refresh(z, n_mats, rows, cols, rank, a_out, b_out, out_t == KVC_BF16, sigma_out, oversample,
                             power_iters, seed, workspace, ws_bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "svd refresh");
  return ok();
}

// ------------------------------------------------------------------ pool updates (App. A.3)
kvc_status kvc_observed_delta(const void* k_src, const void* v_src, const void* k_tgt, const void* v_tgt,
                              kvc_dtype dtype, kvc_shape shape, int64_t p_src, int64_t p_tgt, const kvc_rope* rope,
                              float* k_base, float* v_base, float* k_delta, float* v_delta, void* stream) {
  kvc_status s;
  if ((s = check_dtype(dtype, "cache")) != KVC_OK) return s;
  if ((s = check_shape(shape)) != KVC_OK) return s;
  if ((s = check_rope(rope)) != KVC_OK) return s;
  if ((k_base || k_delta) && !k_src) return fail(KVC_E_NULL, "k_src is NULL");
  if ((v_base || v_delta) && !v_src) return fail(KVC_E_NULL, "v_src is NULL");
  if (k_delta && !k_tgt) return fail(KVC_E_NULL, "k_tgt is NULL");
  if (v_delta && !v_tgt) return fail(KVC_E_NULL, "v_tgt is NULL");
  const void* ins[4] = {k_src, v_src, k_tgt, v_tgt};
  float* outs[4] = {k_base, v_base, k_delta, v_delta};
  const size_t n = (size_t)shape.n_layers * shape.seq_len * D_of(shape);
  for (int i = 0; i < 4; ++i) {
    if ((ins[i] && !aligned16(ins[i])) || (outs[i] && !aligned16(outs[i])))
      return fail(KVC_E_ALIGN, "observed delta: buffers must be 16-byte aligned");
    for (int j = 0; j < 4; ++j) {
      if (outs[i] && ins[j] && overlaps(outs[i], n * 4, ins[j], n * esize(dtype)))
        return fail(KVC_E_ALIAS, "observed delta: output %d overlaps input %d", i, j);
      if (j != i && outs[i] && outs[j] && overlaps(outs[i], n * 4, outs[j], n * 4))
        return fail(KVC_E_ALIAS, "observed delta: outputs %d and %d overlap", i, j);
    }
  }
  RopeTab can_src, can_tgt, ident;
  if ((s = make_tab(can_src, -p_src, shape.head_dim, rope)) != KVC_OK) return s;
  if ((s = make_tab(can_tgt, -p_tgt, shape.head_dim, rope)) != KVC_OK) return s;
  if ((s = make_tab(ident, 0, shape.head_dim, rope)) != KVC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const int64_t rows = (int64_t)shape.n_layers * shape.seq_len;
  const int bf = dtype == KVC_BF16;
  hipError_t e = hipSuccess;
  if (k_base && e == hipSuccess) e = launch_align(k_src, k_base, bf, 0, rows, shape.n_kv_heads, shape.head_dim, can_src, st);
  if (v_base && e == hipSuccess) e = launch_align(v_src, v_base, bf, 0, rows, shape.n_kv_heads, shape.head_dim, ident, st);
  if (k_delta && e == hipSuccess)
    e = launch_observed_delta(k_tgt, k_src, bf, k_delta, rows, shape.n_kv_heads, shape.head_dim, can_tgt, can_src, st);
  if (v_delta && e == hipSuccess)
    e = launch_observed_delta(v_tgt, v_src, bf, v_delta, rows, shape.n_kv_heads, shape.head_dim, ident, ident, st);
  if (e != hipSuccess) return hip_fail(e, "observed delta kernels");
  return ok();
}

kvc_status kvc_pool_state_init(kvc_pool_state* st, int32_t capacity) {
  if (!st) return fail(KVC_E_NULL, "pool state is NULL");
  if (capacity < 1 || capacity > KVC_MAX_ANCHORS)
    return fail(KVC_E_PARAM, "pool capacity must be in [1, %d] (got %d)", KVC_MAX_ANCHORS, capacity);
  memset(st, 0, sizeof *st);
  st->capacity = capacity;
  return ok();
}

kvc_status kvc_pool_record_hop(kvc_pool_state* st, int32_t consumer, int32_t seg_len, int32_t flagged,
                               int32_t* slot_out, int32_t* evicted_out) {
  if (!st || !slot_out || !evicted_out) return fail(KVC_E_NULL, "pool state / slot_out / evicted_out is NULL");
  if (st->capacity < 1 || st->capacity > KVC_MAX_ANCHORS) return fail(KVC_E_PARAM, "pool state not initialised");
  if (seg_len < 1) return fail(KVC_E_SHAPE, "seg_len must be >= 1");
  *slot_out = -1;
  *evicted_out = -1;
  const int V = st->capacity;
  if (!flagged) {
    // the consumer's correction set: its anchors covering min(S, longest) rows
    int longest = 0;
    for (int a = 0; a < V; ++a)
      if (st->stamp[a] && st->consumer[a] == consumer) longest = std::max(longest, (int)st->len[a]);
    const int s_cov = std::min(seg_len, longest);
    for (int a = 0; a < V; ++a)
      if (st->stamp[a] && st->consumer[a] == consumer && s_cov > 0 && st->len[a] >= s_cov) ++st->uses[a];
    return ok();
  }
  int slot = -1;
  for (int a = 0; a < V && slot < 0; ++a)
    if (!st->stamp[a]) slot = a;
  if (slot < 0) {
    // full: the KVC_POOL_EVICT_WINDOW oldest anchors, then the fewest uses, ties to the oldest
    int order[KVC_MAX_ANCHORS];
    for (int a = 0; a < V; ++a) order[a] = a;
    std::sort(order, order + V, [&](int x, int y) { return st->stamp[x] < st->stamp[y]; });
    const int w = std::min(V, (int)KVC_POOL_EVICT_WINDOW);
    slot = order[0];
    for (int i = 1; i < w; ++i)
      if (st->uses[order[i]] < st->uses[slot]) slot = order[i];
    *evicted_out = slot;
  } else {
    ++st->n_held;
  }
  st->stamp[slot] = ++st->clock;
  st->uses[slot] = 0;
  st->len[slot] = seg_len;
  st->consumer[slot] = consumer;
  *slot_out = slot;
  return ok();
}

int32_t kvc_pool_view(const kvc_pool_state* st, int32_t consumer, int32_t* anchor_len_out, uint8_t* live_out) {
  if (!st || !anchor_len_out || !live_out || st->capacity < 1 || st->capacity > KVC_MAX_ANCHORS) return -1;
  int n = 0;
  for (int a = 0; a < st->capacity; ++a) {
    const bool mine = st->stamp[a] != 0 && st->consumer[a] == consumer;
    live_out[a] = mine ? 1 : 0;
    anchor_len_out[a] = mine ? st->len[a] : 0;
    n += mine;
  }
  return n;
}

namespace {
struct InsertWs {
  size_t z, d, a, b, sig, svd, total;
};
InsertWs insert_layout(const kvc_shape& sh, const kvc_pool& p, int oversample) {
  InsertWs w;
  const size_t L = sh.n_layers, S = sh.seq_len, D = D_of(sh), es = esize(p.dtype);
  const int rmax = std::max(p.rank_base, p.rank_delta);
  size_t off = 0;
  w.z = off; off += up256(L * S * D * 4);
  w.d = off; off += up256(L * S * D * 4);
  w.a = off; off += up256(L * S * rmax * es);
  w.b = off; off += up256(L * rmax * D * es);
  w.sig = off; off += up256(L * rmax * 4);
  w.svd = off;
  off += std::max(svd_workspace_bytes(sh.n_layers, sh.seq_len, D_of(sh), p.rank_base, oversample),
                  svd_workspace_bytes(sh.n_layers, sh.seq_len, D_of(sh), p.rank_delta, oversample));
  w.total = off;
  return w;
}
}  // namespace

size_t kvc_pool_insert_workspace_size(kvc_shape shape, const kvc_pool* arena, int32_t oversample) {
  if (check_shape(shape) != KVC_OK || !arena || arena->rank_base < 1 || arena->rank_delta < 1 || oversample < 0)
    return 0;
  if (arena->dtype != KVC_F32 && arena->dtype != KVC_BF16) return 0;
  return insert_layout(shape, *arena, oversample).total;
}

kvc_status kvc_pool_insert(const void* k_src, const void* v_src, const void* k_tgt, const void* v_tgt,
                           kvc_shape shape, int64_t p_src, int64_t p_tgt, const kvc_rope* rope, const kvc_pool* arena,
                           int32_t slot, int32_t oversample, int32_t power_iters, uint64_t seed, void* workspace,
                           size_t ws_bytes, void* stream) {
  kvc_status s;
  if ((s = check_shape(shape)) != KVC_OK) return s;
  if ((s = check_rope(rope)) != KVC_OK) return s;
  if (!arena) return fail(KVC_E_NULL, "arena is NULL");
  if ((s = check_dtype(arena->dtype, "arena")) != KVC_OK) return s;
  if (!k_src || !v_src || !k_tgt || !v_tgt) return fail(KVC_E_NULL, "k_src/v_src/k_tgt/v_tgt is NULL");
  const void* fac[8] = {arena->baseA_k, arena->baseB_k, arena->baseA_v, arena->baseB_v,
                        arena->deltaA_k, arena->deltaB_k, arena->deltaA_v, arena->deltaB_v};
  for (int i = 0; i < 8; ++i)
    if (!fac[i]) return fail(KVC_E_NULL, "arena factor array %d is NULL", i);
  if (arena->slot_rows < shape.seq_len)
    return fail(KVC_E_SHAPE, "arena slot_rows = %d is below seq_len = %d", arena->slot_rows, shape.seq_len);
  if (arena->n_anchors < 1 || arena->n_anchors > KVC_MAX_ANCHORS)
    return fail(KVC_E_SHAPE, "arena n_anchors must be in [1, %d]", KVC_MAX_ANCHORS);
  if (slot < 0 || slot >= arena->n_anchors) return fail(KVC_E_PARAM, "slot %d outside [0, %d)", slot, arena->n_anchors);
  const int D = D_of(shape), S = shape.seq_len, L = shape.n_layers;
  const int rmax = std::max(arena->rank_base, arena->rank_delta);
  if (arena->rank_base < 1 || arena->rank_delta < 1 || oversample < 0 || rmax + oversample > std::min(S, D) ||
      rmax + oversample > 256)
    return fail(KVC_E_SHAPE, "insert: need ranks >= 1 and rank + oversample <= min(seq_len, D, 256)");
  if (S % 4 || D % 4) return fail(KVC_E_SHAPE, "insert: seq_len and D must be multiples of 4");
  if (power_iters < 0 || power_iters > 16) return fail(KVC_E_PARAM, "insert: power_iters must be in [0, 16]");
  const InsertWs w = insert_layout(shape, *arena, oversample);
  if (!workspace || ws_bytes < w.total) return fail(KVC_E_WORKSPACE, "insert workspace: need %zu bytes", w.total);
  if (!aligned16(workspace)) return fail(KVC_E_ALIGN, "workspace not 16-byte aligned");
  char* ws = (char*)workspace;
  float* z = (float*)(ws + w.z);
  float* d = (float*)(ws + w.d);
  hipStream_t st = (hipStream_t)stream;
  const size_t es = esize(arena->dtype);
  const size_t V = arena->n_anchors, R = arena->slot_rows;
  for (int side = 0; side < 2; ++side) {
    const bool keys = side == 0;
    if ((s = kvc_observed_delta(keys ? k_src : nullptr, keys ? nullptr : v_src, keys ? k_tgt : nullptr,
                                keys ? nullptr : v_tgt, arena->dtype, shape, p_src, p_tgt, rope, keys ? z : nullptr,
                                keys ? nullptr : z, keys ? d : nullptr, keys ? nullptr : d, stream)) != KVC_OK)
      return s;
    for (int which = 0; which < 2; ++which) {   // 0: base (source), 1: correction
      const int r = which ? arena->rank_delta : arena->rank_base;
      void* A = (void*)(which ? (keys ? arena->deltaA_k : arena->deltaA_v) : (keys ? arena->baseA_k : arena->baseA_v));
      void* B = (void*)(which ? (keys ? arena->deltaB_k : arena->deltaB_v) : (keys ? arena->baseB_k : arena->baseB_v));
      hipError_t e = svd_refresh(which ? d : z, L, S, D, r, ws + w.a, ws + w.b, arena->dtype == KVC_BF16,
                                 (float*)(ws + w.sig), oversample, power_iters, seed * 4 + side * 2 + which,
                                 ws + w.svd, w.total - w.svd, st);
      if (e != hipSuccess) return hip_fail(e, "insert factorisation");
      // A: layer l's rows go to [slot * slot_rows, + S) of the layer's block; B: anchor `slot`
      e = hipMemcpy2DAsync((char*)A + (size_t)slot * R * r * es, V * R * r * es, ws + w.a, (size_t)S * r * es,
                           (size_t)S * r * es, L, hipMemcpyDeviceToDevice, st);
      if (e == hipSuccess)
        e = hipMemcpy2DAsync((char*)B + (size_t)slot * r * D * es, V * r * D * es, ws + w.b, (size_t)r * D * es,
                             (size_t)r * D * es, L, hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return hip_fail(e, "insert copy into the arena");
    }
  }
  return ok();
}

// ------------------------------------------------------------------ measurement kernels
static kvc_status peak_args(const void* sink, int32_t n_blocks, int32_t iters) {
  if (!sink) return fail(KVC_E_NULL, "sink is NULL");
  if (!aligned16(sink)) return fail(KVC_E_ALIGN, "sink not 16-byte aligned");
  if (n_blocks < 1 || n_blocks > 65536) return fail(KVC_E_SHAPE, "n_blocks must be in [1, 65536]");
  if (iters < 1 || iters > (1 << 20)) return fail(KVC_E_PARAM, "iters must be in [1, 2^20]");
  return KVC_OK;
}

kvc_status kvc_peak_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src) return fail(KVC_E_NULL, "dst/src is NULL");
  if (!aligned16(dst) || !aligned16(src)) return fail(KVC_E_ALIGN, "dst/src not 16-byte aligned");
  if (bytes == 0 || bytes % 16) return fail(KVC_E_SHAPE, "bytes must be a positive multiple of 16");
  if (overlaps(dst, bytes, src, bytes)) return fail(KVC_E_ALIAS, "dst overlaps src");
  hipError_t e = launch_peak_copy(dst, src, bytes, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "copy kernel");
}

kvc_status kvc_peak_mfma_bf16(float* sink, int32_t n_blocks, int32_t iters, void* stream) {
  kvc_status s = peak_args(sink, n_blocks, iters);
  if (s != KVC_OK) return s;
  hipError_t e = launch_peak_mfma(sink, n_blocks, iters, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "mfma loop");
}

kvc_status kvc_peak_lds_read(uint32_t* sink, int32_t n_blocks, int32_t iters, void* stream) {
  kvc_status s = peak_args(sink, n_blocks, iters);
  if (s != KVC_OK) return s;
  hipError_t e = launch_peak_lds(sink, n_blocks, iters, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "lds loop");
}

kvc_status kvc_peak_valu(float* sink, int32_t n_blocks, int32_t iters, void* stream) {
  kvc_status s = peak_args(sink, n_blocks, iters);
  if (s != KVC_OK) return s;
  hipError_t e = launch_peak_valu(sink, n_blocks, iters, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "valu loop");
}

}  // extern "C"
