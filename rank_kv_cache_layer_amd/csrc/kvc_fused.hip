// Fused per-hop correction for gfx950 (CDNA4), bf16 caches: one pass over the source K/V
// scores the segment against the anchor pool, forms the token weights and applies the
// weighted low-rank delta with both positional rotations and the residual add.
//
// KVCMAS (arXiv 2609.34060):
//  * scoring, App. A.3 "Correction Weighting and Positional Alignment": per token and per
//    side, the mean absolute distance between the canonical-frame source row and each
//    anchor's reconstructed base row (Eq. 7 factors A B);
//  * gate sums, App. A.3 Eq. 9: squared Frobenius distance of the value rows over the
//    prefix k, per (layer, anchor); reduced across tiles in double precision elsewhere;
//  * weights: softmax over the correction set, separately for keys and values (Eq. 8 with
//    the token index restored, as App. A.3 states);
//  * apply, Sec. 3.3 Eq. 8 and App. A.3 Eq. 12: out = R(s) Z + R(p_tgt) sum_a w_a A_a B_a for
//    keys, out = Z + sum_a w_a A_a B_a for values.
//
// Work-group = 64 tokens x all D channels of one (layer, side), D / 128 waves; wave w owns
// channels [128 w, 128 w + 128).  Every contraction uses v_mfma_f32_32x32x16_bf16 with
// channels as MFMA rows and tokens as MFMA columns: lane l (col = l % 32, hi = l / 32) owns
// token col of a 32-token block and rows 8 (j / 4) + 4 hi + j % 4 (j = 0..15) of a
// 32-channel block, so per-token reductions over channels stay in the lane and the
// rotate-half partners c and c + d_h/2 sit in the same lane and register slot of two blocks.
//
// Phase 1 (scores): the canonical source tile is held in fp32 registers and is the MFMA
//   accumulator input, the base B^T operands are pre-negated, so each anchor's MFMA chain
//   yields E = Z_can - A B directly; the epilogue adds |E| per token and, for values inside
//   the prefix k, E^2.  Base A rows are staged through LDS (double-buffered).
// Phase 2 (weights): per-token softmax in LDS.
// Phase 3 (apply): the same registers are re-initialised with the residual (R(s) Z for keys,
//   Z for values) and accumulate [w (.) A_delta] B'_delta over (anchor, rank), where the key
//   delta rows B' were turned by R(p_tgt) when they were packed, then round to bf16.
#include <string.h>

#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
// 8 bf16 values times a scalar, rounded back to bf16
__device__ __forceinline__ uint4 scale8(uint4 r, float w) {
  return make_uint4(pack2(lo16(r.x) * w, hi16(r.x) * w), pack2(lo16(r.y) * w, hi16(r.y) * w),
                    pack2(lo16(r.z) * w, hi16(r.z) * w), pack2(lo16(r.w) * w, hi16(r.w) * w));
}

constexpr int kT = kFusedTile;        // tokens per work-group
constexpr int kChunk = 512;           // bf16 elements of one packed MFMA operand chunk (64 lanes x 8)
constexpr int kWRow = kMaxAnchors + 1;

// rotate-half partner layout of a wave's 4 channel blocks (one head of 128 or two of 64)
template <int HD> __device__ __forceinline__ constexpr bool lower_blk(int b) { return ((b * 32) % HD) < HD / 2; }
template <int HD> __device__ __forceinline__ constexpr int partner_blk(int b) { return b + HD / 64; }
template <int HD> __device__ __forceinline__ int pair_index(int b, int row) { return (b * 32) % HD + row; }

// Source tile rows t0 .. t0+63, channels d0 .. d0+127, in accumulator layout (fp32).
__device__ __forceinline__ void load_tile(f32x16 (&z)[2][4], const uint16_t* zl, int t0, int S, int D, int d0,
                                          int col, int hi) {
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = t0 + tb * 32 + col;
    const uint16_t* row = zl + (int64_t)t * D + d0 + 4 * hi;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        uint2 v = make_uint2(0, 0);
        if (t < S) v = *reinterpret_cast<const uint2*>(row + db * 32 + 8 * jg);
        z[tb][db][4 * jg + 0] = lo16(v.x);
        z[tb][db][4 * jg + 1] = hi16(v.x);
        z[tb][db][4 * jg + 2] = lo16(v.y);
        z[tb][db][4 * jg + 3] = hi16(v.y);
      }
  }
}

template <int HD>
__device__ __forceinline__ void rotate_tile(f32x16 (&z)[2][4], const float* cs, const float* sn, int hi) {
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    if (!lower_blk<HD>(db)) continue;
    const int du = partner_blk<HD>(db);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = pair_index<HD>(db, 8 * (j >> 2) + 4 * hi + (j & 3));
      const float cv = cs[c], sv = sn[c];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float ox, oy;
        rot_pair(z[tb][db][j], z[tb][du][j], cv, sv, ox, oy);
        z[tb][db][j] = ox;
        z[tb][du][j] = oy;
      }
    }
  }
}

__device__ __forceinline__ float abs_sum(const f32x16& e) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int j = 0; j < 16; j += 4) {
    s0 += fabsf(e[j]);
    s1 += fabsf(e[j + 1]);
    s2 += fabsf(e[j + 2]);
    s3 += fabsf(e[j + 3]);
  }
  return (s0 + s1) + (s2 + s3);
}

__device__ __forceinline__ float sq_sum(const f32x16& e) {
  float q0 = 0.f, q1 = 0.f;
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    q0 = fmaf(e[j], e[j], q0);
    q1 = fmaf(e[j + 1], e[j + 1], q1);
  }
  return q0 + q1;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Staging ring for the A rows of one tile, shared by both phases.  Chunk j of the tile's
// sequence holds 64 rows x rank of one anchor:
//   j <  nl : base A of list[j]            (phase 1, rank r_b)
//   j >= nl : delta A of corr[j - nl]      (phase 3, rank r_d)
// Chunk j lives in LDS slot j & 1.  The threads form two writer groups; group j & 1 loads
// chunk j into registers two steps before it is consumed and writes it to its slot at the
// end of the step before, so each load has two steps of latency budget and the LDS holds
// only two chunks.  Units beyond U per thread are loaded when the chunk is written.
template <int U>
struct Ring {
  const uint16_t* ab;       // base A of this layer/side, packed rows
  const uint16_t* ad;       // delta A of this layer/side
  const uint8_t* list;      // phase-1 anchors (LDS)
  const uint8_t* corr;      // correction set (LDS)
  const int32_t* off;       // packed first row per anchor (LDS)
  const int32_t* len;       // stored rows per anchor (LDS)
  uint16_t* slots;          // 2 slots x 64 rows x RS elements
  int nl, nj, rb, rd, t0, S, s_cov, RS;
  int grp, gi, G;
  uint4 v[U];

  __device__ __forceinline__ bool mine(int j) const { return j < nj && (j & 1) == grp; }
  __device__ __forceinline__ void unit_src(int j, int u, uint4& out) const {
    const bool base = j < nl;
    const int a = base ? list[j] : corr[j - nl];
    const int r = base ? rb : rd;
    const int row = u / (r >> 3), c = u - row * (r >> 3);
    const int t = t0 + row;
    const int lim = base ? min(S, len[a]) : min(s_cov, len[a]);
    out = make_uint4(0, 0, 0, 0);
    if (t < lim) out = *reinterpret_cast<const uint4*>((base ? ab : ad) + ((int64_t)off[a] + t) * r + c * 8);
  }
  __device__ __forceinline__ int units(int j) const { return kFusedTile * ((j < nl ? rb : rd) >> 3); }
  __device__ __forceinline__ void issue(int j) {
    if (!mine(j)) return;
    const int n = units(j);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int u = gi + k * G;
      if (u < n) unit_src(j, u, v[k]);
    }
  }
  __device__ __forceinline__ void put(int j, int u, uint4 x) {
    const int r = j < nl ? rb : rd;
    const int row = u / (r >> 3), c = u - row * (r >> 3);
    *reinterpret_cast<uint4*>(slots + (j & 1) * kFusedTile * RS + row * RS + c * 8) = x;
  }
  __device__ __forceinline__ void commit(int j) {
    if (!mine(j)) return;
    const int n = units(j);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int u = gi + k * G;
      if (u < n) put(j, u, v[k]);
    }
    for (int u = gi + U * G; u < n; u += G) {
      uint4 x;
      unit_src(j, u, x);
      put(j, u, x);
    }
  }
  __device__ __forceinline__ const uint16_t* slot(int j) const { return slots + (j & 1) * kFusedTile * RS; }
};

// One anchor of phase 1 for a wave: E = Z_can - A B over the wave's 64 tokens x 128 channels
// (8 accumulator blocks), reduced to per-lane |E| sums (ms0: token t0 + col, ms1: t0 + 32 + col)
// and, when Q, the masked E^2 sum.  An empty asm statement that "redefines" the A operands
// after each block's epilogue keeps the compiler from hoisting later MFMA chains above it
// (which would need up to 8 live result blocks); the second wave of the SIMD fills the
// MFMA-to-epilogue latency.  B operands are fetched two channel blocks ahead: b0/b1 hold
// blocks 0/1 on entry and the next anchor's blocks 0/1 (from Bn) on exit.
template <int RK, bool Q>
__device__ __forceinline__ void score_anchor(const f32x16 (&z)[2][4], const uint16_t* as, int RS, int col, int hi,
                                             const uint16_t* Bw, const uint16_t* Bn, bf16x8 (&b0)[RK],
                                             bf16x8 (&b1)[RK], float qm0, float qm1, float& ms0, float& ms1,
                                             float& qs) {
  constexpr int kC = 512;
  bf16x8 av[2][RK];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ks = 0; ks < RK; ++ks)
      av[tb][ks] = as_bf8(*reinterpret_cast<const uint4*>(as + (tb * 32 + col) * RS + ks * 16 + 8 * hi));
  bf16x8 b2[RK], b3[RK];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    // fetch two blocks ahead
#pragma unroll
    for (int ks = 0; ks < RK; ++ks) {
      const uint4 x = db < 2 ? *reinterpret_cast<const uint4*>(Bw + ((db + 2) * RK + ks) * kC)
                             : *reinterpret_cast<const uint4*>(Bn + ((db - 2) * RK + ks) * kC);
      if (db == 0) b2[ks] = as_bf8(x);
      else if (db == 1) b3[ks] = as_bf8(x);
      else if (db == 2) b0[ks] = as_bf8(x);   // b0 already consumed
      else b1[ks] = as_bf8(x);
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const bf16x8* bc = db == 0 ? b0 : db == 1 ? b1 : db == 2 ? b2 : b3;
      f32x16 e = mfma(bc[0], av[tb][0], z[tb][db]);
#pragma unroll
      for (int ks = 1; ks < RK; ++ks) e = mfma(bc[ks], av[tb][ks], e);
      const float s = abs_sum(e);
      if (tb == 0) ms0 += s; else ms1 += s;
      if (Q) qs = fmaf(sq_sum(e), tb == 0 ? qm0 : qm1, qs);
      if constexpr (RK == 1)
        asm volatile("" : "+v"(av[0][0]), "+v"(av[1][0]), "+v"(ms0), "+v"(ms1), "+v"(qs));
      else if constexpr (RK == 2)
        asm volatile("" : "+v"(av[0][0]), "+v"(av[0][1]), "+v"(av[1][0]), "+v"(av[1][1]), "+v"(ms0), "+v"(ms1),
                     "+v"(qs));
    }
  }
}

// Large ranks (r >= 64): B of one channel block held for both token blocks, A read from LDS
// per rank slice.
template <int RK, bool Q>
__device__ __forceinline__ void score_anchor_wide(const f32x16 (&z)[2][4], const uint16_t* as, int RS, int col, int hi,
                                                  const uint16_t* Bw, float qm0, float qm1, float& ms0, float& ms1,
                                                  float& qs) {
  constexpr int kC = 512;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    bf16x8 bv[RK];
#pragma unroll
    for (int ks = 0; ks < RK; ++ks) bv[ks] = as_bf8(*reinterpret_cast<const uint4*>(Bw + (db * RK + ks) * kC));
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x16 e = z[tb][db];
#pragma unroll
      for (int ks = 0; ks < RK; ++ks)
        e = mfma(bv[ks], as_bf8(*reinterpret_cast<const uint4*>(as + (tb * 32 + col) * RS + ks * 16 + 8 * hi)), e);
      const float s = abs_sum(e);
      if (tb == 0) ms0 += s; else ms1 += s;
      if (Q) qs = fmaf(sq_sum(e), tb == 0 ? qm0 : qm1, qs);
      asm volatile("" : "+v"(ms0), "+v"(ms1), "+v"(qs));
    }
  }
}

template <int HD, int RK, int MODE>
__global__ void __launch_bounds__(512) fused_hop(FusedArgs p) {
  extern __shared__ uint16_t ring_lds[];       // 2 slots x 64 rows x RS
  __shared__ float mp[2][8][kT];
  __shared__ float wsh[kT * kWRow];
  __shared__ float qp[8][kMaxAnchors];
  __shared__ float tab[4][kFusedHalf];
  __shared__ int32_t s_off[kMaxAnchors], s_len[kMaxAnchors];
  __shared__ uint8_t s_use[kMaxAnchors], s_corr[kMaxAnchors];

  const int n_tiles = p.n_tiles;
  const int64_t lb = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = (int)(lb % n_tiles);
  const int layer = (int)((lb / n_tiles) % p.n_layers);
  const int side = (int)(lb / ((int64_t)n_tiles * p.n_layers));
  const bool keys = side == 0;
  const int nthr = blockDim.x, tid = threadIdx.x, nw = nthr >> 6;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, hi = lane >> 5;
  const int D = p.D, S = p.S, N = p.N;
  const int NCB = D >> 5;
  const int t0 = tile * kT, d0 = wave * 128;

  for (int i = tid; i < HD / 2; i += nthr) {
    tab[0][i] = p.can.cs[i];
    tab[1][i] = p.can.sn[i];
    tab[2][i] = p.shift.cs[i];
    tab[3][i] = p.shift.sn[i];
  }
  for (int i = tid; i < kMaxAnchors; i += nthr) {
    s_off[i] = p.off[i];
    s_len[i] = p.len[i];
    s_use[i] = p.use[i];
    s_corr[i] = p.corr[i];
  }
  for (int i = tid; i < kT * kWRow; i += nthr) wsh[i] = 0.f;
  __syncthreads();

  const uint16_t* zl = p.z[side] + (int64_t)layer * S * D;
  f32x16 z[2][4];
  bool z_raw = false;   // z holds the stored (unrotated) source tile

  // phase-1 anchors and phase-3 chunks of this tile
  int nl = 0;
  if (MODE == FUSED_PAGES) {
    nl = keys ? p.n_corr : p.n_use;
    const int s_work = keys ? (p.n_corr ? p.s_cov : 0)
                            : max(p.n_corr ? p.s_cov : 0, p.mask_gate ? p.k_gate : 0);
    if (t0 >= s_work) nl = 0;
  }
  const int nc = (p.apply && t0 < p.s_cov) ? p.n_corr : 0;
  Ring<(RK <= 2 ? 1 : 2)> ring;
  ring.ab = p.Ab[side] ? p.Ab[side] + layer * p.ab_layer : nullptr;
  ring.ad = p.Ad[side] ? p.Ad[side] + layer * p.ad_layer : nullptr;
  ring.list = keys ? s_corr : s_use;
  ring.corr = s_corr;
  ring.off = s_off;
  ring.len = s_len;
  ring.slots = ring_lds;
  ring.nl = nl;
  ring.nj = nl + nc;
  ring.rb = p.r_b;
  ring.rd = p.r_d;
  ring.t0 = t0;
  ring.S = S;
  ring.s_cov = p.s_cov;
  ring.RS = p.ring_stride;
  ring.G = nthr >> 1;
  ring.grp = tid >= ring.G;
  ring.gi = tid - ring.grp * ring.G;
  ring.issue(0);
  ring.issue(1);
  ring.commit(0);
  ring.issue(2);

  // ------------------------------------------------------------------ phase 1: scores
  if (MODE == FUSED_PAGES) {
    if (nl > 0) {
      load_tile(z, zl, t0, S, D, d0, col, hi);
      z_raw = true;
      if (keys && p.can.active) {
        rotate_tile<HD>(z, tab[0], tab[1], hi);
        z_raw = false;
      }
    }
    __syncthreads();
    // this wave's packed B operand chunks of the layer: anchor a starts at Bl + a * NCB * RK * 512
    const uint16_t* Bl = p.Bb[side] + ((int64_t)layer * N * NCB + wave * 4) * RK * kChunk + lane * 8;
    const int64_t bstride = (int64_t)NCB * RK * kChunk;
    bf16x8 b0[RK], b1[RK];
    if (RK <= 2 && nl > 0) {
      const uint16_t* B0 = Bl + ring.list[0] * bstride;
#pragma unroll
      for (int ks = 0; ks < RK; ++ks) {
        b0[ks] = as_bf8(*reinterpret_cast<const uint4*>(B0 + ks * kChunk));
        b1[ks] = as_bf8(*reinterpret_cast<const uint4*>(B0 + (RK + ks) * kChunk));
      }
    }
    const float qm0 = (t0 + col < p.k_gate && t0 + col < S) ? 1.f : 0.f;
    const float qm1 = (t0 + 32 + col < p.k_gate && t0 + 32 + col < S) ? 1.f : 0.f;
    for (int ui = 0; ui < nl; ++ui) {
      const int a = ring.list[ui];
      const int buf = ui & 1;
      const bool want_m = (p.mask_corr >> a) & 1;
      const bool want_q = !keys && ((p.mask_gate >> a) & 1) && t0 < p.k_gate;
      const uint16_t* Bw = Bl + a * bstride;
      const uint16_t* Bn = Bl + ring.list[ui + 1 < nl ? ui + 1 : ui] * bstride;
      const uint16_t* as = ring.slot(ui);
      float ms0 = 0.f, ms1 = 0.f, qs = 0.f;
      if constexpr (RK <= 2) {
        if (want_q)
          score_anchor<RK, true>(z, as, ring.RS, col, hi, Bw, Bn, b0, b1, qm0, qm1, ms0, ms1, qs);
        else
          score_anchor<RK, false>(z, as, ring.RS, col, hi, Bw, Bn, b0, b1, qm0, qm1, ms0, ms1, qs);
      } else {
        if (want_q)
          score_anchor_wide<RK, true>(z, as, ring.RS, col, hi, Bw, qm0, qm1, ms0, ms1, qs);
        else
          score_anchor_wide<RK, false>(z, as, ring.RS, col, hi, Bw, qm0, qm1, ms0, ms1, qs);
      }
      if (want_m) {
        ms0 += __shfl_xor(ms0, 32);
        ms1 += __shfl_xor(ms1, 32);
        if (hi == 0) {
          mp[buf][wave][col] = ms0;
          mp[buf][wave][32 + col] = ms1;
        }
      }
      if (want_q) {
        qs = wave_sum(qs);
        if (lane == 0) qp[wave][a] = qs;
      }
      if (ui + 1 == nl && p.apply && !z_raw) {
        // the canonical tile is no longer needed: start fetching the stored keys for the residual
        load_tile(z, zl, t0, S, D, d0, col, hi);
        z_raw = true;
      }
      ring.commit(ui + 1);
      ring.issue(ui + 3);
      __syncthreads();
      if (want_m && tid < kT) {
        float s = 0.f;
        for (int w = 0; w < nw; ++w) s += mp[buf][w][tid];
        wsh[tid * kWRow + a] = s / (float)D;
      }
    }
    __syncthreads();
    if (!keys && p.partials) {
      float* part = p.partials + ((int64_t)layer * n_tiles + tile) * N;
      for (int a = tid; a < N; a += nthr) {
        if (!((p.mask_gate >> a) & 1)) continue;
        float s = 0.f;
        if (t0 < p.k_gate && nl > 0)
          for (int w = 0; w < nw; ++w) s += qp[w][a];
        part[a] = s;
      }
    }
  } else {
    // given weights (explicit apply) or given cosine scores (second scoring mode)
    const float* src = p.w_in[side] + (int64_t)layer * S * N;
    for (int i = tid; i < kT * N; i += nthr) {
      const int tl = i / N, a = i - tl * N;
      const int t = t0 + tl;
      if (t < p.s_cov && ((p.mask_corr >> a) & 1)) wsh[tl * kWRow + a] = src[(int64_t)t0 * N + i];
    }
    __syncthreads();
  }

  // ------------------------------------------------------------------ phase 2: weights
  if (MODE != FUSED_GIVEN) {
    if (tid < kT) {
      float* row = wsh + tid * kWRow;
      const int t = t0 + tid;
      if (t < p.s_cov && p.n_corr > 0) {
        const float sg = MODE == FUSED_PAGES ? -p.inv_temp : p.inv_temp;
        float mx = -INFINITY;
        for (int ci = 0; ci < p.n_corr; ++ci) mx = fmaxf(mx, row[s_corr[ci]] * sg);
        float sum = 0.f;
        for (int ci = 0; ci < p.n_corr; ++ci) {
          const int a = s_corr[ci];
          const float e = expf(row[a] * sg - mx);
          row[a] = e;
          sum += e;
        }
        const float inv = 1.f / sum;
        for (int ci = 0; ci < p.n_corr; ++ci) row[s_corr[ci]] *= inv;
      } else {
        for (int ci = 0; ci < p.n_corr; ++ci) row[s_corr[ci]] = 0.f;
      }
    }
    __syncthreads();
    if (p.w_out[side]) {
      float* dst = p.w_out[side] + (int64_t)layer * S * N;
      for (int i = tid; i < kT * N; i += nthr) {
        const int tl = i / N, a = i - tl * N;
        if (t0 + tl < S) dst[(int64_t)t0 * N + i] = wsh[tl * kWRow + a];
      }
    }
  }
  if (!p.apply) return;

  // ------------------------------------------------------------------ phase 3: apply
  if (!z_raw) load_tile(z, zl, t0, S, D, d0, col, hi);
  if (keys && p.shift.active) rotate_tile<HD>(z, tab[2], tab[3], hi);
  // sub-steps s over (chunk c of the correction set, 16-wide rank slice ks); B operands of
  // sub-step s + 1 are fetched while sub-step s runs its 8 MFMAs (two register sets)
  const int rd = p.r_d, RKD = rd >> 4;
  const int nsub = nc * RKD;
  if (nsub > 0) {
    const uint16_t* Bl = p.Bd[side] + ((int64_t)layer * N * NCB + wave * 4) * RKD * kChunk + lane * 8;
    auto fetch_b = [&](int s, uint4 (&bv)[4]) {
      const int c = s / RKD, ks = s - c * RKD;
      const uint16_t* Bw = Bl + ((int64_t)s_corr[c] * NCB * RKD + ks) * kChunk;
#pragma unroll
      for (int db = 0; db < 4; ++db) bv[db] = *reinterpret_cast<const uint4*>(Bw + db * RKD * kChunk);
    };
    auto step = [&](int s, const uint4 (&bv)[4]) {
      const int c = s / RKD, ks = s - c * RKD;
      const int a = s_corr[c];
      const float w0 = wsh[col * kWRow + a], w1 = wsh[(32 + col) * kWRow + a];
      const uint16_t* as = ring.slot(nl + c) + ks * 16 + 8 * hi;
      const uint4 r0 = *reinterpret_cast<const uint4*>(as + col * ring.RS);
      const uint4 r1 = *reinterpret_cast<const uint4*>(as + (32 + col) * ring.RS);
      const bf16x8 a0 = as_bf8(scale8(r0, w0)), a1 = as_bf8(scale8(r1, w1));
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        z[0][db] = mfma(as_bf8(bv[db]), a0, z[0][db]);
        z[1][db] = mfma(as_bf8(bv[db]), a1, z[1][db]);
      }
      if (ks == RKD - 1) {   // chunk done: advance the ring
        ring.commit(nl + c + 1);
        ring.issue(nl + c + 3);
        __syncthreads();
      }
    };
    uint4 bx[4], by[4];
    fetch_b(0, bx);
    for (int s = 0; s < nsub; s += 2) {
      if (s + 1 < nsub) fetch_b(s + 1, by);
      step(s, bx);
      if (s + 1 < nsub) {
        if (s + 2 < nsub) fetch_b(s + 2, bx);
        step(s + 1, by);
      }
    }
  }
  uint16_t* ol = p.out[side] + (int64_t)layer * S * D;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = t0 + tb * 32 + col;
    if (t >= S) continue;
    uint16_t* row = ol + (int64_t)t * D + d0 + 4 * hi;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        uint2 v;
        v.x = pack2(z[tb][db][4 * jg + 0], z[tb][db][4 * jg + 1]);
        v.y = pack2(z[tb][db][4 * jg + 2], z[tb][db][4 * jg + 3]);
        *reinterpret_cast<uint2*>(row + db * 32 + 8 * jg) = v;
      }
  }
}

// ------------------------------------------------------------------------ B packing

__global__ void __launch_bounds__(256) pack_b(PackArgs p) {
  __shared__ float cs[kFusedHalf], sn[kFusedHalf];
  for (int i = threadIdx.x; i < p.head_dim / 2; i += blockDim.x) { cs[i] = p.tab.cs[i]; sn[i] = p.tab.sn[i]; }
  __syncthreads();
  const int RK = (p.r + 15) >> 4, NCB = p.D >> 5, D = p.D, hd = p.head_dim, h = hd >> 1;   // ranks padded to 16
  const int64_t per_mat = (int64_t)NCB * RK * 64;
  const int64_t per_arr = per_mat * p.n_layers * p.n_anchors;
  const int64_t total = per_arr * p.n_arrays;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
    const int arr = (int)(u / per_arr);
    const int64_t rem = u - arr * per_arr;
    const int64_t mat = rem / per_mat;
    int v = (int)(rem - mat * per_mat);
    const int lane = v & 63;
    v >>= 6;
    const int ks = v % RK, cb = v / RK;
    const int d = cb * 32 + (lane & 31);
    const int k0 = ks * 16 + 8 * (lane >> 5);
    const uint16_t* B = p.src[arr] + mat * p.r * D;
    const bool rot = p.rotate[arr] && p.tab.active;
    const int c = d % hd;
    const int partner = c < h ? d + h : d - h;
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool in = k0 + i < p.r;   // rows past the rank pack as zeros
      const float x = in ? bf2f(B[(int64_t)(k0 + i) * D + d]) : 0.f;
      float val = x;
      if (rot) {
        const float y = in ? bf2f(B[(int64_t)(k0 + i) * D + partner]) : 0.f;
        float lo, up;
        if (c < h) {
          rot_pair(x, y, cs[c], sn[c], lo, up);
          val = lo;
        } else {
          rot_pair(y, x, cs[c - h], sn[c - h], lo, up);
          val = up;
        }
      }
      o[i] = p.negate[arr] ? -val : val;
    }
    const uint4 w = make_uint4(pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7]));
    *reinterpret_cast<uint4*>(p.dst[arr] + (mat * NCB * RK + (int64_t)cb * RK + ks) * kChunk + lane * 8) = w;
  }
}

size_t fused_ring_bytes(const FusedArgs& a) { return sizeof(uint16_t) * 2 * kFusedTile * (size_t)a.ring_stride; }

template <typename K>
void fused_go(K kernel, const FusedArgs& a, hipStream_t st) {
  const int64_t nblk = (int64_t)a.n_tiles * a.n_layers * 2;
  const size_t shmem = fused_ring_bytes(a);
  if (shmem > 64 * 1024)   // a refusal surfaces as the launch's error, which the caller reads
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
  kernel<<<dim3((unsigned)nblk), dim3((a.D / 128) * 64), shmem, st>>>(a);
}

template <int HD>
hipError_t fused_dispatch(const FusedArgs& a, int mode, hipStream_t st) {
  if (mode == FUSED_PAGES) {
    switch (a.r_b) {
      case 16: fused_go(fused_hop<HD, 1, FUSED_PAGES>, a, st); break;
      case 32: fused_go(fused_hop<HD, 2, FUSED_PAGES>, a, st); break;
      case 64: fused_go(fused_hop<HD, 4, FUSED_PAGES>, a, st); break;
      case 128: fused_go(fused_hop<HD, 8, FUSED_PAGES>, a, st); break;
      default: return hipErrorInvalidValue;
    }
  } else if (mode == FUSED_SCORES) {
    fused_go(fused_hop<HD, 1, FUSED_SCORES>, a, st);
  } else {
    fused_go(fused_hop<HD, 1, FUSED_GIVEN>, a, st);
  }
  return hipGetLastError();
}

}  // namespace

// The same packing with 16-byte row reads: a work-group takes one 16-row rank slice (ks) of one
// factor matrix, stages it in LDS row-major (rows past the rank as zeros), and every thread then
// gathers its chunk lanes' 8 rank values of one channel (and of its rotary partner) from LDS and
// writes them as one 16-byte store.  Output identical to pack_b.
constexpr int kPackPad = 8;   // LDS row padding (elements)
__device__ __forceinline__ void pack_rows(const PackArgs& p, int64_t blk, uint16_t* rows_s, float* cs, float* sn) {
  const int D = p.D, hd = p.head_dim, h = hd >> 1, RK = (p.r + 15) >> 4, NCB = D >> 5, ld = D + kPackPad;
  const int tid = threadIdx.x;
  const int ks = (int)(blk % RK);
  blk /= RK;
  const int64_t mats = (int64_t)p.n_layers * p.n_anchors;
  const int64_t mat = blk % mats;
  const int arr = (int)(blk / mats);
  for (int i = tid; i < h; i += blockDim.x) { cs[i] = p.tab.cs[i]; sn[i] = p.tab.sn[i]; }
  const uint16_t* B = p.src[arr] + mat * p.r * D;
  const int units = 16 * (D >> 3);   // 16-byte units of the slice
  for (int u = tid; u < units; u += blockDim.x) {
    const int row = u / (D >> 3), c8 = (u - row * (D >> 3)) * 8;
    const int k = ks * 16 + row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k < p.r) v = *reinterpret_cast<const uint4*>(B + (int64_t)k * D + c8);
    *reinterpret_cast<uint4*>(rows_s + row * ld + c8) = v;
  }
  __syncthreads();
  const bool rot = p.rotate[arr] && p.tab.active;
  const bool neg = p.negate[arr];
  for (int o = tid; o < NCB * 64; o += blockDim.x) {
    const int cb = o >> 6, lane = o & 63;
    const int d = cb * 32 + (lane & 31);
    const int r0 = 8 * (lane >> 5);
    const int c = d % hd;
    const int partner = c < h ? d + h : d - h;
    float out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = bf2f(rows_s[(r0 + i) * ld + d]);
      float val = x;
      if (rot) {
        const float y = bf2f(rows_s[(r0 + i) * ld + partner]);
        float lo, up;
        if (c < h) {
          rot_pair(x, y, cs[c], sn[c], lo, up);
          val = lo;
        } else {
          rot_pair(y, x, cs[c - h], sn[c - h], lo, up);
          val = up;
        }
      }
      out[i] = neg ? -val : val;
    }
    const uint4 w = make_uint4(pack2(out[0], out[1]), pack2(out[2], out[3]), pack2(out[4], out[5]), pack2(out[6], out[7]));
    *reinterpret_cast<uint4*>(p.dst[arr] + (mat * NCB * RK + (int64_t)cb * RK + ks) * kChunk + lane * 8) = w;
  }
}

__global__ void __launch_bounds__(256) pack_b_rows(PackArgs p) {
  extern __shared__ uint16_t rows_s[];   // [16][D + kPackPad]
  __shared__ float cs[kFusedHalf], sn[kFusedHalf];
  pack_rows(p, blockIdx.x, rows_s, cs, sn);
}

// batched: descriptor h owns blocks [start[h], start[h + 1])
__global__ void __launch_bounds__(256) pack_b_rows_batch(const PackArgs* __restrict__ d, BatchTab bt) {
  extern __shared__ uint16_t rows_s[];
  __shared__ float cs[kFusedHalf], sn[kFusedHalf];
  const int64_t b = blockIdx.x;
  int h = 0;
  while (h + 1 < bt.n && b >= bt.start[h + 1]) ++h;
  pack_rows(d[h], b - bt.start[h], rows_s, cs, sn);
}

static int64_t pack_blocks(const PackArgs& a) {
  return (int64_t)a.n_arrays * a.n_layers * a.n_anchors * ((a.r + 15) / 16);
}

bool make_pack_args(PackArgs& a, const uint16_t* const* src, uint16_t* const* dst, const int* negate,
                    const FusedTab* const* tabs, int n_arrays, int n_layers, int n_anchors, int r, int D,
                    int head_dim) {
  if (n_arrays < 1 || n_arrays > 4 || r < 1 || (D & 31) || n_anchors < 1 || head_dim > 2 * kFusedHalf) return false;
  memset(&a, 0, sizeof a);
  for (int i = 0; i < n_arrays; ++i) {
    a.src[i] = src[i];
    a.dst[i] = dst[i];
    a.negate[i] = negate[i];
    a.rotate[i] = tabs[i] != nullptr;
    if (tabs[i]) a.tab = *tabs[i];   // at most one distinct rotation per descriptor
  }
  a.n_arrays = n_arrays; a.n_layers = n_layers; a.n_anchors = n_anchors; a.r = r; a.D = D; a.head_dim = head_dim;
  return true;
}

hipError_t launch_pack_b_batch(const PackArgs* d, const PackArgs* h, int n, hipStream_t st) {
  if (n < 1 || n > kMaxBatch) return hipErrorInvalidValue;
  BatchTab bt;
  bt.n = n;
  int64_t total = 0;
  for (int i = 0; i < n; ++i) {
    if (h[i].D != h[0].D) return hipErrorInvalidValue;
    bt.start[i] = (int32_t)total;
    bt.hop[i] = i;
    total += pack_blocks(h[i]);
  }
  bt.start[n] = (int32_t)total;
  const size_t lds = sizeof(uint16_t) * 16 * (size_t)(h[0].D + kPackPad);
  if (lds > 64 * 1024 || total >= (1ll << 31)) return hipErrorInvalidValue;
  if (total == 0) return hipSuccess;
  pack_b_rows_batch<<<(unsigned)total, 256, lds, st>>>(d, bt);
  return hipGetLastError();
}

hipError_t launch_pack_b(const uint16_t* const* src, uint16_t* const* dst, const int* negate,
                         const FusedTab* const* tabs, int n_arrays, int n_layers, int n_anchors, int r, int D,
                         int head_dim, hipStream_t st) {
  PackArgs a;
  if (!make_pack_args(a, src, dst, negate, tabs, n_arrays, n_layers, n_anchors, r, D, head_dim))
    return hipErrorInvalidValue;
  const size_t lds = sizeof(uint16_t) * 16 * (size_t)(D + kPackPad);
  if (lds <= 64 * 1024) {   // rows up to 2040 channels: staged through LDS
    pack_b_rows<<<(unsigned)pack_blocks(a), 256, lds, st>>>(a);
    return hipGetLastError();
  }
  const int64_t units = (int64_t)n_arrays * n_layers * n_anchors * (D / 32) * ((r + 15) / 16) * 64;
  int64_t blocks = (units + 255) / 256;
  if (blocks > 1 << 20) blocks = 1 << 20;
  pack_b<<<(unsigned)blocks, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fused(const FusedArgs& args, int mode, int head_dim, hipStream_t st) {
  FusedArgs a = args;
  if (a.D % 128 || a.D > 1024 || a.N > kMaxAnchors || (a.r_d & 15) || a.r_d > 256) return hipErrorInvalidValue;
  a.ring_stride = std::max(mode == FUSED_PAGES ? a.r_b : 0, a.apply ? a.r_d : 0) + 8;
  if (head_dim == 128) return fused_dispatch<128>(a, mode, st);
  if (head_dim == 64) return fused_dispatch<64>(a, mode, st);
  return hipErrorInvalidValue;
}

}  // namespace kvc
