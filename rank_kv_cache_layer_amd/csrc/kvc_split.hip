// Two-pass per-hop correction for gfx950 (CDNA4), bf16 caches, tiled for operand reuse:
// every work-group covers 128 tokens x 256 channels of one (layer, side) with 4 waves, wave
// (tw, cw) owning tokens [64 tw, 64 tw + 64) and channels [128 cw, 128 cw + 128) of the tile;
// two work-groups share a CU.  Anchor factors stream through double-buffered LDS slots shared
// by the waves, so each anchor's A rows are read once per 256 channels and its B slice once
// per 128 tokens.
//
// KVCMAS (arXiv 2609.34060):
//  * split_score: App. A.3 "Correction Weighting and Positional Alignment" -- per token, side
//    and anchor, the sum over the tile's channels of |Z_can - A B| (Eq. 7 factors), written as
//    partial sums per channel tile; and App. A.3 Eq. 9 -- the value rows' squared distance
//    over the prefix k, per (layer, anchor, tile).
//  * split_apply: the token weights (softmax over the correction set of -m / T_w, or of
//    cosine / T_w in the second scoring mode, or given), then Sec. 3.3 Eq. 8 / App. A.3
//    Eq. 12: out = R(s) Z + sum_a w_a A_a B'_a with B' = B turned by R(p_tgt) for keys.
//
// MFMA: v_mfma_f32_32x32x16_bf16 with channels as MFMA rows and tokens as MFMA columns; lane
// l (col = l % 32, hi = l / 32) holds token col of a 32-token block and rows
// 8 (j / 4) + 4 hi + j % 4 (j = 0..15) of a 32-channel block.  In split_score the source tile
// (fp32, canonical frame) is the accumulator input and B is pre-negated, so the MFMA chain
// yields E = Z_can - A B directly.  In split_apply the accumulators start from the residual.
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kSW = kSplitWidth;  // channels per work-group
constexpr int kC = 512;           // bf16 elements of one packed operand chunk (64 lanes x 8)
constexpr int kNCBW = kSW / 32;   // 32-channel blocks per work-group

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ uint4 scale8(uint4 r, float w) {
  return make_uint4(pack2(lo16(r.x) * w, hi16(r.x) * w), pack2(lo16(r.y) * w, hi16(r.y) * w),
                    pack2(lo16(r.z) * w, hi16(r.z) * w), pack2(lo16(r.w) * w, hi16(r.w) * w));
}

// wave-uniform value held in a VGPR (e.g. read from LDS) -> scalar register
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
// entry j (wave-uniform) of a table held one entry per lane -> scalar register
__device__ __forceinline__ int lane_get(int v, int j) { return __builtin_amdgcn_readlane(v, j); }

// Anchor slot tables of a work-group, one slot per lane (at most 64 anchors): slot j's anchor,
// first packed A row and readable row count, fetched once per wave; the pipelined loops pick
// slot j with a lane read instead of a chain of dependent memory lookups.
struct Slots {
  int a, off, lim;
};
__device__ __forceinline__ Slots load_slots(const uint8_t* list, int n, const int32_t* off, const int32_t* len,
                                            int row_cap, int lane) {
  Slots s{0, 0, 0};
  if (lane < n) {
    s.a = list[lane];
    s.off = off[s.a];
    s.lim = min(row_cap, len[s.a]);
  }
  return s;
}

// Raw buffer access: a 128-bit descriptor (base, size in bytes) in scalar registers plus a
// 32-bit per-lane byte offset; loads past the size return 0 and stores past it are dropped,
// which is how tile tails and rows beyond an anchor's length are handled without branches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped) 32-bit data, gfx9 family
constexpr int kStream = 2;               // non-temporal: streamed once, keep it out of the way in L2
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
template <int AUX = 0>
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int AUX = 0>
__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, AUX);
  return make_uint2(v.x, v.y);
}
template <int AUX = 0>
__device__ __forceinline__ void bstore8(rsrc_t r, uint32_t off, uint2 v) {
  const u32x2 x = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(x, r, (int)off, 0, AUX);
}

template <int HD> __device__ __forceinline__ constexpr bool lower_blk(int b) { return ((b * 32) % HD) < HD / 2; }
template <int HD> __device__ __forceinline__ constexpr int partner_blk(int b) { return b + HD / 64; }
template <int HD> __device__ __forceinline__ int pair_index(int b, int row) { return (b * 32) % HD + row; }

// Wave-private LDS staging of a 32-token x 128-channel bf16 half tile, rows padded to 132
// elements (264 bytes: consecutive rows start 2 banks apart, so the accumulator-layout 8-byte
// accesses of 16 lanes hit 32 distinct banks).  Global traffic goes through it with 16-byte
// row-contiguous accesses (each token row is 256 contiguous bytes) instead of row-strided
// 8-byte accesses in accumulator layout.
constexpr int kStRow = 132;
constexpr int kStage = 32 * kStRow;            // elements per wave

// 64 tokens x 128 channels (rows tw0.., channels d0..) of a layer's stored cache, buffer over
// its S rows (rows >= S read as 0), into accumulator layout (fp32).
__device__ __forceinline__ void load_tile(f32x16 (&z)[2][4], rsrc_t zr, int tw0, int D, int d0, uint16_t* stage,
                                          int lane, int col, int hi) {
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 4 + (lane >> 4), ch = (lane & 15) * 8;
      v[i] = bload16<kStream>(zr, (uint32_t)((tw0 + tb * 32 + row) * D + d0 + ch) * 2u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 4 + (lane >> 4), ch = (lane & 15) * 8;
      *reinterpret_cast<uint4*>(stage + row * kStRow + ch) = v[i];
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const uint2 x = *reinterpret_cast<const uint2*>(stage + col * kStRow + db * 32 + 8 * jg + 4 * hi);
        z[tb][db][4 * jg + 0] = lo16(x.x);
        z[tb][db][4 * jg + 1] = hi16(x.x);
        z[tb][db][4 * jg + 2] = lo16(x.y);
        z[tb][db][4 * jg + 3] = hi16(x.y);
      }
  }
}

// Accumulator tile (64 tokens x 128 channels) rounded to bf16 and stored through the staging
// area; rows >= S are dropped by the buffer.
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[2][4], rsrc_t orr, int tw0, int D, int d0,
                                           uint16_t* stage, int lane, int col, int hi) {
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        uint2 v;
        v.x = pack2(acc[tb][db][4 * jg + 0], acc[tb][db][4 * jg + 1]);
        v.y = pack2(acc[tb][db][4 * jg + 2], acc[tb][db][4 * jg + 3]);
        *reinterpret_cast<uint2*>(stage + col * kStRow + db * 32 + 8 * jg + 4 * hi) = v;
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 4 + (lane >> 4), ch = (lane & 15) * 8;
      const uint4 x = *reinterpret_cast<const uint4*>(stage + row * kStRow + ch);
      const u32x4 y = {x.x, x.y, x.z, x.w};
      __builtin_amdgcn_raw_buffer_store_b128(y, orr, (int)((tw0 + tb * 32 + row) * D + d0 + ch) * 2, 0, kStream);
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

// Tile decode: the channel tile is the fastest index so the channel tiles of one token tile
// run side by side on one XCD (they share the anchors' A rows through its L2), then token
// tiles, layers, sides.
struct TileId {
  int cq, tt, layer, side;
};
__device__ __forceinline__ TileId tile_id(const SplitArgs& p) {
  const int64_t lb = xcd_remap(blockIdx.x, gridDim.x);
  TileId t;
  t.cq = (int)(lb % p.nct);
  t.tt = (int)((lb / p.nct) % p.ntt);
  t.layer = (int)((lb / ((int64_t)p.nct * p.ntt)) % p.n_layers);
  t.side = (int)(lb / ((int64_t)p.nct * p.ntt * p.n_layers));
  return t;
}

// ================================================================== pass 1: scores
// One anchor for a wave: 8 accumulator blocks (2 token x 4 channel), each E = Z_can - A B
// reduced to per-lane |E| sums and (Q) masked E^2 sums.  The empty asm statement after each
// block's epilogue "redefines" the A operands, so the compiler cannot hoist later MFMA chains
// above it (which would need up to 8 live result blocks); the other wave of the SIMD fills
// the MFMA-to-epilogue latency.
template <int RK, bool Q>
__device__ __forceinline__ void score_anchor(const f32x16 (&z)[2][4], const uint16_t* as, const uint16_t* bs,
                                             int col, int hi, int lane, float qm0, float qm1, float& ms0,
                                             float& ms1, float& qs) {
  constexpr int RS = RK * 16 + 8;
  bf16x8 av[2][RK];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ks = 0; ks < RK; ++ks)
      av[tb][ks] = as_bf8(*reinterpret_cast<const uint4*>(as + (tb * 32 + col) * RS + ks * 16 + 8 * hi));
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    bf16x8 bv[RK];
#pragma unroll
    for (int ks = 0; ks < RK; ++ks) bv[ks] = as_bf8(*reinterpret_cast<const uint4*>(bs + (db * RK + ks) * kC + lane * 8));
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x16 e = mfma(bv[0], av[tb][0], z[tb][db]);
#pragma unroll
      for (int ks = 1; ks < RK; ++ks) e = mfma(bv[ks], av[tb][ks], e);
      const float s = abs_sum(e);
      if (tb == 0) ms0 += s; else ms1 += s;
      if (Q) qs = fmaf(sq_sum(e), tb == 0 ? qm0 : qm1, qs);
      if constexpr (RK == 1)
        asm volatile("" : "+v"(av[0][0]), "+v"(av[1][0]), "+v"(ms0), "+v"(ms1), "+v"(qs));
      else if constexpr (RK == 2)
        asm volatile("" : "+v"(av[0][0]), "+v"(av[0][1]), "+v"(av[1][0]), "+v"(av[1][1]), "+v"(ms0), "+v"(ms1),
                     "+v"(qs));
      else
        asm volatile("" : "+v"(av[0][0]), "+v"(av[1][0]), "+v"(ms0), "+v"(ms1), "+v"(qs));
    }
  }
}

// Streams one anchor's operands into LDS: A rows t0 .. t0+127 (rank R, rows >= lim are 0) and
// the work-group's packed B slice (kNCBW x RK chunks, contiguous).  Thread tid owns RK units
// of A and 2 RK of B; `issue` loads them into registers, `commit` writes them to a slot.
template <int UA, int UB>
struct Operands {
  uint4 a[UA], b[UB];
  float w[UA];
};

// A: buffer over the anchor's first `lim` rows (R bf16 each, rows >= lim read as 0); B: buffer
// over the work-group's packed slice.  With TT tokens and NT threads, A unit u = tid + NT i
// (i < UA = TT R / 8 / NT) is row u / (R/8), 16-byte column u % (R/8) of the tile; B unit
// u = tid + NT i (i < UB = 512 RK / NT) is bytes [16 u, 16 u + 16) of the slice.
template <int RK, int TT, int NT>
struct Stream {
  static constexpr int R = RK * 16, RS = R + 8;
  static constexpr int UA = TT * (R / 8) / NT, UB = kNCBW * RK * 64 / NT;
  using Ops = Operands<UA, UB>;
  static __device__ __forceinline__ void issue(Ops& o, rsrc_t A, rsrc_t B, int t0, int tid) {
#pragma unroll
    for (int i = 0; i < UA; ++i) {
      const int u = tid + i * NT;
      const int row = u / (R / 8), c = u - row * (R / 8);
      o.a[i] = bload16<kStream>(A, (uint32_t)(((t0 + row) * R + c * 8) * 2));
    }
#pragma unroll
    for (int i = 0; i < UB; ++i) o.b[i] = bload16(B, (uint32_t)(tid + i * NT) * 16u);
  }
  // with the token weights of the A rows (buffer over one anchor's weight row, fp32)
  static __device__ __forceinline__ void issue_w(Ops& o, rsrc_t A, rsrc_t B, rsrc_t W, int t0, int tid) {
    issue(o, A, B, t0, tid);
#pragma unroll
    for (int i = 0; i < UA; ++i) {
      const int row = (tid + i * NT) / (R / 8);
      o.w[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(W, (t0 + row) * 4, 0, 0));
    }
  }
  template <bool SCALE>
  static __device__ __forceinline__ void commit(const Ops& o, uint16_t* as, uint16_t* bs, int tid) {
#pragma unroll
    for (int i = 0; i < UA; ++i) {
      const int u = tid + i * NT;
      const int row = u / (R / 8), c = u - row * (R / 8);
      const uint4 x = SCALE ? scale8(o.a[i], o.w[i]) : o.a[i];
      *reinterpret_cast<uint4*>(as + row * RS + c * 8) = x;
    }
#pragma unroll
    for (int i = 0; i < UB; ++i) *reinterpret_cast<uint4*>(bs + (tid + i * NT) * 8) = o.b[i];
  }
};

template <int HD, int RK>
__global__ void __launch_bounds__(kScoreThreads) split_score(SplitArgs p) {
  constexpr int kST = kScoreTile, kNT = kScoreThreads, kNW = kNT / 64;
  using SM = Stream<RK, kST, kNT>;
  constexpr int R = RK * 16, RS = R + 8;
  constexpr int ASZ = kST * RS, BSZ = kNCBW * RK * kC;
  extern __shared__ __attribute__((aligned(16))) uint16_t dyn[];   // As[2][ASZ], Bs[2][BSZ]
  __shared__ float mp[2][2][kST];
  __shared__ float qp[kNW][kMaxAnchors];
  __shared__ float tab[2][kFusedHalf];

  const TileId id = tile_id(p);
  const bool keys = id.side == 0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, hi = lane >> 5;
  const int tw = wave >> 1, cw = wave & 1;
  const int D = p.D, S = p.S, N = p.N, NCB = D >> 5;
  const int t0 = id.tt * kST, tw0 = t0 + tw * 64;
  const int d0 = id.cq * kSW + cw * 128;
  uint16_t* As = dyn;
  uint16_t* Bs = dyn + 2 * ASZ;

  const uint8_t* list = keys ? p.corr : p.use;
  int nl = keys ? p.n_corr : p.n_use;
  const int s_work = keys ? (p.n_corr ? p.s_cov : 0) : max(p.n_corr ? p.s_cov : 0, p.mask_gate ? p.k_gate : 0);
  if (t0 >= s_work) nl = 0;

  for (int i = tid; i < HD / 2; i += kNT) {
    tab[0][i] = p.can.cs[i];
    tab[1][i] = p.can.sn[i];
  }
  const Slots sl = load_slots(list, keys ? p.n_corr : p.n_use, p.off, p.len, S, lane);
  __syncthreads();

  const uint16_t* Al = p.Ab[id.side] + id.layer * p.ab_layer;
  const uint16_t* Bl = p.Bb[id.side] + (((int64_t)id.layer * N) * NCB + id.cq * kNCBW) * RK * kC;
  const int64_t bstride = (int64_t)NCB * RK * kC;
  // past the end of the list the descriptors have size 0: the loads return 0 and fetch nothing,
  // so the pipeline below issues and commits unconditionally (no branches around memory ops)
  auto src = [&](int j, typename SM::Ops& o) {
    const bool live = j < nl;
    const int js = live ? j : 0;
    const int a = lane_get(sl.a, js);
    const int lim = live ? lane_get(sl.lim, js) : 0;
    SM::issue(o, make_rsrc(Al + (int64_t)lane_get(sl.off, js) * R, (uint32_t)lim * R * 2),
                       make_rsrc(Bl + a * bstride, live ? BSZ * 2 : 0), t0, tid);
  };

  // two register sets: set j & 1 holds anchor j's operands from two steps before it is used
  typename SM::Ops o0, o1;
  src(0, o0);
  src(1, o1);
  f32x16 z[2][4];
  if (nl > 0) {
    load_tile(z, make_rsrc(p.z[id.side] + (int64_t)id.layer * S * D, (uint32_t)S * D * 2), tw0, D, d0,
              dyn + wave * kStage, lane, col, hi);
    if (keys && p.can.active) rotate_tile<HD>(z, tab[0], tab[1], hi);
  }
  __syncthreads();   // the staging area overlaps the operand slots
  SM::template commit<false>(o0, As, Bs, tid);
  src(2, o0);
  __syncthreads();

  const float qm0 = (tw0 + col < p.k_gate && tw0 + col < S) ? 1.f : 0.f;
  const float qm1 = (tw0 + 32 + col < p.k_gate && tw0 + 32 + col < S) ? 1.f : 0.f;
  float* mpart = p.mpart + (((int64_t)id.cq * 2 + id.side) * p.n_layers + id.layer) * N * S;

  // the two pipeline stages are instantiated separately (compile-time slot, distinct marker),
  // so the compiler cannot fold them into one body that shares a single register set
  auto step = [&](auto stage, int j, typename SM::Ops& onext) {
    constexpr int buf = decltype(stage)::value;
    asm volatile("; pipeline stage %0" ::"n"(buf));
    const bool live = j < nl;
    const int a = lane_get(sl.a, live ? j : 0);
    const bool want_m = live && ((p.mask_corr >> a) & 1);
    const bool want_q = live && !keys && ((p.mask_gate >> a) & 1) && t0 < p.k_gate;
    if (live) {
      const uint16_t* as = As + buf * ASZ + tw * 64 * RS;
      const uint16_t* bs = Bs + buf * BSZ + cw * 4 * RK * kC;
      float ms0 = 0.f, ms1 = 0.f, qs = 0.f;
      if (want_q)
        score_anchor<RK, true>(z, as, bs, col, hi, lane, qm0, qm1, ms0, ms1, qs);
      else
        score_anchor<RK, false>(z, as, bs, col, hi, lane, qm0, qm1, ms0, ms1, qs);
      if (want_m) {
        ms0 += __shfl_xor(ms0, 32);
        ms1 += __shfl_xor(ms1, 32);
        if (hi == 0) {
          mp[buf][cw][tw * 64 + col] = ms0;
          mp[buf][cw][tw * 64 + 32 + col] = ms1;
        }
      }
      if (want_q) {
        qs = wave_sum(qs);
        if (lane == 0) qp[wave][a] = qs;
      }
    }
    // anchor j + 1 (fetched two steps ago into onext) goes to the other slot; anchor j + 3 is
    // fetched into the freed registers
    SM::template commit<false>(onext, As + (buf ^ 1) * ASZ, Bs + (buf ^ 1) * BSZ, tid);
    src(j + 3, onext);
    __syncthreads();
    if (want_m && tid < kST) {
      const int t = t0 + tid;
      if (t < S) mpart[(int64_t)a * S + t] = mp[buf][0][tid] + mp[buf][1][tid];
    }
  };
  for (int j = 0; j < nl; j += 2) {
    step(std::integral_constant<int, 0>{}, j, o1);
    step(std::integral_constant<int, 1>{}, j + 1, o0);
  }
  __syncthreads();
  if (!keys && p.partials) {
    float* part = p.partials + ((int64_t)id.layer * p.ntt * p.nct + (int64_t)id.tt * p.nct + id.cq) * N;
    for (int a = tid; a < N; a += kNT) {
      if (!((p.mask_gate >> a) & 1)) continue;
      float s = 0.f;
      if (t0 < p.k_gate && nl > 0)
        for (int w = 0; w < kNW; ++w) s += qp[w][a];
      part[a] = s;
    }
  }
}

// ================================================================== token weights
// App. A.3 "Correction Weighting": per token and side, softmax over the correction set of
// -m / T_w (first mode, m = mean |Z_can - A B| from the per-channel-tile partials) or of
// cosine / T_w (second mode), or the caller's weights as given; 0 past S_cov.  Written
// anchor-major (w[side][layer][a][t], the apply kernel's operand order) and, if requested,
// token-major for the caller (w_out[side][layer][t][a], 0 outside the correction set).
__global__ void __launch_bounds__(256) split_weights(SplitArgs p, int wmode) {
  extern __shared__ float xs[];   // [n_corr][256]
  const int tid = threadIdx.x;
  const int t = blockIdx.x * 256 + tid;
  const int layer = blockIdx.y, side = blockIdx.z;
  const int S = p.S, N = p.N, L = p.n_layers, nc = p.n_corr;
  const bool in = t < S, cov = t < p.s_cov;
  float mx = -INFINITY;
  for (int j = 0; j < nc; ++j) {
    const int a = p.corr[j];
    float x = 0.f;
    if (cov) {
      if (wmode == SPLIT_W_PARTIALS) {
        float m = 0.f;
        for (int q = 0; q < p.nct; ++q) m += p.mpart[((((int64_t)q * 2 + side) * L + layer) * N + a) * S + t];
        x = -(m * p.inv_d) * p.inv_temp;
      } else if (wmode == SPLIT_W_SCORES) {
        x = p.w_in[side][((int64_t)layer * S + t) * N + a] * p.inv_temp;
      } else {
        x = p.w_in[side][((int64_t)layer * S + t) * N + a];
      }
    }
    xs[j * 256 + tid] = x;
    mx = fmaxf(mx, x);
  }
  if (wmode != SPLIT_W_GIVEN) {
    float sum = 0.f;
    for (int j = 0; j < nc; ++j) {
      const float e = expf(xs[j * 256 + tid] - mx);
      xs[j * 256 + tid] = e;
      sum += e;
    }
    const float inv = 1.f / sum;
    for (int j = 0; j < nc; ++j) xs[j * 256 + tid] *= inv;
  }
  if (!in) return;
  float* wa = p.wa + ((int64_t)side * L + layer) * N * S;
  for (int j = 0; j < nc; ++j) wa[(int64_t)p.corr[j] * S + t] = cov ? xs[j * 256 + tid] : 0.f;
  if (p.w_out[side]) {
    float* dst = p.w_out[side] + ((int64_t)layer * S + t) * N;
    for (int a = 0; a < N; ++a) dst[a] = 0.f;
    for (int j = 0; j < nc; ++j) dst[p.corr[j]] = cov ? xs[j * 256 + tid] : 0.f;
  }
}

// ================================================================== pass 2: apply
// Sec. 3.3 Eq. 8 / App. A.3 Eq. 12: out = R(s) Z + sum_a w_a A_a B'_a, the token weights read
// anchor-major (split_weights) and folded into the A rows on their way into LDS.
template <int HD, int RKD>
__global__ void __launch_bounds__(kApplyThreads, 2) split_apply(SplitArgs p) {
  constexpr int kST = kApplyTile, kNT = kApplyThreads;
  using SM = Stream<RKD, kST, kNT>;
  constexpr int R = RKD * 16, RS = R + 8;
  constexpr int ASZ = kST * RS, BSZ = kNCBW * RKD * kC;
  extern __shared__ __attribute__((aligned(16))) uint16_t dyn[];   // As[2][ASZ], Bs[2][BSZ] | staging
  __shared__ float tab[2][kFusedHalf];

  const TileId id = tile_id(p);
  const bool keys = id.side == 0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, hi = lane >> 5;
  const int tw = wave >> 1, cw = wave & 1;
  const int D = p.D, S = p.S, N = p.N, NCB = D >> 5;
  const int t0 = id.tt * kST, tw0 = t0 + tw * 64;
  const int d0 = id.cq * kSW + cw * 128;
  uint16_t* As = dyn;
  uint16_t* Bs = dyn + 2 * ASZ;

  for (int i = tid; i < HD / 2; i += kNT) {
    tab[0][i] = p.shift.cs[i];
    tab[1][i] = p.shift.sn[i];
  }
  const int nc = (t0 < p.s_cov) ? p.n_corr : 0;
  const Slots sl = load_slots(p.corr, p.n_corr, p.off, p.len, min(S, p.s_cov), lane);
  const uint16_t* Al = p.Ad[id.side] + id.layer * p.ad_layer;
  const uint16_t* Bl = p.Bd[id.side] + (((int64_t)id.layer * N) * NCB + id.cq * kNCBW) * RKD * kC;
  const float* Wl = p.wa + ((int64_t)id.side * p.n_layers + id.layer) * N * S;
  const int64_t bstride = (int64_t)NCB * RKD * kC;
  // zero-size descriptors past the correction set (see split_score)
  auto src = [&](int j, typename SM::Ops& o) {
    const bool live = j < nc;
    const int js = live ? j : 0;
    const int a = lane_get(sl.a, js);
    const int lim = live ? lane_get(sl.lim, js) : 0;
    SM::issue_w(o, make_rsrc(Al + (int64_t)lane_get(sl.off, js) * R, (uint32_t)lim * R * 2),
                make_rsrc(Bl + a * bstride, live ? BSZ * 2 : 0), make_rsrc(Wl + (int64_t)a * S, (uint32_t)lim * 4),
                t0, tid);
  };
  typename SM::Ops o0, o1;
  src(0, o0);
  src(1, o1);

  // ---- residual: R(s) K or V
  f32x16 acc[2][4];
  const uint32_t layer_bytes = (uint32_t)S * D * 2;
  __syncthreads();   // rotation table
  load_tile(acc, make_rsrc(p.z[id.side] + (int64_t)id.layer * S * D, layer_bytes), tw0, D, d0, dyn + wave * kStage,
            lane, col, hi);
  if (keys && p.shift.active) rotate_tile<HD>(acc, tab[0], tab[1], hi);
  __syncthreads();   // the staging area overlaps the operand slots
  SM::template commit<true>(o0, As, Bs, tid);
  src(2, o0);
  __syncthreads();
  // the two pipeline stages are instantiated separately (compile-time slot, distinct marker),
  // so the compiler cannot fold them into one body that shares a single register set
  auto step = [&](auto stage, int j, typename SM::Ops& onext) {
    constexpr int buf = decltype(stage)::value;
    asm volatile("; pipeline stage %0" ::"n"(buf));
    if (j < nc) {
      const uint16_t* as = As + buf * ASZ + tw * 64 * RS;
      const uint16_t* bs = Bs + buf * BSZ + cw * 4 * RKD * kC;
#pragma unroll
      for (int ks = 0; ks < RKD; ++ks) {
        const bf16x8 a0 = as_bf8(*reinterpret_cast<const uint4*>(as + col * RS + ks * 16 + 8 * hi));
        const bf16x8 a1 = as_bf8(*reinterpret_cast<const uint4*>(as + (32 + col) * RS + ks * 16 + 8 * hi));
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 b = as_bf8(*reinterpret_cast<const uint4*>(bs + (db * RKD + ks) * kC + lane * 8));
          acc[0][db] = mfma(b, a0, acc[0][db]);
          acc[1][db] = mfma(b, a1, acc[1][db]);
        }
      }
    }
    SM::template commit<true>(onext, As + (buf ^ 1) * ASZ, Bs + (buf ^ 1) * BSZ, tid);
    src(j + 3, onext);
    __syncthreads();
  };
  for (int j = 0; j < nc; j += 2) {
    step(std::integral_constant<int, 0>{}, j, o1);
    step(std::integral_constant<int, 1>{}, j + 1, o0);
  }

  // the last step ended with a barrier: the operand slots are free for the output staging
  store_tile(acc, make_rsrc(p.out[id.side] + (int64_t)id.layer * S * D, layer_bytes), tw0, D, d0, dyn + wave * kStage,
             lane, col, hi);
}

template <typename K>
hipError_t go(K kernel, const SplitArgs& args, int tile, int threads, size_t shmem, hipStream_t st) {
  if (shmem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  SplitArgs a = args;
  a.ntt = (a.S + tile - 1) / tile;
  const int64_t nblk = (int64_t)a.nct * a.ntt * a.n_layers * 2;
  kernel<<<dim3((unsigned)nblk), dim3(threads), shmem, st>>>(a);
  return hipGetLastError();
}

template <int HD>
hipError_t score_dispatch(const SplitArgs& a, hipStream_t st) {
  switch (a.r_b) {
    case 16: return go(split_score<HD, 1>, a, kScoreTile, kScoreThreads, split_score_lds(a.r_b), st);
    case 32: return go(split_score<HD, 2>, a, kScoreTile, kScoreThreads, split_score_lds(a.r_b), st);
    case 64: return go(split_score<HD, 4>, a, kScoreTile, kScoreThreads, split_score_lds(a.r_b), st);
    default: return hipErrorInvalidValue;
  }
}

template <int HD>
hipError_t apply_dispatch(const SplitArgs& a, hipStream_t st) {
  const size_t lds = split_apply_lds(a.r_d);
  switch (a.r_d) {
    case 16: return go(split_apply<HD, 1>, a, kApplyTile, kApplyThreads, lds, st);
    case 32: return go(split_apply<HD, 2>, a, kApplyTile, kApplyThreads, lds, st);
    case 64: return go(split_apply<HD, 4>, a, kApplyTile, kApplyThreads, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// dynamic LDS: two operand slots (A rows + packed B slice) or the 8 waves' staging areas,
// whichever is larger, then (apply) the token weights
size_t split_score_lds(int r_b) {
  const int RK = r_b / 16;
  return std::max(sizeof(uint16_t) * 2 * ((size_t)kScoreTile * (r_b + 8) + (size_t)kNCBW * RK * kC),
                  sizeof(uint16_t) * (kScoreThreads / 64) * kStage);
}

size_t split_apply_lds(int r_d) {
  const int RKD = r_d / 16;
  return std::max(sizeof(uint16_t) * 2 * ((size_t)kApplyTile * (r_d + 8) + (size_t)kNCBW * RKD * kC),
                  sizeof(uint16_t) * (kApplyThreads / 64) * kStage);
}

hipError_t launch_split_score(const SplitArgs& a, int head_dim, hipStream_t st) {
  if (a.D % kSW || a.N > kMaxAnchors) return hipErrorInvalidValue;
  if (head_dim == 128) return score_dispatch<128>(a, st);
  if (head_dim == 64) return score_dispatch<64>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_split_apply(const SplitArgs& a, int head_dim, hipStream_t st) {
  if (a.D % kSW || a.N > kMaxAnchors || !a.wa) return hipErrorInvalidValue;
  if (head_dim == 128) return apply_dispatch<128>(a, st);
  if (head_dim == 64) return apply_dispatch<64>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_split_weights(const SplitArgs& a, int wmode, hipStream_t st) {
  if (a.N > kMaxAnchors || !a.wa || a.n_corr < 1) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.S + 255) / 256), (unsigned)a.n_layers, 2);
  split_weights<<<grid, 256, sizeof(float) * 256 * (size_t)a.n_corr, st>>>(a, wmode);
  return hipGetLastError();
}

}  // namespace kvc
