// Two-pass per-hop correction for gfx950 (CDNA4), bf16 caches, tiled for operand reuse:
// every work-group covers 128 tokens x 256 channels of one (layer, side) with 4 waves, wave
// (tw, cw) owning tokens [64 tw, 64 tw + 64) and channels [128 cw, 128 cw + 128) of the tile;
// two scoring or three apply work-groups share a CU.  Anchor factors stream through LDS slots
// shared by the waves, so each anchor's A rows are read once per 256 channels and its B slice
// once per 128 tokens.
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
template <typename L8, typename L32>
__device__ __forceinline__ Slots load_slots(L8 list, int n, L32 off, L32 len, int row_cap, int lane) {
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

// LDS byte offset of a shared-memory pointer, and typed LDS reads at a byte offset
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_char*)p);
}
__device__ __forceinline__ uint4 lds_u4(uint32_t off) {
  const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((uintptr_t)off);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float lds_f(uint32_t off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) float*>((uintptr_t)off);
}

template <int HD> __device__ __forceinline__ constexpr bool lower_blk(int b) { return ((b * 32) % HD) < HD / 2; }
template <int HD> __device__ __forceinline__ constexpr int partner_blk(int b) { return b + HD / 64; }
template <int HD> __device__ __forceinline__ int pair_index(int b, int row) { return (b * 32) % HD + row; }

// Wave-private LDS staging of a 32-token x 128-channel bf16 half tile, rows padded to 136
// elements (272 bytes: every row stays 16-byte aligned for the 16-byte accesses, and
// consecutive rows start 4 banks apart, so the accumulator-layout 8-byte accesses of 16 lanes
// hit 32 distinct banks).  Global traffic goes through it with 16-byte row-contiguous accesses
// (each token row is 256 contiguous bytes) instead of row-strided 8-byte accesses in
// accumulator layout.
constexpr int kStRow = 136;
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
      // four table entries at a time: the compiler would otherwise load all 32 of a block pair
      // up front, which pushes the apply kernel (168 VGPRs) into spilling
      if ((j & 3) == 3) asm volatile("" ::: "memory");
    }
  }
}

// Cross-lane sums on the VALU (DPP and the gfx950 lane swap), no LDS round trips.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}
// sum over the 64 lanes, complete in lane 63: within quads, within rows of 16 (rotations by
// 4 and 8), then row 0 into row 1, row 2 into row 3, and row 1 into rows 2 and 3
__device__ __forceinline__ float wave_sum63(float v) {
  v += dpp<0xB1>(v);          // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);          // quad_perm [2,3,0,1]
  v += dpp<0x124>(v);         // row_ror:4
  v += dpp<0x128>(v);         // row_ror:8
  v += dpp<0x142, 0xa>(v);    // row_bcast:15
  v += dpp<0x143, 0xc>(v);    // row_bcast:31
  return v;
}
// v + (v of lane ^ 32)
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Tile decode: the channel tile is the fastest index so the channel tiles of one token tile
// run side by side on one XCD (they share the anchors' A rows through its L2), then token
// tiles, layers, sides.  With `side_first` the side is the fastest index instead: the scoring
// pass then keeps key tiles (|E| sums only) and value tiles (|E| and E^2 sums, twice the
// vector work) side by side on every CU, so the matrix and vector units are loaded evenly.
struct TileId {
  int cq, tt, layer, side;
};
template <bool side_first = false, typename P>
__device__ __forceinline__ TileId tile_id(P& p, int64_t lb) {
  TileId t;
  if constexpr (side_first) {
    t.side = (int)(lb & 1);
    lb >>= 1;
    t.cq = (int)(lb % p.nct);
    t.tt = (int)((lb / p.nct) % p.ntt);
    t.layer = p.layer0 + (int)((lb / ((int64_t)p.nct * p.ntt)) % p.n_grp);
    return t;
  }
  t.cq = (int)(lb % p.nct);
  t.tt = (int)((lb / p.nct) % p.ntt);
  t.layer = p.layer0 + (int)((lb / ((int64_t)p.nct * p.ntt)) % p.n_grp);
  t.side = (int)(lb / ((int64_t)p.nct * p.ntt * p.n_grp));
  return t;
}

// ================================================================== pass 1: scores
// The operands an anchor's first products need (its A fragments and the first two channel
// blocks' B fragments), read as soon as the anchor's slot has landed, ahead of the step's scalar
// bookkeeping, so their latency is not paid in front of the first products.
template <int RK>
struct ScoreFrags {
  bf16x8 av[2][RK], bv[RK], bn[RK];
};
template <int RK>
__device__ __forceinline__ ScoreFrags<RK> score_frags(uint32_t slot, const uint32_t (&aoff)[2][RK], uint32_t boff) {
  ScoreFrags<RK> f;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ks = 0; ks < RK; ++ks) f.av[tb][ks] = as_bf8(lds_u4(slot + aoff[tb][ks]));
  const uint32_t bs = slot + boff;
#pragma unroll
  for (int ks = 0; ks < RK; ++ks) {
    f.bv[ks] = as_bf8(lds_u4(bs + ks * 1024));
    f.bn[ks] = as_bf8(lds_u4(bs + (RK + ks) * 1024));
  }
  return f;
}

// One anchor for a wave: 8 accumulator blocks (2 token x 4 channel, channel-block major), each
// E = Z_can - A B reduced to per-lane |E| sums and (Q) E^2 sums.  Software-pipelined one block
// deep: the MFMA chain of block b + 1 is issued before the VALU reduction of block b, and the
// empty asm statement after each reduction "redefines" the A operands, so the compiler cannot
// hoist the chain of block b + 2 above it (two live result blocks, not eight).
// `slot`: LDS byte offset of the anchor's slot; `fr`: its first fragments (score_frags);
// `boff`: this lane's offset of its first B chunk inside a slot; `dma(u)`: issues transfer u of
// this wave's share of a later anchor's operands, called once per result block while u is below
// the share's size.
template <int RK, bool Q, typename RG, typename DMA>
__device__ __forceinline__ void score_anchor(const f32x16 (&z)[2][4], const ScoreFrags<RK>& fr, uint32_t slot,
                                             uint32_t boff, float qm0, float qm1, float& ms0, float& ms1,
                                             float& qs, DMA&& dma) {
  bf16x8 av[2][RK];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ks = 0; ks < RK; ++ks) av[tb][ks] = fr.av[tb][ks];
  const uint32_t bs = slot + boff;
  float m[2] = {0.f, 0.f}, q[2] = {0.f, 0.f};
  auto chain = [&](const bf16x8* bv, int tb, int db) {
    f32x16 e = mfma(bv[0], av[tb][0], z[tb][db]);
#pragma unroll
    for (int ks = 1; ks < RK; ++ks) e = mfma(bv[ks], av[tb][ks], e);
    return e;
  };
  auto reduce = [&](const f32x16& e, int tb) {
#pragma unroll
    for (int j = 0; j < 16; ++j) m[tb] += fabsf(e[j]);
    if (Q) {
#pragma unroll
      for (int j = 0; j < 16; ++j) q[tb] = fmaf(e[j], e[j], q[tb]);
    }
  };
  // B fragments of channel block db (bv) and db + 1 (bn): each block's are read from LDS two
  // result blocks before their first use
  bf16x8 bv[RK], bn[RK];
#pragma unroll
  for (int ks = 0; ks < RK; ++ks) {
    bv[ks] = fr.bv[ks];
    bn[ks] = fr.bn[ks];
  }
  f32x16 e = chain(bv, 0, 0);
#pragma unroll
  for (int b = 1; b <= 8; ++b) {
    f32x16 en;
    if (b < 8) {
      const int db = b >> 1, tb = b & 1;
      if (tb == 0) {
#pragma unroll
        for (int ks = 0; ks < RK; ++ks) bv[ks] = bn[ks];
      }
      en = chain(bv, tb, db);
      if (tb == 0 && db < 3) {
#pragma unroll
        for (int ks = 0; ks < RK; ++ks) bn[ks] = as_bf8(lds_u4(bs + ((db + 1) * RK + ks) * 1024));
      }
    }
    if (b - 1 < RG::DMA_PER_WAVE) dma(b - 1);
    reduce(e, (b - 1) & 1);
    // the q sums are tied too: left free, their FMAs sink and keep every block alive
    if constexpr (RK == 1)
      asm volatile("" : "+v"(av[0][0]), "+v"(av[1][0]), "+v"(m[0]), "+v"(m[1]), "+v"(q[0]), "+v"(q[1]));
    else
      asm volatile("" : "+v"(av[0][0]), "+v"(av[0][1]), "+v"(av[1][0]), "+v"(av[1][1]), "+v"(m[0]), "+v"(m[1]),
                   "+v"(q[0]), "+v"(q[1]));
    if (b < 8) e = en;
  }
  ms0 += m[0];
  ms1 += m[1];
  if (Q) qs = fmaf(q[0], qm0, fmaf(q[1], qm1, qs));
}

// ------------------------------------------------------------ operand ring (LDS, DMA-filled)
// Anchor operands stream from memory straight into LDS with buffer->LDS DMA (each lane of a
// wave instruction moves 16 bytes to LDS base + 16 * lane; lanes past the descriptor's size
// write zeros), into a ring of slots: slot j % (slots) holds anchor j's A rows, its B slice and
// (apply) its token weights.  The scoring pass has three slots and fetches anchor j + 2 while
// anchor j is consumed; the apply pass has two and fetches anchor j + 1.  A step waits only for
// its own slot (vmcnt), then a bare barrier (no release fence, which would drain every DMA in
// flight).
constexpr int kSlots = 3;        // scoring pass
constexpr int kApplySlots = 2;   // apply pass (three work-groups per CU)
typedef __attribute__((address_space(3))) void lds_void;

// The transfer is issued through inline assembly: the compiler then neither reorders LDS
// accesses around it nor makes every later LDS read wait for all transfers in flight (it cannot
// tell ring slots apart); the explicit waits below order each slot's transfer before its reads.
// LDS address in M0 (wave-uniform), 16 bytes per lane at M0 + 16 * lane.
// M0 is written only here (nothing else in these kernels uses it).
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t lds_addr, uint32_t voff) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)lds_addr);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory");
}


// s_waitcnt with vmcnt <= N and lgkmcnt = 0 (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] in [15:14]), then the work-group barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
}

// Slot layout for rank 16 RK, TT tokens, NW waves: A rows (TT x R bf16, 16-byte units
// swizzled so the fragment reads of 16 consecutive rows hit distinct banks), the B slice
// (kNCBW x RK packed 1 KiB chunks), the TT token weights (fp32, apply only).  RA = the rank
// of the A rows taken (<= R): the units of an LDS row past it are filled with zeros; RS = the
// A rows' stride in memory (elements, >= RA: a slice of the columns of wider rows).
template <int RK, int TT, int NW, bool W, int RA = RK * 16, int RS = RA>
struct Ring {
  static constexpr int R = RK * 16;
  static_assert(RA % 8 == 0 && RA <= R && RS >= RA && RS % 8 == 0, "A row rank");
  static constexpr int U = R / 8;                       // 16-byte units per A row
  static constexpr int A_BYTES = TT * R * 2;
  static constexpr int B_BYTES = kNCBW * RK * 1024;
  static constexpr int W_BYTES = W ? TT * 4 : 0;
  static constexpr int SLOT = A_BYTES + B_BYTES + W_BYTES;
  static constexpr int A_PER_WAVE = A_BYTES / 1024 / NW;
  static constexpr int B_PER_WAVE = B_BYTES / 1024 / NW;
  static constexpr int W_LANES = W ? TT / 4 / NW : 0;    // lanes per wave moving weights
  static constexpr int DMA_PER_WAVE = A_PER_WAVE + B_PER_WAVE + (W ? 1 : 0);
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "ring split");
  static_assert(!W || (TT % (4 * NW) == 0 && W_LANES <= 64), "weight split");

  // 16-byte unit of A row `row`, column unit `c`, inside the slot
  static __device__ __forceinline__ int a_unit(int row, int c) { return row * U + (c ^ ((row / (16 / U)) & (U - 1))); }

  // DMA anchor operands into `slot`: A rows t0.. of buffer `Ar` (rows past its size read 0),
  // B slice of buffer `Br`, weights t0.. of buffer `Wr`.
  // `slot`: LDS byte offset of the slot (wave-uniform); `wave` must be wave-uniform too
  static __device__ __forceinline__ void fetch(uint32_t slot, rsrc_t Ar, rsrc_t Br, rsrc_t Wr, int t0, int wave,
                                               int lane) {
#pragma unroll
    for (int i = 0; i < A_PER_WAVE; ++i) {
      const int u = (wave * A_PER_WAVE + i) * 64 + lane;     // LDS unit this lane fills
      const int row = u / U, cpos = u % U;
      const int c = cpos ^ ((row / (16 / U)) & (U - 1));     // global unit stored there
      // units past the stored rank read out of range: the transfer writes zeros there
      const uint32_t voff = c * 8 < RA ? (uint32_t)(((t0 + row) * RS + c * 8) * 2) : 0x80000000u;
      dma16(Ar, slot + (wave * A_PER_WAVE + i) * 1024, voff);
    }
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
      const int kc = wave * B_PER_WAVE + i;
      dma16(Br, slot + A_BYTES + kc * 1024, (uint32_t)(kc * 1024 + lane * 16));
    }
    if constexpr (W) {
      if (lane < W_LANES)
        dma16(Wr, slot + A_BYTES + B_BYTES + wave * W_LANES * 16, (uint32_t)((t0 + (wave * W_LANES + lane) * 4) * 4));
    }
  }

  // Transfer `i` (< A_PER_WAVE + B_PER_WAVE; a compile-time constant after unrolling) of this
  // wave's share of fetch() without weights, so a step can spread its transfers over its work.
  static __device__ __forceinline__ void fetch_unit(int i, uint32_t slot, rsrc_t Ar, rsrc_t Br, int t0, int wave,
                                                    int lane) {
    if (i < A_PER_WAVE) {
      const int u = (wave * A_PER_WAVE + i) * 64 + lane;
      const int row = u / U, cpos = u % U;
      const int c = cpos ^ ((row / (16 / U)) & (U - 1));
      const uint32_t voff = c * 8 < RA ? (uint32_t)(((t0 + row) * RS + c * 8) * 2) : 0x80000000u;
      dma16(Ar, slot + (wave * A_PER_WAVE + i) * 1024, voff);
    } else {
      const int kc = wave * B_PER_WAVE + (i - A_PER_WAVE);
      dma16(Br, slot + A_BYTES + kc * 1024, (uint32_t)(kc * 1024 + lane * 16));
    }
  }
};

// Static LDS of a scoring work-group (the operand ring is dynamic LDS).
struct ScoreShared {
  float mp[2][2][kScoreTile];                    // |E| sums of two anchors, both channel halves
  float qp[kScoreThreads / 64][kMaxAnchors];     // per-wave gate sums
  float tab[2][kFusedHalf];                      // R(-p_src) table
};

// One scoring tile (logical block `lb` of the hop described by `p`).
template <int HD, int RK, typename P>
__device__ __forceinline__ void score_tile(P& p, int64_t lb, char* ring, ScoreShared& sh) {
  constexpr int kST = kScoreTile, kNT = kScoreThreads, kNW = kNT / 64;
  using RG = Ring<RK, kST, kNW, false>;
  constexpr int R = RK * 16;
  auto& mp = sh.mp;
  auto& qp = sh.qp;
  auto& tab = sh.tab;

  const TileId id = tile_id<true>(p, lb);
  const bool keys = id.side == 0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, hi = lane >> 5;
  const int tw = wave >> 1, cw = wave & 1;
  const int D = p.D, S = p.S, N = p.N, NCB = D >> 5;
  const int t0 = id.tt * kST, tw0 = t0 + tw * 64;
  const int d0 = id.cq * kSW + cw * 128;

  const auto list = keys ? p.corr : p.use;
  int nl = keys ? p.n_corr : p.n_use;
  const int s_work = keys ? (p.n_corr ? p.s_cov : 0) : max(p.n_corr ? p.s_cov : 0, p.mask_gate ? p.k_gate : 0);
  if (t0 >= s_work) nl = 0;

  for (int i = tid; i < HD / 2; i += kNT) {
    tab[0][i] = p.can.cs[i];
    tab[1][i] = p.can.sn[i];
  }
  const Slots sl = load_slots(list, keys ? p.n_corr : p.n_use, p.off, p.len, S, lane);

  const uint16_t* Al = p.Ab[id.side] + id.layer * p.ab_layer;
  const uint16_t* Bl = p.Bb[id.side] + (((int64_t)id.layer * N) * NCB + id.cq * kNCBW) * RK * kC;
  const int64_t bstride = (int64_t)NCB * RK * kC;
  // past the end of the list the descriptors have size 0: the DMA writes zeros and fetches
  // nothing, so every step issues the same number of transfers
  const uint32_t ring0 = lds_off(ring);
  const int wv = uni(wave);
  auto fetch = [&](int j) {
    const bool live = j < nl;
    const int js = live ? j : 0;
    const int a = lane_get(sl.a, js);
    const int lim = live ? lane_get(sl.lim, js) : 0;
    RG::fetch(ring0 + (uint32_t)(j % kSlots) * RG::SLOT,
              make_rsrc(Al + (int64_t)lane_get(sl.off, js) * R, (uint32_t)lim * R * 2),
              make_rsrc(Bl + a * bstride, live ? RG::B_BYTES : 0), make_rsrc(nullptr, 0), t0, wv, lane);
  };
  // The same transfers for the steady state, issued one per result block of the step two
  // anchors earlier (score_anchor's `dma`), not all right after the step's barrier where every
  // wave of the CU would queue its transfers at once in front of its first products.
  struct Plan {
    uint32_t slot;
    rsrc_t Ar, Br;
  };
  auto plan = [&](int j) {
    const bool live = j < nl;
    const int js = live ? j : 0;
    const int a = lane_get(sl.a, js);
    const int lim = live ? lane_get(sl.lim, js) : 0;
    return Plan{ring0 + (uint32_t)(j % kSlots) * RG::SLOT,
                make_rsrc(Al + (int64_t)lane_get(sl.off, js) * R, (uint32_t)lim * R * 2),
                make_rsrc(Bl + a * bstride, live ? RG::B_BYTES : 0)};
  };
  uint32_t aoff[2][RK];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ks = 0; ks < RK; ++ks) aoff[tb][ks] = RG::a_unit(tw * 64 + tb * 32 + col, ks * 2 + hi) * 16;
  const uint32_t boff = RG::A_BYTES + cw * 4 * RK * 1024 + lane * 16;

  const float qm0 = (tw0 + col < p.k_gate && tw0 + col < S) ? 1.f : 0.f;
  const float qm1 = (tw0 + 32 + col < p.k_gate && tw0 + 32 + col < S) ? 1.f : 0.f;
  float* mpart = p.mpart + (((int64_t)id.cq * 2 + id.side) * p.n_layers + id.layer) * N * S;
  auto store_m = [&](int j) {   // partial |E| sums of anchor j (LDS buffer j & 1), both channel halves
    const int a = lane_get(sl.a, j);
    if (((p.mask_corr >> a) & 1) && tid < kST) {
      const int t = t0 + tid;
      if (t < S) mpart[(int64_t)a * S + t] = mp[j & 1][0][tid] + mp[j & 1][1][tid];
    }
  };

  // value rows also accumulate the gate sums (Eq. 9), masked per anchor afterwards
  auto run = [&](const f32x16 (&z)[2][4], auto values) {
    constexpr bool Q = decltype(values)::value;
#pragma nounroll
    for (int j = 0; j < nl; ++j) {
      wait_vm_barrier<RG::DMA_PER_WAVE>();   // anchor j landed for every wave; slot (j + 2) % 3 is free
      // through a lane read the base is opaque: each operand address is then one add to it
      // plus an immediate offset, not a re-derivation of j % kSlots per access
      const uint32_t slot = (uint32_t)uni((int)(ring0 + (uint32_t)(j % kSlots) * RG::SLOT));
      const ScoreFrags<RK> fr = score_frags<RK>(slot, aoff, boff);
      const Plan fp = plan(j + 2);
      const int a = lane_get(sl.a, j);
      float ms0 = 0.f, ms1 = 0.f, qs = 0.f;
      score_anchor<RK, Q, RG>(z, fr, slot, boff, qm0, qm1, ms0, ms1, qs,
                              [&](int u) { RG::fetch_unit(u, fp.slot, fp.Ar, fp.Br, t0, wv, lane); });
      if ((p.mask_corr >> a) & 1) {
        ms0 = xor32_sum(ms0);
        ms1 = xor32_sum(ms1);
        if (hi == 0) {
          mp[j & 1][cw][tw * 64 + col] = ms0;
          mp[j & 1][cw][tw * 64 + 32 + col] = ms1;
        }
      }
      if (Q && ((p.mask_gate >> a) & 1)) {
        qs = wave_sum63(qs);
        if (lane == 63) qp[wave][a] = qs;
      }
      // anchor j - 1's sums (written by every wave before this step's barrier; this step writes
      // the other buffer, and the next step's barrier orders this read before its reuse)
      if (j > 0) store_m(j - 1);
    }
  };
  __syncthreads();   // rotation table (before any transfer: the barrier's fence would wait for them)
  if (nl > 0) {
    f32x16 z[2][4];
    fetch(0);   // in flight together with the source tile's loads
    // staging (wave-private) in the ring past slot 0, free until anchor 1 is fetched
    load_tile(z, make_rsrc(p.z[id.side] + (int64_t)id.layer * S * D, (uint32_t)S * D * 2), tw0, D, d0,
              reinterpret_cast<uint16_t*>(ring + RG::SLOT) + wave * kStage, lane, col, hi);
    if (keys && p.can.active) rotate_tile<HD>(z, tab[0], tab[1], hi);
    wait_vm_barrier<63>();   // every wave is done with the staging area
    fetch(1);
    if (keys)
      run(z, std::false_type{});
    else
      run(z, std::true_type{});
  }
  wait_vm_barrier<0>();   // also drains the trailing (empty) transfers
  if (nl > 0) store_m(nl - 1);
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

template <int HD, int RK>
__global__ void __launch_bounds__(kScoreThreads, 2) split_score(SplitArgs p) {
  extern __shared__ __attribute__((aligned(16))) char ring[];   // kSlots x slot | staging
  __shared__ ScoreShared sh;
  score_tile<HD, RK>(p, xcd_remap(blockIdx.x, gridDim.x), ring, sh);
}

// A batched launch's descriptor, read through the constant address space: like a kernel argument
// it is known not to change during the kernel, so its fields stay in scalar registers (or are
// re-read at will) across the operand transfers' memory clobbers instead of being re-read
// after each of them.
typedef const __attribute__((address_space(4))) SplitArgs CSplitArgs;
__device__ __forceinline__ CSplitArgs& desc_of(const SplitArgs* d, int h) { return *(CSplitArgs*)(d + h); }

// Hop of logical block `lb` in a batched launch: the hops' block ranges are consecutive.
__device__ __forceinline__ int batch_hop(const BatchTab& bt, int64_t lb) {
  int h = 0;
  while (h + 1 < bt.n && lb >= bt.start[h + 1]) ++h;
  return h;
}

// Logical tile of hardware block `b` in a batched launch, or -1 for a padding block.  The hops'
// block ranges follow one another in dispatch order, each starting at a multiple of the XCD
// count, and the XCD remap runs inside each hop: every hop is spread over all XCDs (hops of
// unequal cost per tile would otherwise leave whole XCDs idle at the end of the launch), and a
// hop's tiles that share operands stay on one XCD, as in a launch of that hop alone.
template <typename P>
__device__ __forceinline__ int64_t batch_tile(P& p, const BatchTab& bt, int h, int64_t b) {
  const int64_t n = bt.start[h + 1] - bt.start[h];
  const int64_t lb = xcd_remap(b - bt.start[h], n);
  const int64_t real = (int64_t)p.nct * ((p.S + kScoreTile - 1) / kScoreTile) * p.n_grp * 2;
  return lb < real ? lb : -1;
}

// Several independent hops of one base rank (16 or 32; ragged pools) in one grid; descriptors in
// device memory.  Hops of the other rank go to a grid of their own, so each instance keeps the
// single-hop kernel's register allocation.
template <int HD, int RK>
__global__ void __launch_bounds__(kScoreThreads, 2) split_score_batch(const SplitArgs* __restrict__ d, BatchTab bt) {
  extern __shared__ __attribute__((aligned(16))) char ring[];
  __shared__ ScoreShared sh;
  const int h = batch_hop(bt, blockIdx.x);
  CSplitArgs& p = desc_of(d, bt.hop[h]);
  const int64_t lb = batch_tile(p, bt, h, blockIdx.x);
  if (lb < 0) return;
  score_tile<HD, RK>(p, lb, ring, sh);
}

// ------------------------------------------------- first-mode scores at base ranks 64 and 128
// The contraction over an anchor's rank runs in ring steps of 64 ranks (two of the packed rank-32
// slices, NS / 2 steps per anchor, the slot 48 KiB); the reconstruction Z - sum_s A_s B_s of an
// anchor is complete only after its last step, so every wave keeps its result blocks live
// across the steps.  To fit them next to the source tile each wave covers 64 tokens x 64
// channels; a work-group of 8 waves (two token halves x four channel pairs, one work-group per
// CU) covers 128 tokens x 256 channels, so a step's A rows and B slices (six transfers per wave)
// feed 16 products per wave, and an anchor takes half the barriers of steps of 32 ranks.  A
// wave's two 32-channel blocks are the two halves of its rotary pairs (head_dim 128: blocks b
// and b + 2 of a head, head_dim 64: one head), so the keys' rotation to the canonical frame
// stays in registers.
constexpr int kSlTile = 128;                   // tokens per work-group
constexpr int kSlThreads = 512;                // 8 waves: 2 token halves x 4 channel pairs
constexpr int kSlPitch = 72;                   // staging row pitch (elements): 64 channels + 8

struct ScoreShared64 {
  float mp[2][4][kSlTile];                      // |E| sums of two anchors, per wave (64 channels)
  float qp[kSlThreads / 64][kMaxAnchors];       // per-wave gate sums
  float tab[2][kFusedHalf];                     // R(-p_src) table
};

// channel offset (within the 256-channel tile) of wave w's lower and upper 32-channel blocks
template <int HD> __device__ __forceinline__ int sl_block(int w) { return HD == 128 ? 4 * (w >> 1) + (w & 1) : 2 * w; }

// 64 tokens x the wave's two 32-channel blocks (channels c0 .. c0 + 31 and c1 .. c1 + 31 of the
// layer's rows), through wave-private staging, into accumulator layout (fp32); rows >= S read 0
__device__ __forceinline__ void load_tile2(f32x16 (&z)[2][2], rsrc_t zr, int t0, int D, int c0, int c1,
                                           uint16_t* stage, int lane, int col, int hi) {
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // 32 rows x 2 blocks x 64 bytes: 8 lanes per row
      const int row = i * 8 + (lane >> 3), u = lane & 7, ch = (u >> 2 ? c1 : c0) + (u & 3) * 8;
      v[i] = bload16<kStream>(zr, (uint32_t)((t0 + tb * 32 + row) * D + ch) * 2u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i * 8 + (lane >> 3), u = lane & 7;
      *reinterpret_cast<uint4*>(stage + row * kSlPitch + u * 8) = v[i];
    }
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const uint2 x = *reinterpret_cast<const uint2*>(stage + col * kSlPitch + db * 32 + 8 * jg + 4 * hi);
        z[tb][db][4 * jg + 0] = lo16(x.x);
        z[tb][db][4 * jg + 1] = hi16(x.x);
        z[tb][db][4 * jg + 2] = lo16(x.y);
        z[tb][db][4 * jg + 3] = hi16(x.y);
      }
  }
}

// keys: the pairs (block 0 row, block 1 row) turned by the table's angles; `pc` = pair index of
// the lower block's first row
__device__ __forceinline__ void rotate_tile2(f32x16 (&z)[2][2], const float* cs, const float* sn, int pc, int hi) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int c = pc + 8 * (j >> 2) + 4 * hi + (j & 3);
    const float cv = cs[c], sv = sn[c];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float ox, oy;
      rot_pair(z[tb][0][j], z[tb][1][j], cv, sv, ox, oy);
      z[tb][0][j] = ox;
      z[tb][1][j] = oy;
    }
  }
}

template <int HD, int NS, typename P>
__device__ __forceinline__ void score_tile_sliced(P& p, int64_t lb, char* ring, ScoreShared64& sh) {
  constexpr int kST = kSlTile, kNT = kSlThreads, kNW = kNT / 64, RS = 32 * NS;
  constexpr int NS2 = NS / 2;   // ring steps per anchor, two rank-32 slices each
  static_assert(NS % 2 == 0, "ranks 64 and 128: whole steps of 64");
  using RG = Ring<4, kST, kNW, false, 64, RS>;
  auto& mp = sh.mp;
  auto& qp = sh.qp;
  auto& tab = sh.tab;

  const TileId id = tile_id<true>(p, lb);
  const bool keys = id.side == 0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, hi = lane >> 5;
  const int D = p.D, S = p.S, N = p.N, NCB = D >> 5;
  const int t0 = id.tt * kST;
  const int tw = wave >> 2, wc = wave & 3, tw0 = t0 + tw * 64;
  const int blk0 = sl_block<HD>(wc), blk1 = blk0 + HD / 64;
  const int c0 = id.cq * kSW + blk0 * 32, c1 = id.cq * kSW + blk1 * 32;

  const auto list = keys ? p.corr : p.use;
  int nl = keys ? p.n_corr : p.n_use;
  const int s_work = keys ? (p.n_corr ? p.s_cov : 0) : max(p.n_corr ? p.s_cov : 0, p.mask_gate ? p.k_gate : 0);
  if (t0 >= s_work) nl = 0;
  const int steps = nl * NS2;

  for (int i = tid; i < HD / 2; i += kNT) {
    tab[0][i] = p.can.cs[i];
    tab[1][i] = p.can.sn[i];
  }
  const Slots sl = load_slots(list, keys ? p.n_corr : p.n_use, p.off, p.len, S, lane);

  const uint16_t* Al = p.Ab[id.side] + id.layer * p.ab_layer;
  // the packed base B holds each rank slice as a matrix of its own: index a NS + ks
  const uint16_t* Bl = p.Bb[id.side] + (((int64_t)id.layer * N * NS) * NCB + id.cq * kNCBW) * 2 * kC;
  const int64_t bstride = (int64_t)NCB * 2 * kC;
  const uint32_t ring0 = lds_off(ring);
  const int wv = uni(wave);
  auto fetch = [&](int j) {   // slices 2 (j % NS2) and 2 (j % NS2) + 1 of scored anchor j / NS2 into slot j % 3
    const bool live = j < steps;
    const int js = live ? j / NS2 : 0, ks = live ? j % NS2 : 0;
    const int a = lane_get(sl.a, js);
    const int lim = live ? lane_get(sl.lim, js) : 0;
    const int a_elems = lim * RS - ks * 64;   // the step's rows end where the stored rows do
    const uint32_t slot = ring0 + (uint32_t)(j % kSlots) * RG::SLOT;
    const rsrc_t Ar = make_rsrc(Al + (int64_t)lane_get(sl.off, js) * RS + ks * 64, (uint32_t)(live ? a_elems : 0) * 2);
#pragma unroll
    for (int i = 0; i < RG::A_PER_WAVE; ++i) {
      const int u = (wv * RG::A_PER_WAVE + i) * 64 + lane;
      const int row = u / RG::U, cpos = u % RG::U;
      const int c = cpos ^ ((row / (16 / RG::U)) & (RG::U - 1));
      dma16(Ar, slot + (wv * RG::A_PER_WAVE + i) * 1024, (uint32_t)(((t0 + row) * RS + c * 8) * 2));
    }
    // the two slices' packed matrices (each [block][k16] 1 KiB chunks) interleaved into the
    // slot's [block][k16 of the step] order
    const rsrc_t Br = make_rsrc(Bl + (a * NS + 2 * ks) * bstride, live ? (uint32_t)(2 * bstride * 2) : 0u);
#pragma unroll
    for (int i = 0; i < RG::B_PER_WAVE; ++i) {
      const int kc = wv * RG::B_PER_WAVE + i, db = kc >> 2, kk = kc & 3;
      dma16(Br, slot + RG::A_BYTES + kc * 1024,
            (uint32_t)((((kk >> 1) * bstride + (db * 2 + (kk & 1)) * kC)) * 2 + lane * 16));
    }
  };
  uint32_t aoff[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) aoff[tb][ks] = RG::a_unit(tw * 64 + tb * 32 + col, ks * 2 + hi) * 16;
  const uint32_t boff0 = RG::A_BYTES + blk0 * 4 * 1024 + lane * 16, boff1 = RG::A_BYTES + blk1 * 4 * 1024 + lane * 16;

  const float qm0 = (tw0 + col < p.k_gate && tw0 + col < S) ? 1.f : 0.f;
  const float qm1 = (tw0 + 32 + col < p.k_gate && tw0 + 32 + col < S) ? 1.f : 0.f;
  float* mpart = p.mpart + (((int64_t)id.cq * 2 + id.side) * p.n_layers + id.layer) * N * S;
  auto store_m = [&](int ja) {   // partial |E| sums of anchor ja over the tile's 256 channels
    const int a = lane_get(sl.a, ja);
    if (((p.mask_corr >> a) & 1) && tid < kST) {
      const int t = t0 + tid, b = ja & 1;
      if (t < S) mpart[(int64_t)a * S + t] = (mp[b][0][tid] + mp[b][1][tid]) + (mp[b][2][tid] + mp[b][3][tid]);
    }
  };

  auto run = [&](const f32x16 (&z)[2][2], auto values) {
    constexpr bool Q = decltype(values)::value;
#pragma nounroll
    for (int ja = 0; ja < nl; ++ja) {
      f32x16 e[2][2];
#pragma unroll
      for (int ks = 0; ks < NS2; ++ks) {
        const int j = ja * NS2 + ks;
        wait_vm_barrier<RG::DMA_PER_WAVE>();   // step j landed for every wave; slot (j + 2) % 3 is free
        const uint32_t slot = (uint32_t)uni((int)(ring0 + (uint32_t)(j % kSlots) * RG::SLOT));
        // the step's fragments first: their reads are in flight while the transfers issue
        bf16x8 av[2][4], bv[2][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) av[tb][kk] = as_bf8(lds_u4(slot + aoff[tb][kk]));
          bv[0][kk] = as_bf8(lds_u4(slot + boff0 + kk * 1024));
          bv[1][kk] = as_bf8(lds_u4(slot + boff1 + kk * 1024));
        }
        fetch(j + 2);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            f32x16 acc = ks == 0 ? z[tb][db] : e[tb][db];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma(bv[db][kk], av[tb][kk], acc);
            e[tb][db] = acc;
          }
      }
      // E = Z_can - A B complete: |E| per token column, E^2 for the gate
      float m0 = 0.f, m1 = 0.f, q0 = 0.f, q1 = 0.f;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          m0 += fabsf(e[0][db][jj]);
          m1 += fabsf(e[1][db][jj]);
          if (Q) {
            q0 = fmaf(e[0][db][jj], e[0][db][jj], q0);
            q1 = fmaf(e[1][db][jj], e[1][db][jj], q1);
          }
        }
      const int a = lane_get(sl.a, ja);
      if ((p.mask_corr >> a) & 1) {
        m0 = xor32_sum(m0);
        m1 = xor32_sum(m1);
        if (hi == 0) {
          mp[ja & 1][wc][tw * 64 + col] = m0;
          mp[ja & 1][wc][tw * 64 + 32 + col] = m1;
        }
      }
      if (Q && ((p.mask_gate >> a) & 1)) {
        float qs = fmaf(q0, qm0, q1 * qm1);
        qs = wave_sum63(qs);
        if (lane == 63) qp[wave][a] = qs;
      }
      // anchor ja - 1's sums (written by every wave before this anchor's first barrier; this
      // anchor wrote the other buffer, and the next anchor's first barrier orders this read
      // before that buffer is written again)
      if (ja > 0) store_m(ja - 1);
    }
  };
  __syncthreads();   // rotation table
  if (nl > 0) {
    f32x16 z[2][2];
    fetch(0);
    // staging (wave-private) in the ring past slot 0, free until step 1 is fetched
    load_tile2(z, make_rsrc(p.z[id.side] + (int64_t)id.layer * S * D, (uint32_t)S * D * 2), tw0, D, c0, c1,
               reinterpret_cast<uint16_t*>(ring + RG::SLOT) + wave * 32 * kSlPitch, lane, col, hi);
    if (keys && p.can.active) rotate_tile2(z, tab[0], tab[1], (blk0 * 32) % HD, hi);
    wait_vm_barrier<63>();   // every wave is done with the staging area
    fetch(1);
    if (keys)
      run(z, std::false_type{});
    else
      run(z, std::true_type{});
  }
  wait_vm_barrier<0>();
  if (nl > 0) store_m(nl - 1);
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

template <int HD, int NS>
__global__ void __launch_bounds__(kSlThreads, 1) split_score_sliced(SplitArgs p) {
  extern __shared__ __attribute__((aligned(16))) char ring[];
  __shared__ ScoreShared64 sh;
  score_tile_sliced<HD, NS>(p, xcd_remap(blockIdx.x, gridDim.x), ring, sh);
}

// ================================================================== token weights
// App. A.3 "Correction Weighting": per token and side, softmax over the correction set of
// -m / T_w (first mode, m = mean |Z_can - A B| from the per-channel-tile partials) or of
// cosine / T_w (second mode), or the caller's weights as given; 0 past S_cov.  Written
// anchor-major (w[side][layer][a][t], the apply kernel's operand order) and, if requested,
// token-major for the caller (w_out[side][layer][t][a], 0 outside the correction set).
template <typename P>
__device__ __forceinline__ void weights_rows(P& p, int wmode, int bx, int by, int side, float* xs) {
  const int tid = threadIdx.x;
  const int t = bx * 256 + tid;
  const int layer = p.layer0 + by;
  const int S = p.S, N = p.N, L = p.n_layers, nc = p.n_corr;
  const bool in = t < S, cov = t < p.s_cov;
  float mx = -INFINITY;
  // four anchors at a time, every load issued before the values are used (the channel-tile
  // partials are still summed in ascending order)
  const int64_t plane = (int64_t)2 * L * N * S;
  const float* mp0 = p.mpart + (((int64_t)side * L + layer) * N) * S + t;
  const float* wi = wmode == SPLIT_W_PARTIALS ? nullptr : p.w_in[side] + ((int64_t)layer * S + t) * N;
  for (int j0 = 0; j0 < nc; j0 += 4) {
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    if (cov) {
      if (wmode == SPLIT_W_PARTIALS) {
#pragma unroll 4
        for (int q = 0; q < p.nct; ++q) {
          float v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = j0 + u < nc ? mp0[q * plane + (int64_t)p.corr[j0 + u] * S] : 0.f;
#pragma unroll
          for (int u = 0; u < 4; ++u) x[u] += v[u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = -(x[u] * p.inv_d) * p.inv_temp;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = j0 + u < nc ? wi[p.corr[j0 + u]] : 0.f;
        if (wmode == SPLIT_W_SCORES) {
#pragma unroll
          for (int u = 0; u < 4; ++u) x[u] *= p.inv_temp;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (j0 + u >= nc) break;
      xs[(j0 + u) * 256 + tid] = x[u];
      mx = fmaxf(mx, x[u]);
    }
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

__global__ void __launch_bounds__(256) split_weights(SplitArgs p, int wmode) {
  extern __shared__ float xs[];   // [n_corr][256]
  weights_rows(p, wmode, blockIdx.x, blockIdx.y, blockIdx.z, xs);
}

// batched: blockIdx.z = 2 hop + side; every hop's weights come from its distance partials
__global__ void __launch_bounds__(256) split_weights_batch(const SplitArgs* __restrict__ d) {
  extern __shared__ float xs[];
  CSplitArgs& p = desc_of(d, blockIdx.z >> 1);
  if ((int)blockIdx.x * 256 >= p.S || p.n_corr < 1) return;
  weights_rows(p, SPLIT_W_PARTIALS, blockIdx.x, blockIdx.y, blockIdx.z & 1, xs);
}

// ================================================================== pass 2: apply
// Sec. 3.3 Eq. 8 / App. A.3 Eq. 12: out = R(s) Z + sum_a w_a A_a B'_a, the token weights read
// anchor-major (split_weights) and folded into the A fragments after they leave LDS.
// Three work-groups share a CU (at most 168 VGPRs per lane, a two-slot ring of ~49 KB): the
// extra waves cover the tile's load and store phases and the operand waits, which pays more
// than a third slot or operands held in registers across a step.
// NS > 1: a delta of rank NS x RA runs as NS steps of rank RA per anchor (the contraction over
// the rank splits into column slices of A and row slices of B): step j takes slice j % NS of
// correction anchor j / NS, the same ring slot size as rank RA.  The packed B operand then holds
// each slice as its own matrix (rows RA k .. RA k + RA - 1 of anchor a at index a NS + k).
template <int HD, int RKD, int RA, int NS = 1, typename P>
__device__ __forceinline__ void apply_tile(P& p, int64_t lb, char* ring, float (*tab)[kFusedHalf]) {
  constexpr int kST = kApplyTile, kNT = kApplyThreads, kNW = kNT / 64;
  constexpr int RS = RA * NS;   // stored rank of the A rows
  using RG = Ring<RKD, kST, kNW, true, RA, RS>;

  const TileId id = tile_id<true>(p, lb);
  const bool keys = id.side == 0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, hi = lane >> 5;
  const int tw = wave >> 1, cw = wave & 1;
  const int D = p.D, S = p.S, N = p.N, NCB = D >> 5;
  const int t0 = id.tt * kST, tw0 = t0 + tw * 64;
  const int d0 = id.cq * kSW + cw * 128;

  for (int i = tid; i < HD / 2; i += kNT) {
    tab[0][i] = p.shift.cs[i];
    tab[1][i] = p.shift.sn[i];
  }
  const int nc = (t0 < p.s_cov) ? p.n_corr * NS : 0;   // steps
  Slots sl;   // loaded after the tile's rotation (below), so it holds no registers through it
  const uint16_t* Al = p.Ad[id.side] + id.layer * p.ad_layer;
  const uint16_t* Bl = p.Bd[id.side] + (((int64_t)id.layer * N * NS) * NCB + id.cq * kNCBW) * RKD * kC;
  const float* Wl = p.wa + ((int64_t)id.side * p.n_layers + id.layer) * N * S;
  const int64_t bstride = (int64_t)NCB * RKD * kC;
  // zero-size descriptors past the correction set (see split_score)
  const uint32_t ring0 = lds_off(ring);
  const int wv = uni(wave);
  auto fetch = [&](int j) {
    const bool live = j < nc;
    const int js = live ? j / NS : 0, ks = live ? j % NS : 0;   // anchor, rank slice
    const int a = lane_get(sl.a, js);
    const int lim = live ? lane_get(sl.lim, js) : 0;
    // the slice's rows end RA (NS - 1 - ks) elements before the stored rows do (a live anchor
    // has lim >= 1 rows, so this is positive; past the list lim = ks = 0)
    const int a_elems = lim * RS - ks * RA;
    RG::fetch(ring0 + (uint32_t)(j % kApplySlots) * RG::SLOT,
              make_rsrc(Al + (int64_t)lane_get(sl.off, js) * RS + ks * RA, (uint32_t)a_elems * 2),
              make_rsrc(Bl + (a * NS + ks) * bstride, live ? RG::B_BYTES : 0),
              make_rsrc(Wl + (int64_t)a * S, (uint32_t)lim * 4), t0, wv, lane);
  };
  // A fragment offsets: the second token block's rows lie 32 rows further with the same
  // swizzle (the swizzle depends on the row through row / (16 / U) mod U, and 32 rows are a
  // multiple of 16 / U x U), so they are an immediate offset from the first block's and take
  // no registers of their own
  uint32_t aoff[2][RKD];
#pragma unroll
  for (int ks = 0; ks < RKD; ++ks) {
    aoff[0][ks] = RG::a_unit(tw * 64 + col, ks * 2 + hi) * 16;
    aoff[1][ks] = aoff[0][ks] + 32 * RG::U * 16;
  }
  const uint32_t boff = RG::A_BYTES + cw * 4 * RKD * 1024 + lane * 16;
  const uint32_t woff = RG::A_BYTES + RG::B_BYTES + (tw * 64 + col) * 4;
  uint16_t* stage = reinterpret_cast<uint16_t*>(ring) + wave * kStage;   // over the ring, before anchor 0

  __syncthreads();   // rotation table
  // ---- residual: R(s) K or V
  f32x16 acc[2][4];
  const uint32_t layer_bytes = (uint32_t)S * D * 2;
  load_tile(acc, make_rsrc(p.z[id.side] + (int64_t)id.layer * S * D, layer_bytes), tw0, D, d0, stage, lane, col, hi);
  if (keys && p.shift.active) rotate_tile<HD>(acc, tab[0], tab[1], hi);
  {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    sl = load_slots(p.corr, p.n_corr, p.off, p.len, min(S, p.s_cov), ln);
  }
  if (nc > 0) {
    wait_vm_barrier<63>();   // every wave is done with the staging area
    fetch(0);
  }
#pragma nounroll
  for (int j = 0; j < nc; ++j) {
    // anchor j landed for every wave, and every wave is past step j - 1, the last reader of
    // the other slot, which now takes anchor j + 1
    wait_vm_barrier<0>();
    fetch(j + 1);
    const uint32_t slot = (uint32_t)uni((int)(ring0 + (uint32_t)(j % kApplySlots) * RG::SLOT));   // opaque base
    const float w0 = lds_f(slot + woff), w1 = lds_f(slot + woff + 128);
#pragma unroll
    for (int ks = 0; ks < RKD; ++ks) {
      const bf16x8 a0 = as_bf8(scale8(lds_u4(slot + aoff[0][ks]), w0));
      const bf16x8 a1 = as_bf8(scale8(lds_u4(slot + aoff[1][ks]), w1));
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 b = as_bf8(lds_u4(slot + boff + (db * RKD + ks) * 1024));
        acc[0][db] = mfma(b, a0, acc[0][db]);
        acc[1][db] = mfma(b, a1, acc[1][db]);
      }
    }
  }
  wait_vm_barrier<0>();   // trailing (empty) transfers drained, every wave past its last reads
  store_tile(acc, make_rsrc(p.out[id.side] + (int64_t)id.layer * S * D, layer_bytes), tw0, D, d0, stage, lane, col, hi);
}

template <int HD, int RKD, int RA, int NS = 1>
__global__ void __launch_bounds__(kApplyThreads, 3) split_apply(SplitArgs p) {
  extern __shared__ __attribute__((aligned(16))) char ring[];   // kApplySlots x slot | staging
  __shared__ float tab[2][kFusedHalf];
  apply_tile<HD, RKD, RA, NS>(p, xcd_remap(blockIdx.x, gridDim.x), ring, tab);
}

// Several independent hops of one delta rank in one grid (descriptors in device memory); hops
// of other ranks go to grids of their own, so every instance keeps the single-hop kernel's
// register allocation.
template <int HD, int RKD, int RA, int NS>
__global__ void __launch_bounds__(kApplyThreads, 3) split_apply_batch(const SplitArgs* __restrict__ d, BatchTab bt) {
  extern __shared__ __attribute__((aligned(16))) char ring[];
  __shared__ float tab[2][kFusedHalf];
  const int h = batch_hop(bt, blockIdx.x);
  CSplitArgs& p = desc_of(d, bt.hop[h]);
  const int64_t b = batch_tile(p, bt, h, blockIdx.x);
  if (b < 0) return;
  apply_tile<HD, RKD, RA, NS>(p, b, ring, tab);
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
  const int64_t nblk = (int64_t)a.nct * a.ntt * a.n_grp * 2;
  kernel<<<dim3((unsigned)nblk), dim3(threads), shmem, st>>>(a);
  return hipGetLastError();
}

template <int HD>
hipError_t score_dispatch(const SplitArgs& a, hipStream_t st) {
  switch (a.r_b) {
    case 16: return go(split_score<HD, 1>, a, kScoreTile, kScoreThreads, split_score_lds(a.r_b), st);
    case 32: return go(split_score<HD, 2>, a, kScoreTile, kScoreThreads, split_score_lds(a.r_b), st);
    case 64: return go(split_score_sliced<HD, 2>, a, kSlTile, kSlThreads, split_score_lds(a.r_b), st);
    case 128: return go(split_score_sliced<HD, 4>, a, kSlTile, kSlThreads, split_score_lds(a.r_b), st);
    default: return hipErrorInvalidValue;
  }
}

template <int HD>
hipError_t apply_dispatch(const SplitArgs& a, hipStream_t st) {
  const size_t lds = split_apply_lds(a.r_d);
  switch (a.r_d) {
    case 8: return go(split_apply<HD, 1, 8>, a, kApplyTile, kApplyThreads, lds, st);
    case 16: return go(split_apply<HD, 1, 16>, a, kApplyTile, kApplyThreads, lds, st);
    case 32: return go(split_apply<HD, 2, 32>, a, kApplyTile, kApplyThreads, lds, st);
    case 64: return go(split_apply<HD, 2, 32, 2>, a, kApplyTile, kApplyThreads, lds, st);
    case 128: return go(split_apply<HD, 2, 32, 4>, a, kApplyTile, kApplyThreads, lds, st);
    case 256: return go(split_apply<HD, 2, 32, 8>, a, kApplyTile, kApplyThreads, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// dynamic LDS: the operand ring, or the waves' staging areas (scoring: past slot 0, which is
// filled during the tile load; apply: from the start, before anchor 0 is fetched), whichever
// is larger
size_t split_score_lds(int r_b) {
  if (r_b == 64 || r_b == 128) {   // steps of 64 ranks, 8 waves' staging
    const size_t slot = (size_t)kSlTile * 64 * 2 + (size_t)kNCBW * 4 * 1024;
    return std::max((size_t)kSlots * slot, slot + sizeof(uint16_t) * (kSlThreads / 64) * 32 * kSlPitch);
  }
  const size_t slot = (size_t)kScoreTile * r_b * 2 + (size_t)kNCBW * (r_b / 16) * 1024;
  return std::max((size_t)kSlots * slot, slot + sizeof(uint16_t) * (kScoreThreads / 64) * kStage);
}

int split_score_tile(int r_b) { return r_b == 64 || r_b == 128 ? kSlTile : kScoreTile; }

size_t split_apply_lds(int r_d) {
  const int rp = split_apply_slices(r_d) > 1 ? 32 : (r_d + 15) & ~15;   // on chip: padded to 16, or slices of 32
  const size_t slot = (size_t)kApplyTile * rp * 2 + (size_t)kNCBW * (rp / 16) * 1024 + (size_t)kApplyTile * 4;
  return std::max((size_t)kApplySlots * slot, sizeof(uint16_t) * (kApplyThreads / 64) * kStage);
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

namespace {
// block ranges of the hops of a batched two-pass launch (128-token x 256-channel tiles, both sides)
// grid of the hops idx[0..m) of h (128-token x 256-channel tiles, both sides)
bool batch_tab(BatchTab& bt, const SplitArgs* h, const int* idx, int m, int64_t& total) {
  if (m < 1 || m > kMaxBatch) return false;
  bt.n = m;
  total = 0;
  for (int i = 0; i < m; ++i) {
    const SplitArgs& a = h[idx[i]];
    bt.start[i] = (int32_t)total;
    bt.hop[i] = idx[i];
    const int64_t ntt = (a.S + kScoreTile - 1) / kScoreTile;
    const int64_t blocks = (int64_t)a.nct * ntt * a.n_grp * 2;
    total += (blocks + 7) / 8 * 8;   // each hop starts on XCD 0 (blocks are dealt round-robin over 8)
    if (a.D % kSW || a.N > kMaxAnchors) return false;
  }
  bt.start[m] = (int32_t)total;
  return total < (1ll << 31);
}

template <int HD>
hipError_t apply_batch_dispatch(int r, const SplitArgs* d, const BatchTab& bt, int64_t total, size_t lds,
                                hipStream_t st);

template <typename K>
hipError_t go_batch(K kernel, const SplitArgs* d, const BatchTab& bt, int64_t total, size_t shmem, hipStream_t st) {
  if (shmem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  kernel<<<dim3((unsigned)total), dim3(kScoreThreads), shmem, st>>>(d, bt);
  return hipGetLastError();
}
}  // namespace

// one grid per distinct base rank among the hops, in order of first appearance
hipError_t launch_split_score_batch(const SplitArgs* d, const SplitArgs* h, int n, int head_dim, hipStream_t st) {
  static_assert(kScoreThreads == kApplyThreads && kScoreTile == kApplyTile, "one tile grid for both passes");
  if (n < 1 || n > kMaxBatch || (head_dim != 128 && head_dim != 64)) return hipErrorInvalidValue;
  for (int i = 0; i < n; ++i)
    if (h[i].r_b != 16 && h[i].r_b != 32) return hipErrorInvalidValue;
  bool done[kMaxBatch] = {};
  for (int i = 0; i < n; ++i) {
    if (done[i]) continue;
    int idx[kMaxBatch], m = 0;
    for (int j = i; j < n; ++j)
      if (!done[j] && h[j].r_b == h[i].r_b) {
        idx[m++] = j;
        done[j] = true;
      }
    BatchTab bt;
    int64_t total;
    if (!batch_tab(bt, h, idx, m, total)) return hipErrorInvalidValue;
    if (total == 0) continue;
    const size_t lds = split_score_lds(h[i].r_b);
    hipError_t e;
    if (head_dim == 128)
      e = h[i].r_b == 16 ? go_batch(split_score_batch<128, 1>, d, bt, total, lds, st)
                         : go_batch(split_score_batch<128, 2>, d, bt, total, lds, st);
    else
      e = h[i].r_b == 16 ? go_batch(split_score_batch<64, 1>, d, bt, total, lds, st)
                         : go_batch(split_score_batch<64, 2>, d, bt, total, lds, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

namespace {
template <int HD>
hipError_t apply_batch_dispatch(int r, const SplitArgs* d, const BatchTab& bt, int64_t total, size_t lds,
                                hipStream_t st) {
  switch (r) {
    case 8: return go_batch(split_apply_batch<HD, 1, 8, 1>, d, bt, total, lds, st);
    case 16: return go_batch(split_apply_batch<HD, 1, 16, 1>, d, bt, total, lds, st);
    case 32: return go_batch(split_apply_batch<HD, 2, 32, 1>, d, bt, total, lds, st);
    case 64: return go_batch(split_apply_batch<HD, 2, 32, 2>, d, bt, total, lds, st);
    case 128: return go_batch(split_apply_batch<HD, 2, 32, 4>, d, bt, total, lds, st);
    case 256: return go_batch(split_apply_batch<HD, 2, 32, 8>, d, bt, total, lds, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

// one grid per distinct delta rank among the hops, in order of first appearance
hipError_t launch_split_apply_batch(const SplitArgs* d, const SplitArgs* h, int n, int head_dim, hipStream_t st) {
  if (n < 1 || n > kMaxBatch || (head_dim != 128 && head_dim != 64)) return hipErrorInvalidValue;
  for (int i = 0; i < n; ++i) {
    const int r = h[i].r_d;
    if ((r != 8 && r != 16 && r != 32 && split_apply_slices(r) == 1) || !h[i].wa) return hipErrorInvalidValue;
  }
  bool done[kMaxBatch] = {};
  for (int i = 0; i < n; ++i) {
    if (done[i]) continue;
    int idx[kMaxBatch], m = 0;
    for (int j = i; j < n; ++j)
      if (!done[j] && h[j].r_d == h[i].r_d) {
        idx[m++] = j;
        done[j] = true;
      }
    BatchTab bt;
    int64_t total;
    if (!batch_tab(bt, h, idx, m, total)) return hipErrorInvalidValue;
    if (total == 0) continue;
    const size_t lds = split_apply_lds(h[i].r_d);
    const hipError_t e = head_dim == 128 ? apply_batch_dispatch<128>(h[i].r_d, d, bt, total, lds, st)
                                         : apply_batch_dispatch<64>(h[i].r_d, d, bt, total, lds, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_split_weights_batch(const SplitArgs* d, const SplitArgs* h, int n, hipStream_t st) {
  if (n < 1 || n > kMaxBatch) return hipErrorInvalidValue;
  int nc = 1;
  for (int i = 0; i < n; ++i) {
    if (h[i].N > kMaxAnchors || !h[i].wa || h[i].S != h[0].S || h[i].n_grp != h[0].n_grp) return hipErrorInvalidValue;
    nc = std::max(nc, h[i].n_corr);
  }
  const dim3 grid((unsigned)((h[0].S + 255) / 256), (unsigned)h[0].n_grp, 2u * n);
  split_weights_batch<<<grid, 256, sizeof(float) * 256 * (size_t)nc, st>>>(d);
  return hipGetLastError();
}

hipError_t launch_split_weights(const SplitArgs& a, int wmode, hipStream_t st) {
  if (a.N > kMaxAnchors || !a.wa || a.n_corr < 1) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.S + 255) / 256), (unsigned)a.n_grp, 2);
  split_weights<<<grid, 256, sizeof(float) * 256 * (size_t)a.n_corr, st>>>(a, wmode);
  return hipGetLastError();
}

}  // namespace kvc
