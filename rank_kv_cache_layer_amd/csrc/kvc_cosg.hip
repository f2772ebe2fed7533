// Second scoring mode as one bf16 GEMM per (layer, side) for gfx950 (CDNA4): the projection
// of the canonical source on every scored anchor's basis, P = Z_can B^T (the Eq. 7 factor B
// of KVCMAS, arXiv 2609.34060, Sec. 3.3), with tokens as one GEMM dimension, (anchor, rank)
// as the other and the channels as the contraction; then, per token and anchor, the cosine of
// P with the anchor coordinates A, and over the prefix k the value-side sums of the segment
// cosine that the gate reads (App. A.3 "Reliability Gate", second mode).
//
// The key re-alignment to the canonical frame is folded into the packed operand: with
// Z_can = R Z (R = R(-p_src), rotate-half pairs), P = Z_can B^T = Z (R^T B)^T, so the kernel
// contracts the stored keys with B' = R^T B, each row of B turned by +p_src.  Values use B as
// stored.
//
// Work-group: 128 tokens x all scored anchors (passes of 20) of one (layer, side), 8 waves.
// Wave (tw, ag) owns tokens [64 tw, 64 tw + 64) and anchors [5 ag, 5 ag + 5) of the pass, i.e.
// a 64 x 160 block of P in 160 accumulator registers.  The contraction runs over 32-channel
// chunks: each chunk's source rows (128 x 64 B) and packed B' rows (20 x 32 x 64 B) are copied
// from memory straight into a three-slot LDS ring by buffer->LDS transfers two chunks ahead.  At
// rank 32 the transfers past the last chunk carry the epilogue's A rows instead of nothing.
//
// MFMA: v_mfma_f32_32x32x16_bf16, operand A = 32 rank rows of B' x 16 channels, operand B =
// 32 tokens x 16 channels; result register j of lane l holds rank row 8 (j / 4) + 4 (l / 32)
// + j % 4 and token l % 32, so the cosine's sums over the rank stay in the lane (plus one
// exchange with lane l ^ 32).
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kTok = kCosGemmTile;   // tokens per work-group
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kAnch = 5;             // anchors per wave and pass
constexpr int kPass = 4 * kAnch;     // anchors per pass (four anchor groups)
constexpr int kKc = 32;              // channels per chunk
constexpr int kRowB = kKc * 2;       // bytes per LDS row (token or rank row of one chunk)
constexpr int kZBytes = kTok * kRowB;                 // 8 KiB
constexpr int kBBytes = kPass * 32 * kRowB;           // 40 KiB
constexpr int kSlot = kZBytes + kBBytes;              // 48 KiB
constexpr int kRing = 3;
constexpr int kZDma = kZBytes / 1024 / kWaves;        // 1 transfer per wave
constexpr int kBDma = kBBytes / 1024 / kWaves;        // 5 transfers per wave
constexpr int kDmaPerWave = kZDma + kBDma;
static_assert(kZBytes % (1024 * kWaves) == 0 && kBBytes % (1024 * kWaves) == 0, "ring split");

constexpr int kRsrcWord3 = 0x00020000;   // raw 32-bit data, gfx9 family
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// 16-byte unit of row `row`, logical unit c (0..3) of a 64-byte LDS row: units XOR-swizzled by
// row / 4, so the fragment reads of 16 consecutive rows (same logical unit) hit distinct banks.
__device__ __forceinline__ int unit_of(int row, int c) { return row * 4 + (c ^ ((row >> 2) & 3)); }

// buffer->LDS transfer of 16 bytes per lane to LDS M0 + 16 * lane (lanes past the descriptor's
// size write zeros).  Inline assembly so the compiler neither reorders LDS accesses around it
// nor waits for every transfer in flight before later LDS reads; the ring's explicit waits
// order each slot.  M0 is written only here.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t lds_addr, uint32_t voff) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)lds_addr);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory");
}

// s_waitcnt vmcnt <= N, lgkmcnt = 0 (gfx9 encoding), then the work-group barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
}

typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_char*)p);
}
__device__ __forceinline__ bf16x8 lds_frag(uint32_t off) {
  const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((uintptr_t)off);
  return __builtin_bit_cast(bf16x8, v);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 lds_u2(uint32_t off) {
  const u32x2 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>((uintptr_t)off);
  return make_uint2(v.x, v.y);
}
// s_waitcnt vmcnt <= N only
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// --------------------------------------------------------------------- operand packing
// B' rows of the scored anchors, in scoring order u, chunked by 32 channels:
// dst[side][layer][chunk][u][k][32] bf16 (each row 64 contiguous bytes).  Key rows are turned
// by the transpose of the canonical rotation (cs, sn of R(-p_src)): b'_c = b_c cs + b_{c+h} sn,
// b'_{c+h} = b_{c+h} cs - b_c sn.  One thread per (side, layer, u, k) row and 8 rotary pairs:
// 16-byte loads of the 8 lower and the 8 upper channels, 16-byte stores of each.
__global__ void __launch_bounds__(256) pack_cos(CosGemmArgs p, uint16_t* __restrict__ dst) {
  const int D = p.D, h = p.head_dim / 2, r = p.r;
  const int per_row = D / 16;   // groups of 8 pairs
  const int64_t rows = (int64_t)2 * p.n_layers * p.n_use * r;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * per_row) return;
  const int g = (int)(i % per_row);
  int64_t row = i / per_row;
  const int k = (int)(row % r);
  row /= r;
  const int u = (int)(row % p.n_use);
  row /= p.n_use;
  const int layer = (int)(row % p.n_layers);
  const int side = (int)(row / p.n_layers);
  const int gph = h / 8;                            // groups per head
  const int head = g / gph, c0 = (g % gph) * 8;
  const int dl = head * p.head_dim + c0, du = dl + h;
  const int a = p.use[u];
  const uint16_t* b = p.B[side] + (int64_t)layer * p.b_layer_stride + ((int64_t)a * r + k) * D;
  uint4 xv = *reinterpret_cast<const uint4*>(b + dl), yv = *reinterpret_cast<const uint4*>(b + du);
  if (side == 0 && p.can.active) {
    uint32_t* xw = &xv.x;
    uint32_t* yw = &yv.x;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float x[2] = {__uint_as_float(xw[w] << 16), __uint_as_float(xw[w] & 0xffff0000u)};
      float y[2] = {__uint_as_float(yw[w] << 16), __uint_as_float(yw[w] & 0xffff0000u)};
      uint16_t ox[2], oy[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float cs = p.can.cs[c0 + 2 * w + e], sn = p.can.sn[c0 + 2 * w + e];
        ox[e] = f2bf(fmaf(x[e], cs, y[e] * sn));
        oy[e] = f2bf(fmaf(y[e], cs, -(x[e] * sn)));
      }
      xw[w] = (uint32_t)ox[0] | ((uint32_t)ox[1] << 16);
      yw[w] = (uint32_t)oy[0] | ((uint32_t)oy[1] << 16);
    }
  }
  const int nkc = D / kKc;
  uint16_t* o = dst + ((((int64_t)side * p.n_layers + layer) * nkc) * p.n_use) * r * kKc;
  *reinterpret_cast<uint4*>(o + (((int64_t)(dl / kKc) * p.n_use + u) * r + k) * kKc + dl % kKc) = xv;
  *reinterpret_cast<uint4*>(o + (((int64_t)(du / kKc) * p.n_use + u) * r + k) * kKc + du % kKc) = yv;
}

// Cosines at rank 32 NS from slice sums (NS > 1).  Each wave forms, per token of its 64 and per
// column group of its five, the slice's sums <P, A>, |P|^2, |A|^2 and stores them in LDS
// (red[tw][group][3][64], 30 KiB over the ring, free once every transfer has drained); after a
// barrier, wave (tw, ag) finishes anchors ag, ag + 4, ... of the pass for its 64 tokens: the
// sums over the slices, the cosine, and the value-side gate sums of its 64-token tile.  Ends
// with a barrier, so the next pass may refill the ring.
template <int NS>
__device__ __forceinline__ void slice_cosines(const CosGemmArgs& p, const f32x16 (&acc)[kAnch][2], float* red,
                                              int u0, int np, int side, int layer, int tt, int t0, int tw, int ag,
                                              int lane, int col, int hi) {
  constexpr int R = 32 * NS;
  const int S = p.S;
#pragma unroll
  for (int x = 0; x < kAnch; ++x) {
    const int qp = ag * kAnch + x;   // column group within the pass
    if (qp >= np) break;
    const int q = u0 + qp, a = p.use[q / NS], sl = q % NS;
    const int alen = p.len[a];
    const uint16_t* Aa = p.A[side] + layer * p.a_layer_stride + (int64_t)p.off[a] * R + sl * 32;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int t = t0 + tw * 64 + tb * 32 + col;
      const bool ok = t < alen && t < S;
      float num = 0.f, pp = 0.f, aa = 0.f;
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        uint2 av = make_uint2(0, 0);
        if (ok) av = *reinterpret_cast<const uint2*>(Aa + (int64_t)t * R + 8 * jg + 4 * hi);
        const float a4[4] = {__uint_as_float(av.x << 16), __uint_as_float(av.x & 0xffff0000u),
                             __uint_as_float(av.y << 16), __uint_as_float(av.y & 0xffff0000u)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = acc[x][tb][4 * jg + i];
          num = fmaf(pv, a4[i], num);
          pp = fmaf(pv, pv, pp);
          aa = fmaf(a4[i], a4[i], aa);
        }
      }
      num += __shfl_xor(num, 32);
      pp += __shfl_xor(pp, 32);
      aa += __shfl_xor(aa, 32);
      if (hi == 0) {
        float* o = red + ((tw * kPass + qp) * 3) * 64 + tb * 32 + col;
        o[0] = num;
        o[64] = pp;
        o[128] = aa;
      }
    }
  }
  __syncthreads();
  const int t = t0 + tw * 64 + lane;
  const int tile = tt * (kTok / kCosTile) + tw;
  for (int ap = ag; ap < np / NS; ap += 4) {
    const int a = p.use[u0 / NS + ap];
    float num = 0.f, pp = 0.f, aa = 0.f;
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const float* o = red + ((tw * kPass + ap * NS + sl) * 3) * 64 + lane;
      num += o[0];
      pp += o[64];
      aa += o[128];
    }
    const float den = sqrtf(pp) * sqrtf(aa);
    const float cval = den > 0.f ? num / den : 0.f;
    if (t < S && tile < p.n_tiles) p.scores[(((int64_t)side * p.n_layers + layer) * S + t) * p.N + a] = cval;
    if (side == 1 && ((p.mask_gate >> a) & 1) && tile < p.n_tiles) {
      const float qm = (t < p.len[a] && t < S && t < p.k_gate) ? 1.f : 0.f;
      float gnum = num * qm, gpp = pp * qm, gaa = aa * qm;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        gnum += __shfl_xor(gnum, o);
        gpp += __shfl_xor(gpp, o);
        gaa += __shfl_xor(gaa, o);
      }
      if (lane == 0) {
        const int64_t plane = (int64_t)p.n_layers * p.n_tiles * p.N;
        const int64_t o = ((int64_t)layer * p.n_tiles + tile) * p.N + a;
        p.partials[o] = gnum;
        p.partials[plane + o] = gpp;
        p.partials[2 * plane + o] = gaa;
      }
    }
  }
  __syncthreads();
}

// --------------------------------------------------------------------- the GEMM and cosines
// NS = rank / 32: GEMM column group q = u NS + s is slice s (rows 32 s .. 32 s + 31 of B',
// columns of A) of scored anchor u; the packed rows [u][r] are the same memory as [u NS + s][32].
// At NS > 1 the cosine's three sums are formed per slice, summed over the slices through LDS
// (the slices of one anchor sit in different waves), then finished per (token, anchor).
template <int NS>
__global__ void __launch_bounds__(kThreads, 1) score_cos_gemm(CosGemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char ring[];   // kRing x kSlot
  const int nwg = (p.n_tiles * kCosTile + kTok - 1) / kTok;   // token range of the scored tiles
  const int64_t lb = xcd_remap(blockIdx.x, gridDim.x);
  const int tt = (int)(lb % nwg);
  const int layer = (int)((lb / nwg) % p.n_layers);
  const int side = (int)(lb / ((int64_t)nwg * p.n_layers));
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, hi = lane >> 5;
  const int tw = wave >> 2, ag = wave & 3;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int D = p.D, S = p.S, nkc = D / kKc, r = 32;
  const int nq = p.n_use * NS;   // GEMM column groups of 32
  const int t0 = tt * kTok;
  const uint32_t ring0 = lds_off(ring);

  const uint16_t* zl = p.z[side] + (int64_t)layer * S * D;
  const rsrc_t zr = make_rsrc(zl, (uint32_t)S * D * 2);
  const uint16_t* bside = p.packed + (((int64_t)side * p.n_layers + layer) * nkc) * nq * r * kKc;

  // fragment offsets inside a slot: token rows (operand B) and rank rows (operand A)
  uint32_t zoff[2][2], boff[kAnch][2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int s = 0; s < 2; ++s) zoff[tb][s] = unit_of(tw * 64 + tb * 32 + col, s * 2 + hi) * 16;
#pragma unroll
  for (int x = 0; x < kAnch; ++x)
#pragma unroll
    for (int s = 0; s < 2; ++s) boff[x][s] = kZBytes + unit_of((ag * kAnch + x) * 32 + col, s * 2 + hi) * 16;

  static_assert(kPass % NS == 0, "a pass holds whole anchors");
  for (int u0 = 0; u0 < nq; u0 += kPass) {
    const int np = min(kPass, nq - u0);
    // chunk kc of this pass into slot kc % kRing; past the last chunk the descriptors have
    // size 0 (zeros written, nothing fetched), so every step issues the same transfers
    auto fetch = [&](int kc) {
      const bool live = kc < nkc;
      const uint32_t slot = ring0 + (uint32_t)(kc % kRing) * kSlot;
      const rsrc_t zs = live ? zr : make_rsrc(zl, 0);
#pragma unroll
      for (int i = 0; i < kZDma; ++i) {
        const int unit = (wv * kZDma + i) * 64 + lane;
        const int row = unit >> 2, c = (unit & 3) ^ ((row >> 2) & 3);
        dma16(zs, slot + (uint32_t)(wv * kZDma + i) * 1024,
              (uint32_t)(((int64_t)(t0 + row) * D + kc * kKc + c * 8) * 2));
      }
      const uint16_t* bc = bside + ((int64_t)(live ? kc : 0) * nq + u0) * r * kKc;
      const rsrc_t bs = make_rsrc(bc, live ? (uint32_t)np * r * kRowB : 0u);
#pragma unroll
      for (int i = 0; i < kBDma; ++i) {
        const int unit = (wv * kBDma + i) * 64 + lane;
        const int row = unit >> 2, c = (unit & 3) ^ ((row >> 2) & 3);
        dma16(bs, slot + kZBytes + (uint32_t)(wv * kBDma + i) * 1024, (uint32_t)(row * kRowB + c * 16));
      }
    };
    // transfer u (< kDmaPerWave, a compile-time constant after unrolling) of fetch(kc): the
    // steady state spreads a chunk's transfers over the previous chunk's products
    auto fetch_unit = [&](int kc, int u) {
      const bool live = kc < nkc;
      const uint32_t slot = ring0 + (uint32_t)(kc % kRing) * kSlot;
      if (u < kZDma) {
        const rsrc_t zs = live ? zr : make_rsrc(zl, 0);
        const int unit = (wv * kZDma + u) * 64 + lane;
        const int row = unit >> 2, c = (unit & 3) ^ ((row >> 2) & 3);
        dma16(zs, slot + (uint32_t)(wv * kZDma + u) * 1024,
              (uint32_t)(((int64_t)(t0 + row) * D + kc * kKc + c * 8) * 2));
      } else {
        const int i = u - kZDma;
        const uint16_t* bc = bside + ((int64_t)(live ? kc : 0) * nq + u0) * r * kKc;
        const rsrc_t bs = make_rsrc(bc, live ? (uint32_t)np * r * kRowB : 0u);
        const int unit = (wv * kBDma + i) * 64 + lane;
        const int row = unit >> 2, c = (unit & 3) ^ ((row >> 2) & 3);
        dma16(bs, slot + kZBytes + (uint32_t)(wv * kBDma + i) * 1024, (uint32_t)(row * kRowB + c * 16));
      }
    };

    // Rank 32: the epilogue's A rows (per wave, its 5 anchors x 64 tokens x 64 bytes, four 1 KiB
    // units per anchor, 16-byte units swizzled as the ring's) come into LDS through the ring's
    // transfers instead of global loads after the products: units 0-11 (anchors 0-2) take the
    // places of the empty transfers of the last two chunks (slots nkc % 3 and (nkc + 1) % 3, six
    // units per wave each), units 12-17 (anchor 3, half of anchor 4) the last chunk's slot once
    // every wave is past it, units 18-19 anchor 0's first two places once this wave has read
    // them.  Every unit is written and read by one wave only.
    auto a_place = [&](int i) -> uint32_t {
      int sl, pos;
      if (i < 12) { sl = (nkc + i / 6) % kRing; pos = i % 6; }
      else if (i < 18) { sl = (nkc + 2) % kRing; pos = i - 12; }
      else { sl = nkc % kRing; pos = i - 18; }
      return ring0 + (uint32_t)sl * kSlot + (uint32_t)(wv * 6 + pos) * 1024;
    };
    auto stage_a = [&](int i) {
      const int x = i >> 2, k = i & 3;
      const int u = u0 + __builtin_amdgcn_readfirstlane(ag) * kAnch + x;   // wave-uniform: the descriptor is scalar
      const bool un = u < p.n_use;
      const int a = un ? p.use[u] : 0;
      const int rows = un ? min(p.len[a], S) : 0;
      const rsrc_t ar = make_rsrc(p.A[side] + layer * p.a_layer_stride + (int64_t)p.off[a] * r, (uint32_t)rows * r * 2);
      const int row = 16 * k + (lane >> 2), c = (lane & 3) ^ ((row >> 2) & 3);
      dma16(ar, a_place(i), (uint32_t)(((t0 + tw * 64 + row) * r + c * 8) * 2));
    };
    static_assert(NS > 1 || kDmaPerWave == 6, "the last two chunks carry anchors 0-2 of the epilogue");

    f32x16 acc[kAnch][2];
#pragma unroll
    for (int x = 0; x < kAnch; ++x)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[x][tb][j] = 0.f;

    fetch(0);
    fetch(1);
#pragma nounroll
    for (int kc = 0; kc < nkc; ++kc) {
      wait_vm_barrier<kDmaPerWave>();   // chunk kc landed everywhere; slot (kc + 2) % 3 is free
      const uint32_t slot = (uint32_t)__builtin_amdgcn_readfirstlane((int)(ring0 + (uint32_t)(kc % kRing) * kSlot));
      // the first half-chunk's fragments are in flight while the next transfers issue
      const bf16x8 f0 = lds_frag(slot + zoff[0][0]), f1 = lds_frag(slot + zoff[1][0]);
      bf16x8 fb[kAnch];
#pragma unroll
      for (int x = 0; x < kAnch; ++x) fb[x] = lds_frag(slot + boff[x][0]);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 z0 = s == 0 ? f0 : lds_frag(slot + zoff[0][s]), z1 = s == 0 ? f1 : lds_frag(slot + zoff[1][s]);
#pragma unroll
        for (int x = 0; x < kAnch; ++x) {
          const bf16x8 bx = s == 0 ? fb[x] : lds_frag(slot + boff[x][s]);
          acc[x][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bx, z0, acc[x][0], 0, 0, 0);
          acc[x][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bx, z1, acc[x][1], 0, 0, 0);
          if (s * kAnch + x < kDmaPerWave) {
            if (NS == 1 && kc + 2 >= nkc) stage_a((kc + 2 - nkc) * kDmaPerWave + s * kAnch + x);
            else fetch_unit(kc + 2, s * kAnch + x);
          }
        }
      }
    }
    wait_vm_barrier<0>();   // trailing transfers drained; every wave past the last chunk
    if constexpr (NS > 1) {
      slice_cosines<NS>(p, acc, reinterpret_cast<float*>(ring), u0, np, side, layer, tt, t0, tw, ag, lane, col, hi);
      continue;
    }

    // cosines of P with A per token, and the value-side gate sums over the prefix
#pragma unroll
    for (int i = 12; i < 18; ++i) stage_a(i);
#pragma unroll
    for (int x = 0; x < kAnch; ++x) {
      const int u = u0 + ag * kAnch + x;
      if (u >= p.n_use) break;
      if (x == 1) {   // anchor 0's reads are done (their values were used)
        stage_a(18);
        stage_a(19);
      }
      if (x == 3) wait_vm<0>();
      const int a = p.use[u];
      const int alen = p.len[a];
      const bool gate = side == 1 && ((p.mask_gate >> a) & 1);
      float gnum = 0.f, gpp = 0.f, gaa = 0.f;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int t = t0 + tw * 64 + tb * 32 + col;
        const bool ok = t < alen && t < S;
        float num = 0.f, pp = 0.f, aa = 0.f;
        // this lane's row of the wave's 64 (unit k = row / 16 of the anchor's four)
        const int row = tb * 32 + col;
        const uint32_t ub = (col >> 4) ? a_place(4 * x + 2 * tb + 1) : a_place(4 * x + 2 * tb);
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          // rows past the anchor or the layer were transferred as zeros
          const uint2 av = lds_u2(ub + (uint32_t)(((row & 15) * 4 + (jg ^ ((row >> 2) & 3))) * 16 + 8 * hi));
          const float a4[4] = {__uint_as_float(av.x << 16), __uint_as_float(av.x & 0xffff0000u),
                               __uint_as_float(av.y << 16), __uint_as_float(av.y & 0xffff0000u)};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = acc[x][tb][4 * jg + i];
            num = fmaf(pv, a4[i], num);
            pp = fmaf(pv, pv, pp);
            aa = fmaf(a4[i], a4[i], aa);
          }
        }
        const float qm = (gate && ok && t < p.k_gate) ? 1.f : 0.f;
        gnum = fmaf(num, qm, gnum);
        gpp = fmaf(pp, qm, gpp);
        gaa = fmaf(aa, qm, gaa);
        num += __shfl_xor(num, 32);
        pp += __shfl_xor(pp, 32);
        aa += __shfl_xor(aa, 32);
        const float den = sqrtf(pp) * sqrtf(aa);
        const float cval = den > 0.f ? num / den : 0.f;
        if (hi == 0 && t < S && tt * (kTok / kCosTile) + tw < p.n_tiles) p.scores[(((int64_t)side * p.n_layers + layer) * S + t) * p.N + a] = cval;
      }
      const int tile = tt * (kTok / kCosTile) + tw;
      if (gate && tile < p.n_tiles) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          gnum += __shfl_xor(gnum, o);
          gpp += __shfl_xor(gpp, o);
          gaa += __shfl_xor(gaa, o);
        }
        if (lane == 0) {
          const int64_t plane = (int64_t)p.n_layers * p.n_tiles * p.N;
          const int64_t o = ((int64_t)layer * p.n_tiles + tile) * p.N + a;
          p.partials[o] = gnum;
          p.partials[plane + o] = gpp;
          p.partials[2 * plane + o] = gaa;
        }
      }
    }
    wait_vm<0>();   // no transfer into this work-group's LDS outlives the pass
    if (u0 + kPass < nq) __syncthreads();   // every wave done with its A rows before the next pass's transfers
  }
}

}  // namespace

size_t cos_gemm_lds() { return (size_t)kRing * kSlot; }

size_t cos_gemm_packed_elems(int n_layers, int n_use, int r, int D) { return (size_t)2 * n_layers * n_use * r * D; }

hipError_t launch_pack_cos(const CosGemmArgs& a, uint16_t* dst, hipStream_t st) {
  if (a.n_use < 1) return hipSuccess;
  if (a.head_dim % 16 || (a.r != 32 && a.r != 64 && a.r != 128)) return hipErrorInvalidValue;
  const int64_t n = (int64_t)2 * a.n_layers * a.n_use * a.r * (a.D / 16);
  pack_cos<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(a, dst);
  return hipGetLastError();
}

hipError_t launch_score_cos_gemm(const CosGemmArgs& a, hipStream_t st) {
  if (a.n_use < 1) return hipSuccess;
  if (a.D % kKc || (a.head_dim != 64 && a.head_dim != 128)) return hipErrorInvalidValue;
  const void* k = a.r == 32    ? reinterpret_cast<const void*>(score_cos_gemm<1>)
                  : a.r == 64  ? reinterpret_cast<const void*>(score_cos_gemm<2>)
                  : a.r == 128 ? reinterpret_cast<const void*>(score_cos_gemm<4>)
                               : nullptr;
  if (!k) return hipErrorInvalidValue;
  const size_t lds = cos_gemm_lds();
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t nblk = (int64_t)((a.n_tiles * kCosTile + kTok - 1) / kTok) * a.n_layers * 2;
  if (nblk == 0) return hipSuccess;
  if (a.r == 32) score_cos_gemm<1><<<dim3((unsigned)nblk), kThreads, lds, st>>>(a);
  else if (a.r == 64) score_cos_gemm<2><<<dim3((unsigned)nblk), kThreads, lds, st>>>(a);
  else score_cos_gemm<4><<<dim3((unsigned)nblk), kThreads, lds, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvc
