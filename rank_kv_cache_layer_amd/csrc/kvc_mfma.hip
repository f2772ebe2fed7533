// bf16 MFMA kernels of the per-hop correction for gfx950 (CDNA4).
//
// KVCMAS (arXiv 2609.34060):
//  * scoring (App. A.3 "Correction Weighting and Positional Alignment", Eq. 7 bases, Eq. 9
//    gate sums): E = Z_can - A_a B_a for every anchor a, reduced to the per-token mean |E|
//    and, for values, to the Frobenius sum over the prefix k;
//  * the second scoring mode projects the canonical source on each anchor basis, P = Z B^T,
//    and compares P with the anchor coordinates A by cosine;
//  * apply (Sec. 3.3 Eq. 8, App. A.3 Eq. 12): out = R(s) Z + R(p_tgt) [w (.) A_D] B_D, one
//    contraction over (anchor, rank) fused with both rotations and the residual add.
//
// MFMA used: v_mfma_f32_32x32x16_bf16.  Lane l (col = l % 32, hi = l / 32) supplies
//   operand A: row col, k = 8*hi .. 8*hi+7;  operand B: column col, k = 8*hi .. 8*hi+7;
//   result register j holds row 8*(j/4) + 4*hi + (j%4), column col.
// Every contraction is arranged with channels d (or rank rows) as MFMA rows and tokens as
// MFMA columns, so one lane owns one token and 16 channels of each 32x32 block: per-token
// reductions over channels stay in registers, and the rotate-half partners c and c + h of a
// head sit in the same lane and register slot of two blocks.
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// Flattened block index -> logical tile, XCD-aware (consecutive tiles share an XCD L2).
__device__ __forceinline__ int64_t logical_block() {
  return xcd_remap(blockIdx.x, gridDim.x);
}

// ------------------------------------------------------------------ B^T pre-pass
struct TransArgs {
  const uint16_t* src[4];
  uint16_t* dst[4];
  int32_t negate[4];
  int32_t n_arrays, n_layers, n_anchors, r, D;
};

// grid (ceil(D/64), n_anchors, n_layers * n_arrays); B [r][D] -> Bt [D][r] per (layer, anchor)
__global__ void __launch_bounds__(256) transpose_b(TransArgs p) {
  __shared__ uint16_t tile[256][66];
  const int arr = blockIdx.z % p.n_arrays, layer = blockIdx.z / p.n_arrays, a = blockIdx.y;
  const int d0 = blockIdx.x * 64, r = p.r, D = p.D;
  const int64_t mat = ((int64_t)layer * p.n_anchors + a);
  const uint16_t* src = p.src[arr] + mat * r * D;
  uint16_t* dst = p.dst[arr] + mat * D * r;
  const uint16_t flip = p.negate[arr] ? 0x8000u : 0u;
  for (int i = threadIdx.x; i < r * 64; i += 256) {
    const int k = i >> 6, dd = i & 63;
    tile[k][dd] = (d0 + dd < D) ? (uint16_t)(src[(int64_t)k * D + d0 + dd] ^ flip) : (uint16_t)0;
  }
  __syncthreads();
  const int kc_n = r >> 3;
  for (int i = threadIdx.x; i < 64 * kc_n; i += 256) {
    const int dd = i / kc_n, kc = i - dd * kc_n;
    if (d0 + dd >= D) continue;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)tile[kc * 8 + 2 * j][dd] | ((uint32_t)tile[kc * 8 + 2 * j + 1][dd] << 16);
    *reinterpret_cast<uint4*>(dst + (int64_t)(d0 + dd) * r + kc * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Rotate-half partner layout for a wave covering 128 channels (one head of 128 or two of 64):
// lower block b pairs with block b + HD/64; rotary index of row `row` in block b.
template <int HD> __device__ __forceinline__ bool is_lower(int b) { return ((b * 32) % HD) < HD / 2; }
template <int HD> __device__ __forceinline__ int rot_index(int b, int row) { return (b * 32) % HD + row; }

// ---------------------------------------------------------- PAGES scoring (MFMA)
// Work-group = 64 tokens of one (layer, side); D/128 waves, wave w owns channels
// [128w, 128w + 128) of all 64 tokens with the canonical source held in fp32 registers as
// the MFMA accumulator input, so every anchor's E = Z_can - A B needs no extra copy.
template <int HD, int RK>
__global__ void __launch_bounds__(512) score_pages_mfma(ScoreArgs p) {
  extern __shared__ float lds[];
  __shared__ float cs_s[64], sn_s[64];
  constexpr bool kHoldA = RK <= 2;
  const int nu = p.n_use;
  const int NW = blockDim.x >> 6;
  float* mpart = lds;                         // [NW][64][nu]
  float* qpart = lds + NW * 64 * nu;          // [NW][nu]

  const int64_t lb = logical_block();
  const int tile = (int)(lb % p.n_tiles);
  const int layer = (int)((lb / p.n_tiles) % p.n_layers);
  const int side = (int)(lb / ((int64_t)p.n_tiles * p.n_layers));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 31, hi = lane >> 5;
  const int D = p.D, S = p.S;
  const int t0 = tile * 64, d0 = wave * 128;
  for (int i = threadIdx.x; i < HD / 2; i += blockDim.x) { cs_s[i] = p.can.cs[i]; sn_s[i] = p.can.sn[i]; }
  __syncthreads();

  // canonical source tile, MFMA accumulator layout
  float zc[2][4][16];
  const uint16_t* z = (const uint16_t*)p.z[side] + (int64_t)layer * S * D;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = t0 + tb * 32 + col;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        uint2 v = make_uint2(0, 0);
        if (t < S) v = *reinterpret_cast<const uint2*>(z + (int64_t)t * D + d0 + db * 32 + 8 * jg + 4 * hi);
        zc[tb][db][4 * jg + 0] = __uint_as_float(v.x << 16);
        zc[tb][db][4 * jg + 1] = __uint_as_float(v.x & 0xffff0000u);
        zc[tb][db][4 * jg + 2] = __uint_as_float(v.y << 16);
        zc[tb][db][4 * jg + 3] = __uint_as_float(v.y & 0xffff0000u);
      }
  }
  if (side == 0 && p.can.active) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      if (!is_lower<HD>(db)) continue;
      const int du = db + HD / 64;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int c = rot_index<HD>(db, 8 * (j >> 2) + 4 * hi + (j & 3));
        const float cs = cs_s[c], sn = sn_s[c];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const float x = zc[tb][db][j], y = zc[tb][du][j];
          zc[tb][db][j] = x * cs - y * sn;
          zc[tb][du][j] = x * sn + y * cs;
        }
      }
    }
  }

  const int r = RK * 16;
  const uint16_t* Abase = (const uint16_t*)p.A[side] + layer * p.g.a_layer_stride;
  const uint16_t* Btb = p.Bt[side] + (int64_t)layer * p.g.n * D * r;
  for (int ui = 0; ui < nu; ++ui) {
    const int a = p.use[ui];
    const bool gate = side == 1 && ((p.mask_gate >> a) & 1);
    const int alen = p.g.len[a];
    const uint16_t* Aa = Abase + (int64_t)p.g.off[a] * r;
    const uint16_t* Bta = Btb + (int64_t)a * D * r;
    float qmask[2];
    bf16x8 af[2][kHoldA ? RK : 1];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int t = t0 + tb * 32 + col;
      qmask[tb] = (t < p.k_gate && t < alen && t < S) ? 1.f : 0.f;
      if (kHoldA)
#pragma unroll
        for (int ks = 0; ks < (kHoldA ? RK : 1); ++ks)
          af[tb][ks] = (t < alen && t < S) ? ld8(Aa + (int64_t)t * r + ks * 16 + 8 * hi) : zero8();
    }
    float msum[2] = {0.f, 0.f};
    float qsum = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      bf16x8 bf[RK];
#pragma unroll
      for (int ks = 0; ks < RK; ++ks) bf[ks] = ld8(Bta + (int64_t)(d0 + db * 32 + col) * r + ks * 16 + 8 * hi);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        f32x16 acc;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = zc[tb][db][j];
#pragma unroll
        for (int ks = 0; ks < RK; ++ks) {
          bf16x8 av;
          if (kHoldA) {
            av = af[tb][kHoldA ? ks : 0];
          } else {
            const int t = t0 + tb * 32 + col;
            av = (t < alen && t < S) ? ld8(Aa + (int64_t)t * r + ks * 16 + 8 * hi) : zero8();
          }
          acc = mfma32(bf[ks], av, acc);     // Z_can - B^T A^T (B^T pre-negated)
        }
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          s0 += fabsf(acc[j]);
          s1 += fabsf(acc[j + 1]);
          s2 += fabsf(acc[j + 2]);
          s3 += fabsf(acc[j + 3]);
        }
        msum[tb] += (s0 + s1) + (s2 + s3);
        if (gate) {
          float q0 = 0.f, q1 = 0.f;
#pragma unroll
          for (int j = 0; j < 16; j += 2) {
            q0 = fmaf(acc[j], acc[j], q0);
            q1 = fmaf(acc[j + 1], acc[j + 1], q1);
          }
          qsum = fmaf(q0 + q1, qmask[tb], qsum);
        }
      }
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const float m = msum[tb] + __shfl_xor(msum[tb], 32);
      if (hi == 0) mpart[(wave * 64 + tb * 32 + col) * nu + ui] = m;
    }
    if (gate) {
      float q = qsum;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) q += __shfl_xor(q, o);
      if (lane == 0) qpart[wave * nu + ui] = q;
    }
  }
  __syncthreads();
  const float invD = 1.f / (float)D;
  for (int i = threadIdx.x; i < 64 * nu; i += blockDim.x) {
    const int tl = i / nu, ui = i - tl * nu;
    float s = 0.f;
    for (int w = 0; w < NW; ++w) s += mpart[(w * 64 + tl) * nu + ui];
    const int t = t0 + tl;
    if (t < S) p.scores[(((int64_t)side * p.n_layers + layer) * S + t) * p.g.n + p.use[ui]] = s * invD;
  }
  if (side == 1) {
    for (int ui = threadIdx.x; ui < nu; ui += blockDim.x) {
      const int a = p.use[ui];
      if (!((p.mask_gate >> a) & 1)) continue;
      float s = 0.f;
      for (int w = 0; w < NW; ++w) s += qpart[w * nu + ui];
      p.partials[((int64_t)layer * p.n_tiles + tile) * p.g.n + a] = s;
    }
  }
}

// ---------------------------------------------------------- COS_R scoring (MFMA)
// Work-group = 64 tokens of one (layer, side), 4 waves.  The canonical source tile is staged
// once in LDS as bf16; each wave takes whole anchors and contracts P = B_a Z^T over D with
// B read in its stored [r][D] layout, then forms per-token cosines with A_a.
template <int HD, int RB>
__global__ void __launch_bounds__(256) score_cos_mfma(ScoreArgs p) {
  extern __shared__ uint16_t zs[];            // [64][D + 8]
  __shared__ float cs_s[64], sn_s[64];
  constexpr int ANCH = RB == 1 ? 2 : 1;       // anchors per pass per wave
  const int64_t lb = logical_block();
  const int tile = (int)(lb % p.n_tiles);
  const int layer = (int)((lb / p.n_tiles) % p.n_layers);
  const int side = (int)(lb / ((int64_t)p.n_tiles * p.n_layers));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 31, hi = lane >> 5;
  const int D = p.D, S = p.S, ld = D + 8;
  const int t0 = tile * 64;
  const int h = HD / 2;
  const uint16_t* z = (const uint16_t*)p.z[side] + (int64_t)layer * S * D;
  const bool rot = side == 0 && p.can.active;
  for (int i = threadIdx.x; i < h; i += blockDim.x) { cs_s[i] = p.can.cs[i]; sn_s[i] = p.can.sn[i]; }
  __syncthreads();
  // stage: 8 rotary pairs per thread-iteration
  const int units = 64 * (D / HD) * (h / 8);
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const int tl = u / ((D / HD) * (h / 8));
    const int rem = u - tl * ((D / HD) * (h / 8));
    const int head = rem / (h / 8), c0 = (rem - head * (h / 8)) * 8;
    const int t = t0 + tl;
    uint4 xv = make_uint4(0, 0, 0, 0), yv = make_uint4(0, 0, 0, 0);
    const int dx = head * HD + c0;
    if (t < S) {
      xv = *reinterpret_cast<const uint4*>(z + (int64_t)t * D + dx);
      yv = *reinterpret_cast<const uint4*>(z + (int64_t)t * D + dx + h);
    }
    if (rot) {
      uint32_t* xw = &xv.x;
      uint32_t* yw = &yv.x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x0 = __uint_as_float(xw[i] << 16), x1 = __uint_as_float(xw[i] & 0xffff0000u);
        float y0 = __uint_as_float(yw[i] << 16), y1 = __uint_as_float(yw[i] & 0xffff0000u);
        const float c_0 = cs_s[c0 + 2 * i], s_0 = sn_s[c0 + 2 * i];
        const float c_1 = cs_s[c0 + 2 * i + 1], s_1 = sn_s[c0 + 2 * i + 1];
        const float nx0 = x0 * c_0 - y0 * s_0, ny0 = x0 * s_0 + y0 * c_0;
        const float nx1 = x1 * c_1 - y1 * s_1, ny1 = x1 * s_1 + y1 * c_1;
        xw[i] = (uint32_t)f2bf(nx0) | ((uint32_t)f2bf(nx1) << 16);
        yw[i] = (uint32_t)f2bf(ny0) | ((uint32_t)f2bf(ny1) << 16);
      }
    }
    *reinterpret_cast<uint4*>(zs + tl * ld + dx) = xv;
    *reinterpret_cast<uint4*>(zs + tl * ld + dx + h) = yv;
  }
  __syncthreads();

  const int r = RB * 32;
  const uint16_t* Abase = (const uint16_t*)p.A[side] + layer * p.g.a_layer_stride;
  const uint16_t* Bbase = (const uint16_t*)p.B[side] + layer * p.g.b_layer_stride;
  const int64_t plane = (int64_t)p.n_layers * p.n_tiles * p.g.n;
  for (int u0 = wave * ANCH; u0 < p.n_use; u0 += 4 * ANCH) {
    f32x16 acc[ANCH][RB][2];
#pragma unroll
    for (int x = 0; x < ANCH; ++x)
#pragma unroll
      for (int kb = 0; kb < RB; ++kb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[x][kb][tb][j] = 0.f;
    const uint16_t* Bx[ANCH];
#pragma unroll
    for (int x = 0; x < ANCH; ++x) {
      const int ui = u0 + x < p.n_use ? u0 + x : u0;
      Bx[x] = Bbase + (int64_t)p.use[ui] * r * D;
    }
    for (int ks = 0; ks < D / 16; ++ks) {
      bf16x8 zf[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) zf[tb] = ld8(zs + (tb * 32 + col) * ld + ks * 16 + 8 * hi);
#pragma unroll
      for (int x = 0; x < ANCH; ++x)
#pragma unroll
        for (int kb = 0; kb < RB; ++kb) {
          const bf16x8 bfr = ld8(Bx[x] + (int64_t)(kb * 32 + col) * D + ks * 16 + 8 * hi);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) acc[x][kb][tb] = mfma32(bfr, zf[tb], acc[x][kb][tb]);
        }
    }
#pragma unroll
    for (int x = 0; x < ANCH; ++x) {
      const int ui = u0 + x;
      if (ui >= p.n_use) break;
      const int a = p.use[ui];
      const int alen = p.g.len[a];
      const uint16_t* Aa = Abase + (int64_t)p.g.off[a] * r;
      const bool gate = side == 1 && ((p.mask_gate >> a) & 1);
      float gnum = 0.f, gpp = 0.f, gaa = 0.f;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int t = t0 + tb * 32 + col;
        const bool ok = t < alen && t < S;
        float num = 0.f, pp = 0.f, aa = 0.f;
#pragma unroll
        for (int kb = 0; kb < RB; ++kb)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            uint2 av = make_uint2(0, 0);
            if (ok) av = *reinterpret_cast<const uint2*>(Aa + (int64_t)t * r + kb * 32 + 8 * jg + 4 * hi);
            const float a4[4] = {__uint_as_float(av.x << 16), __uint_as_float(av.x & 0xffff0000u),
                                 __uint_as_float(av.y << 16), __uint_as_float(av.y & 0xffff0000u)};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float pv = acc[x][kb][tb][4 * jg + i];
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
        if (hi == 0 && t < S) p.scores[(((int64_t)side * p.n_layers + layer) * S + t) * p.g.n + a] = cval;
      }
      if (gate) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          gnum += __shfl_xor(gnum, o);
          gpp += __shfl_xor(gpp, o);
          gaa += __shfl_xor(gaa, o);
        }
        if (lane == 0) {
          const int64_t o = ((int64_t)layer * p.n_tiles + tile) * p.g.n + a;
          p.partials[o] = gnum;
          p.partials[plane + o] = gpp;
          p.partials[2 * plane + o] = gaa;
        }
      }
    }
  }
}

// -------------------------------------------------------------------- apply (MFMA)
// Work-group = 128 tokens x (128 * waves) channels of one (layer, side); wave w owns 128
// channels x 128 tokens = 16 accumulator blocks.  Per anchor the work-group scales the
// anchor's delta rows A_D by the token weights into LDS (bf16), then each wave contracts
// them with its slice of B_D^T.  Epilogue: R(p_tgt) on the accumulated delta (keys),
// + R(s) Z (keys) or + Z (values), round to bf16.
template <int HD, int RK>
__global__ void __launch_bounds__(256) apply_mfma(ApplyArgs p, int n_ttiles, int n_dtiles) {
  extern __shared__ float smem[];
  constexpr int R = RK * 16;
  constexpr int LDA = R + 8;                  // padded bf16 row of the scaled delta rows
  __shared__ float cts[64], sts[64], css[64], sss[64];
  const int N = p.g.n;
  float* wsh = smem;                                            // [128][N]
  uint16_t* ash = reinterpret_cast<uint16_t*>(smem + 128 * N);  // [2][128][LDA]

  const int64_t lb = logical_block();
  const int dt = (int)(lb % n_dtiles);
  const int tt = (int)((lb / n_dtiles) % n_ttiles);
  const int layer = (int)((lb / ((int64_t)n_dtiles * n_ttiles)) % p.n_layers);
  const int side = (int)(lb / ((int64_t)n_dtiles * n_ttiles * p.n_layers));
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 31, hi = lane >> 5;
  const int D = p.D, S = p.S;
  const int t0 = tt * 128;
  const int dw0 = (dt * nw + wave) * 128;
  for (int i = threadIdx.x; i < HD / 2; i += blockDim.x) {
    cts[i] = p.tgt.cs[i]; sts[i] = p.tgt.sn[i];
    css[i] = p.shift.cs[i]; sss[i] = p.shift.sn[i];
  }
  const float* wg = p.w[side] + ((int64_t)layer * S) * N;
  for (int i = threadIdx.x; i < 128 * N; i += blockDim.x) {
    const int t = t0 + i / N;
    wsh[i] = t < S ? wg[(int64_t)t0 * N + i] : 0.f;
  }
  __syncthreads();

  const uint16_t* Abase = (const uint16_t*)p.A[side] + layer * p.g.a_layer_stride;
  const uint16_t* Btb = p.Bt[side] + (int64_t)layer * N * D * R;
  const int climit = p.s_cov < S ? p.s_cov : S;

  auto stage = [&](int ci, int buf) {
    const int a = p.corr[ci];
    const int lim = p.g.len[a] < climit ? p.g.len[a] : climit;
    const uint16_t* Aa = Abase + (int64_t)p.g.off[a] * R;
    uint16_t* dstb = ash + buf * 128 * LDA;
    for (int u = threadIdx.x; u < 128 * (R / 8); u += blockDim.x) {
      const int tl = u / (R / 8), kc = u - tl * (R / 8);
      const int t = t0 + tl;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < lim) {
        const uint4 x = *reinterpret_cast<const uint4*>(Aa + (int64_t)t * R + kc * 8);
        const float wv = wsh[tl * N + a];
        const uint32_t* xw = &x.x;
        uint32_t* vw = &v.x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float(xw[i] << 16) * wv;
          const float hv = __uint_as_float(xw[i] & 0xffff0000u) * wv;
          vw[i] = (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hv) << 16);
        }
      }
      *reinterpret_cast<uint4*>(dstb + tl * LDA + kc * 8) = v;
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[tb][db][j] = 0.f;

  if (p.n_corr > 0 && t0 < climit) {
    stage(0, 0);
    __syncthreads();
    for (int ci = 0; ci < p.n_corr; ++ci) {
      const int buf = ci & 1;
      if (ci + 1 < p.n_corr) stage(ci + 1, buf ^ 1);
      const int a = p.corr[ci];
      const uint16_t* Bta = Btb + (int64_t)a * D * R;
      const uint16_t* as = ash + buf * 128 * LDA;
#pragma unroll
      for (int ks = 0; ks < RK; ++ks) {
        bf16x8 bf[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) bf[db] = ld8(Bta + (int64_t)(dw0 + db * 32 + col) * R + ks * 16 + 8 * hi);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const bf16x8 af = ld8(as + (tb * 32 + col) * LDA + ks * 16 + 8 * hi);
#pragma unroll
          for (int db = 0; db < 4; ++db) acc[tb][db] = mfma32(bf[db], af, acc[tb][db]);
        }
      }
      __syncthreads();
    }
  }

  // epilogue
  const uint16_t* z = (const uint16_t*)p.z[side] + (int64_t)layer * S * D;
  uint16_t* out = (uint16_t*)p.out[side] + (int64_t)layer * S * D;
  const bool rot_t = side == 0 && p.tgt.active;
  const bool rot_s = side == 0 && p.shift.active;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int t = t0 + tb * 32 + col;
    if (t >= S) continue;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      if (!is_lower<HD>(db)) continue;
      const int du = db + HD / 64;
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int dl = dw0 + db * 32 + 8 * jg + 4 * hi;
        const int dh = dw0 + du * 32 + 8 * jg + 4 * hi;
        const uint2 zl = *reinterpret_cast<const uint2*>(z + (int64_t)t * D + dl);
        const uint2 zh = *reinterpret_cast<const uint2*>(z + (int64_t)t * D + dh);
        const float xl[4] = {__uint_as_float(zl.x << 16), __uint_as_float(zl.x & 0xffff0000u),
                             __uint_as_float(zl.y << 16), __uint_as_float(zl.y & 0xffff0000u)};
        const float xh[4] = {__uint_as_float(zh.x << 16), __uint_as_float(zh.x & 0xffff0000u),
                             __uint_as_float(zh.y << 16), __uint_as_float(zh.y & 0xffff0000u)};
        float ol[4], oh[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * jg + i;
          float el = acc[tb][db][j], eh = acc[tb][du][j];
          float bl = xl[i], bh = xh[i];
          const int c = rot_index<HD>(db, 8 * jg + 4 * hi + i);
          if (rot_t) {
            const float c_ = cts[c], s_ = sts[c];
            const float nl = el * c_ - eh * s_, nh = el * s_ + eh * c_;
            el = nl;
            eh = nh;
          }
          if (rot_s) {
            const float c_ = css[c], s_ = sss[c];
            const float nl = bl * c_ - bh * s_, nh = bl * s_ + bh * c_;
            bl = nl;
            bh = nh;
          }
          ol[i] = bl + el;
          oh[i] = bh + eh;
        }
        uint2 vl, vh;
        vl.x = (uint32_t)f2bf(ol[0]) | ((uint32_t)f2bf(ol[1]) << 16);
        vl.y = (uint32_t)f2bf(ol[2]) | ((uint32_t)f2bf(ol[3]) << 16);
        vh.x = (uint32_t)f2bf(oh[0]) | ((uint32_t)f2bf(oh[1]) << 16);
        vh.y = (uint32_t)f2bf(oh[2]) | ((uint32_t)f2bf(oh[3]) << 16);
        *reinterpret_cast<uint2*>(out + (int64_t)t * D + dl) = vl;
        *reinterpret_cast<uint2*>(out + (int64_t)t * D + dh) = vh;
      }
    }
  }
}

// Dynamic LDS above the default limit must be enabled per kernel instance.
template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

#define KVC_LAUNCH(kern, grid, block, shmem, st, ...)                  \
  do {                                                                 \
    hipError_t e_ = allow_lds(kern, shmem);                            \
    if (e_ != hipSuccess) return e_;                                   \
    kern<<<grid, block, shmem, st>>>(__VA_ARGS__);                     \
  } while (0)

template <int HD>
hipError_t pages_dispatch(const ScoreArgs& a, dim3 grid, int threads, size_t shmem, hipStream_t st) {
  switch (a.g.r / 16) {
    case 1: KVC_LAUNCH((score_pages_mfma<HD, 1>), grid, threads, shmem, st, a); break;
    case 2: KVC_LAUNCH((score_pages_mfma<HD, 2>), grid, threads, shmem, st, a); break;
    case 4: KVC_LAUNCH((score_pages_mfma<HD, 4>), grid, threads, shmem, st, a); break;
    case 8: KVC_LAUNCH((score_pages_mfma<HD, 8>), grid, threads, shmem, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int HD>
hipError_t cos_dispatch(const ScoreArgs& a, dim3 grid, size_t shmem, hipStream_t st) {
  switch (a.g.r / 32) {
    case 1: KVC_LAUNCH((score_cos_mfma<HD, 1>), grid, 256, shmem, st, a); break;
    case 2: KVC_LAUNCH((score_cos_mfma<HD, 2>), grid, 256, shmem, st, a); break;
    case 4: KVC_LAUNCH((score_cos_mfma<HD, 4>), grid, 256, shmem, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int HD>
hipError_t apply_dispatch(const ApplyArgs& a, dim3 grid, int threads, size_t shmem, int ntt, int ndt,
                          hipStream_t st) {
  switch (a.g.r / 16) {
    case 1: KVC_LAUNCH((apply_mfma<HD, 1>), grid, threads, shmem, st, a, ntt, ndt); break;
    case 2: KVC_LAUNCH((apply_mfma<HD, 2>), grid, threads, shmem, st, a, ntt, ndt); break;
    case 4: KVC_LAUNCH((apply_mfma<HD, 4>), grid, threads, shmem, st, a, ntt, ndt); break;
    case 8: KVC_LAUNCH((apply_mfma<HD, 8>), grid, threads, shmem, st, a, ntt, ndt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_transpose_b(const uint16_t* const* src, uint16_t* const* dst, int n_arrays, const int* negate,
                              int n_layers, int n_anchors, int r, int D, hipStream_t st) {
  if (n_arrays < 1 || n_arrays > 4 || r > 256 || (r % 8) != 0 || n_anchors < 1) return hipErrorInvalidValue;
  TransArgs a;
  for (int i = 0; i < 4; ++i) {
    a.src[i] = i < n_arrays ? src[i] : nullptr;
    a.dst[i] = i < n_arrays ? dst[i] : nullptr;
    a.negate[i] = i < n_arrays ? negate[i] : 0;
  }
  a.n_arrays = n_arrays; a.n_layers = n_layers; a.n_anchors = n_anchors; a.r = r; a.D = D;
  dim3 grid((D + 63) / 64, n_anchors, n_layers * n_arrays);
  transpose_b<<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_score_pages_mfma(const ScoreArgs& a, hipStream_t st) {
  const int nw = a.D / 128;
  const size_t shmem = sizeof(float) * ((size_t)nw * 64 * a.n_use + (size_t)nw * a.n_use);
  const int64_t nblk = (int64_t)a.n_tiles * a.n_layers * 2;
  dim3 grid((unsigned)nblk);
  if (a.head_dim == 128) return pages_dispatch<128>(a, grid, nw * 64, shmem, st);
  if (a.head_dim == 64) return pages_dispatch<64>(a, grid, nw * 64, shmem, st);
  return hipErrorInvalidValue;
}

hipError_t launch_score_cos_mfma(const ScoreArgs& a, hipStream_t st) {
  const size_t shmem = sizeof(uint16_t) * 64 * (size_t)(a.D + 8);
  const int64_t nblk = (int64_t)a.n_tiles * a.n_layers * 2;
  dim3 grid((unsigned)nblk);
  if (a.head_dim == 128) return cos_dispatch<128>(a, grid, shmem, st);
  if (a.head_dim == 64) return cos_dispatch<64>(a, grid, shmem, st);
  return hipErrorInvalidValue;
}

hipError_t launch_apply_mfma(const ApplyArgs& a, hipStream_t st) {
  const int groups = a.D / 128;
  int nw = 4;
  while (groups % nw) --nw;
  const int ndt = groups / nw;
  const int ntt = (a.S + 127) / 128;
  const size_t shmem = sizeof(float) * 128 * a.g.n + sizeof(uint16_t) * 2 * 128 * (a.g.r + 8);
  const int64_t nblk = (int64_t)ndt * ntt * a.n_layers * 2;
  dim3 grid((unsigned)nblk);
  if (a.head_dim == 128) return apply_dispatch<128>(a, grid, nw * 64, shmem, ntt, ndt, st);
  if (a.head_dim == 64) return apply_dispatch<64>(a, grid, nw * 64, shmem, ntt, ndt, st);
  return hipErrorInvalidValue;
}

}  // namespace kvc
