// bf16 MFMA scoring kernel of the second scoring mode for gfx950 (CDNA4): the canonical
// source is projected on each anchor's basis, P = Z B^T (the Eq. 7 factor B of KVCMAS,
// arXiv 2609.34060, Sec. 3.3), and P is compared with the anchor coordinates A by cosine,
// per token; value-side sums over the prefix k feed the segment cosine of the gate.
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

// Flattened block index -> logical tile, XCD-aware (consecutive tiles share an XCD L2).
__device__ __forceinline__ int64_t logical_block() {
  return xcd_remap(blockIdx.x, gridDim.x);
}

// Rotate-half partner layout for a wave covering 128 channels (one head of 128 or two of 64):
// lower block b pairs with block b + HD/64; rotary index of row `row` in block b.
template <int HD> __device__ __forceinline__ bool is_lower(int b) { return ((b * 32) % HD) < HD / 2; }
template <int HD> __device__ __forceinline__ int rot_index(int b, int row) { return (b * 32) % HD + row; }

// ---------------------------------------------------------- COS_R scoring (MFMA)
// Work-group = 64 tokens of one (layer, side), 4 waves.  The canonical source tile is staged
// once in LDS as bf16; each wave takes ANCH anchors per pass and contracts P = B_a Z^T over D
// with B read in its stored [r][D] layout, then forms per-token cosines with A_a.  The staged
// tile fills the LDS of a CU, so one wave runs per SIMD and may hold up to 512 VGPRs: more
// anchors per pass share each source fragment read and give the matrix core independent work.
template <int HD, int RB, int ANCH>
__global__ void __launch_bounds__(256) score_cos_mfma(ScoreArgs p) {
  extern __shared__ uint16_t zs[];            // [64][D + 8]
  __shared__ float cs_s[64], sn_s[64];
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

// rank 32: anchors per wave and pass among 2, 3, 5, whichever needs the fewest anchor-passes
// per wave for n_use anchors over 4 waves (ties to the smaller)
int cos_anch(int n_use) {
  int best = 2, cost = 1 << 30;
  for (int c : {2, 3, 5}) {
    const int passes = (n_use + 4 * c - 1) / (4 * c);
    if (passes * c < cost) { cost = passes * c; best = c; }
  }
  return best;
}

template <int HD>
hipError_t cos_dispatch(const ScoreArgs& a, dim3 grid, size_t shmem, hipStream_t st) {
  switch (a.g.r / 32) {
    case 1:
      switch (cos_anch(a.n_use)) {
        case 5: KVC_LAUNCH((score_cos_mfma<HD, 1, 5>), grid, 256, shmem, st, a); break;
        case 3: KVC_LAUNCH((score_cos_mfma<HD, 1, 3>), grid, 256, shmem, st, a); break;
        default: KVC_LAUNCH((score_cos_mfma<HD, 1, 2>), grid, 256, shmem, st, a); break;
      }
      break;
    case 2: KVC_LAUNCH((score_cos_mfma<HD, 2, 1>), grid, 256, shmem, st, a); break;
    case 4: KVC_LAUNCH((score_cos_mfma<HD, 4, 1>), grid, 256, shmem, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_cos_mfma(const ScoreArgs& a, hipStream_t st) {
  const size_t shmem = sizeof(uint16_t) * 64 * (size_t)(a.D + 8);
  const int64_t nblk = (int64_t)a.n_tiles * a.n_layers * 2;
  dim3 grid((unsigned)nblk);
  if (a.head_dim == 128) return cos_dispatch<128>(a, grid, shmem, st);
  if (a.head_dim == 64) return cos_dispatch<64>(a, grid, shmem, st);
  return hipErrorInvalidValue;
}

}  // namespace kvc
