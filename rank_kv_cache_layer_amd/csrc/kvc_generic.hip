// Generic (any shape, f32 or bf16) kernels of the per-hop correction: token scores, token
// weights, and the delta apply.  Plain VALU code with fp32 accumulation; the bf16 MFMA
// kernels in kvc_mfma.hip replace the score and apply steps for the common shapes.
//
// KVCMAS (arXiv 2609.34060) App. A.3 "Correction Weighting and Positional Alignment":
// token-wise weights from the mean absolute distance between the canonical source and each
// anchor's reconstructed base (Eq. 7 factors), softmax over anchors, separately for keys
// and values; Eq. 9 gate sums on values over the prefix k; Eq. 8 / Eq. 12 apply.
#include "kvc_internal.h"

namespace kvc {
namespace {

// Canonical-frame source element (keys rotated by R(-p_src), values as stored).
template <typename T>
__device__ __forceinline__ float zcan(const T* row, int d, int head_dim, const float* cs, const float* sn,
                                      bool rot) {
  const float x = ldf(row, d);
  if (!rot) return x;
  const int h = head_dim >> 1;
  const int c = d % head_dim;
  if (c < h) {
    const float y = ldf(row, d + h);
    return x * cs[c] - y * sn[c];
  }
  const float y = ldf(row, d - h);  // partner in the lower half
  return y * sn[c - h] + x * cs[c - h];
}

// grid (n_tiles, N_l, 2); block 256 threads = TT tokens x n_use anchors (thread -> (t, ai)).
template <typename T, int MODE>
__global__ void __launch_bounds__(256) score_generic(ScoreArgs p, int TT) {
  __shared__ float cs[kMaxHalf], sn[kMaxHalf];
  __shared__ float red[3][256];
  const int side = blockIdx.z, layer = blockIdx.y, tile = blockIdx.x;
  const int nu = p.n_use;
  const int tid = threadIdx.x;
  const int h = p.head_dim >> 1;
  for (int i = tid; i < h; i += blockDim.x) { cs[i] = p.can.cs[i]; sn[i] = p.can.sn[i]; }
  __syncthreads();
  const bool rot = side == 0 && p.can.active;
  const int tl = tid / nu, ai = tid % nu;
  const int t = tile * TT + tl;
  float m = 0.f, g0 = 0.f, g1 = 0.f, g2 = 0.f;
  const bool active = tl < TT && t < p.s_work;
  if (active) {
    const int a = p.use[ai];
    const int D = p.D, r = p.g.r;
    const T* row = (const T*)p.z[side] + ((int64_t)layer * p.S + t) * D;
    const bool has_row = t < p.g.len[a];
    const T* Arow = (const T*)p.A[side] + layer * p.g.a_layer_stride + ((int64_t)p.g.off[a] + t) * r;
    const T* B = (const T*)p.B[side] + layer * p.g.b_layer_stride + (int64_t)a * r * D;
    const bool want_gate = side == 1 && ((p.mask_gate >> a) & 1) && t < p.k_gate && has_row;
    if (MODE == KVC_SCORE_PAGES) {
      float q = 0.f;
      for (int d = 0; d < D; ++d) {
        float rec = 0.f;
        if (has_row)
          for (int k = 0; k < r; ++k) rec = fmaf(ldf(Arow, k), ldf(B, (int64_t)k * D + d), rec);
        const float e = zcan(row, d, p.head_dim, cs, sn, rot) - rec;
        m += fabsf(e);
        q = fmaf(e, e, q);
      }
      m = m / (float)D;
      if (want_gate) g0 = q;
    } else {
      float num = 0.f, pp = 0.f, aa = 0.f;
      if (has_row) {
        for (int k = 0; k < r; ++k) {
          float pk = 0.f;
          for (int d = 0; d < D; ++d) pk = fmaf(zcan(row, d, p.head_dim, cs, sn, rot), ldf(B, (int64_t)k * D + d), pk);
          const float av = ldf(Arow, k);
          num = fmaf(pk, av, num);
          pp = fmaf(pk, pk, pp);
          aa = fmaf(av, av, aa);
        }
      }
      const float den = sqrtf(pp) * sqrtf(aa);
      m = den > 0.f ? num / den : 0.f;
      if (want_gate) { g0 = num; g1 = pp; g2 = aa; }
    }
    if (t < p.S) p.scores[(((int64_t)side * p.n_layers + layer) * p.S + t) * p.g.n + a] = m;
  }
  if (side == 1) {
    red[0][tid] = g0;
    red[1][tid] = g1;
    red[2][tid] = g2;
    __syncthreads();
    // fixed-order per-anchor reduction over the tile's tokens
    if (tid < nu) {
      const int a = p.use[tid];
      float s0 = 0.f, s1 = 0.f, s2 = 0.f;
      for (int j = 0; j < TT; ++j) {
        s0 += red[0][j * nu + tid];
        s1 += red[1][j * nu + tid];
        s2 += red[2][j * nu + tid];
      }
      const int64_t plane = (int64_t)p.n_layers * p.n_tiles * p.g.n;
      const int64_t o = ((int64_t)layer * p.n_tiles + tile) * p.g.n + a;
      p.partials[o] = s0;
      p.partials[plane + o] = s1;
      p.partials[2 * plane + o] = s2;
    }
  }
}

// One thread per (side, layer, token): softmax over the correction set.
__global__ void __launch_bounds__(256) softmax_kernel(SoftmaxArgs p) {
  const int64_t rows = 2ll * p.n_layers * p.S;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += (int64_t)gridDim.x * blockDim.x) {
    const int side = (int)(i / ((int64_t)p.n_layers * p.S));
    const int64_t lt = i - (int64_t)side * p.n_layers * p.S;
    const int t = (int)(lt % p.S);
    const float* s = p.scores + i * p.N;
    float* w = p.w[side] + lt * p.N;
    if (t >= p.s_cov) {
      for (int a = 0; a < p.N; ++a) w[a] = 0.f;
      continue;
    }
    const float sg = p.mode == KVC_SCORE_PAGES ? -p.inv_temp : p.inv_temp;
    float mx = -INFINITY;
    for (int a = 0; a < p.N; ++a)
      if ((p.mask_corr >> a) & 1) mx = fmaxf(mx, s[a] * sg);
    float sum = 0.f;
    float e[kMaxAnchors];
    for (int a = 0; a < p.N; ++a) {
      e[a] = ((p.mask_corr >> a) & 1) ? expf(s[a] * sg - mx) : 0.f;
      sum += e[a];
    }
    const float inv = 1.f / sum;
    for (int a = 0; a < p.N; ++a) w[a] = e[a] * inv;
  }
}

// One thread per (side, layer, token, head, rotary pair c): both channels c and c + h.
template <typename T>
__global__ void __launch_bounds__(256) apply_generic(ApplyArgs p) {
  __shared__ float c_s[kMaxHalf], s_s[kMaxHalf], c_t[kMaxHalf], s_t[kMaxHalf];
  const int h = p.head_dim >> 1;
  for (int i = threadIdx.x; i < h; i += blockDim.x) {
    c_s[i] = p.shift.cs[i]; s_s[i] = p.shift.sn[i];
    c_t[i] = p.tgt.cs[i];   s_t[i] = p.tgt.sn[i];
  }
  __syncthreads();
  const int D = p.D, H = D / p.head_dim, r = p.g.r;
  const int64_t per_side = (int64_t)p.n_layers * p.S * H * h;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < 2 * per_side;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int side = (int)(u / per_side);
    int64_t v = u - side * per_side;
    const int c = (int)(v % h); v /= h;
    const int head = (int)(v % H); v /= H;
    const int t = (int)(v % p.S);
    const int layer = (int)(v / p.S);
    const int d0 = head * p.head_dim + c, d1 = d0 + h;
    const int64_t rowo = ((int64_t)layer * p.S + t) * D;
    const T* z = (const T*)p.z[side] + rowo;
    float e0 = 0.f, e1 = 0.f;
    if (t < p.s_cov) {
      const float* w = p.w[side] + ((int64_t)layer * p.S + t) * p.g.n;
      for (int ci = 0; ci < p.n_corr; ++ci) {
        const int a = p.corr[ci];
        const float wa = w[a];
        if (t >= p.g.len[a]) continue;
        const T* Arow = (const T*)p.A[side] + layer * p.g.a_layer_stride + ((int64_t)p.g.off[a] + t) * r;
        const T* B = (const T*)p.B[side] + layer * p.g.b_layer_stride + (int64_t)a * r * D;
        for (int k = 0; k < r; ++k) {
          const float wa_k = wa * ldf(Arow, k);
          e0 = fmaf(wa_k, ldf(B, (int64_t)k * D + d0), e0);
          e1 = fmaf(wa_k, ldf(B, (int64_t)k * D + d1), e1);
        }
      }
    }
    const float z0 = ldf(z, d0), z1 = ldf(z, d1);
    float o0, o1;
    if (side == 0) {
      float b0 = z0, b1 = z1, r0 = e0, r1 = e1;
      if (p.shift.active) { b0 = z0 * c_s[c] - z1 * s_s[c]; b1 = z0 * s_s[c] + z1 * c_s[c]; }
      if (p.tgt.active) { r0 = e0 * c_t[c] - e1 * s_t[c]; r1 = e0 * s_t[c] + e1 * c_t[c]; }
      o0 = b0 + r0;
      o1 = b1 + r1;
    } else {
      o0 = z0 + e0;
      o1 = z1 + e1;
    }
    T* out = (T*)p.out[side] + rowo;
    stf(out, d0, o0);
    stf(out, d1, o1);
  }
}

int64_t clamp_blocks(int64_t units) {
  int64_t b = (units + 255) / 256;
  if (b > 65536) b = 65536;
  return b < 1 ? 1 : b;
}

}  // namespace

hipError_t launch_score_generic(const ScoreArgs& a, int bf16, int mode, int tile_tokens, hipStream_t st) {
  dim3 grid(a.n_tiles, a.n_layers, 2);
  if (bf16) {
    if (mode == KVC_SCORE_PAGES) score_generic<uint16_t, KVC_SCORE_PAGES><<<grid, 256, 0, st>>>(a, tile_tokens);
    else score_generic<uint16_t, KVC_SCORE_COS_R><<<grid, 256, 0, st>>>(a, tile_tokens);
  } else {
    if (mode == KVC_SCORE_PAGES) score_generic<float, KVC_SCORE_PAGES><<<grid, 256, 0, st>>>(a, tile_tokens);
    else score_generic<float, KVC_SCORE_COS_R><<<grid, 256, 0, st>>>(a, tile_tokens);
  }
  return hipGetLastError();
}

hipError_t launch_softmax(const SoftmaxArgs& a, hipStream_t st) {
  softmax_kernel<<<(unsigned)clamp_blocks(2ll * a.n_layers * a.S), 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_apply_generic(const ApplyArgs& a, int bf16, hipStream_t st) {
  const int64_t units = 2ll * a.n_layers * a.S * (a.D / 2);
  if (bf16) apply_generic<uint16_t><<<(unsigned)clamp_blocks(units), 256, 0, st>>>(a);
  else apply_generic<float><<<(unsigned)clamp_blocks(units), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvc
