// Anchor pool updates of KVCMAS (arXiv 2609.34060), App. A.3 "Cache Materialization and Pool
// Updates":
//  * after a dense fallback the observed correction is Delta = C_j - Align(C_i) (Eq. 12); the
//    source cache and Delta are factorised (Eq. 7, kvc_anchor_refresh_svd) and inserted as a
//    new anchor, into a slot of a caller-owned arena (kvc_pool_insert);
//  * accepted corrections are not reinserted; when the pool is full, the least frequently
//    used anchor among the five oldest is evicted (kvc_pool_record_hop, host only).
// Key factors are stored in the canonical frame (position 0): the key base is R(-p_src) K_i,
// and the key correction R(-p_tgt) (K_j - R(p_tgt - p_src) K_i) = R(-p_tgt) K_j - R(-p_src) K_i,
// which is how the kernel forms it (one rotation per operand).
#include <string.h>

#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace {

// 8 consecutive elements as fp32, one 16-byte (bf16) or two 16-byte (fp32) loads
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

// out (fp32) = R(tt) tgt - R(ts) src per rotate-half pair; an inactive table is the identity
// (values).  VEC = 8: each thread owns pairs c0..c0+7 of one head of one row and moves them
// with 16-byte accesses (head_dim / 2 a multiple of 8); VEC = 1: one pair per thread.
template <typename T, int VEC>
__global__ void __launch_bounds__(256) observed_delta(const T* __restrict__ tgt, const T* __restrict__ src,
                                                      float* __restrict__ out, int64_t n_units, int n_heads,
                                                      int head_dim, RopeTab tt, RopeTab ts) {
  __shared__ float ct[kMaxHalf], st_[kMaxHalf], cs[kMaxHalf], ss[kMaxHalf];
  const int h = head_dim >> 1;
  for (int i = threadIdx.x; i < h; i += blockDim.x) {
    ct[i] = tt.cs[i];
    st_[i] = tt.sn[i];
    cs[i] = ts.cs[i];
    ss[i] = ts.sn[i];
  }
  __syncthreads();
  const int per_head = h / VEC, per_row = per_head * n_heads, D = n_heads * head_dim;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = u / per_row;
    const int rem = (int)(u - row * per_row);
    const int head = rem / per_head;
    const int c0 = (rem - head * per_head) * VEC;
    const int64_t base = row * D + (int64_t)head * head_dim + c0;
    float xt[VEC], yt[VEC], xs[VEC], ys[VEC];
    if constexpr (VEC == 8) {
      load8(tgt + base, xt);
      load8(tgt + base + h, yt);
      load8(src + base, xs);
      load8(src + base + h, ys);
    } else {
      xt[0] = ldf(tgt, base); yt[0] = ldf(tgt, base + h);
      xs[0] = ldf(src, base); ys[0] = ldf(src, base + h);
    }
    float ox[VEC], oy[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      float at = xt[i], bt = yt[i], as = xs[i], bs = ys[i];
      if (tt.active) rot_pair(xt[i], yt[i], ct[c0 + i], st_[c0 + i], at, bt);
      if (ts.active) rot_pair(xs[i], ys[i], cs[c0 + i], ss[c0 + i], as, bs);
      ox[i] = at - as;
      oy[i] = bt - bs;
    }
    if constexpr (VEC == 8) {
      store8(out + base, ox);
      store8(out + base + h, oy);
    } else {
      out[base] = ox[0];
      out[base + h] = oy[0];
    }
  }
}

template <typename T>
hipError_t go_delta(const void* tgt, const void* src, float* out, int64_t n_rows, int n_heads, int head_dim,
                    const RopeTab& tt, const RopeTab& ts, hipStream_t st) {
  const int h = head_dim / 2;
  const bool vec = (h % 8) == 0;
  const int64_t units = n_rows * n_heads * (vec ? h / 8 : h);
  const int64_t blocks = std::min<int64_t>(std::max<int64_t>((units + 255) / 256, 1), 65536);
  if (vec)
    observed_delta<T, 8><<<(unsigned)blocks, 256, 0, st>>>((const T*)tgt, (const T*)src, out, units, n_heads,
                                                             head_dim, tt, ts);
  else
    observed_delta<T, 1><<<(unsigned)blocks, 256, 0, st>>>((const T*)tgt, (const T*)src, out, units, n_heads,
                                                             head_dim, tt, ts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_observed_delta(const void* tgt, const void* src, int bf16, float* out, int64_t n_rows,
                                 int n_heads, int head_dim, const RopeTab& tt, const RopeTab& ts, hipStream_t st) {
  return bf16 ? go_delta<uint16_t>(tgt, src, out, n_rows, n_heads, head_dim, tt, ts, st)
              : go_delta<float>(tgt, src, out, n_rows, n_heads, head_dim, tt, ts, st);
}

}  // namespace kvc
