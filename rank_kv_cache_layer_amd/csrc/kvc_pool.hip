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

// out (fp32) = R(tt) tgt - R(ts) src per rotate-half pair, 8 pairs per thread (or 1 when
// head_dim / 2 is not a multiple of 8); an inactive table is the identity (values).
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
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float xt = ldf(tgt, base + i), yt = ldf(tgt, base + h + i);
      const float xs = ldf(src, base + i), ys = ldf(src, base + h + i);
      float at = xt, bt = yt, as = xs, bs = ys;
      if (tt.active) rot_pair(xt, yt, ct[c0 + i], st_[c0 + i], at, bt);
      if (ts.active) rot_pair(xs, ys, cs[c0 + i], ss[c0 + i], as, bs);
      out[base + i] = at - as;
      out[base + h + i] = bt - bs;
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
