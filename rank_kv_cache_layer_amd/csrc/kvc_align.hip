// Key re-alignment: a constant rotate-half RoPE rotation of every row of a key cache
// (KVCMAS Sec. 2.2 and App. A.3 "Correction Weighting and Positional Alignment": cached
// keys are re-aligned to the target positions before reuse; values need no rotation).
//
// Pure HBM streaming: each thread owns 8 rotary pairs (c..c+7, c+h..c+h+7) of one head of
// one row and moves them with 16-byte (bf16) or 2x16-byte (f32) loads/stores, so every
// wave touches whole 128-byte lines.
#include "kvc_internal.h"

namespace kvc {
namespace {

template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
  uint4 v;
  __device__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ void store(uint16_t* p) const { *reinterpret_cast<uint4*>(p) = v; }
  __device__ float get(int i) const {
    uint32_t w = (&v.x)[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ void set8(const float* f) {
    uint32_t* w = &v.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(f[2 * i]) | ((uint32_t)f2bf(f[2 * i + 1]) << 16);
  }
};
template <> struct Vec8<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ void store(float* p) const {
    reinterpret_cast<float4*>(p)[0] = a;
    reinterpret_cast<float4*>(p)[1] = b;
  }
  __device__ float get(int i) const { return i < 4 ? (&a.x)[i] : (&b.x)[i - 4]; }
  __device__ void set8(const float* f) {
    a = make_float4(f[0], f[1], f[2], f[3]);
    b = make_float4(f[4], f[5], f[6], f[7]);
  }
};

// VEC = 8 pairs per thread when head_dim/2 is a multiple of 8, else 1.
template <typename Tin, typename Tout>
__global__ void __launch_bounds__(256) align_rope_vec8(const Tin* __restrict__ in, Tout* __restrict__ out,
                                                       int64_t n_units, int n_heads, int head_dim,
                                                       RopeTab tab) {
  __shared__ float cs[kMaxHalf], sn[kMaxHalf];
  const int h = head_dim >> 1;
  for (int i = threadIdx.x; i < h; i += blockDim.x) { cs[i] = tab.cs[i]; sn[i] = tab.sn[i]; }
  __syncthreads();
  const int per_head = h >> 3;
  const int per_row = per_head * n_heads;
  const int D = n_heads * head_dim;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = u / per_row;
    const int rem = (int)(u - row * per_row);
    const int head = rem / per_head;
    const int c0 = (rem - head * per_head) * 8;
    const int64_t base = row * D + (int64_t)head * head_dim + c0;
    Vec8<Tin> x, y;
    x.load(in + base);
    y.load(in + base + h);
    float ox[8], oy[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = x.get(i), b = y.get(i);
      if (tab.active) {
        rot_pair(a, b, cs[c0 + i], sn[c0 + i], ox[i], oy[i]);
      } else {
        ox[i] = a;
        oy[i] = b;
      }
    }
    Vec8<Tout> X, Y;
    X.set8(ox);
    Y.set8(oy);
    X.store(out + base);
    Y.store(out + base + h);
  }
}

template <typename Tin, typename Tout>
__global__ void __launch_bounds__(256) align_rope_scalar(const Tin* __restrict__ in, Tout* __restrict__ out,
                                                         int64_t n_units, int n_heads, int head_dim,
                                                         RopeTab tab) {
  const int h = head_dim >> 1;
  const int D = n_heads * head_dim;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = u / (h * n_heads);
    const int rem = (int)(u - row * h * n_heads);
    const int head = rem / h, c = rem - head * h;
    const int64_t i0 = row * D + (int64_t)head * head_dim + c;
    const float a = ldf(in, i0), b = ldf(in, i0 + h);
    float x = a, y = b;
    if (tab.active) rot_pair(a, b, tab.cs[c], tab.sn[c], x, y);
    stf(out, i0, x);
    stf(out, i0 + h, y);
  }
}

template <typename Tin, typename Tout>
hipError_t go(const void* in, void* out, int64_t n_rows, int n_heads, int head_dim, const RopeTab& tab,
              hipStream_t st) {
  const int h = head_dim / 2;
  const bool vec = (h % 8) == 0;
  const int64_t units = n_rows * n_heads * (vec ? h / 8 : h);
  int64_t blocks = (units + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (vec)
    align_rope_vec8<Tin, Tout><<<(unsigned)blocks, 256, 0, st>>>((const Tin*)in, (Tout*)out, units, n_heads,
                                                                   head_dim, tab);
  else
    align_rope_scalar<Tin, Tout><<<(unsigned)blocks, 256, 0, st>>>((const Tin*)in, (Tout*)out, units, n_heads,
                                                                     head_dim, tab);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) fill_f32(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  fill_f32<<<(unsigned)blocks, 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_align(const void* in, void* out, int in_bf16, int out_bf16, int64_t n_rows, int n_heads,
                        int head_dim, const RopeTab& tab, hipStream_t st) {
  if (in_bf16 && out_bf16) return go<uint16_t, uint16_t>(in, out, n_rows, n_heads, head_dim, tab, st);
  if (in_bf16) return go<uint16_t, float>(in, out, n_rows, n_heads, head_dim, tab, st);
  if (out_bf16) return go<float, uint16_t>(in, out, n_rows, n_heads, head_dim, tab, st);
  return go<float, float>(in, out, n_rows, n_heads, head_dim, tab, st);
}

}  // namespace kvc
