// Measurement kernels: sustained HBM copy, bf16 MFMA, LDS read and fp32 VALU throughput of
// the device, the ceilings the correction kernels are reported against.
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// one 16-byte unit per thread over a grid that covers the buffer: on the device this sustains
// more than grid-stride loops with 1-8 loads in flight per lane (measured 6.5 vs 4.2-5.4 TB/s at
// 1 GiB with 2048-16384 work-groups); non-temporal, streamed once
__global__ void __launch_bounds__(256) peak_copy(u32x4* __restrict__ dst, const u32x4* __restrict__ src, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ void __launch_bounds__(256) peak_mfma(float* sink, int iters) {
  const int tid = threadIdx.x;
  // operands differ per lane and round so nothing folds; four independent accumulator chains
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (tid + i));
    b[i] = (__bf16)(0.002f * (tid - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  sink[(size_t)blockIdx.x * 256 + tid] = s;
}

__global__ void __launch_bounds__(256) peak_lds(uint32_t* sink, int iters) {
  __shared__ uint4 buf[4096];   // 64 KiB
  const int tid = threadIdx.x;
  for (int i = tid; i < 4096; i += 256) buf[i] = make_uint4(i, i * 3u, i * 5u, i * 7u);
  __syncthreads();
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int it = 0; it < iters; ++it) {
    // lane-consecutive 16-byte words: conflict-free; the round index moves the window
    const int base = (it * 8 * 256) & 4095;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint4 v = buf[(base + u * 256 + tid) & 4095];
      acc.x ^= v.x;
      acc.y += v.y;
      acc.z ^= v.z;
      acc.w += v.w;
    }
  }
  sink[(size_t)blockIdx.x * 256 + tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ void __launch_bounds__(256) peak_valu(float* sink, int iters) {
  const int tid = threadIdx.x;
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.5f * (tid + i);
  const float y = 1e-7f * (tid + 1);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = x[i] + y;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  sink[(size_t)blockIdx.x * 256 + tid] = s;
}

}  // namespace

hipError_t launch_peak_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 16;
  const size_t grid = (n + 255) / 256;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffu) return hipErrorInvalidValue;
  peak_copy<<<(unsigned)grid, 256, 0, st>>>(static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), n);
  return hipGetLastError();
}

hipError_t launch_peak_mfma(float* sink, int n_blocks, int iters, hipStream_t st) {
  peak_mfma<<<n_blocks, 256, 0, st>>>(sink, iters);
  return hipGetLastError();
}

hipError_t launch_peak_lds(uint32_t* sink, int n_blocks, int iters, hipStream_t st) {
  peak_lds<<<n_blocks, 256, 0, st>>>(sink, iters);
  return hipGetLastError();
}

hipError_t launch_peak_valu(float* sink, int n_blocks, int iters, hipStream_t st) {
  peak_valu<<<n_blocks, 256, 0, st>>>(sink, iters);
  return hipGetLastError();
}

}  // namespace kvc
