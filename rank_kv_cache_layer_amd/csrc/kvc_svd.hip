// Rank-r factor refresh (KVCMAS Sec. 3.3 Eq. 7, App. B.1 "Factorization and Measurement"):
// Z ~ A B with A = U_r Sigma_r and B = R_r^T, for a batch of fp32 matrices Z [rows][cols].
//
// The pages name no method; this is randomised subspace iteration (Halko, Martinsson & Tropp,
// "Finding structure with randomness", SIAM Review 2011, Alg. 4.4) with a Gaussian sketch of
// l = rank + oversample columns and `power_iters` power iterations.  The bases between power
// iterations take one CholeskyQR round and the final basis Q two (CholeskyQR2, Fukaya et al.
// 2014), each with an fp64 Gram matrix.  Directions whose Cholesky pivot vanishes
// (rank-deficient sketches, e.g. an exactly rank-r Z) are dropped (their basis columns set to
// zero).  The small problem is solved as the symmetric eigenproblem of the l x l Gram matrix of
// Bsk = Q^T Z (fp64) by parallel cyclic Jacobi (Golub & Van Loan, Matrix Computations,
// Sec. 8.5): Bsk Bsk^T = W Lambda W^T, sigma = sqrt(lambda), A = Q W_r Sigma_r,
// B = Sigma_r^-1 W_r^T Bsk.  Each component is signed so that the largest-magnitude entry of its
// left singular vector (column of A) is positive.
//
// Precision: the products that only steer the sketch's span (Z Omega, every Z^T Y, every Z W
// but the last, the one-round CholeskyQR products) run with each fp32 operand split into two
// bf16 parts on the matrix cores (about 16 significant bits); the last Z W, the final
// CholeskyQR2 products, Q^T Z and A run in fp32 on the matrix cores, the Grams, the Cholesky
// factorisation and the eigensolver in fp64.
//
// Kernels: sketch (counter-based Gaussian draws); gemm_bf3_wide / gemm_f32_mfma_wide (narrow
// products, N <= 160), gemm_f32_mfma (wider fp32 products), gemm_f64_tn (split-K fp64 Grams) and
// the VALU GEMMs for the remaining shapes; chol_inv_reg (l <= 160, registers), chol_inv_lds and
// chol_inv (wider); jacobi_step (l <= 192: sweeps in LDS, eigenvector replay spread over the
// device) and jacobi (wider); select_top; the three sign-convention passes.
#include <math.h>

#include <type_traits>

#include <utility>

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef uint16_t bf16_bits;

// ------------------------------------------------------------------ counter-based sketch
// splitmix64 finaliser (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
// OOPSLA 2014), applied to (seed, element index); two 32-bit halves -> Box-Muller normal.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

__global__ void __launch_bounds__(256) sketch(float* om, int64_t count, uint64_t seed) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const uint64_t r = splitmix64(seed ^ splitmix64((uint64_t)i));
  const double u1 = ((double)(uint32_t)(r >> 32) + 1.0) * (1.0 / 4294967296.0);   // (0, 1]
  const double u2 = (double)(uint32_t)r * (1.0 / 4294967296.0);                    // [0, 1)
  om[i] = (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

// ------------------------------------------------------------------ batched tiled GEMM
// C[b] (M x N) = opA(A[b]) (M x K) * opB(B[b]) (K x N), products and sums in ACC.
// opA[i][k] = TRA ? A[k * lda + i] : A[i * lda + k]; opB[k][j] = TRB ? B[j * ldb + k] : B[k * ldb + j].
// 64 x 64 tile per work-group of 256 threads (4 x 4 outputs each), K in steps of 16 through LDS;
// every tail is bounds-checked.
template <typename T> __device__ __forceinline__ double to_d(T x) { return (double)x; }
template <typename T> __device__ __forceinline__ T from_acc(double x);
template <> __device__ __forceinline__ float from_acc<float>(double x) { return (float)x; }
template <> __device__ __forceinline__ double from_acc<double>(double x) { return x; }
template <> __device__ __forceinline__ bf16_bits from_acc<bf16_bits>(double x) {
  return __builtin_bit_cast(bf16_bits, (__bf16)(float)x);
}

template <typename TA, typename TB, typename TC, typename ACC, bool TRA, bool TRB>
__global__ void __launch_bounds__(256) gemm(const TA* __restrict__ A, const TB* __restrict__ B, TC* __restrict__ C,
                                            int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int64_t sA,
                                            int64_t sB, int64_t sC) {
  __shared__ ACC As[16][64 + 1];
  __shared__ ACC Bs[16][64 + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  A += (int64_t)blockIdx.z * sA;
  B += (int64_t)blockIdx.z * sB;
  C += (int64_t)blockIdx.z * sC;
  ACC acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = (ACC)0;
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      int i, k;
      if (TRA) { i = e & 63; k = e >> 6; } else { i = e >> 4; k = e & 15; }
      const int gi = i0 + i, gk = k0 + k;
      ACC x = (ACC)0;
      if (gi < M && gk < K) x = (ACC)(TRA ? A[(int64_t)gk * lda + gi] : A[(int64_t)gi * lda + gk]);
      As[k][i] = x;
      int j, kb;
      if (TRB) { j = e >> 4; kb = e & 15; } else { j = e & 63; kb = e >> 6; }
      const int gj = j0 + j, gkb = k0 + kb;
      ACC y = (ACC)0;
      if (gj < N && gkb < K) y = (ACC)(TRB ? B[(int64_t)gj * ldb + gkb] : B[(int64_t)gkb * ldb + gj]);
      Bs[kb][j] = y;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      ACC a[4], b[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = As[k][ty * 4 + r];
#pragma unroll
      for (int c = 0; c < 4; ++c) b[c] = Bs[k][tx * 4 + c];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fma(a[r], b[c], acc[r][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gi = i0 + ty * 4 + r;
    if (gi >= M) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int gj = j0 + tx * 4 + c;
      if (gj < N) C[(int64_t)gi * ldc + gj] = from_acc<TC>((double)acc[r][c]);
    }
  }
}

// ------------------------------------------------------------------ fp64 GEMM on matrix cores
// C[b] (M x N) = opA(A[b]) (M x K) * opB(B[b]) (K x N) with fp64 products and sums on
// v_mfma_f64_16x16x4_f64 (inputs widened to fp64 as they are loaded, so fp32 products are
// exact).  A work-group of 4 waves owns a 32 x 32 tile of C (2 x 2 blocks of 16 x 16); K goes
// in groups of 16, group g to wave g % 4, and the waves' partial tiles are added in wave order
// at the end.  Inside a group, step s (4 MFMA k-slices) takes k = 4 (l / 16) + s in lane l:
// the same order for both operands, so the sum is unchanged, and a lane's 4 k of a row-major
// operand are contiguous (one vector load).  Element v of a block's result in lane l is
// (4 v + l / 16, l % 16).
typedef double f64x4 __attribute__((ext_vector_type(4)));
template <typename T> struct Vec4;
template <> struct Vec4<float> { typedef float4 type; };
template <> struct Vec4<double> { typedef double4 type; };

// 4 consecutive elements p[0..3] of a row (k < K guarded per element at the tail)
template <typename T>
__device__ __forceinline__ void load4(const T* p, int k, int K, double (&x)[4]) {
  if (k + 3 < K && (reinterpret_cast<uintptr_t>(p) % sizeof(typename Vec4<T>::type)) == 0) {
    const typename Vec4<T>::type v = *reinterpret_cast<const typename Vec4<T>::type*>(p);
    x[0] = (double)v.x; x[1] = (double)v.y; x[2] = (double)v.z; x[3] = (double)v.w;
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] = k + s < K ? to_d(p[s]) : 0.0;
  }
}

template <typename TA, typename TB, typename TC, bool TRA, bool TRB>
__global__ void __launch_bounds__(256) gemm_f64(const TA* __restrict__ A, const TB* __restrict__ B, TC* __restrict__ C,
                                                int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int64_t sA,
                                                int64_t sB, int64_t sC, int lower) {
  __shared__ double red[3][16][64];   // partial tiles of waves 1..3
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15, kq = lane >> 4;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  if (lower && j0 >= i0 + 32) return;   // tile strictly above the diagonal of a Gram nobody reads
  A += (int64_t)blockIdx.z * sA;
  B += (int64_t)blockIdx.z * sB;
  C += (int64_t)blockIdx.z * sC;
  const int ia[2] = {i0 + r16, i0 + 16 + r16}, jb[2] = {j0 + r16, j0 + 16 + r16};
  f64x4 acc[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) acc[t][u] = (f64x4){0.0, 0.0, 0.0, 0.0};
  const int n_groups = (K + 15) / 16;
#pragma unroll 2
  for (int g = wave; g < n_groups; g += 4) {
    const int k = g * 16 + 4 * kq;   // this lane's k at step 0; k + s at step s
    double a[2][4], b[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool in_a = ia[t] < M, in_b = jb[t] < N;
      if (TRA) {
#pragma unroll
        for (int s = 0; s < 4; ++s) a[t][s] = in_a && k + s < K ? to_d(A[(int64_t)(k + s) * lda + ia[t]]) : 0.0;
      } else if (in_a) {
        load4(A + (int64_t)ia[t] * lda + k, k, K, a[t]);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) a[t][s] = 0.0;
      }
      if (!TRB) {
#pragma unroll
        for (int s = 0; s < 4; ++s) b[t][s] = in_b && k + s < K ? to_d(B[(int64_t)(k + s) * ldb + jb[t]]) : 0.0;
      } else if (in_b) {
        load4(B + (int64_t)jb[t] * ldb + k, k, K, b[t]);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) b[t][s] = 0.0;
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[t][u] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[t][s], b[u][s], acc[t][u], 0, 0, 0);
  }
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave - 1][(t * 2 + u) * 4 + v][lane] = acc[t][u][v];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        double x = acc[t][u][v];
#pragma unroll
        for (int w = 0; w < 3; ++w) x += red[w][(t * 2 + u) * 4 + v][lane];
        const int i = i0 + 16 * t + 4 * v + kq, j = j0 + 16 * u + r16;
        if (i < M && j < N) C[(int64_t)i * ldc + j] = from_acc<TC>(x);
      }
}

// four consecutive floats at p + base, of which `avail` exist (the rest read as 0)
__device__ __forceinline__ float4 ld4_guard(const float* p, int64_t base, int avail) {
  if (avail >= 4) return *reinterpret_cast<const float4*>(p + base);
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (avail > 0) v.x = p[base];
  if (avail > 1) v.y = p[base + 1];
  if (avail > 2) v.z = p[base + 2];
  return v;
}

// C (M x N, fp64) = A^T B with A stored [K][M] and B stored [K][N], both fp32 (exact in fp64),
// for M <= 160 (the sketch width: Gram matrices Y^T Y): one work-group holds all M rows x 64
// columns, each wave one 16-column block against the ten 16-row blocks, K in chunks of 16
// through double-buffered LDS.  Every operand is read once per 64 columns.  Split K: work-group
// y sums rows [y kc, (y + 1) kc) of A and B into C + y sP.  With `lower` (a Gram read only below
// its diagonal), row blocks wholly above a wave's columns are skipped and left zero.
constexpr int kTnRows = 160;
__global__ void __launch_bounds__(256) gemm_f64_tn(const float* __restrict__ A, const float* __restrict__ B,
                                                   double* __restrict__ C, int M, int N, int K, int64_t lda,
                                                   int64_t ldb, int64_t ldc, int64_t sA, int64_t sB, int64_t sC,
                                                   int kc, int64_t sP, int lower) {
  constexpr int AQ = kTnRows / 4, NAV = (16 * AQ + 255) / 256;
  __shared__ __attribute__((aligned(16))) float As[2][16][kTnRows + 4];
  __shared__ __attribute__((aligned(16))) float Bs[2][16][64 + 4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, kq = lane >> 4;
  const int j0 = blockIdx.x * 64;
  const int kb = blockIdx.y * kc;
  A += (int64_t)blockIdx.z * sA + (int64_t)kb * lda;
  B += (int64_t)blockIdx.z * sB + (int64_t)kb * ldb;
  C += (int64_t)blockIdx.z * sC + (int64_t)blockIdx.y * sP;
  K = min(K - kb, kc);
  const int t0 = lower ? (j0 + wave * 16) / 16 : 0;   // first row block that meets the lower triangle
  float4 ra[NAV], rb;
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < NAV; ++u) {
      const int idx = tid + 256 * u, k = idx / AQ, m4 = (idx % AQ) * 4;
      ra[u] = (idx < 16 * AQ && k0 + k < K) ? ld4_guard(A, (int64_t)(k0 + k) * lda + m4, M - m4)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int k = tid >> 4, n4 = (tid & 15) * 4;
    rb = (k0 + k < K) ? ld4_guard(B, (int64_t)(k0 + k) * ldb + j0 + n4, N - j0 - n4) : make_float4(0.f, 0.f, 0.f, 0.f);
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NAV; ++u) {
      const int idx = tid + 256 * u, k = idx / AQ, m4 = (idx % AQ) * 4;
      if (idx < 16 * AQ) *reinterpret_cast<float4*>(&As[buf][k][m4]) = ra[u];
    }
    *reinterpret_cast<float4*>(&Bs[buf][tid >> 4][(tid & 15) * 4]) = rb;
  };
  f64x4 acc[kTnRows / 16];
#pragma unroll
  for (int t = 0; t < kTnRows / 16; ++t) acc[t] = (f64x4){0.0, 0.0, 0.0, 0.0};
  load(0);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const bool more = k0 + 16 < K;
    if (more) load(k0 + 16);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = 4 * s + kq;
      const double b = (double)Bs[buf][k][wave * 16 + r16];
#pragma unroll
      for (int t = 0; t < kTnRows / 16; ++t)
        if (t >= t0)
          acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)As[buf][k][16 * t + r16], b, acc[t], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  const int j = j0 + wave * 16 + r16;
  if (j >= N) return;
#pragma unroll
  for (int t = 0; t < kTnRows / 16; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = 16 * t + 4 * v + kq;
      if (i < M) C[(int64_t)i * ldc + j] = acc[t][v];
    }
}

// lower_only: C is a symmetric Gram whose consumers read only its lower triangle (fp64 path):
// tiles strictly above the diagonal are skipped
template <typename TA, typename TB, typename TC, typename ACC, bool TRA, bool TRB>
hipError_t run_gemm(const TA* A, const TB* B, TC* C, int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc,
                    int64_t sA, int64_t sB, int64_t sC, int batch, hipStream_t st, bool lower_only = false) {
  if constexpr (std::is_same<ACC, double>::value && std::is_same<TA, float>::value &&
                std::is_same<TB, float>::value && std::is_same<TC, double>::value && TRA && !TRB) {
    if (M <= kTnRows && lda % 4 == 0 && ldb % 4 == 0 && sA % 4 == 0 && sB % 4 == 0) {
      const dim3 grid((unsigned)((N + 63) / 64), 1u, (unsigned)batch);
      gemm_f64_tn<<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, K, 0, lower_only ? 1 : 0);
      return hipGetLastError();
    }
  }
  if constexpr (std::is_same<ACC, double>::value) {
    const dim3 grid((unsigned)((N + 31) / 32), (unsigned)((M + 31) / 32), (unsigned)batch);
    gemm_f64<TA, TB, TC, TRA, TRB><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC,
                                                         lower_only ? 1 : 0);
  } else {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64), (unsigned)batch);
    gemm<TA, TB, TC, ACC, TRA, TRB><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ fp32 GEMM on matrix cores
// C[b] (M x N, fp32) = opA(A[b]) (M x K) * B[b] (K x N, row-major), fp32 products and sums on
// v_mfma_f32_32x32x2_f32: 128 x 128 tile per work-group of 4 waves (64 x 64 each, 2 x 2 blocks),
// K in chunks of 16 through double-buffered LDS (next chunk loaded into registers while the
// current one is multiplied).  opA = A (row-major, lda) or, with TRA, A^T (A stored K x M).
// Requires lda, ldb, ldc and the batch strides to be multiples of 4 (16-byte vector loads);
// tails in M, N, K are bounds-checked.
typedef float f32x16v __attribute__((ext_vector_type(16)));


template <bool TRA>
__global__ void __launch_bounds__(256) gemm_f32_mfma(const float* __restrict__ A, const float* __restrict__ B,
                                                     float* __restrict__ C, int M, int N, int K, int64_t lda,
                                                     int64_t ldb, int64_t ldc, int64_t sA, int64_t sB, int64_t sC) {
  __shared__ __attribute__((aligned(16))) float As[2][16][128 + 4];   // [buffer][k][m]
  __shared__ __attribute__((aligned(16))) float Bs[2][16][128 + 4];   // [buffer][k][n]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, kh = lane >> 5;
  const int i0 = blockIdx.y * 128, j0 = blockIdx.x * 128;
  A += (int64_t)blockIdx.z * sA;
  B += (int64_t)blockIdx.z * sB;
  C += (int64_t)blockIdx.z * sC;
  float4 ra[2], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + 256 * u;
      if (TRA) {   // A stored [k][m]: 16 rows of 32 float4 along m
        const int k = idx >> 5, m4 = (idx & 31) * 4;
        ra[u] = (k0 + k < K) ? ld4_guard(A, (int64_t)(k0 + k) * lda + i0 + m4, M - i0 - m4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {     // A stored [m][k]: 128 rows of 4 float4 along k
        const int m = idx >> 2, k4 = (idx & 3) * 4;
        ra[u] = (i0 + m < M) ? ld4_guard(A, (int64_t)(i0 + m) * lda + k0 + k4, K - k0 - k4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      const int k = idx >> 5, n4 = (idx & 31) * 4;
      rb[u] = (k0 + k < K) ? ld4_guard(B, (int64_t)(k0 + k) * ldb + j0 + n4, N - j0 - n4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + 256 * u;
      if (TRA) {
        const int k = idx >> 5, m4 = (idx & 31) * 4;
        *reinterpret_cast<float4*>(&As[buf][k][m4]) = ra[u];
      } else {
        const int m = idx >> 2, k4 = (idx & 3) * 4;
        As[buf][k4 + 0][m] = ra[u].x;
        As[buf][k4 + 1][m] = ra[u].y;
        As[buf][k4 + 2][m] = ra[u].z;
        As[buf][k4 + 3][m] = ra[u].w;
      }
      const int k = idx >> 5, n4 = (idx & 31) * 4;
      *reinterpret_cast<float4*>(&Bs[buf][k][n4]) = rb[u];
    }
  };
  f32x16v acc[2][2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[tb][db][j] = 0.f;
  load(0);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const bool more = k0 + 16 < K;
    if (more) load(k0 + 16);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int k = 2 * kk + kh;
      float a[2], b[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) a[tb] = As[buf][k][wm * 64 + tb * 32 + l32];
#pragma unroll
      for (int db = 0; db < 2; ++db) b[db] = Bs[buf][k][wn * 64 + db * 32 + l32];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int db = 0; db < 2; ++db)
          acc[tb][db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[tb], b[db], acc[tb][db], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int j = j0 + wn * 64 + db * 32 + l32;
      if (j >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + wm * 64 + tb * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        if (i < M) C[(int64_t)i * ldc + j] = acc[tb][db][r];
      }
    }
}

// The same product for narrow N (the sketch width l = r + p, at most 160): a 128 x 32 NB tile per
// work-group, each wave 32 rows x all NB column blocks, so no matrix-core work is spent on
// columns past N (a 128 x 128 tile at N = 160 computes 256 columns).
template <bool TRA, int NB, int KC = 16>
__global__ void __launch_bounds__(256) gemm_f32_mfma_wide(const float* __restrict__ A, const float* __restrict__ B,
                                                          float* __restrict__ C, int M, int N, int K, int64_t lda,
                                                          int64_t ldb, int64_t ldc, int64_t sA, int64_t sB,
                                                          int64_t sC) {
  constexpr int BN = 32 * NB, BQ = BN / 4, NBV = (KC * BQ + 255) / 256, NAV = KC / 8;
  __shared__ __attribute__((aligned(16))) float As[2][KC][128 + 4];   // [buffer][k][m]
  __shared__ __attribute__((aligned(16))) float Bs[2][KC][BN + 4];    // [buffer][k][n]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, kh = lane >> 5;
  const int i0 = blockIdx.y * 128, j0 = blockIdx.x * BN;
  A += (int64_t)blockIdx.z * sA;
  B += (int64_t)blockIdx.z * sB;
  C += (int64_t)blockIdx.z * sC;
  float4 ra[NAV], rb[NBV];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < NAV; ++u) {
      const int idx = tid + 256 * u;
      if (TRA) {   // A stored [k][m]: KC rows of 32 float4 along m
        const int k = idx >> 5, m4 = (idx & 31) * 4;
        ra[u] = (k0 + k < K) ? ld4_guard(A, (int64_t)(k0 + k) * lda + i0 + m4, M - i0 - m4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {     // A stored [m][k]: 128 rows of KC / 4 float4 along k
        const int m = idx / (KC / 4), k4 = (idx % (KC / 4)) * 4;
        ra[u] = (i0 + m < M) ? ld4_guard(A, (int64_t)(i0 + m) * lda + k0 + k4, K - k0 - k4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < NBV; ++u) {
      const int idx = tid + 256 * u, k = idx / BQ, n4 = (idx % BQ) * 4;
      rb[u] = (idx < KC * BQ && k0 + k < K) ? ld4_guard(B, (int64_t)(k0 + k) * ldb + j0 + n4, N - j0 - n4)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NAV; ++u) {
      const int idx = tid + 256 * u;
      if (TRA) {
        const int k = idx >> 5, m4 = (idx & 31) * 4;
        *reinterpret_cast<float4*>(&As[buf][k][m4]) = ra[u];
      } else {
        const int m = idx / (KC / 4), k4 = (idx % (KC / 4)) * 4;
        As[buf][k4 + 0][m] = ra[u].x;
        As[buf][k4 + 1][m] = ra[u].y;
        As[buf][k4 + 2][m] = ra[u].z;
        As[buf][k4 + 3][m] = ra[u].w;
      }
    }
#pragma unroll
    for (int u = 0; u < NBV; ++u) {
      const int idx = tid + 256 * u, k = idx / BQ, n4 = (idx % BQ) * 4;
      if (idx < KC * BQ) *reinterpret_cast<float4*>(&Bs[buf][k][n4]) = rb[u];
    }
  };
  f32x16v acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[nb][j] = 0.f;
  load(0);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < K; k0 += KC) {
    const bool more = k0 + KC < K;
    if (more) load(k0 + KC);
    // operands of step kk + 1 are read from LDS before the products of step kk are issued
    float a_cur = As[buf][kh][wave * 32 + l32], b_cur[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b_cur[nb] = Bs[buf][kh][nb * 32 + l32];
#pragma unroll
    for (int kk = 0; kk < KC / 2; ++kk) {
      float a_nxt = 0.f, b_nxt[NB];
      if (kk + 1 < KC / 2) {
        const int k = 2 * kk + 2 + kh;
        a_nxt = As[buf][k][wave * 32 + l32];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) b_nxt[nb] = Bs[buf][k][nb * 32 + l32];
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a_cur, b_cur[nb], acc[nb], 0, 0, 0);
      // keep the next step's LDS reads ahead of this step's products
      __builtin_amdgcn_sched_group_barrier(0x100, NB + 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
      a_cur = a_nxt;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) b_cur[nb] = b_nxt[nb];
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int j = j0 + nb * 32 + l32;
    if (j >= N) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + wave * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (i < M) C[(int64_t)i * ldc + j] = acc[nb][r];
    }
  }
}

// fp32 products: matrix cores when every leading dimension allows 16-byte loads, else VALU
template <bool TRA>
hipError_t gemm_f32(const float* A, const float* B, float* C, int M, int N, int K, int64_t lda, int64_t ldb,
                    int64_t ldc, int64_t sA, int64_t sB, int64_t sC, int batch, hipStream_t st) {
  if (lda % 4 == 0 && ldb % 4 == 0 && sA % 4 == 0 && sB % 4 == 0 && N <= 160) {
    // narrow products (the sketch and power iterations): one column tile of 32 ceil(N / 32)
    const dim3 grid(1u, (unsigned)((M + 127) / 128), (unsigned)batch);
    switch ((N + 31) / 32) {
      case 1: gemm_f32_mfma_wide<TRA, 1><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC); break;
      case 2: gemm_f32_mfma_wide<TRA, 2><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC); break;
      case 3: gemm_f32_mfma_wide<TRA, 3><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC); break;
      case 4: gemm_f32_mfma_wide<TRA, 4><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC); break;
      default: gemm_f32_mfma_wide<TRA, 5><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC); break;
    }
    return hipGetLastError();
  }
  if (lda % 4 == 0 && ldb % 4 == 0 && sA % 4 == 0 && sB % 4 == 0) {
    const dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128), (unsigned)batch);
    gemm_f32_mfma<TRA><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC);
    return hipGetLastError();
  }
  return run_gemm<float, float, float, float, TRA, false>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, st);
}

// The same narrow product on bf16 matrix cores to about 16 significant bits ("bf16x3"): every
// operand is split x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), and
// C = Ahi Bhi + Ahi Blo + Alo Bhi with fp32 sums (v_mfma_f32_32x32x16_bf16); the dropped
// Alo Blo and the split residues stay below about 2^-16 of |a b|.  For products whose result
// only has to keep its span: the power-iteration bases.  A 128 x 32 NB tile per work-group,
// each wave 32 rows x NB column blocks; K in chunks of 32 staged through LDS as bf16 [row][k]
// (the next chunk is loaded into registers while the current one is multiplied).
constexpr int kB3K = 32, kB3Pitch = kB3K + 8;   // 80-byte LDS rows: conflict-free 16-byte reads
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split8(const float* x, uint4& hi, uint4& lo) {
  uint16_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 bh = (__bf16)x[i];
    const __bf16 bl = (__bf16)(x[i] - (float)bh);
    h[i] = __builtin_bit_cast(uint16_t, bh);
    l[i] = __builtin_bit_cast(uint16_t, bl);
  }
  hi = make_uint4(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16, h[4] | (uint32_t)h[5] << 16,
                  h[6] | (uint32_t)h[7] << 16);
  lo = make_uint4(l[0] | (uint32_t)l[1] << 16, l[2] | (uint32_t)l[3] << 16, l[4] | (uint32_t)l[5] << 16,
                  l[6] | (uint32_t)l[7] << 16);
}

template <bool TRA, int NB>
__global__ void __launch_bounds__(256) gemm_bf3_wide(const float* __restrict__ A, const float* __restrict__ B,
                                                     float* __restrict__ C, int M, int N, int K, int64_t lda,
                                                     int64_t ldb, int64_t ldc, int64_t sA, int64_t sB, int64_t sC) {
  constexpr int BN = 32 * NB;
  __shared__ __attribute__((aligned(16))) uint16_t Ah[128][kB3Pitch], Al[128][kB3Pitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bh[BN][kB3Pitch], Bl[BN][kB3Pitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, kh = lane >> 5;
  const int i0 = blockIdx.y * 128, j0 = blockIdx.x * BN;
  A += (int64_t)blockIdx.z * sA;
  B += (int64_t)blockIdx.z * sB;
  C += (int64_t)blockIdx.z * sC;
  // staging: a thread takes 8 consecutive k of one LDS row (a row of A or a column of B), so the
  // 16-byte LDS writes of a wave go to consecutive rows; A stored [m][k] is read as two float4
  // per item, operands stored [k][row] as eight coalesced scalars
  constexpr int NBI = (4 * BN + 255) / 256;   // B items per thread
  float ra[16], rb[8 * NBI];
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  auto put4 = [](float* d, float4 v) {
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
  };
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int it = tid + 256 * u;
      if (TRA) {   // item: row it & 127, k-octet it >> 7
        const int m = it & 127, k = k0 + 8 * (it >> 7);
        const bool in = i0 + m < M;
#pragma unroll
        for (int j = 0; j < 8; ++j) ra[8 * u + j] = (in && k + j < K) ? A[(int64_t)(k + j) * lda + i0 + m] : 0.f;
      } else {     // item: row it >> 2, k-octet it & 3
        const int m = it >> 2, k = k0 + 8 * (it & 3);
        const bool in = i0 + m < M;
        const int64_t base = (int64_t)(i0 + m) * lda + k;
        put4(ra + 8 * u, in ? ld4_guard(A, base, K - k) : z4);
        put4(ra + 8 * u + 4, in ? ld4_guard(A, base + 4, K - k - 4) : z4);
      }
    }
#pragma unroll
    for (int u = 0; u < NBI; ++u) {   // item: column it % BN, k-octet it / BN
      const int it = tid + 256 * u, n = it % BN, k = k0 + 8 * (it / BN);
      const bool in = it < 4 * BN && j0 + n < N;
#pragma unroll
      for (int j = 0; j < 8; ++j) rb[8 * u + j] = (in && k + j < K) ? B[(int64_t)(k + j) * ldb + j0 + n] : 0.f;
    }
  };
  auto store = [&]() {
    uint4 h, l;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int it = tid + 256 * u;
      const int m = TRA ? (it & 127) : (it >> 2), g = TRA ? (it >> 7) : (it & 3);
      split8(ra + 8 * u, h, l);
      *reinterpret_cast<uint4*>(&Ah[m][8 * g]) = h;
      *reinterpret_cast<uint4*>(&Al[m][8 * g]) = l;
    }
#pragma unroll
    for (int u = 0; u < NBI; ++u) {
      const int it = tid + 256 * u;
      if (it < 4 * BN) {
        split8(rb + 8 * u, h, l);
        *reinterpret_cast<uint4*>(&Bh[it % BN][8 * (it / BN)]) = h;
        *reinterpret_cast<uint4*>(&Bl[it % BN][8 * (it / BN)]) = l;
      }
    }
  };
  f32x16v acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[nb][j] = 0.f;
  load(0);
  for (int k0 = 0; k0 < K; k0 += kB3K) {
    __syncthreads();   // every wave is done with the previous chunk
    store();
    __syncthreads();
    if (k0 + kB3K < K) load(k0 + kB3K);
#pragma unroll
    for (int s = 0; s < kB3K / 16; ++s) {
      const int kc = 16 * s + 8 * kh;
      const bf16x8v ah = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(&Ah[wave * 32 + l32][kc]));
      const bf16x8v al = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(&Al[wave * 32 + l32][kc]));
      bf16x8v bh[NB], bl[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        bh[nb] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(&Bh[nb * 32 + l32][kc]));
        bl[nb] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(&Bl[nb * 32 + l32][kc]));
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh[nb], acc[nb], 0, 0, 0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl[nb], acc[nb], 0, 0, 0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh[nb], acc[nb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int j = j0 + nb * 32 + l32;
    if (j >= N) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + wave * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (i < M) C[(int64_t)i * ldc + j] = acc[nb][r];
    }
  }
}

// the same products through gemm_bf3_wide where the operands allow it, else fp32
template <bool TRA>
hipError_t gemm_bf3(const float* A, const float* B, float* C, int M, int N, int K, int64_t lda, int64_t ldb,
                    int64_t ldc, int64_t sA, int64_t sB, int64_t sC, int batch, hipStream_t st) {
  if (!(lda % 4 == 0 && ldb % 4 == 0 && sA % 4 == 0 && sB % 4 == 0 && N <= 160))
    return gemm_f32<TRA>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, st);
  const dim3 grid(1u, (unsigned)((M + 127) / 128), (unsigned)batch);
  switch ((N + 31) / 32) {
    case 1: gemm_bf3_wide<TRA, 1><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC); break;
    case 2: gemm_bf3_wide<TRA, 2><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC); break;
    case 3: gemm_bf3_wide<TRA, 3><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC); break;
    case 4: gemm_bf3_wide<TRA, 4><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC); break;
    default: gemm_bf3_wide<TRA, 5><<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ Gram matrices
// G (fp64, l x l) = Y^T Y for Y [rows][l] fp32; with `lower` only the lower triangle (zero above).  The rows are split
// over `splits` work-groups per column tile so the grid covers the device; their partial sums
// land in `part` and are added in split order (deterministic).
constexpr int kGramSplitMax = 4;
__global__ void __launch_bounds__(256) sum_splits(const double* __restrict__ part, double* __restrict__ G,
                                                  int64_t n, int splits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  double s = part[i];
  for (int y = 1; y < splits; ++y) s += part[(int64_t)y * n + i];
  G[i] = s;
}

hipError_t gram_f64(const float* Y, double* G, double* part, int rows, int l, int b, bool lower, hipStream_t st) {
  const int64_t sY = (int64_t)rows * l, sG = (int64_t)l * l;
  if (l > kTnRows || l % 4)
    return run_gemm<float, float, double, double, true, false>(Y, Y, G, l, l, rows, l, l, l, sY, sY, sG, b, st, lower);
  const int tiles = (l + 63) / 64 * b;
  int splits = std::min(kGramSplitMax, std::max(1, (2048 + tiles - 1) / tiles));
  splits = std::min(splits, std::max(1, rows / 256));
  const int kc = (rows + splits - 1) / splits;
  const dim3 grid((unsigned)((l + 63) / 64), (unsigned)splits, (unsigned)b);
  if (splits == 1) {
    gemm_f64_tn<<<grid, 256, 0, st>>>(Y, Y, G, l, l, rows, l, l, l, sY, sY, sG, rows, 0, lower ? 1 : 0);
    return hipGetLastError();
  }
  const int64_t n = (int64_t)b * sG;
  gemm_f64_tn<<<grid, 256, 0, st>>>(Y, Y, part, l, l, rows, l, l, l, sY, sY, sG, kc, n, lower ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e) return e;
  sum_splits<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(part, G, n, splits);
  return hipGetLastError();
}

// ------------------------------------------------------------------ Cholesky with dropping
// In: G [l][l] (symmetric positive semi-definite Gram matrix, fp64).  Out: Li [l][l] = L^-1
// with G ~ L L^T, rows and columns of dropped pivots zero, so that Y Li^T has orthonormal or
// zero columns.  A pivot is dropped when it falls below `rel_tol` times the largest diagonal
// entry of G.  One work-group per matrix; G is overwritten by L.
__global__ void __launch_bounds__(1024) chol_inv(double* G, double* Li, int l, double rel_tol) {
  __shared__ double diag_max;
  __shared__ double piv;
  __shared__ int dead[256];
  const int tid = threadIdx.x, nt = blockDim.x;
  G += (int64_t)blockIdx.x * l * l;
  Li += (int64_t)blockIdx.x * l * l;
  if (tid == 0) {
    double m = 0.0;
    for (int i = 0; i < l; ++i) m = fmax(m, G[(int64_t)i * l + i]);
    diag_max = m;
  }
  __syncthreads();
  const double tol = rel_tol * diag_max;
  for (int k = 0; k < l; ++k) {
    if (tid == 0) {
      const double d = G[(int64_t)k * l + k];
      const bool drop = !(d > tol);
      dead[k] = drop;
      piv = drop ? 0.0 : sqrt(d);
      G[(int64_t)k * l + k] = drop ? 1.0 : sqrt(d);
    }
    __syncthreads();
    const double p = piv;
    for (int i = k + 1 + tid; i < l; i += nt) G[(int64_t)i * l + k] = p > 0.0 ? G[(int64_t)i * l + k] / p : 0.0;
    __syncthreads();
    // trailing update of the lower triangle: G[i][j] -= L[i][k] L[j][k], k < j <= i
    const int rem = l - k - 1;
    for (int e = tid; e < rem * rem; e += nt) {
      const int i = k + 1 + e / rem, j = k + 1 + e % rem;
      if (j <= i) G[(int64_t)i * l + j] -= G[(int64_t)i * l + k] * G[(int64_t)j * l + k];
    }
    __syncthreads();
  }
  // Li = L^-1 by forward substitution, one column per thread
  for (int c = tid; c < l; c += nt) {
    for (int i = 0; i < c; ++i) Li[(int64_t)i * l + c] = 0.0;
    if (dead[c]) {
      for (int i = c; i < l; ++i) Li[(int64_t)i * l + c] = 0.0;
      continue;
    }
    Li[(int64_t)c * l + c] = 1.0 / G[(int64_t)c * l + c];
    for (int i = c + 1; i < l; ++i) {
      double s = 0.0;
      for (int k = c; k < i; ++k) s += G[(int64_t)i * l + k] * Li[(int64_t)k * l + c];
      Li[(int64_t)i * l + c] = dead[i] ? 0.0 : -s / G[(int64_t)i * l + i];
    }
  }
  __syncthreads();
  // dropped directions contribute nothing: zero their rows
  for (int e = tid; e < l * l; e += nt)
    if (dead[e / l]) Li[e] = 0.0;
}

// Same factorisation and inverse with L resident in LDS as its packed lower triangle (fp64),
// for l up to kJacobiLdsMax.  Right-looking Cholesky with dropping: step k takes the pivot,
// scales column k (kept in `col`) and updates the trailing lower triangle row by row (one wave
// per row, lanes along the row).  Then the inverse X = L^-1 in place by forward elimination of
// [L | I]: step k divides row k of X (columns <= k) by L_kk and subtracts L_ik times it from
// every later row i, so each step is one parallel rank-1 update; row i's X entries take the
// places of L entries already used (column c of L is last read at step c).  A dropped pivot
// gets X_kk = 0 and a zero column below it, which zeroes its row and column of the inverse.
// Li is written in full (upper triangle zero).
__global__ void __launch_bounds__(1024) chol_inv_lds(const double* G, double* Li, int l, double rel_tol) {
  extern __shared__ double T[];   // packed lower triangle: entry (i, j), j <= i, at ro[i] + j
  __shared__ double col[256];
  __shared__ double diag_max;
  __shared__ int ro[256];
  __shared__ int dead[256];
  const int tid = threadIdx.x, nt = blockDim.x, wave = tid >> 6, lane = tid & 63, nw = nt >> 6;
  G += (int64_t)blockIdx.x * l * l;
  Li += (int64_t)blockIdx.x * l * l;
  for (int i = tid; i < l; i += nt) ro[i] = i * (i + 1) / 2;
  for (int i = wave; i < l; i += nw)
    for (int j = lane; j <= i; j += 64) T[i * (i + 1) / 2 + j] = G[(int64_t)i * l + j];
  __syncthreads();
  if (tid == 0) {
    double m = 0.0;
    for (int i = 0; i < l; ++i) m = fmax(m, T[ro[i] + i]);
    diag_max = m;
  }
  __syncthreads();
  const double tol = rel_tol * diag_max;
  for (int k = 0; k < l; ++k) {
    const double d = T[ro[k] + k];   // every thread: the same value
    const bool drop = !(d > tol);
    const double piv = drop ? 0.0 : sqrt(d);
    for (int i = k + 1 + tid; i < l; i += nt) {
      const double x = drop ? 0.0 : T[ro[i] + k] / piv;
      T[ro[i] + k] = x;
      col[i] = x;
    }
    __syncthreads();   // column k complete; every thread has read the pivot
    if (tid == 0) {
      dead[k] = drop;
      T[ro[k] + k] = drop ? 1.0 : piv;
    }
    for (int i = k + 1 + wave; i < l; i += nw) {
      const double ci = col[i];
      const int r = ro[i];
      for (int j = k + 1 + lane; j <= i; j += 64) T[r + j] -= ci * col[j];
    }
    __syncthreads();
  }
  // inverse by forward elimination
  for (int k = 0; k < l; ++k) {
    const double xkk = dead[k] ? 0.0 : 1.0 / T[ro[k] + k];   // every thread: the same value
    const int rk = ro[k];
    for (int c = tid; c < k; c += nt) T[rk + c] *= xkk;
    for (int i = k + 1 + tid; i < l; i += nt) col[i] = T[ro[i] + k];   // L_ik, about to be replaced
    __syncthreads();   // row k of X final (but X_kk); every thread has read L_kk
    if (tid == 0) T[rk + k] = xkk;
    for (int i = k + 1 + wave; i < l; i += nw) {
      const double li = col[i];
      const int r = ro[i];
      for (int c = lane; c < k; c += 64) T[r + c] -= li * T[rk + c];
      if (lane == 0) T[r + k] = -li * xkk;
    }
    __syncthreads();
  }
  for (int i = wave; i < l; i += nw) {
    const int r = ro[i];
    for (int j = lane; j < l; j += 64) Li[(int64_t)i * l + j] = j <= i ? T[r + j] : 0.0;
  }
}

// The same factorisation and inverse for l <= kCholRegMax with both L (as the trailing Gram
// block) and X = L^-1 in registers: thread (a, b) of 16 x 32 holds entries (a + 16 u, b + 32 v),
// u < 10, v < 5, of the full symmetric T and of X, so a step moves only one column of L and one
// row of X through LDS.  Step k: the sixteen threads holding column k of T take the pivot
// (dropped below rel_tol times the largest diagonal entry of G) and publish
// L[:, k] = T[:, k] / L_kk below the diagonal and L_kk (0 when dropped); the threads holding
// row k of X publish it unscaled.  After one barrier every thread applies the trailing update
// T_ij -= L_ik L_jk (i, j > k) and the forward elimination X_i. -= L_ik X_k. / L_kk (i > k), and
// row k of X is divided by L_kk (zeroed for a dropped pivot, which also leaves its column of X
// zero).  The buffers alternate between steps, so one barrier per step suffices.  The steps
// run in blocks of 16 with the block index a template argument, so every register index is a
// constant and the register blocks wholly before the step are skipped at compile time.
// Writes LiT [l][l] (fp32) = (L^-1)^T, the right operand of Y (L^-1)^T.
constexpr int kCholRegMax = 160;
constexpr int kCholNU = kCholRegMax / 16, kCholNV = kCholRegMax / 32;
struct CholShared {
  double colb[2][kCholRegMax], rowb[2][kCholRegMax], lkk[2];
};

template <int KU>
__device__ __forceinline__ void chol_steps(double (&T)[kCholNU][kCholNV], double (&X)[kCholNU][kCholNV],
                                           CholShared& sh, int l, double tol, int a, int b, int lane) {
  constexpr int KV = KU >> 1;
  for (int kk = 0; kk < 16; ++kk) {
    const int k = 16 * KU + kk, buf = k & 1;
    if (k >= l) return;
    // pivot from lane a == kk of this thread's 16-lane group (the group shares b)
    const double d = __shfl(T[KU][KV], (lane & 48) | kk, 64);
    if (b == (k & 31)) {
      const bool drop = !(d > tol);
      const double piv = drop ? 0.0 : sqrt(d);
      const double rp = drop ? 0.0 : 1.0 / piv;
#pragma unroll
      for (int u = KU; u < kCholNU; ++u) {
        const int i = a + 16 * u;
        if (i > k && i < l) sh.colb[buf][i] = T[u][KV] * rp;
      }
      if (a == kk) sh.lkk[buf] = piv;
    }
    if (a == kk) {
#pragma unroll
      for (int v = 0; v < kCholNV; ++v) {
        const int j = b + 32 * v;
        if (j < l) sh.rowb[buf][j] = X[KU][v];
      }
    }
    __syncthreads();
    const double lk = sh.lkk[buf];
    const double inv = lk > 0.0 ? 1.0 / lk : 0.0;
    double cc[kCholNV], rw[kCholNV];
#pragma unroll
    for (int v = 0; v < kCholNV; ++v) {
      const int j = b + 32 * v;
      cc[v] = (v >= KV && j > k && j < l) ? sh.colb[buf][j] : 0.0;
      rw[v] = (v <= KV && j <= k) ? sh.rowb[buf][j] * inv : 0.0;
    }
#pragma unroll
    for (int u = KU; u < kCholNU; ++u) {
      const int i = a + 16 * u;
      const double cr = (i > k && i < l) ? sh.colb[buf][i] : 0.0;
#pragma unroll
      for (int v = KV; v < kCholNV; ++v) T[u][v] -= cr * cc[v];
#pragma unroll
      for (int v = 0; v <= KV; ++v) X[u][v] -= cr * rw[v];
    }
    if (a == kk) {
#pragma unroll
      for (int v = 0; v <= KV; ++v) X[KU][v] = rw[v];
    }
  }
}

template <int... KU>
__device__ __forceinline__ void chol_all(double (&T)[kCholNU][kCholNV], double (&X)[kCholNU][kCholNV],
                                         CholShared& sh, int l, double tol, int a, int b, int lane,
                                         std::integer_sequence<int, KU...>) {
  (chol_steps<KU>(T, X, sh, l, tol, a, b, lane), ...);
}

__global__ void __launch_bounds__(512) chol_inv_reg(const double* G, float* LiT, int l, double rel_tol) {
  __shared__ CholShared sh;
  __shared__ double diag_max;
  const int tid = threadIdx.x, a = tid & 15, b = tid >> 4, lane = tid & 63;
  G += (int64_t)blockIdx.x * l * l;
  LiT += (int64_t)blockIdx.x * l * l;
  double T[kCholNU][kCholNV], X[kCholNU][kCholNV];
#pragma unroll
  for (int u = 0; u < kCholNU; ++u)
#pragma unroll
    for (int v = 0; v < kCholNV; ++v) {
      const int i = a + 16 * u, j = b + 32 * v;
      const bool in = i < l && j < l;
      T[u][v] = in ? (i >= j ? G[(int64_t)i * l + j] : G[(int64_t)j * l + i]) : 0.0;   // lower triangle
      X[u][v] = (in && i == j) ? 1.0 : 0.0;
    }
  if (tid < 64) {
    double m = 0.0;
    for (int i = lane; i < l; i += 64) m = fmax(m, G[(int64_t)i * l + i]);
    for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
    if (lane == 0) diag_max = m;
  }
  __syncthreads();
  chol_all(T, X, sh, l, rel_tol * diag_max, a, b, lane, std::make_integer_sequence<int, kCholNU>());
#pragma unroll
  for (int u = 0; u < kCholNU; ++u)
#pragma unroll
    for (int v = 0; v < kCholNV; ++v) {
      const int i = a + 16 * u, j = b + 32 * v;
      if (i < l && j < l) LiT[(int64_t)j * l + i] = (float)X[u][v];
    }
}

// ------------------------------------------------------------------ Jacobi eigensolver
// Symmetric A [l][l] (fp64, overwritten; its diagonal ends as the eigenvalues) and V [l][l]
// (out: eigenvectors as columns).  Parallel cyclic Jacobi with round-robin pairing: each round
// rotates l/2 disjoint index pairs, (c, s) from Golub & Van Loan's symmetric 2x2 Schur step,
// A <- J^T A J, V <- V J.  Sweeps until the off-diagonal mass is below tol^2 of the total, or
// max_sweeps.  One work-group per matrix.
__global__ void __launch_bounds__(1024) jacobi(double* A, double* V, int l, int max_sweeps, double tol) {
  __shared__ double cs[128], sn[128];
  __shared__ int pp[128], qq[128];
  __shared__ double red[2][32];
  __shared__ int done;
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 31, warp = tid >> 5;
  A += (int64_t)blockIdx.x * l * l;
  V += (int64_t)blockIdx.x * l * l;
  for (int e = tid; e < l * l; e += nt) V[e] = (e / l == e % l) ? 1.0 : 0.0;
  const int lp = (l + 1) & ~1, half = lp / 2;
  __syncthreads();
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    // convergence test
    double off = 0.0, tot = 0.0;
    for (int e = tid; e < l * l; e += nt) {
      const double x = A[e] * A[e];
      tot += x;
      if (e / l != e % l) off += x;
    }
    for (int o = 16; o >= 1; o >>= 1) {
      off += __shfl_xor(off, o, 32);
      tot += __shfl_xor(tot, o, 32);
    }
    if (lane == 0) {
      red[0][warp] = off;
      red[1][warp] = tot;
    }
    __syncthreads();
    if (tid == 0) {
      double o = 0.0, t = 0.0;
      for (int w = 0; w < (nt + 31) / 32; ++w) {
        o += red[0][w];
        t += red[1][w];
      }
      done = !(o > tol * tol * t);
    }
    __syncthreads();
    if (done) break;
    for (int round = 0; round < lp - 1; ++round) {
      if (tid < half) {
        auto pos = [&](int x) { return x == 0 ? 0 : 1 + (x - 1 + round) % (lp - 1); };
        int p = pos(tid), q = pos(lp - 1 - tid);
        if (p > q) { const int t = p; p = q; q = t; }
        double c = 1.0, s = 0.0;
        if (q < l) {
          const double apq = A[(int64_t)p * l + q];
          if (apq != 0.0) {
            const double tau = (A[(int64_t)q * l + q] - A[(int64_t)p * l + p]) / (2.0 * apq);
            const double t = tau >= 0.0 ? 1.0 / (tau + sqrt(1.0 + tau * tau)) : -1.0 / (-tau + sqrt(1.0 + tau * tau));
            c = 1.0 / sqrt(1.0 + t * t);
            s = t * c;
          }
        }
        pp[tid] = p;
        qq[tid] = q < l ? q : p;
        cs[tid] = c;
        sn[tid] = q < l ? s : 0.0;
      }
      __syncthreads();
      for (int e = tid; e < half * l; e += nt) {   // rows: A <- J^T A
        const int k = e / l, j = e % l, p = pp[k], q = qq[k];
        if (p == q) continue;
        const double c = cs[k], s = sn[k], x = A[(int64_t)p * l + j], y = A[(int64_t)q * l + j];
        A[(int64_t)p * l + j] = c * x - s * y;
        A[(int64_t)q * l + j] = s * x + c * y;
      }
      __syncthreads();
      for (int e = tid; e < half * l; e += nt) {   // columns: A <- A J, V <- V J
        const int k = e / l, i = e % l, p = pp[k], q = qq[k];
        if (p == q) continue;
        const double c = cs[k], s = sn[k];
        const double x = A[(int64_t)i * l + p], y = A[(int64_t)i * l + q];
        A[(int64_t)i * l + p] = c * x - s * y;
        A[(int64_t)i * l + q] = s * x + c * y;
        const double vx = V[(int64_t)i * l + p], vy = V[(int64_t)i * l + q];
        V[(int64_t)i * l + p] = c * vx - s * vy;
        V[(int64_t)i * l + q] = s * vx + c * vy;
      }
      __syncthreads();
    }
  }
}

// Same eigenproblem with the matrix resident in LDS as its packed lower triangle (index
// i (i + 1) / 2 + j, j <= i; fp64), for l up to kJacobiLdsMax.  The eigenvector accumulation is
// taken off the one work-group that owns a matrix, and overlapped with it:
//  - sweep blocks (one 1024-thread work-group per matrix) run up to kJacobiChunkSweeps sweeps
//    on the triangle.  A round rotates the l/2 disjoint pairs at once: the thread that computes
//    pair P's rotation turns its diagonal block into diag(a'_pp, a'_qq) (a'_pq = 0), then each
//    2 x 2 block between two pairs P, Q (stored once, P > Q) becomes J_P^T B J_Q.  Every round's (c, s) go to a rotation log; the
//    triangle is kept in global memory between launches.
//  - replay blocks replay the previous launch's log on VT (row k = eigenvector k): V <- V J acts
//    on rows p and q of VT independently in every column, so a work-group takes kApplyCols
//    columns of one matrix into LDS and applies all logged rounds to them.
// Launch c runs sweep chunk c and replays chunk c - 1 (two logs alternate); the host launches
// ceil(max_sweeps / kJacobiChunkSweeps) + 1 of them and chunks after convergence return at once.
// Per-matrix state: [0] converged (or out of sweeps), [1 + buffer] rounds logged in that
// buffer, [3] sweeps done.  An odd l is padded with a zero row that is never rotated.
constexpr int kJacobiLdsMax = 192;
constexpr int kJacobiChunkSweeps = 2;
constexpr int kApplyCols = 64, kApplyPitch = kApplyCols + 1, kApplyGroups = 1024 / kApplyCols;
__device__ __forceinline__ int tri(int i, int j) { return i >= j ? i * (i + 1) / 2 + j : j * (j + 1) / 2 + i; }

// Round-robin pairing (lp even): position 0 stays, positions 1 .. lp-1 advance by one each
// round; round `round` (0 .. lp-2) pairs position k with position lp-1-k.  Returns p < q.
__device__ __forceinline__ void jacobi_pair(int k, int round, int lp, int& p, int& q) {
  auto pos = [&](int x) {
    if (x == 0) return 0;
    int v = x - 1 + round;   // < 2 (lp - 1)
    if (v >= lp - 1) v -= lp - 1;
    return 1 + v;
  };
  p = pos(k);
  q = pos(lp - 1 - k);
  if (p > q) {
    const int t = p;
    p = q;
    q = t;
  }
}

__device__ __forceinline__ int tri_row(int e) {   // i with i (i + 1) / 2 <= e < (i + 1) (i + 2) / 2
  int i = (int)((sqrt(8.0 * e + 1.0) - 1.0) * 0.5);
  while (i * (i + 1) / 2 > e) --i;
  while ((i + 1) * (i + 2) / 2 <= e) ++i;
  return i;
}

__host__ __device__ size_t jacobi_log_pairs(int l) {   // (c, s) entries per matrix and log buffer
  const size_t lp = (l + 1) & ~1;
  return (size_t)kJacobiChunkSweeps * (lp - 1) * (lp / 2);
}

__device__ void jacobi_sweeps(double* T, double* A, double* Tg, double2* rot, int* stt, int l, int first, int buf,
                              int max_sweeps, double tol) {
  __shared__ double2 csn[kJacobiLdsMax / 2];   // (c, s) of pair k this round
  __shared__ int4 pq[kJacobiLdsMax / 2];       // (p, q, p (p + 1) / 2, q (q + 1) / 2) of pair k this round
  __shared__ double red[2][32];
  __shared__ int done;
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 31, warp = tid >> 5;
  const int lp = (l + 1) & ~1, half = lp / 2, ntri = lp * (lp + 1) / 2;
  if (!first && stt[0]) {
    if (tid == 0) stt[1 + buf] = 0;
    return;
  }
  const int swept = first ? 0 : stt[3];
  for (int e = tid; e < ntri; e += nt) {
    if (first) {
      const int i = tri_row(e), j = e - i * (i + 1) / 2;
      T[e] = (i < l && j < l) ? A[(int64_t)i * l + j] : 0.0;
    } else {
      T[e] = Tg[e];
    }
  }
  const int nblk = half * (half - 1) / 2;
  // this thread's off-diagonal rotation-pair blocks (K1, K2), K2 < K1 (index e = K1 (K1 - 1) / 2
  // + K2), decoded once: with 1024 threads and half <= kJacobiLdsMax / 2, at most 5 per thread.
  // The diagonal block of each pair is rotated by the thread that computes the pair's rotation.
  constexpr int kMaxBlk = 5;
  static_assert((kJacobiLdsMax / 2) * (kJacobiLdsMax / 2 - 1) / 2 <= kMaxBlk * 1024, "blocks per thread");
  int bk1[kMaxBlk], bk2[kMaxBlk];
#pragma unroll
  for (int c = 0; c < kMaxBlk; ++c) {
    const int e = tid + c * nt;
    const int k1 = tri_row(e) + 1;   // K1 (K1 - 1) / 2 <= e < K1 (K1 + 1) / 2
    bk1[c] = e < nblk ? k1 : -1;
    bk2[c] = e - k1 * (k1 - 1) / 2;
  }
  __syncthreads();
  int sweeps = 0, logged = 0;
  bool conv = false;
  for (; sweeps < kJacobiChunkSweeps && swept + sweeps < max_sweeps; ++sweeps) {
    double off = 0.0, tot = 0.0;
    for (int e = tid; e < ntri; e += nt) {
      const int i = tri_row(e), j = e - i * (i + 1) / 2;
      const double x = T[e] * T[e];
      if (i == j) tot += x;
      else { off += 2.0 * x; tot += 2.0 * x; }
    }
    for (int o = 16; o >= 1; o >>= 1) {
      off += __shfl_xor(off, o, 32);
      tot += __shfl_xor(tot, o, 32);
    }
    if (lane == 0) {
      red[0][warp] = off;
      red[1][warp] = tot;
    }
    __syncthreads();
    if (tid == 0) {
      double o = 0.0, t = 0.0;
      for (int w = 0; w < (nt + 31) / 32; ++w) {
        o += red[0][w];
        t += red[1][w];
      }
      done = !(o > tol * tol * t);
    }
    __syncthreads();
    if (done) {
      conv = true;
      break;
    }
    for (int round = 0; round < lp - 1; ++round, ++logged) {
      if (tid < half) {
        int p, q;
        jacobi_pair(tid, round, lp, p, q);
        const int rp = p * (p + 1) / 2, rq = q * (q + 1) / 2;
        double c = 1.0, s = 0.0;
        if (q < l) {
          const double app = T[rp + p], aqq = T[rq + q], apq = T[rq + p];
          if (apq != 0.0) {
            const double tau = (aqq - app) / (2.0 * apq);
            const double t = tau >= 0.0 ? 1.0 / (tau + sqrt(1.0 + tau * tau)) : -1.0 / (-tau + sqrt(1.0 + tau * tau));
            c = 1.0 / sqrt(1.0 + t * t);
            s = t * c;
            // the pair's own 2 x 2 diagonal block: J^T B J = diag(a'_pp, a'_qq)
            T[rp + p] = c * c * app - 2.0 * c * s * apq + s * s * aqq;
            T[rq + q] = s * s * app + 2.0 * c * s * apq + c * c * aqq;
            T[rq + p] = 0.0;
          }
        }
        pq[tid] = make_int4(p, q, rp, rq);
        csn[tid] = make_double2(c, s);
        rot[(int64_t)logged * half + tid] = make_double2(c, s);
      }
      __syncthreads();
      // the blocks of one round are disjoint: read a group of blocks first, then write them
      auto blocks = [&](auto c0_, auto c1_) {
        constexpr int c0 = decltype(c0_)::value, c1 = decltype(c1_)::value;
        double b[c1 - c0][4];
        int ix[c1 - c0][4];
#pragma unroll
        for (int c = c0; c < c1; ++c) {   // block (K1, K2), K2 < K1
          const int k1 = bk1[c], k2 = bk2[c];
          if (k1 < 0) continue;
          const int4 r1 = pq[k1], r2 = pq[k2];
          // packed index of (i, j) from the row offsets: the larger index owns the row
          auto at = [](int i, int ri, int j, int rj) { return i >= j ? ri + j : rj + i; };
          int* x = ix[c - c0];
          x[0] = at(r1.x, r1.z, r2.x, r2.z);
          x[1] = at(r1.x, r1.z, r2.y, r2.w);
          x[2] = at(r1.y, r1.w, r2.x, r2.z);
          x[3] = at(r1.y, r1.w, r2.y, r2.w);
#pragma unroll
          for (int u = 0; u < 4; ++u) b[c - c0][u] = T[x[u]];
        }
#pragma unroll
        for (int c = c0; c < c1; ++c) {
          const int k1 = bk1[c], k2 = bk2[c];
          if (k1 < 0) continue;
          const int* x = ix[c - c0];
          const double* v = b[c - c0];
          const double2 j1 = csn[k1], j2 = csn[k2];
          const double c1v = j1.x, s1 = j1.y, c2 = j2.x, s2 = j2.y;
          // B rows {p1, q1}, columns {p2, q2}; B' = J1^T B J2
          const double r00 = c1v * v[0] - s1 * v[2], r01 = c1v * v[1] - s1 * v[3];
          const double r10 = s1 * v[0] + c1v * v[2], r11 = s1 * v[1] + c1v * v[3];
          T[x[0]] = c2 * r00 - s2 * r01;
          T[x[1]] = s2 * r00 + c2 * r01;
          T[x[2]] = c2 * r10 - s2 * r11;
          T[x[3]] = s2 * r10 + c2 * r11;
        }
      };
      blocks(std::integral_constant<int, 0>(), std::integral_constant<int, 3>());
      blocks(std::integral_constant<int, 3>(), std::integral_constant<int, kMaxBlk>());
      __syncthreads();
    }
  }
  for (int e = tid; e < ntri; e += nt) Tg[e] = T[e];
  for (int i = tid; i < l; i += nt) A[(int64_t)i * l + i] = T[tri(i, i)];
  if (tid == 0) {
    stt[0] = conv || swept + sweeps >= max_sweeps;
    stt[1 + buf] = logged;
    stt[3] = swept + sweeps;
  }
}

// Replays `rounds` logged rounds on kApplyCols columns of VT (identity before the first
// chunk): thread (column, group g) applies the rotations of pairs g, g + kApplyGroups, ... of
// every round, the round's rows read first (its pairs are disjoint), then written; the next
// round's (c, s) are loaded while this one is applied.
__device__ void jacobi_replay(double* Vs, double* VT, const double2* __restrict__ rot, int rounds, int l, int c0,
                              int first) {
  const int tid = threadIdx.x, col = tid % kApplyCols, g = tid / kApplyCols;
  const int lp = (l + 1) & ~1, half = lp / 2, ncyc = lp - 1;
  const int gc = c0 + col;
  for (int i = g; i < l; i += kApplyGroups)
    Vs[i * kApplyPitch + col] = first ? (i == gc ? 1.0 : 0.0) : (gc < l ? VT[(int64_t)i * l + gc] : 0.0);
  constexpr int kMaxPairs = (kJacobiLdsMax / 2 + kApplyGroups - 1) / kApplyGroups;
  double2 nxt[kMaxPairs];
  auto fetch = [&](int r) {
#pragma unroll
    for (int u = 0; u < kMaxPairs; ++u) {
      const int k = g + u * kApplyGroups;
      nxt[u] = (r < rounds && k < half) ? rot[(int64_t)r * half + k] : make_double2(1.0, 0.0);
    }
  };
  fetch(0);
  __syncthreads();
  int round = 0;
  for (int r = 0; r < rounds; ++r) {
    double2 cur[kMaxPairs];
#pragma unroll
    for (int u = 0; u < kMaxPairs; ++u) cur[u] = nxt[u];
    fetch(r + 1);
    int pi[kMaxPairs], qi[kMaxPairs];
    double x[kMaxPairs], y[kMaxPairs];
#pragma unroll
    for (int u = 0; u < kMaxPairs; ++u) {
      const int k = g + u * kApplyGroups;
      int p = 0, q = l;
      if (k < half) jacobi_pair(k, round, lp, p, q);
      pi[u] = p;
      qi[u] = q;
      if (q < l) {
        x[u] = Vs[p * kApplyPitch + col];
        y[u] = Vs[q * kApplyPitch + col];
      }
    }
#pragma unroll
    for (int u = 0; u < kMaxPairs; ++u) {
      if (qi[u] >= l) continue;
      const double c = cur[u].x, s = cur[u].y;
      Vs[pi[u] * kApplyPitch + col] = c * x[u] - s * y[u];
      Vs[qi[u] * kApplyPitch + col] = s * x[u] + c * y[u];
    }
    __syncthreads();
    if (++round == ncyc) round = 0;
  }
  if (gc < l)
    for (int i = g; i < l; i += kApplyGroups) VT[(int64_t)i * l + gc] = Vs[i * kApplyPitch + col];
}

// Launch c: work-groups [0, b) run sweep chunk c (c < n_chunks), the next b * ceil(l /
// kApplyCols) replay chunk c - 1 (c >= 1) on their column slices.
__global__ void __launch_bounds__(1024) jacobi_step(double* A, double* Tg, double* VT, double2* rot, int* state,
                                                    int l, int b, int c, int n_chunks, int max_sweeps, double tol) {
  extern __shared__ double lds[];
  const size_t per = jacobi_log_pairs(l);
  const int nsl = (l + kApplyCols - 1) / kApplyCols;
  if ((int)blockIdx.x < b) {
    if (c >= n_chunks) return;
    const int m = blockIdx.x, lp = (l + 1) & ~1;
    jacobi_sweeps(lds, A + (int64_t)m * l * l, Tg + (int64_t)m * (lp * (lp + 1) / 2),
                  rot + ((size_t)(c & 1) * b + m) * per, state + 4 * m, l, c == 0, c & 1, max_sweeps, tol);
  } else {
    if (c == 0) return;
    const int w = blockIdx.x - b, m = w / nsl, sl = w % nsl, pb = (c - 1) & 1;
    const int rounds = state[4 * m + 1 + pb];
    if (c - 1 > 0 && rounds == 0) return;
    jacobi_replay(lds, VT + (int64_t)m * l * l, rot + ((size_t)pb * b + m) * per, rounds, l, sl * kApplyCols,
                  c - 1 == 0);
  }
}

// ------------------------------------------------------------------ top-r selection
// From the eigenpairs (diag of E, columns of V) of matrix b: sigma_i = sqrt(lambda_(i)) for the
// r largest eigenvalues in descending order (ties by index), M1 = V_r Sigma_r [l][r] and
// M2 = Sigma_r^-1 V_r^T [r][l] (zero rows for sigma = 0); M1f is M1 rounded to fp32.
__global__ void __launch_bounds__(256) select_top(const double* E, const double* V, float* sigma, double* M1,
                                                  float* M1f, double* M2, int l, int r, int v_transposed) {
  __shared__ int order[256];
  __shared__ double sig[256];
  const int tid = threadIdx.x;
  E += (int64_t)blockIdx.x * l * l;
  V += (int64_t)blockIdx.x * l * l;
  M1 += (int64_t)blockIdx.x * l * r;
  M1f += (int64_t)blockIdx.x * l * r;
  M2 += (int64_t)blockIdx.x * r * l;
  sigma += (int64_t)blockIdx.x * r;
  for (int i = tid; i < l; i += blockDim.x) {
    const double li = E[(int64_t)i * l + i];
    int rank = 0;
    for (int j = 0; j < l; ++j) {
      const double lj = E[(int64_t)j * l + j];
      rank += (lj > li) || (lj == li && j < i);
    }
    if (rank < r) {
      order[rank] = i;
      sig[rank] = sqrt(fmax(li, 0.0));
    }
  }
  __syncthreads();
  for (int i = tid; i < r; i += blockDim.x) sigma[i] = (float)sig[i];
  for (int e = tid; e < l * r; e += blockDim.x) {
    const int row = e / r, c = e % r;
    const double x = (v_transposed ? V[(int64_t)order[c] * l + row] : V[(int64_t)row * l + order[c]]) * sig[c];
    M1[e] = x;
    M1f[e] = (float)x;
  }
  for (int e = tid; e < r * l; e += blockDim.x) {
    const int c = e / l, col = e % l;
    const double vv = v_transposed ? V[(int64_t)order[c] * l + col] : V[(int64_t)col * l + order[c]];
    M2[e] = sig[c] > 0.0 ? vv / sig[c] : 0.0;
  }
}

// ------------------------------------------------------------------ sign convention
// Component c of matrix b: if the largest-magnitude entry of A[:, c] (the lowest row among
// equals) is negative, A[:, c] and B[c, :] are negated.  Three passes so the row scan covers the
// device: sign_partial reduces row slices (kSignSplits per matrix, 64 columns per work-group,
// coalesced rows), sign_decide merges the slices in row order, sign_negate flips the flagged
// entries of A and B.
template <typename T>
__device__ __forceinline__ double sign_val(T v) {
  if constexpr (sizeof(T) == 2) return (double)__builtin_bit_cast(__bf16, (uint16_t)v);
  else return (double)v;
}
template <typename T>
__device__ __forceinline__ T negated(T v) {
  if constexpr (sizeof(T) == 2) return (T)(v ^ 0x8000u);
  else return -v;
}

constexpr int kSignSplits = 16;
struct SignPart {
  double mag;
  int idx, neg;
};
// (mag, idx) beats (bm, bi): larger magnitude, or equal magnitude at a lower row
__device__ __forceinline__ bool sign_better(double mag, int idx, double bm, int bi) {
  return mag > bm || (mag == bm && idx < bi);
}

template <typename T>
__global__ void __launch_bounds__(256) sign_partial(const T* __restrict__ A, SignPart* __restrict__ part, int rows,
                                                    int r) {
  __shared__ double bv[4][64];
  __shared__ int bi[4][64], bn[4][64];
  const int tid = threadIdx.x, cl = tid & 63, ph = tid >> 6;
  const int c = blockIdx.x * 64 + cl;
  const int rs = (rows + kSignSplits - 1) / kSignSplits, r0 = blockIdx.y * rs, r1 = min(rows, r0 + rs);
  A += (int64_t)blockIdx.z * rows * r;
  double best = -1.0;
  int bidx = 0, neg = 0;
  if (c < r) {
    for (int i = r0 + ph; i < r1; i += 4) {
      const double x = sign_val(A[(int64_t)i * r + c]);
      if (fabs(x) > best) {
        best = fabs(x);
        bidx = i;
        neg = x < 0.0;
      }
    }
  }
  bv[ph][cl] = best;
  bi[ph][cl] = bidx;
  bn[ph][cl] = neg;
  __syncthreads();
  if (ph == 0 && c < r) {
    for (int q = 1; q < 4; ++q) {
      if (sign_better(bv[q][cl], bi[q][cl], best, bidx)) {
        best = bv[q][cl];
        bidx = bi[q][cl];
        neg = bn[q][cl];
      }
    }
    SignPart o;
    o.mag = best;
    o.idx = bidx;
    o.neg = neg;
    part[((int64_t)blockIdx.z * kSignSplits + blockIdx.y) * r + c] = o;
  }
}

__global__ void __launch_bounds__(256) sign_decide(const SignPart* __restrict__ part, int* __restrict__ flag, int r,
                                                   int n_mats) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_mats * r) return;
  const int z = i / r, c = i % r;
  double best = -1.0;
  int bidx = 0, neg = 0;
  for (int y = 0; y < kSignSplits; ++y) {
    const SignPart p = part[((int64_t)z * kSignSplits + y) * r + c];
    if (sign_better(p.mag, p.idx, best, bidx)) {
      best = p.mag;
      bidx = p.idx;
      neg = p.neg;
    }
  }
  flag[i] = neg;
}

// A [b][rows][r] and B [b][r][cols]: entries of flagged components negated, one per thread
template <typename T>
__global__ void __launch_bounds__(256) sign_negate(T* __restrict__ A, T* __restrict__ B, const int* __restrict__ flag,
                                                   int rows, int cols, int r, int64_t na, int64_t nb) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < na) {
    const int64_t z = i / ((int64_t)rows * r);
    const int c = (int)(i % r);
    if (flag[z * r + c]) A[i] = negated(A[i]);
  } else if (i < na + nb) {
    const int64_t j = i - na;
    const int64_t zc = j / cols;   // z * r + c
    if (flag[zc]) B[j] = negated(B[j]);
  }
}

template <typename T>
hipError_t fix_signs(T* A, T* B, SignPart* part, int* flag, int b, int rows, int cols, int r, hipStream_t st) {
  sign_partial<T><<<dim3((r + 63) / 64, kSignSplits, b), 256, 0, st>>>(A, part, rows, r);
  hipError_t e = hipGetLastError();
  if (e) return e;
  sign_decide<<<(b * r + 255) / 256, 256, 0, st>>>(part, flag, r, b);
  if ((e = hipGetLastError())) return e;
  const int64_t na = (int64_t)b * rows * r, nb = (int64_t)b * r * cols;
  sign_negate<T><<<(unsigned)((na + nb + 255) / 256), 256, 0, st>>>(A, B, flag, rows, cols, r, na, nb);
  return hipGetLastError();
}

// ------------------------------------------------------------------ workspace layout
struct SvdWs {
  size_t om, y0, y1, w0, w1, g, li, part, bskt, g2, v, m1, m1f, m2, jt, jr, js, sp, sf, total;
};
size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
SvdWs layout(int n_mats, int rows, int cols, int rank, int oversample) {
  const size_t b = (size_t)n_mats, m = rows, n = cols, l = (size_t)rank + oversample, r = rank;
  SvdWs w;
  size_t o = 0;
  w.om = o;  o += al(b * n * l * 4);
  w.y0 = o;  o += al(b * m * l * 4);
  w.y1 = o;  o += al(b * m * l * 4);
  w.w0 = o;  o += al(b * n * l * 4);
  w.w1 = o;  o += al(b * n * l * 4);
  w.g = o;   o += al(b * l * l * 8);
  w.li = o;  o += al(b * l * l * 8);
  w.part = o; o += al(kGramSplitMax * b * l * l * 8);                 // split Gram partial sums
  w.bskt = o; o += al(b * n * l * 4);                                  // Bsk^T = Z^T Q (fp32)
  w.g2 = o;  o += al(b * l * l * 8);
  w.v = o;   o += al(b * l * l * 8);
  w.m1 = o;  o += al(b * l * r * 8);
  w.m1f = o; o += al(b * l * r * 4);
  w.m2 = o;  o += al(b * r * l * 8);
  const size_t lp = (l + 1) & ~(size_t)1;
  w.jt = o;  o += al(b * lp * (lp + 1) / 2 * 8);                       // Jacobi triangles
  w.jr = o;  o += al(2 * b * jacobi_log_pairs((int)l) * 16);            // two rotation logs
  w.js = o;  o += al(b * 4 * 4);                                        // Jacobi state
  w.sp = o;  o += al(b * kSignSplits * r * sizeof(SignPart));           // sign scan partials
  w.sf = o;  o += al(b * r * 4);                                        // sign flags
  w.total = o;
  return w;
}

// Y [b][rows][l] (fp32) <- orthonormal (or zero) columns spanning it: `passes` rounds of
// CholeskyQR with pivot dropping (two = CholeskyQR2).  Rounds alternate between Y and `tmp`; with
// an odd number the result is in `tmp` and the caller swaps the two.  A single round (a basis
// between power iterations) multiplies Y L^-T in split bf16; two rounds (the final basis) in
// fp32.  `part`: the Gram's split-K partial sums.
hipError_t orth(float* Y, float* tmp, double* G, double* Li, double* part, int b, int rows, int l, int passes,
                hipStream_t st) {
  hipError_t e;
  float* src = Y;
  float* dst = tmp;
  for (int pass = 0; pass < passes; ++pass) {
    // G = Y^T Y (fp64); the Cholesky kernels read only its lower triangle
    if ((e = gram_f64(src, G, part, rows, l, b, true, st))) return e;
    const double tolr = pass == 0 ? 1e-12 : 1e-10;
    if (l <= kCholRegMax) {
      // dst = src Li^T on matrix cores; Li^T (fp32) takes the place of Li
      float* lit = reinterpret_cast<float*>(Li);
      chol_inv_reg<<<b, 512, 0, st>>>(G, lit, l, tolr);
      if ((e = hipGetLastError())) return e;
      // a one-round basis between power iterations only has to keep its span: split bf16
      if ((e = passes == 1 ? gemm_bf3<false>(src, lit, dst, rows, l, l, l, l, l, (int64_t)rows * l, (int64_t)l * l,
                                             (int64_t)rows * l, b, st)
                           : gemm_f32<false>(src, lit, dst, rows, l, l, l, l, l, (int64_t)rows * l, (int64_t)l * l,
                                             (int64_t)rows * l, b, st)))
        return e;
    } else {
      const size_t tri_bytes = sizeof(double) * (size_t)l * (l + 1) / 2;
      if (l <= kJacobiLdsMax) {
        if (tri_bytes > 64 * 1024 &&
            (e = hipFuncSetAttribute(reinterpret_cast<const void*>(chol_inv_lds),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)tri_bytes)))
          return e;
        chol_inv_lds<<<b, 1024, tri_bytes, st>>>(G, Li, l, tolr);
      } else {
        chol_inv<<<b, 1024, 0, st>>>(G, Li, l, tolr);
      }
      if ((e = hipGetLastError())) return e;
      // dst = src Li^T
      if ((e = run_gemm<float, double, float, double, false, true>(src, Li, dst, rows, l, l, l, l, l,
                                                                    (int64_t)rows * l, (int64_t)l * l,
                                                                    (int64_t)rows * l, b, st)))
        return e;
    }
    float* t = src;
    src = dst;
    dst = t;
  }
  return hipSuccess;
}

}  // namespace

size_t svd_workspace_bytes(int n_mats, int rows, int cols, int rank, int oversample) {
  return layout(n_mats, rows, cols, rank, oversample).total;
}

hipError_t svd_refresh(const float* z, int n_mats, int rows, int cols, int rank, void* a_out, void* b_out,
                       int out_bf16, float* sigma_out, int oversample, int power_iters, uint64_t seed, void* ws,
                       size_t ws_bytes, hipStream_t st) {
  const SvdWs L = layout(n_mats, rows, cols, rank, oversample);
  if (ws_bytes < L.total) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  float* om = reinterpret_cast<float*>(base + L.om);
  float* y0 = reinterpret_cast<float*>(base + L.y0);
  float* y1 = reinterpret_cast<float*>(base + L.y1);
  float* w0 = reinterpret_cast<float*>(base + L.w0);
  float* w1 = reinterpret_cast<float*>(base + L.w1);
  double* G = reinterpret_cast<double*>(base + L.g);
  double* Li = reinterpret_cast<double*>(base + L.li);
  double* part = reinterpret_cast<double*>(base + L.part);
  double* g2 = reinterpret_cast<double*>(base + L.g2);
  double* V = reinterpret_cast<double*>(base + L.v);
  double* m1 = reinterpret_cast<double*>(base + L.m1);
  double* m2 = reinterpret_cast<double*>(base + L.m2);
  const int m = rows, n = cols, l = rank + oversample, r = rank, b = n_mats;
  const int64_t sZ = (int64_t)m * n, sY = (int64_t)m * l, sW = (int64_t)n * l;
  hipError_t e;

  // Omega [b][n][l] ~ N(0, 1)
  const int64_t cnt = (int64_t)b * n * l;
  sketch<<<(unsigned)((cnt + 255) / 256), 256, 0, st>>>(om, cnt, seed);
  if ((e = hipGetLastError())) return e;
  // Y = Z Omega, orthonormalised; the bases between power iterations take one CholeskyQR round
  // (their Gram is formed in fp64, so one round leaves them orthonormal to the fp32 storage
  // precision, and the next product only needs their span), the final basis Q two.  Every
  // product but the one that forms the final basis runs in split bf16 (about 16 significant
  // bits: it only steers the span); the final Y = Z W and Bsk^T = Z^T Q run in fp32, so error
  // components of W outside the row space of Z are annihilated and the span of Q and the
  // projection keep fp32 accuracy.
  if ((e = power_iters > 0 ? gemm_bf3<false>(z, om, y0, m, l, n, n, l, l, sZ, sW, sY, b, st)
                           : gemm_f32<false>(z, om, y0, m, l, n, n, l, l, sZ, sW, sY, b, st)))
    return e;
  auto orth_swap = [&](float*& X, float*& Xt, int rows_, int passes) -> hipError_t {
    hipError_t r = orth(X, Xt, G, Li, part, b, rows_, l, passes, st);
    if (passes & 1) std::swap(X, Xt);
    return r;
  };
  float *Y = y0, *Yt = y1, *Wb = w0, *Wt = w1;
  if ((e = orth_swap(Y, Yt, m, power_iters > 0 ? 1 : 2))) return e;
  for (int it = 0; it < power_iters; ++it) {
    // W = Z^T Y, orthonormalised; Y = Z W, orthonormalised
    const bool last = it + 1 == power_iters;
    if ((e = gemm_bf3<true>(z, Y, Wb, n, l, m, n, l, l, sZ, sY, sW, b, st))) return e;
    if ((e = orth_swap(Wb, Wt, n, 1))) return e;
    if ((e = last ? gemm_f32<false>(z, Wb, Y, m, l, n, n, l, l, sZ, sW, sY, b, st)
                  : gemm_bf3<false>(z, Wb, Y, m, l, n, n, l, l, sZ, sW, sY, b, st)))
      return e;
    if ((e = orth_swap(Y, Yt, m, it + 1 < power_iters ? 1 : 2))) return e;
  }
  y0 = Y;
  // Bsk^T = Z^T Q (fp32 matrix cores), the Gram Bsk Bsk^T in fp64, its eigenpairs
  float* bskt = reinterpret_cast<float*>(base + L.bskt);
  if ((e = gemm_f32<true>(z, y0, bskt, n, l, m, n, l, l, sZ, sY, sW, b, st))) return e;
  const int lp = (l + 1) & ~1;
  const size_t tri_bytes = sizeof(double) * (size_t)lp * (lp + 1) / 2;
  const bool in_lds = lp <= kJacobiLdsMax;
  // the LDS eigensolver reads only the lower triangle of the Gram; the global one all of it
  if ((e = gram_f64(bskt, g2, part, n, l, b, in_lds, st))) return e;
  if (in_lds) {
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(jacobi_step), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)std::max(tri_bytes, sizeof(double) * (size_t)l * kApplyPitch))))
      return e;
    double* jt = reinterpret_cast<double*>(base + L.jt);
    double2* jr = reinterpret_cast<double2*>(base + L.jr);
    int* js = reinterpret_cast<int*>(base + L.js);
    const int max_sweeps = 40, n_chunks = (max_sweeps + kJacobiChunkSweeps - 1) / kJacobiChunkSweeps;
    const int nsl = (l + kApplyCols - 1) / kApplyCols;
    const size_t lds = std::max(tri_bytes, sizeof(double) * (size_t)l * kApplyPitch);
    for (int c = 0; c <= n_chunks; ++c) {
      jacobi_step<<<b * (1 + nsl), 1024, lds, st>>>(g2, jt, V, jr, js, l, b, c, n_chunks, max_sweeps, 1e-13);
      if ((e = hipGetLastError())) return e;
    }
  } else {
    jacobi<<<b, 1024, 0, st>>>(g2, V, l, 40, 1e-13);
  }
  if ((e = hipGetLastError())) return e;
  float* m1f = reinterpret_cast<float*>(base + L.m1f);
  select_top<<<b, 256, 0, st>>>(g2, V, sigma_out, m1, m1f, m2, l, r, in_lds ? 1 : 0);
  if ((e = hipGetLastError())) return e;
  // A = Q (W_r Sigma_r), B = (Sigma_r^-1 W_r^T) Bsk, then the sign convention
  SignPart* sp = reinterpret_cast<SignPart*>(base + L.sp);
  int* sf = reinterpret_cast<int*>(base + L.sf);
  if (out_bf16) {
    bf16_bits* A = static_cast<bf16_bits*>(a_out);
    bf16_bits* Bo = static_cast<bf16_bits*>(b_out);
    if ((e = run_gemm<float, double, bf16_bits, double, false, false>(y0, m1, A, m, r, l, l, r, r, sY, (int64_t)l * r,
                                                                       (int64_t)m * r, b, st)))
      return e;
    if ((e = run_gemm<double, float, bf16_bits, double, false, true>(m2, bskt, Bo, r, n, l, l, l, n, (int64_t)r * l,
                                                                      sW, (int64_t)r * n, b, st)))
      return e;
    return fix_signs<bf16_bits>(A, Bo, sp, sf, b, m, n, r, st);
  }
  float* A = static_cast<float*>(a_out);
  float* Bo = static_cast<float*>(b_out);
  if ((e = gemm_f32<false>(y0, m1f, A, m, r, l, l, r, r, sY, (int64_t)l * r, (int64_t)m * r, b, st))) return e;
  if ((e = run_gemm<double, float, float, double, false, true>(m2, bskt, Bo, r, n, l, l, l, n, (int64_t)r * l, sW,
                                                                (int64_t)r * n, b, st)))
    return e;
  return fix_signs<float>(A, Bo, sp, sf, b, m, n, r, st);
}

}  // namespace kvc
