// Reliability gate finalisation (KVCMAS App. A.3 "Reliability Gate", Eq. 9-11).
//
// Per-tile fp32 partial sums from the scoring kernels are reduced in double precision in a
// fixed order (per layer: strided thread sums over the tiles, a fixed shuffle tree per wave,
// the waves in order; then the layers in order), so distances, entropies and flags are
// bit-reproducible.  One work-group per layer does the tile sums (`gate_layer_sums`); a single
// work-group then forms the hop row and the decisions (`gate_finalize`).
//   PAGES:  d_v = sqrt(sum_l sum_{t<k} ||V - A_v B_v||^2)            (Eq. 9)
//           g = softmax(-d / T)                                       (Eq. 10)
//           H = -sum g log2 g / log2 |A_k|                            (Eq. 11)
//           accept iff H <= tau; |A_k| < 2 flags; capacity 1 bypasses (App. C.3)
//   COS_R:  cos_v = sum <P, A> / sqrt(sum |P|^2 sum |A|^2) over values, prefix k;
//           flagged when the best cosine is below tau.
// Row 0 is the hop (sums over all layers); row 1 + l restricts the sums to layer l.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kMaxLayersGate = 256;

// gsum [3][1 + N_l][N] (row 1 + l): layer l's sums over all tiles, fp64
__device__ __forceinline__ void layer_sums(const GateArgs& p, int l, double (*wsum)[kMaxAnchors]) {
  const int N = p.N, L = p.n_layers;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int64_t plane_in = (int64_t)L * p.n_tiles * N;
  const int planes = p.mode == KVC_SCORE_PAGES ? 1 : 3;
  for (int pl = 0; pl < planes; ++pl) {
    const float* src = p.partials + pl * plane_in + (int64_t)l * p.n_tiles * N;
    for (int a = 0; a < N; ++a) {
      double s = 0.0;
      if ((p.mask_gate >> a) & 1)
        for (int t = tid; t < p.n_tiles; t += blockDim.x) s += (double)src[(int64_t)t * N + a];
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      if (lane == 0) wsum[wave][a] = s;
    }
    __syncthreads();
    for (int a = tid; a < N; a += blockDim.x) {
      double s = 0.0;
      for (int w = 0; w < nw; ++w) s += wsum[w][a];
      p.gsum[((int64_t)pl * (1 + L) + 1 + l) * N + a] = s;
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(1024) gate_layer_sums(GateArgs p) {
  __shared__ double wsum[16][kMaxAnchors];
  layer_sums(p, blockIdx.x, wsum);
}

// batched: blockIdx.y = hop (layers past a hop's count have nothing to do)
__global__ void __launch_bounds__(1024) gate_layer_sums_batch(const GateArgs* __restrict__ d) {
  __shared__ double wsum[16][kMaxAnchors];
  const GateArgs& p = d[blockIdx.y];
  if ((int)blockIdx.x < p.n_layers) layer_sums(p, blockIdx.x, wsum);
}

__device__ __forceinline__ void finalize(const GateArgs& p, double* sh) {   // sh: [3][1 + N_l][N]
  const int N = p.N, L = p.n_layers;
  const int rows = 1 + L;
  const int planes = p.mode == KVC_SCORE_PAGES ? 1 : 3;
  // 1) per (layer, anchor) sums from gate_layer_sums
  for (int i = threadIdx.x; i < planes * L * N; i += blockDim.x) {
    const int pl = i / (L * N), l = (i / N) % L, a = i % N;
    sh[(pl * rows + 1 + l) * N + a] = p.gsum[((int64_t)pl * rows + 1 + l) * N + a];
  }
  __syncthreads();
  // 2) hop row: fixed-order sum over layers
  for (int i = threadIdx.x; i < planes * N; i += blockDim.x) {
    const int pl = i / N, a = i % N;
    double s = 0.0;
    for (int l = 0; l < L; ++l) s += sh[(pl * rows + 1 + l) * N + a];
    sh[(pl * rows + 0) * N + a] = s;
  }
  __syncthreads();
  // 3) one thread per row: decision
  for (int row = threadIdx.x; row < rows; row += blockDim.x) {
    int n_gate = 0;
    for (int a = 0; a < N; ++a) n_gate += (int)((p.mask_gate >> a) & 1);
    double* dist = p.dist + (int64_t)row * N;
    int flag = 0;
    double stat = __builtin_nan("");
    if (p.mode == KVC_SCORE_PAGES) {
      double dmin = INFINITY;
      for (int a = 0; a < N; ++a) {
        if ((p.mask_gate >> a) & 1) {
          const double d = sqrt(sh[(0 * rows + row) * N + a]);
          dist[a] = d;
          dmin = fmin(dmin, d);
        } else {
          dist[a] = __builtin_nan("");
        }
      }
      if (n_gate >= 2) {
        double z = 0.0;
        for (int a = 0; a < N; ++a)
          if ((p.mask_gate >> a) & 1) z += exp(-(dist[a] - dmin) / p.temp_gate);
        double hsum = 0.0;
        for (int a = 0; a < N; ++a) {
          if (!((p.mask_gate >> a) & 1)) continue;
          const double g = exp(-(dist[a] - dmin) / p.temp_gate) / z;
          if (g > 0.0) hsum -= g * log2(g);
        }
        stat = hsum / log2((double)n_gate);
      }
      if (N == 0) flag = KVC_FLAG_FEW_ANCHORS;
      else if (p.capacity == 1) flag = 0;
      else if (n_gate < 2) flag = KVC_FLAG_FEW_ANCHORS;
      else flag = stat > p.tau ? KVC_FLAG_ENTROPY : 0;
    } else {
      double best = -INFINITY;
      for (int a = 0; a < N; ++a) {
        if ((p.mask_gate >> a) & 1) {
          const double pa = sh[(0 * rows + row) * N + a];
          const double pp = sh[(1 * rows + row) * N + a];
          const double aa = sh[(2 * rows + row) * N + a];
          const double den = sqrt(pp * aa);
          const double c = den > 0.0 ? pa / den : 0.0;
          dist[a] = c;
          best = fmax(best, c);
        } else {
          dist[a] = __builtin_nan("");
        }
      }
      if (n_gate > 0) stat = best;
      if (N == 0) flag = KVC_FLAG_FEW_ANCHORS;
      else if (p.capacity == 1) flag = 0;
      else if (n_gate == 0) flag = KVC_FLAG_FEW_ANCHORS;
      else flag = best < p.tau ? KVC_FLAG_COS_BELOW : 0;
    }
    if (p.pred_flags != nullptr && p.pred_flags[0] != 0) flag |= KVC_FLAG_PRED_FLAGGED;
    p.stat[row] = stat;
    p.flags[row] = flag;
  }
}

__global__ void __launch_bounds__(1024) gate_finalize(GateArgs p) {
  extern __shared__ double sh[];
  finalize(p, sh);
}

__global__ void __launch_bounds__(1024) gate_finalize_batch(const GateArgs* __restrict__ d) {
  extern __shared__ double sh[];
  finalize(d[blockIdx.x], sh);
}

}  // namespace

hipError_t launch_gate(const GateArgs& a, hipStream_t st) {
  const size_t shmem = sizeof(double) * 3 * (1 + a.n_layers) * (a.N > 0 ? a.N : 1);
  if (a.n_layers > kMaxLayersGate || shmem > 160 * 1024 || a.N > kMaxAnchors || !a.gsum) return hipErrorInvalidValue;
  if (a.n_layers > 0) {
    gate_layer_sums<<<a.n_layers, 1024, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  gate_finalize<<<1, 1024, shmem, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvc

namespace kvc {
hipError_t launch_gate_batch(const GateArgs* d, const GateArgs* h, int n, hipStream_t st) {
  if (n < 1 || n > 65535) return hipErrorInvalidValue;
  int lmax = 0;
  size_t shmem = 0;
  for (int i = 0; i < n; ++i) {
    const size_t b = sizeof(double) * 3 * (1 + h[i].n_layers) * (h[i].N > 0 ? h[i].N : 1);
    if (h[i].n_layers > kMaxLayersGate || b > 160 * 1024 || h[i].N > kMaxAnchors || !h[i].gsum)
      return hipErrorInvalidValue;
    lmax = lmax > h[i].n_layers ? lmax : h[i].n_layers;
    shmem = shmem > b ? shmem : b;
  }
  if (lmax > 0) {
    gate_layer_sums_batch<<<dim3((unsigned)lmax, (unsigned)n), 1024, 0, st>>>(d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  gate_finalize_batch<<<(unsigned)n, 1024, shmem, st>>>(d);
  return hipGetLastError();
}
}  // namespace kvc
