// Internal declarations shared by the host side of libkvc and its kernels (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

constexpr int kMaxAnchors = KVC_MAX_ANCHORS;
constexpr int kMaxHalf = KVC_MAX_HEAD_DIM / 2;

// cos/sin of one per-hop rotation, one entry per rotary pair c (angles evaluated on the host
// in double precision, rounded to float).  `active` = 0 means the identity (zero shift).
struct RopeTab {
  float cs[kMaxHalf];
  float sn[kMaxHalf];
  int32_t active;
};

// Anchor pool geometry as the kernels see it.
struct PoolGeom {
  int32_t n;                  // anchors
  int32_t r;                  // rank of the factor set in use
  int64_t a_layer_stride;     // elements per layer of the packed A array (sum(len) * r)
  int64_t b_layer_stride;     // elements per layer of the B array (n * r * D)
  int32_t off[kMaxAnchors];   // first packed row of each anchor
  int32_t len[kMaxAnchors];   // stored rows of each anchor
};

// ----------------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  return __builtin_bit_cast(uint16_t, b);
}
template <typename T> __device__ __forceinline__ float ldf(const T* p, int64_t i);
template <> __device__ __forceinline__ float ldf<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p, int64_t i) { return bf2f(p[i]); }
template <typename T> __device__ __forceinline__ void stf(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void stf<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void stf<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = f2bf(v); }

// One rotate-half pair turned by the angle whose cosine/sine are (c, s).  Written with explicit
// fused multiply-adds so every kernel that re-aligns keys rounds identically.
__device__ __forceinline__ void rot_pair(float x, float y, float c, float s, float& ox, float& oy) {
  ox = fmaf(x, c, -(y * s));
  oy = fmaf(x, s, y * c);
}

// Maps the hardware block index so that consecutive logical tiles run on the same XCD
// (blocks are dealt round-robin over the 8 XCDs; each XCD has its own L2).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblk) {
  const int64_t nx = 8;
  if (nblk < nx) return bid;
  const int64_t per = nblk / nx, rem = nblk % nx;
  const int64_t x = bid % nx, i = bid / nx;
  // first `rem` XCDs own per+1 tiles
  const int64_t base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return base + i;
}

// Sets the thread-local reason kvc_last_error() returns; returns s.
kvc_status report(kvc_status s, const char* fmt, ...);

// --------------------------------------------------------------------------- launchers
// All launchers enqueue on `st` and return hipGetLastError() of the launch.

hipError_t launch_align(const void* in, void* out, int in_bf16, int out_bf16, int64_t n_rows,
                        int n_heads, int head_dim, const RopeTab& tab, hipStream_t st);
// p[0 .. n) = v (a kernel, so it also records as a kernel node under graph capture)
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t st);
// out (fp32) = R(tt) tgt - R(ts) src per rotate-half pair (Eq. 12's observed correction)
hipError_t launch_observed_delta(const void* tgt, const void* src, int bf16, float* out, int64_t n_rows,
                                 int n_heads, int head_dim, const RopeTab& tt, const RopeTab& ts, hipStream_t st);

struct ScoreArgs {
  const void* z[2];          // source K, V   [N_l][S][D]
  const void* A[2];          // base A (K, V) packed [N_l][sum len][r]
  const void* B[2];          // base B (K, V) [N_l][N][r][D]  (generic path)
  float* scores;             // [2][N_l][S][N]
  float* partials;           // [3][N_l][n_tiles][N]
  int32_t n_layers, S, D, head_dim;
  int32_t s_cov, k_gate, s_work, n_tiles;
  uint64_t mask_corr, mask_gate;
  int32_t n_use;             // anchors in corr U gate, ascending
  int32_t use[kMaxAnchors];
  PoolGeom g;
  RopeTab can;               // R(-p_src) for keys
};

struct SoftmaxArgs {
  const float* scores;       // [2][N_l][S][N]
  float* w[2];               // K, V weights [N_l][S][N]
  int32_t n_layers, S, N, s_cov, mode;
  uint64_t mask_corr;
  float inv_temp;
};

struct ApplyArgs {
  const void* z[2];          // source K, V
  void* out[2];              // outputs K, V
  const void* A[2];          // delta A (K, V) packed
  const void* B[2];          // delta B (K, V) [N_l][N][r][D] (generic path)
  const float* w[2];         // weights [N_l][S][N]
  int32_t n_layers, S, D, head_dim, s_cov;
  int32_t n_corr;
  int32_t corr[kMaxAnchors];
  PoolGeom g;
  RopeTab shift;             // R(p_tgt - p_src)
  RopeTab tgt;               // R(p_tgt)
};

struct GateArgs {
  const float* partials;     // [3][N_l][n_tiles][N]
  double* gsum;              // [3][1+N_l][N] per-layer sums (workspace)
  double* dist;              // [1+N_l][N]
  double* stat;              // [1+N_l]
  int32_t* flags;            // [1+N_l]
  const int32_t* pred_flags; // flags of the preceding hop (row 0 used) or nullptr
  int32_t n_layers, n_tiles, N, mode, capacity;
  uint64_t mask_gate;
  double tau, temp_gate;
};

hipError_t launch_score_generic(const ScoreArgs& a, int bf16, int mode, int tile_tokens, hipStream_t st);
hipError_t launch_softmax(const SoftmaxArgs& a, hipStream_t st);
hipError_t launch_apply_generic(const ApplyArgs& a, int bf16, hipStream_t st);
hipError_t launch_gate(const GateArgs& a, hipStream_t st);
// `n` hops' gates in two launches; d = device copies of the host descriptors h
hipError_t launch_gate_batch(const GateArgs* d, const GateArgs* h, int n, hipStream_t st);

// second scoring mode, bf16 MFMA
hipError_t launch_score_cos_mfma(const ScoreArgs& a, hipStream_t st);
constexpr int kCosTile = 64;      // tokens per work-group (and per gate partial tile)

// second scoring mode as one GEMM per (layer, side): rank 32, bf16, D a multiple of 32
constexpr int kCosGemmTile = 128; // tokens per work-group (two gate partial tiles)
struct CosGemmArgs {
  const uint16_t* z[2];      // source K, V   [N_l][S][D] bf16
  const uint16_t* A[2];      // base A (K, V) packed [N_l][sum len][r]
  const uint16_t* B[2];      // base B (K, V) [N_l][N][r][D] (read by the packing kernel)
  const uint16_t* packed;    // B' rows [2][N_l][D / 32][n_use][r][32] (workspace)
  float* scores;             // [2][N_l][S][N]
  float* partials;           // [3][N_l][n_tiles][N], tiles of kCosTile tokens
  int64_t a_layer_stride;    // elements per layer of A (sum len * 32)
  int64_t b_layer_stride;    // elements per layer of B (N * 32 * D)
  int32_t n_layers, S, D, head_dim, N;
  int32_t k_gate, n_tiles;
  uint64_t mask_gate;
  int32_t r;                 // base rank: 32, 64 or 128 (slices of 32 GEMM columns)
  int32_t n_use;             // scored anchors (corr U gate), ascending
  int32_t use[kMaxAnchors];
  int32_t off[kMaxAnchors];  // first packed A row of each anchor
  int32_t len[kMaxAnchors];  // stored rows of each anchor
  RopeTab can;               // R(-p_src): keys' B rows are turned by its transpose
};
size_t cos_gemm_lds();
size_t cos_gemm_packed_elems(int n_layers, int n_use, int r, int D);
hipError_t launch_pack_cos(const CosGemmArgs& a, uint16_t* dst, hipStream_t st);
hipError_t launch_score_cos_gemm(const CosGemmArgs& a, hipStream_t st);

// ------------------------------------------------------------------ fused hop (bf16)
// One work-group = 64 tokens x all D channels of one (layer, side); wave w owns channels
// [128 w, 128 w + 128).  Phase 1 scores the tile (or loads given weights/scores), phase 2
// forms the token weights, phase 3 applies the weighted low-rank delta with both rotations
// and the residual folded in.
constexpr int kFusedTile = 64;
constexpr int kFusedHalf = 64;    // rotary pairs per head the fused path supports (head_dim <= 128)

enum FusedMode { FUSED_PAGES = 0, FUSED_SCORES = 1, FUSED_GIVEN = 2 };

struct FusedTab {
  float cs[kFusedHalf];
  float sn[kFusedHalf];
  int32_t active;
};

struct FusedArgs {
  const uint16_t* z[2];       // source K, V        [N_l][S][D]
  uint16_t* out[2];           // corrected K, V     [N_l][S][D]        (apply only)
  const uint16_t* Ab[2];      // base A, packed     [N_l][sum len][r_C]
  const uint16_t* Bb[2];      // base B^T, MFMA operand chunks, negated   (PAGES)
  const uint16_t* Ad[2];      // delta A, packed    [N_l][sum len][r_D]
  const uint16_t* Bd[2];      // delta B^T chunks; key rows turned by R(p_tgt)
  const float* w_in[2];       // GIVEN: weights, SCORES: cosine scores   [N_l][S][N]
  float* w_out[2];            // optional weights out                    [N_l][S][N]
  float* partials;            // PAGES gate sums, value side             [N_l][n_tiles][N]
  int32_t n_layers, S, D, n_tiles;
  int32_t s_cov, k_gate, r_b, r_d;
  int32_t N, n_use, n_corr, apply;
  int32_t ring_stride;               // LDS row stride of the A staging ring (set by the launcher)
  uint64_t mask_corr, mask_gate;
  int64_t ab_layer, ad_layer;       // elements per layer of the packed A arrays
  int32_t off[kMaxAnchors];         // first packed row of each anchor
  int32_t len[kMaxAnchors];         // stored rows of each anchor
  uint8_t use[kMaxAnchors];         // anchors scored (gate U correction set), ascending
  uint8_t corr[kMaxAnchors];        // correction set, ascending
  FusedTab can;                     // R(-p_src), keys' canonical frame
  FusedTab shift;                   // R(p_tgt - p_src), residual of the keys
  float inv_temp;                   // 1 / temp_weight
};

// Packs B [N_l][N][r][D] (bf16) into MFMA operand chunks: chunk (l, a, cb, ks) holds, for lane
// q of a wave, the 8 values B[16 ks + 8 (q / 32) + i][32 cb + q % 32], i = 0..7.  `negate`
// flips signs; `tab` (may be inactive) turns every row by a rotate-half rotation first.
hipError_t launch_pack_b(const uint16_t* const* src, uint16_t* const* dst, const int* negate,
                         const FusedTab* const* tabs, int n_arrays, int n_layers, int n_anchors,
                         int r, int D, int head_dim, hipStream_t st);
hipError_t launch_fused(const FusedArgs& a, int mode, int head_dim, hipStream_t st);

// B packing of several factor sets in one launch (each as launch_pack_b would pack it).
struct PackArgs {
  const uint16_t* src[4];
  uint16_t* dst[4];
  int32_t negate[4];
  int32_t rotate[4];
  FusedTab tab;
  int32_t n_arrays, n_layers, n_anchors, r, D, head_dim;
};
// fills one descriptor (what launch_pack_b would launch); false for an unsupported request
bool make_pack_args(PackArgs& a, const uint16_t* const* src, uint16_t* const* dst, const int* negate,
                    const FusedTab* const* tabs, int n_arrays, int n_layers, int n_anchors, int r, int D,
                    int head_dim);
hipError_t launch_pack_b_batch(const PackArgs* d, const PackArgs* h, int n, hipStream_t st);

// ------------------------------------------------------------ two-pass path (bf16)
// Score work-group = 128 tokens x 256 channels of one (layer, side), 4 waves of 64 x 128, two per
// CU (at base ranks 64 / 128: 8 waves of 64 x 64, one per CU).  Apply work-group = 128 tokens x
// 256 channels, 4 waves of 64 x 128, three per CU, so one's streaming phases (source in,
// corrected cache out) overlap the others' MFMA phases.
constexpr int kScoreTile = 128;
constexpr int kScoreThreads = 256;
constexpr int kApplyTile = 128;
constexpr int kApplyThreads = 256;
constexpr int kSplitWidth = 256;

enum SplitWMode { SPLIT_W_PARTIALS = 0, SPLIT_W_SCORES = 1, SPLIT_W_GIVEN = 2 };

struct SplitArgs {
  const uint16_t* z[2];       // source K, V                  [N_l][S][D]
  uint16_t* out[2];           // corrected K, V               [N_l][S][D]
  const uint16_t* Ab[2];      // base A, packed               [N_l][sum len][r_C]
  const uint16_t* Bb[2];      // base B operand chunks, negated
  const uint16_t* Ad[2];      // delta A, packed              [N_l][sum len][r_D]
  const uint16_t* Bd[2];      // delta B' operand chunks (key rows turned by R(p_tgt))
  float* mpart;               // per channel tile |E| sums    [n_ct][2][N_l][N][S]
  const float* w_in[2];       // given weights / cosine scores [N_l][S][N]
  float* w_out[2];            // optional weights out          [N_l][S][N]
  float* wa;                  // token weights, anchor-major   [2][N_l][N][S]
  float* partials;            // gate sums, value side         [N_l][n_tt * n_ct][N] (score tiles)
  int32_t n_layers, S, D, ntt, nct, N, r_b, r_d;   // ntt: token tiles of the launched kernel
  int32_t s_cov, k_gate, n_use, n_corr, apply, pad_;
  uint64_t mask_corr, mask_gate;
  int64_t ab_layer, ad_layer;       // elements per layer of the packed A arrays
  int32_t off[kMaxAnchors];
  int32_t len[kMaxAnchors];
  uint8_t use[kMaxAnchors];
  uint8_t corr[kMaxAnchors];
  FusedTab can;                     // R(-p_src)
  FusedTab shift;                   // R(p_tgt - p_src)
  float inv_temp, inv_d;            // 1 / temp_weight, 1 / D
  int32_t layer0, n_grp;            // layers [layer0, layer0 + n_grp) in this launch
};

// Several independent hops in one launch: descriptors in device memory, hop h owning the
// logical blocks [start[h], start[h + 1]) of the grid.
constexpr int kMaxBatch = 64;
struct BatchTab {
  int32_t n;
  int32_t start[kMaxBatch + 1];
  int32_t hop[kMaxBatch];   // descriptor index of the grid's i-th hop
};

hipError_t launch_split_score(const SplitArgs& a, int head_dim, hipStream_t st);
// batched forms: `d` = device array of `n` descriptors whose host copies are `h` (read for
// the grid and LDS sizes); the two-pass path's ranks, one shape
hipError_t launch_split_score_batch(const SplitArgs* d, const SplitArgs* h, int n, int head_dim, hipStream_t st);
hipError_t launch_split_weights_batch(const SplitArgs* d, const SplitArgs* h, int n, hipStream_t st);
hipError_t launch_split_apply_batch(const SplitArgs* d, const SplitArgs* h, int n, int head_dim, hipStream_t st);
hipError_t launch_split_weights(const SplitArgs& a, int wmode, hipStream_t st);
hipError_t launch_split_apply(const SplitArgs& a, int head_dim, hipStream_t st);
size_t split_score_lds(int r_b);                   // dynamic LDS bytes
int split_score_tile(int r_b);                     // tokens per scoring tile (128 at every rank)
size_t split_apply_lds(int r_d);
// rank slices of 32 the apply takes per anchor: ranks 64, 128 and 256 run as 2, 4 and 8 slices
// (their packed delta B is then one matrix per slice); ranks 8, 16 and 32 in one step
inline int split_apply_slices(int r_d) { return r_d == 64 ? 2 : r_d == 128 ? 4 : r_d == 256 ? 8 : 1; }

// SVD refresh
hipError_t svd_refresh(const float* z, int n_mats, int rows, int cols, int rank, void* a_out,
                       void* b_out, int out_bf16, float* sigma, int oversample, int power_iters,
                       uint64_t seed, void* ws, size_t ws_bytes, hipStream_t st);
size_t svd_workspace_bytes(int n_mats, int rows, int cols, int rank, int oversample);

// machine-ceiling measurement kernels (kvc_peaks.hip)
hipError_t launch_peak_copy(void* dst, const void* src, size_t bytes, hipStream_t st);
hipError_t launch_peak_mfma(float* sink, int n_blocks, int iters, hipStream_t st);
hipError_t launch_peak_lds(uint32_t* sink, int n_blocks, int iters, hipStream_t st);
hipError_t launch_peak_valu(float* sink, int n_blocks, int iters, hipStream_t st);

}  // namespace kvc
