/*
 * kvc.h -- C ABI of the MI355X (gfx950) per-hop KV-cache correction library (libkvc.so).
 *
 * The library implements the data-parallel hot path of KVCMAS ("KVCMAS: Efficient KV
 * cache Correction for Shared Context in Multi-Agent Systems", arXiv 2609.34060): for a
 * shared context segment handed from a source agent i to a target agent j it
 *   1. re-aligns the cached keys to the target positions (Sec. 2.2; App. A.3
 *      "Correction Weighting and Positional Alignment"),
 *   2. scores the segment against the slot's anchor pool stored as rank-r factors
 *      (Sec. 3.3 Eq. 7),
 *   3. evaluates the reliability gate (App. A.3 Eq. 9-11),
 *   4. forms token-wise anchor weights (App. A.3 "Correction Weighting"), and
 *   5. adds the weighted low-rank delta to the aligned source (Sec. 3.3 Eq. 8, Eq. 12).
 * It also factorises matrices into rank-r factors for anchor refresh (Eq. 7, App. B.1
 * "Factorization and Measurement").
 *
 * Conventions shared by every call
 *  - Ownership: the caller owns every buffer.  Device buffers are plain device pointers
 *    (e.g. from torch tensors); small descriptors are host memory read during the call.
 *    The library never allocates device memory; calls that need scratch take a workspace
 *    pointer and size (query with kvc_workspace_size).
 *  - Streams: all device work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream).  Device results are valid after the stream is synchronised.
 *  - Errors: every call returns a kvc_status.  All validation happens on the host before
 *    any launch, so a non-OK status has no side effect on device memory.  A human-readable
 *    reason is available from kvc_last_error() (thread-local).  No call prints, throws
 *    or exits.
 *  - Layout: caches are row-major [layer][token][head][dim] with D = n_kv_heads*head_dim
 *    contiguous; every device pointer must be 16-byte aligned (KVC_E_ALIGN otherwise).
 *  - Frames: token t of the segment sits at absolute position p + t.  Anchor bases and key
 *    deltas are stored in the canonical frame, where token t sits at position t.
 *  - Rotation: rotate-half RoPE; channel c of each head pairs with c + head_dim/2 and turns
 *    by dp * w_c, w_c = theta^(-2c/head_dim) unless an explicit frequency table is given.
 *    Angles are evaluated in double precision on the host and passed to the GPU as float.
 *  - The library is stateless and reentrant.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 3
#define KVC_MAX_ANCHORS 64
#define KVC_MAX_HEAD_DIM 256

typedef enum {
  KVC_OK = 0,
  KVC_E_NULL = 1,        /* a required pointer is NULL                               */
  KVC_E_SHAPE = 2,       /* a size is out of range or inconsistent                   */
  KVC_E_DTYPE = 3,       /* unsupported dtype or dtype mismatch                      */
  KVC_E_ALIGN = 4,       /* a device pointer is not 16-byte aligned                  */
  KVC_E_ALIAS = 5,       /* an output overlaps an input it must not overlap          */
  KVC_E_WORKSPACE = 6,   /* workspace missing or smaller than kvc_workspace_size()   */
  KVC_E_HIP = 7,         /* the HIP runtime reported an error at launch              */
  KVC_E_PARAM = 8,       /* a scalar parameter is out of range                       */
  KVC_E_UNSUPPORTED = 9  /* valid request the kernels do not implement               */
} kvc_status;

typedef enum { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

/* Anchor scoring mode.
 * KVC_SCORE_PAGES: App. A.3 -- token weights from the mean absolute distance between the
 *   (canonical) source and each anchor's reconstructed base, softmax(-m / temp_weight);
 *   gate on the Frobenius distance of reconstructed values over the prefix k (Eq. 9),
 *   g = softmax(-d / temp_gate) (Eq. 10), normalised entropy (Eq. 11), accept iff <= tau.
 * KVC_SCORE_COS_R: cosine between the source expressed in each anchor's r-dim basis
 *   (P = Z B^T) and the anchor's own coordinates A; weights softmax(c / temp_weight);
 *   the hop is flagged when the best segment cosine (values, prefix k) is below tau.   */
typedef enum { KVC_SCORE_PAGES = 0, KVC_SCORE_COS_R = 1 } kvc_score_mode;

/* Flag bits (0 = accept the correction). */
#define KVC_FLAG_ENTROPY 1        /* normalised entropy above tau (Eq. 11)                 */
#define KVC_FLAG_FEW_ANCHORS 2    /* fewer than two compatible anchors (App. A.3)          */
#define KVC_FLAG_COS_BELOW 4      /* COS_R: best segment cosine below tau                  */
#define KVC_FLAG_PRED_FLAGGED 8   /* batched chains: the preceding hop was flagged         */

typedef struct {
  int32_t n_layers;    /* N_l >= 1                                                         */
  int32_t seq_len;     /* S >= 1, tokens of the shared segment                              */
  int32_t n_kv_heads;  /* >= 1                                                             */
  int32_t head_dim;    /* even, <= KVC_MAX_HEAD_DIM; D = n_kv_heads * head_dim              */
} kvc_shape;

typedef struct {
  double theta;              /* rotary base (e.g. 10000); used when inv_freq is NULL       */
  const double* inv_freq;    /* optional host table of head_dim/2 frequencies w_c          */
} kvc_rope;

/* One slot's anchor pool as seen by one consuming agent (App. A.3: each anchor stores a
 * base representation and corrections for its consumers; Eq. 7 factors).
 *  A factors, slot_rows == 0: packed without padding: anchor a owns rows
 *  [off_a, off_a + anchor_len[a]) with off_a = sum_{b<a} anchor_len[b]; arrays are
 *  [n_layers][sum(len)][rank].  slot_rows > 0: fixed-capacity slots (a pool arena, see
 *  kvc_pool_insert): anchor a owns rows [a * slot_rows, a * slot_rows + anchor_len[a]) and
 *  arrays are [n_layers][n_anchors * slot_rows][rank]; every anchor_len[a] <= slot_rows.
 *  B factors are [n_layers][n_anchors][rank][D].
 *  live (host, optional): anchors with live[a] == 0 take no part in the call (an empty arena
 *  slot, or an anchor holding no correction for this consumer); their length and factors are
 *  not read.  NULL = every anchor live.
 *  Key bases and key deltas are canonical-frame.  All factor arrays share `dtype`, which
 *  must equal the cache dtype.  capacity == 1 bypasses the gate (App. C.3). */
typedef struct {
  int32_t n_anchors;          /* 0 .. KVC_MAX_ANCHORS                                       */
  int32_t rank_base;          /* r_C >= 1                                                   */
  int32_t rank_delta;         /* r_Delta >= 1                                               */
  int32_t capacity;           /* pool capacity V (>= n_anchors, or 0 = n_anchors)           */
  const int32_t* anchor_len;  /* host [n_anchors], each >= 1                                */
  kvc_dtype dtype;
  const void* baseA_k;  const void* baseB_k;  const void* baseA_v;  const void* baseB_v;
  const void* deltaA_k; const void* deltaB_k; const void* deltaA_v; const void* deltaB_v;
  int32_t slot_rows;          /* 0 = packed A rows; > 0 = fixed-capacity slots (above)         */
  int32_t pad_;
  const uint8_t* live;        /* host [n_anchors] or NULL                                      */
} kvc_pool;

/* Optional per-kernel trace for benchmarking.  The caller creates `capacity` pairs of
 * hipEvent_t (passed as void*); for every kernel the call launches, the library records
 * start[i] / stop[i] around it on the call's stream, stores the kernel's id in kernel_id[i]
 * and increments count (launches beyond capacity are not traced).  Nothing synchronises:
 * the caller reads elapsed times after synchronising the stream. */
#define KVC_TRACE_MAX 64
#define KVC_K_PACK_BASE 1        /* base B factors -> MFMA operand chunks                     */
#define KVC_K_SCORE_COS 3        /* second-mode scores (bf16 MFMA)                            */
#define KVC_K_SCORE_GENERIC 4    /* scores, any shape / dtype (VALU)                          */
#define KVC_K_GATE 5             /* Eq. 9-11 finalisation (fp64)                              */
#define KVC_K_SOFTMAX 6          /* token weights from materialised scores                    */
#define KVC_K_PACK_DELTA 7       /* delta B factors -> MFMA operand chunks (keys turned)      */
#define KVC_K_FUSED 8            /* fused score / weights / apply (bf16 MFMA)                 */
#define KVC_K_APPLY_GENERIC 9    /* apply, any shape / dtype (VALU)                           */
#define KVC_K_SCORE_SPLIT 10     /* first-mode scores, 128 x 256 tiles (bf16 MFMA)            */
#define KVC_K_APPLY_SPLIT 11     /* weighted delta + residual, 128 x 256 tiles (bf16 MFMA)    */
#define KVC_K_WEIGHTS_SPLIT 12   /* token weights, anchor-major, for the two-pass apply       */
#define KVC_K_SCORE_COS_GEMM 13  /* second-mode scores as one GEMM per layer-side (bf16 MFMA) */
#define KVC_K_PACK_COS 14        /* base B rows -> second-mode GEMM operand (keys turned)     */
typedef struct {
  int32_t capacity;               /* <= KVC_TRACE_MAX                                      */
  int32_t count;                  /* written by the library                                */
  int32_t kernel_id[KVC_TRACE_MAX];
  void* start[KVC_TRACE_MAX];     /* hipEvent_t                                            */
  void* stop[KVC_TRACE_MAX];      /* hipEvent_t                                            */
} kvc_trace;

typedef struct {
  double tau;           /* acceptance threshold (Eq. 11 / best cosine)                      */
  double temp_gate;     /* Eq. 10 temperature (> 0; the pages use 1)                         */
  double temp_weight;   /* token-weight temperature (> 0)                                     */
  int32_t gate_len;     /* comparison prefix k (0 = seq_len), 1 .. seq_len                    */
  int32_t mode;         /* kvc_score_mode                                                    */
  int32_t options;      /* bit 0: force the generic (non-MFMA) kernels; bit 1: use the
                           single-pass fused kernel instead of the two-pass one; others 0    */
  int32_t pad_;
  kvc_trace* trace;     /* optional kernel trace (NULL = none)                                */
} kvc_params;

/* Match results.  Rows: index 0 = the hop (Eq. 9 sums over all layers), 1 + l = layer l.
 *  dist  : device double [1 + n_layers][n_anchors] -- PAGES: d_v of Eq. 9; COS_R: segment
 *          cosine; NaN for anchors outside the gate set A_k.
 *  stat  : device double [1 + n_layers] -- PAGES: normalised entropy (NaN if |A_k| < 2);
 *          COS_R: best segment cosine (NaN if A_k is empty).
 *  flags : device int32  [1 + n_layers] -- 0 accept, else KVC_FLAG_* bits.
 *  w_k, w_v : optional device float [n_layers][seq_len][n_anchors] token weights (rows
 *          >= S_cov and anchors outside the correction set are 0); NULL = not returned.
 *  s_cov : optional host int32, the covered prefix S_cov = min(S, longest anchor).       */
typedef struct {
  double* dist;
  double* stat;
  int32_t* flags;
  float* w_k;
  float* w_v;
  int32_t* s_cov;
} kvc_match_out;

/* Workspace query.  `call` selects the entry point: */
#define KVC_CALL_MATCH 1
#define KVC_CALL_APPLY 2
#define KVC_CALL_CORRECT 3

int32_t kvc_abi_version(void);
const char* kvc_status_str(kvc_status s);
const char* kvc_last_error(void);

/* Bytes of workspace `call` (KVC_CALL_MATCH / _APPLY / _CORRECT) needs for this
 * shape/pool/params; 0 for an invalid request.  params may be NULL (defaults).  The factor
 * refresh has its own query, kvc_svd_workspace_size. */
size_t kvc_workspace_size(int32_t call, kvc_shape shape, const kvc_pool* pool,
                          const kvc_params* params);

/* Key re-alignment (Sec. 2.2, App. A.3): k_out[l,t] = R(pos_to - pos_from) k_in[l,t] for all
 * layers and tokens.  in_t/out_t may differ (f32 <-> bf16, output rounded to nearest even).
 * k_in == k_out (in place) is allowed when in_t == out_t; other overlaps give KVC_E_ALIAS.
 * A zero shift copies bits unchanged. */
kvc_status kvc_align_rope(const void* k_in, void* k_out, kvc_dtype in_t, kvc_dtype out_t,
                          kvc_shape shape, int64_t pos_from, int64_t pos_to,
                          const kvc_rope* rope, void* stream);

/* Anchor matching and reliability gate (Eq. 7, Eq. 9-11, App. A.3 weights): scores the
 * source segment (keys at start position p_src, values) against `pool`, writes the gate
 * results and optional token weights to `out`.  Needs workspace KVC_CALL_MATCH. */
kvc_status kvc_match_anchors(const void* k_src, const void* v_src, kvc_dtype dtype,
                             kvc_shape shape, int64_t p_src, const kvc_rope* rope,
                             const kvc_pool* pool, const kvc_params* params,
                             kvc_match_out* out, void* workspace, size_t ws_bytes,
                             void* stream);

/* Low-rank delta apply with explicit weights (Eq. 8, Eq. 12 form):
 *   K_out[t] = R(p_tgt - p_src) K_src[t] + R(p_tgt) sum_a w_k[t,a] A_k,a[t] B_k,a
 *   V_out[t] = V_src[t]                  + sum_a w_v[t,a] A_v,a[t] B_v,a
 * for t < s_cov (rows >= s_cov get no delta).  w_k/w_v: device float
 * [n_layers][seq_len][n_anchors].  Outputs must not overlap the sources (KVC_E_ALIAS): the
 * source stays the source agent's live cache.  Needs workspace KVC_CALL_APPLY. */
kvc_status kvc_apply_lowrank_delta(const void* k_src, const void* v_src, void* k_out,
                                   void* v_out, kvc_dtype dtype, kvc_shape shape,
                                   int64_t p_src, int64_t p_tgt, const kvc_rope* rope,
                                   const kvc_pool* pool, const float* w_k, const float* w_v,
                                   int32_t s_cov, void* workspace, size_t ws_bytes,
                                   void* stream);

/* The whole per-hop correction: match + gate + weights + apply (Sec. 3.3, App. A.3).  The
 * corrected cache is always written; flags tell the caller to prefill densely instead.
 * Needs workspace KVC_CALL_CORRECT. */
kvc_status kvc_correct_hop(const void* k_src, const void* v_src, void* k_out, void* v_out,
                           kvc_dtype dtype, kvc_shape shape, int64_t p_src, int64_t p_tgt,
                           const kvc_rope* rope, const kvc_pool* pool,
                           const kvc_params* params, kvc_match_out* out, void* workspace,
                           size_t ws_bytes, void* stream);

/* kvc_correct_hop without a workspace argument, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid allocation).  Scratch
 * is a library-owned device array of KVC_NOALLOC_SCRATCH_BYTES per GPU (one copy per device the
 * library runs on, kept until the process ends; its address is taken on the first call on each
 * device).  Requests whose kvc_workspace_size(KVC_CALL_CORRECT, ...) exceeds it return
 * KVC_E_WORKSPACE before any launch: up to about the 4096-token, 32-layer, 8x128 hop with 20
 * anchors at rank 32, or 10 at rank 128.  Arguments, results and errors are those of
 * kvc_correct_hop.  The call allocates no device memory and copies nothing from the host.
 * Every call on a GPU uses that GPU's one scratch array, so calls that overlap on one GPU
 * (different streams or threads) race; serialise them.  The kernels write every scratch word
 * they read, so nothing left by an earlier call is used. */
#define KVC_NOALLOC_SCRATCH_BYTES (384 << 20)
kvc_status kvc_correct_hop_noalloc(const void* k_src, const void* v_src, void* k_out, void* v_out,
                                   kvc_dtype dtype, kvc_shape shape, int64_t p_src, int64_t p_tgt,
                                   const kvc_rope* rope, const kvc_pool* pool,
                                   const kvc_params* params, kvc_match_out* out, void* stream);

/* One hop of a batch (chained corrections, Eq. 6 and App. A.3 "Cache Materialization"). */
typedef struct {
  const void* k_src;   /* ignored when chain_prev >= 0                                     */
  const void* v_src;
  void* k_out;
  void* v_out;
  int64_t p_src;       /* start position of the source segment                             */
  int64_t p_tgt;       /* start position in the target agent                               */
  int32_t chain_prev;  /* index (< this hop's) whose output is this hop's source, or -1    */
  int32_t pad_;
  kvc_pool pool;
  kvc_match_out out;   /* s_cov may be NULL                                                 */
} kvc_hop_desc;

/* Runs n_hops corrections on one stream (KVCMAS Sec. 3.2 Eq. 6; App. A.3 "Cache
 * Materialization and Pool Updates": a materialised target is the next edge's source; App. B.1
 * "Workflow Structures": chains of agents and fan-in).  Hops are grouped by their depth in the
 * chains (a hop with chain_prev = -1 is at depth 0, otherwise one deeper than chain_prev); the
 * levels run in order, and the hops of one level that take the two-pass bf16 path (first
 * scoring mode, base rank 16 or 32, at least one correcting anchor) run together, one launch of
 * each kernel for the whole level (up to 64 hops per launch) with per-hop descriptors (ragged
 * pools, ranks and positions) in the workspace.  Other hops run one call at a time.  A hop whose
 * predecessor is flagged is still computed and gets KVC_FLAG_PRED_FLAGGED.
 * Workspace: kvc_hops_batched_workspace_size(); given only the largest one-hop workspace
 * (kvc_workspace_size(KVC_CALL_CORRECT, ...) over the hops) every hop runs on its own; less
 * returns KVC_E_WORKSPACE.  Outputs are the same either way. */
size_t kvc_hops_batched_workspace_size(const kvc_hop_desc* hops, int32_t n_hops, kvc_dtype dtype,
                                       kvc_shape shape, const kvc_params* params);
kvc_status kvc_correct_hops_batched(const kvc_hop_desc* hops, int32_t n_hops, kvc_dtype dtype,
                                    kvc_shape shape, const kvc_rope* rope,
                                    const kvc_params* params, void* workspace, size_t ws_bytes,
                                    void* stream);

/* Rank-r factorisation of n_mats fp32 matrices z [n_mats][rows][cols] (Eq. 7, App. B.1):
 * z ~ A B with A = U_r Sigma_r [n_mats][rows][rank] and B = R_r^T [n_mats][rank][cols],
 * sigma_out [n_mats][rank] (device float).  Randomised subspace iteration with `oversample`
 * extra columns and `power_iters` power iterations, seeded by `seed`; each component's
 * sign is fixed so the largest-magnitude entry of its left singular vector is positive.
 * With power_iters >= 1 the basis comes from a last fp32 product of z with an orthonormal
 * factor, and an exactly rank-r input is reconstructed to fp32 accuracy; with power_iters = 0
 * it comes from the fp32 sketch z Omega itself, whose span is exact only to about the fp32
 * unit roundoff times the sketch's condition number (1e-5 to 1e-4 relative on exactly rank-r
 * products of Gaussian factors).  a_out/b_out dtype out_t.  Workspace: kvc_svd_workspace_size. */
size_t kvc_svd_workspace_size(int32_t n_mats, int32_t rows, int32_t cols, int32_t rank,
                              int32_t oversample);
kvc_status kvc_anchor_refresh_svd(const float* z, int32_t n_mats, int32_t rows, int32_t cols,
                                  int32_t rank, void* a_out, void* b_out, kvc_dtype out_t,
                                  float* sigma_out, int32_t oversample, int32_t power_iters,
                                  uint64_t seed, void* workspace, size_t ws_bytes,
                                  void* stream);

/* ---------------------------------------------------------------- pool updates
 * KVCMAS App. A.3 "Cache Materialization and Pool Updates": after a dense fallback at the
 * edge i -> j, the observed correction Delta = C_j - Align(C_i) (Eq. 12) and the source cache
 * are factorised (Eq. 7) and inserted as a new anchor; accepted corrections are not
 * reinserted; when the pool is full, the least frequently used anchor among the five oldest
 * is evicted.  The pool's anchors live in a caller-owned arena: a kvc_pool with
 * slot_rows > 0 and n_anchors = its capacity, read through kvc_pool_view's live mask. */

/* Eq. 12 in fp32, per layer and side, for the factorisation: any output may be NULL.
 *  k_base  = R(-p_src) K_src (the canonical-frame source keys)      needs k_src
 *  v_base  = V_src                                                  needs v_src
 *  k_delta = R(-p_tgt) (K_tgt - R(p_tgt - p_src) K_src), formed as R(-p_tgt) K_tgt - R(-p_src) K_src
 *                                                                   needs k_src, k_tgt
 *  v_delta = V_tgt - V_src                                          needs v_src, v_tgt
 * Inputs [n_layers][seq_len][D] of dtype; outputs fp32, same layout, 16-byte aligned, not
 * overlapping any input or each other.  Enqueued on `stream`; no allocation. */
kvc_status kvc_observed_delta(const void* k_src, const void* v_src, const void* k_tgt, const void* v_tgt,
                              kvc_dtype dtype, kvc_shape shape, int64_t p_src, int64_t p_tgt,
                              const kvc_rope* rope, float* k_base, float* v_base, float* k_delta,
                              float* v_delta, void* stream);

#define KVC_POOL_EVICT_WINDOW 5   /* eviction looks at the five oldest anchors (App. A.3) */

/* Host-side bookkeeping of one shared-context slot's pool (caller-allocated, plain data).
 * Arena slot a is empty when stamp[a] == 0; otherwise it holds one anchor inserted at the
 * stamp-th insertion, with `len` rows and the correction for `consumer`. */
typedef struct {
  int32_t capacity;                   /* V, 1 .. KVC_MAX_ANCHORS                          */
  int32_t n_held;
  int64_t clock;                      /* insertions so far                                */
  int64_t stamp[KVC_MAX_ANCHORS];     /* insertion order, 0 = empty                       */
  int64_t uses[KVC_MAX_ANCHORS];      /* accepted hops whose correction set held it       */
  int32_t len[KVC_MAX_ANCHORS];       /* stored rows                                      */
  int32_t consumer[KVC_MAX_ANCHORS];  /* consuming agent whose correction it stores       */
} kvc_pool_state;

kvc_status kvc_pool_state_init(kvc_pool_state* st, int32_t capacity);

/* Records one hop into `consumer` over a segment of seg_len rows, after its gate decision.
 *  flagged == 0 (accepted correction): nothing is inserted; every anchor of the consumer's
 *    correction set (its anchors covering min(seg_len, its longest anchor) rows) gains a use;
 *    *slot_out = *evicted_out = -1.
 *  flagged != 0 (dense fallback): a slot for the new anchor: the lowest empty slot, or, when
 *    the pool is full, among the KVC_POOL_EVICT_WINDOW oldest anchors the one with the fewest
 *    uses (ties: the oldest), which is evicted (*evicted_out).  The slot is stamped with
 *    seg_len rows and `consumer`; the caller then fills it with kvc_pool_insert.
 * Host only, no GPU work.  Errors leave the state unchanged. */
kvc_status kvc_pool_record_hop(kvc_pool_state* st, int32_t consumer, int32_t seg_len, int32_t flagged,
                               int32_t* slot_out, int32_t* evicted_out);

/* The consumer's view of the arena, for the kvc_pool descriptor of its match / correct calls:
 * anchor_len_out[a] and live_out[a] for a < capacity (live = the slot holds an anchor with a
 * correction for `consumer`).  Returns the number of live anchors, or -1 on bad arguments. */
int32_t kvc_pool_view(const kvc_pool_state* st, int32_t consumer, int32_t* anchor_len_out, uint8_t* live_out);

/* Fills arena slot `slot` with a new anchor after a dense fallback (App. A.3, Eq. 12, Eq. 7):
 * the canonical source (R(-p_src) K_src, V_src) factorised at rank_base and the observed
 * correction (kvc_observed_delta) at rank_delta, both by kvc_anchor_refresh_svd's method
 * (`oversample`, `power_iters`, seeds derived from `seed`), written into the arena's factor
 * arrays (which this call writes through their const pointers): A rows
 * [slot * slot_rows, slot * slot_rows + seq_len) of every layer and B entry `slot`.
 * Caches are arena->dtype; arena->slot_rows >= seq_len.  Workspace:
 * kvc_pool_insert_workspace_size (fp32 source and correction of one side, factor staging and
 * the factorisation's own).  Enqueued on `stream`; no allocation. */
size_t kvc_pool_insert_workspace_size(kvc_shape shape, const kvc_pool* arena, int32_t oversample);
kvc_status kvc_pool_insert(const void* k_src, const void* v_src, const void* k_tgt, const void* v_tgt,
                           kvc_shape shape, int64_t p_src, int64_t p_tgt, const kvc_rope* rope,
                           const kvc_pool* arena, int32_t slot, int32_t oversample, int32_t power_iters,
                           uint64_t seed, void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H_ */
