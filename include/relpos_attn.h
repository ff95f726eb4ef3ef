/*
 * relpos_attn.h -- C ABI of the exact relative-position attention library
 * (gfx950 / MI355X, hand-written HIP kernels).
 *
 * The operation is the one described in "Fast and Exact Relative-Position
 * Attention via Structure-Aware Kernels" (Boychev, Petrov, Dimitrov; digest on
 * nanless.github.io), section on the score formula, Eq. (1):
 *
 *   S_ij = tau * ( q_i.k_j + q_i.aQ[phi(i,j)] + k_j.aK[phi(i,j)] + b[phi(i,j)] ) + M_ij
 *   P    = softmax_j(S),   O = P V,   LSE_i = log sum_j exp(S_ij)
 *
 * computed FlashAttention-style (no N x N matrix is ever stored), forward and
 * backward.  Eq. (2)/(3) of the same section rewrite the two vector terms as
 * scalar lookups Z^Q[i, r] = q_i.aQ[r] and Z^K[j, r] = k_j.aK[r]; the library
 * stores those projections (fp32) for the reachable offset window only
 * (section on the grouped reachable range), adds them on chip, and in the
 * backward accumulates dS per offset with a single writer per entry (section
 * on the backward pass, Eq. (4)), then contracts to the table gradients.
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates or frees device memory; scratch comes from `workspace`.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work on it and return without synchronising the host.
 *  - Every argument is validated before anything is launched; on an error
 *    nothing is written and the status says why (see relpos_last_error()).
 *  - Outputs are overwritten, never accumulated into.
 *  - Results are bitwise reproducible run to run on one device model: no
 *    atomics, fixed summation orders.  Some launch shapes depend on the
 *    device's compute-unit count, so devices with different counts may
 *    differ in the last bits (always within the same error bounds).
 *  - Thread-safe.  The only shared state is a per-device cache of the
 *    compute-unit count (written once, atomically) and the thread-local
 *    error message.
 */
#ifndef RELPOS_ATTN_H
#define RELPOS_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum relpos_status {
  RELPOS_OK = 0,
  RELPOS_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size, bad descriptor */
  RELPOS_ERR_UNSUPPORTED = -2,  /* valid request the kernels do not implement (e.g. d != 64) */
  RELPOS_ERR_WORKSPACE = -3,    /* workspace smaller than relpos_attn_workspace_size() */
  RELPOS_ERR_HIP = -4           /* a HIP launch failed */
} relpos_status;

/* Element type of Q, K, V, O, dO, dQ, dK, dV and of the tables aQ, aK, b. */
typedef enum relpos_dtype { RELPOS_F32 = 0, RELPOS_F16 = 1, RELPOS_BF16 = 2 } relpos_dtype;

/* Offset maps phi(i, j) = phi(o), o = j - i (key index minus query index).
 * The setup section of the page lists the maps per mechanism:
 *  TRUNCATED (Shaw, DeBERTa as configured):  r = clip(o, lo, hi) - lo,  R = hi - lo + 1
 *  BUCKET_T5 (T5): standard T5 relative bucket (num_buckets, max_exact,
 *            max_distance, bidirectional), R = num_buckets.  Inside the
 *            library the bucketed map is unfolded into a truncated map whose
 *            rows are copies of bucket rows (section on constant tiles), and
 *            the copied gradient columns are folded back in ascending offset.
 *  IDENTITY (Transformer-XL): r = o + N - 1, R = 2N - 1.
 *  BUCKET_LOG (DeBERTa; the page names 256 log buckets to distance 512): the
 *            log-bucket positions of DeBERTa (num_buckets = k, max_distance
 *            = m, mid = k / 2): bucket = o for |o| <= mid, otherwise
 *            sign(o) (mid + ceil((mid - 1) ln(|o| / mid) / ln((m - 1) / mid)));
 *            r = clip(bucket + k, 0, 2k - 1), R = 2k.  Unfolded and folded
 *            like BUCKET_T5. */
typedef enum relpos_phi_kind {
  RELPOS_PHI_TRUNCATED = 0,
  RELPOS_PHI_BUCKET_T5 = 1,
  RELPOS_PHI_IDENTITY = 2,
  RELPOS_PHI_BUCKET_LOG = 3
} relpos_phi_kind;

typedef struct relpos_phi {
  int32_t kind;           /* relpos_phi_kind */
  int32_t lo, hi;         /* TRUNCATED: lo <= hi */
  int32_t num_buckets;    /* BUCKET_T5: >= 2 (even when bidirectional);
                             BUCKET_LOG: k, even, in [4, 4096] (the table has 2k rows) */
  int32_t max_exact;      /* BUCKET_T5: 0 = default (half of the buckets per side, halved) */
  int32_t max_distance;   /* BUCKET_T5: > max_exact; BUCKET_LOG: m, k / 2 + 2 <= m <= 2^24 */
  int32_t bidirectional;  /* BUCKET_T5: 1 = keys after the query use the upper half */
} relpos_phi;

/* Additive mask M_ij of Eq. (1): 0 or -inf. */
enum {
  RELPOS_MASK_NONE = 0,
  RELPOS_MASK_CAUSAL = 1,       /* M_ij = -inf for j > i */
  RELPOS_MASK_KEY_PADDING = 2   /* M_ij = -inf for j >= key_len[batch] */
};
typedef struct relpos_mask {
  int32_t flags;            /* OR of the RELPOS_MASK_* bits */
  const int32_t* key_len;   /* device int32[B]; required iff KEY_PADDING; values clamped to [0, N] */
} relpos_mask;

/* Roles of the [B, H, N, d] tensors, used to index relpos_problem.strides. */
enum {
  RELPOS_T_Q = 0, RELPOS_T_K, RELPOS_T_V, RELPOS_T_O,
  RELPOS_T_DO, RELPOS_T_DQ, RELPOS_T_DK, RELPOS_T_DV,
  RELPOS_T_COUNT
};

/* Problem descriptor.
 *  - Attention dropout (the digest page's section on reproduction asks for
 *    dropout whose random numbers the backward recomputes): the weights P of
 *    O = P V are replaced by P * K / (1 - p), with drop probability
 *    p = t / 256, t = dropout_p * 256 rounded to the nearest integer, which
 *    must be in [1, 255]: a dropout_p that rounds to t = 0 or to t = 256 is
 *    RELPOS_ERR_INVALID_ARG, and dropout_p = 0 exactly turns dropout off.
 *    K_ij = 1 iff the random byte u_ij >= t, where u_ij is byte j % 4 of word i % 4 of Philox4x32-10
 *    (Salmon et al., SC 2011) at counter (j / 4, i / 4, batch * H + head,
 *    dropout_offset) under the key dropout_seed (low word first).  The LSE
 *    output is that of the undropped softmax.  The backward must be given
 *    the forward's dropout_p, dropout_seed and dropout_offset.  Dropout is
 *    implemented for fp16 and bf16 (ERR_UNSUPPORTED for fp32).
 *  - Tensors are [B, H, N, d] with d contiguous; strides[role] = {batch, head,
 *    row} strides in ELEMENTS.  Each stride must be a multiple of 8 elements
 *    (16 bytes) and every tensor pointer 16-byte aligned.
 *  - Tables: aQ, aK are [H, R, d] (rows contiguous, row stride d), b is [H, R];
 *    their head strides are given in elements and may be 0 (one table shared
 *    by all heads; its gradient is then summed over heads).
 *  - tau > 0 (the softmax scale of Eq. (1)).
 *  - d must be 64 (ERR_UNSUPPORTED otherwise); any N >= 0 (N = 0 is a no-op).
 *  - zchunk (a multiple of 128, or 0): linear-memory mode for wide relation
 *    windows (the identity map's is N + 127 columns per query).  When
 *    0 < zchunk < N the query-side projection Z^Q and its gradient dZ^Q are
 *    never held for the whole sequence: the forward (unless it computes the
 *    relation in the block, below, and holds no Z^Q at all) and the backward
 *    each recompute them one chunk of zchunk queries at a time inside the
 *    workspace (the digest's section on limitations: recomputing the
 *    projection instead of storing it makes the memory linear), so the
 *    workspace is O(B H zchunk W) plus O(B H N d) for the chunk-summed dK
 *    and dV, and nothing is kept between the passes (zsave must be NULL,
 *    relpos_attn_zsave_size returns 0).  The key-side term must be absent
 *    (ERR_UNSUPPORTED).  Under this mode the stage calls run whole chunks:
 *    FWD_PROJECT and BWD_PREPARE only build the map tables, FWD_ATTEND runs
 *    every chunk's projection and attention (in-block: one attention launch
 *    over all queries), BWD_QUERY_PASS | BWD_KEY_PASS
 *    (both together) every chunk's row terms, passes and contraction, and
 *    BWD_CONTRACT alone does nothing.  Each chunk's results are summed into
 *    dK, dV, daQ and db in chunk order, so the outputs are deterministic;
 *    they may differ from the unchunked ones in the last bits.
 *  - relation: how the forward gets the query-side relation term of the
 *    band tiles (the digest's ablation of keeping the projection against
 *    recomputing it inside each block, and its limitations section).
 *    RELPOS_REL_STORED: projected once into Z^Q (kept in zsave when one is
 *    given).  RELPOS_REL_INBLOCK: computed inside each attention block from
 *    Q and the tables (Q aQ^T of the tile's offsets by MFMA, plus b), so the
 *    forward holds no projection at all (zsave must be NULL and
 *    relpos_attn_zsave_size returns 0; the backward then projects Z^Q
 *    itself, one chunk at a time when zchunk is set).  It needs fp16 or
 *    bf16 inputs and no aK (ERR_UNSUPPORTED otherwise); without aQ it
 *    changes nothing.
 *    RELPOS_REL_AUTO (0) picks by sequence length: in-block where it is
 *    supported and the relation window min(R, N + 127) is at least as wide
 *    as the sequence, i.e. N <= R for a map of R unfolded rows (short
 *    sequences, where a stored window is as large as a dense bias, and the
 *    identity map, R = 2N - 1), else stored. */
enum { RELPOS_REL_AUTO = 0, RELPOS_REL_STORED = 1, RELPOS_REL_INBLOCK = 2 };

typedef struct relpos_problem {
  int64_t B, H, N, d;
  int32_t dtype;            /* relpos_dtype */
  float tau;
  int64_t strides[RELPOS_T_COUNT][3];
  int64_t aq_head_stride;   /* elements; 0 = shared */
  int64_t ak_head_stride;
  int64_t b_head_stride;
  float dropout_p;          /* in [0, 1); 0 = no dropout */
  uint32_t dropout_offset;  /* counter word 3 of the generator */
  uint64_t dropout_seed;    /* generator key */
  int64_t zchunk;           /* query rows per projection chunk; 0 = whole sequence */
  int32_t relation;         /* RELPOS_REL_* */
} relpos_problem;

/* Which relation terms are present (a "= 0" table is simply absent). */
enum { RELPOS_TERM_AQ = 1, RELPOS_TERM_AK = 2, RELPOS_TERM_B = 4 };
/* Pass selector for relpos_attn_workspace_size. */
enum { RELPOS_PASS_FWD = 0, RELPOS_PASS_BWD = 1 };

/* Bytes of device workspace relpos_attn_fwd (pass = FWD) or relpos_attn_bwd
 * (pass = BWD) needs for this problem.  `zsave_given` says whether the caller
 * will pass a zsave buffer (then the projections do not live in the
 * workspace).  Host-only; launches nothing. */
relpos_status relpos_attn_workspace_size(const relpos_problem* prob, const relpos_phi* phi,
                                         const relpos_mask* mask, int32_t terms, int32_t pass,
                                         int32_t zsave_given, size_t* bytes);

/* Bytes of the optional buffer in which the forward keeps the relation
 * projections Z^Q, Z^K (fp32, reachable window only) for the backward
 * (keeping them trades memory for recomputation, section on ablations):
 * B*H*N rows per present vector term, each of the window width rounded up
 * to 32 floats (128 bytes), plus 32 floats when the window is 1024 columns
 * or wider or no narrower than N (the workspace's relation gradients then
 * store each row shifted, and all relation rows share one pitch).  0 when no
 * vector table is present.  Host-only. */
relpos_status relpos_attn_zsave_size(const relpos_problem* prob, const relpos_phi* phi,
                                     int32_t terms, size_t* bytes);

/* Forward of Eq. (1).
 *  Q, K, V   : device [B,H,N,d], dtype prob->dtype (strides Q, K, V).
 *  aQ, aK, b : device tables or NULL when the term is absent.
 *  O         : device [B,H,N,d] output, dtype prob->dtype (strides O).
 *  lse       : device float32 [B,H,N] contiguous output, natural-log LSE
 *              (-inf for a row whose keys are all masked; its O row is 0).
 *  zsave     : device buffer of relpos_attn_zsave_size() bytes or NULL.  When
 *              given, the projections are written there for the backward.
 *  workspace : device scratch of at least relpos_attn_workspace_size(FWD).  */
relpos_status relpos_attn_fwd(const relpos_problem* prob, const relpos_phi* phi,
                              const relpos_mask* mask,
                              const void* Q, const void* K, const void* V,
                              const void* aQ, const void* aK, const void* b,
                              void* O, float* lse, void* zsave,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Backward: gradients of sum(O * dO) (section on the backward pass).
 *  O, lse    : the forward's outputs for the same inputs.
 *  dO        : device [B,H,N,d] (strides DO).
 *  zsave     : the buffer filled by relpos_attn_fwd, or NULL to recompute
 *              the projections into the workspace.
 *  dQ, dK, dV: device [B,H,N,d] outputs, dtype prob->dtype (strides DQ, DK, DV).
 *  daQ, daK  : device float32 [Ho, R, d] contiguous outputs, Ho = H (or 1 for a
 *              shared table); must be NULL exactly when the table is absent.
 *  db        : device float32 [Ho, R] contiguous output; NULL iff b is absent.
 *  workspace : device scratch of at least relpos_attn_workspace_size(BWD).  */
relpos_status relpos_attn_bwd(const relpos_problem* prob, const relpos_phi* phi,
                              const relpos_mask* mask,
                              const void* Q, const void* K, const void* V,
                              const void* aQ, const void* aK, const void* b,
                              const void* O, const float* lse, const void* dO,
                              const void* zsave,
                              void* dQ, void* dK, void* dV,
                              float* daQ, float* daK, float* db,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments and results as relpos_attn_fwd, without the
 * workspace: the forward's scratch (the bucket fold table, the unfolded
 * bias and, when zsave is NULL, the projections Z^Q, Z^K) lives in a static
 * device buffer of RELPOS_NOALLOC_SCRATCH_BYTES inside the library, one per
 * device, held until the process ends.  A problem whose forward workspace
 * (relpos_attn_workspace_size, pass FWD, with the same zsave_given) exceeds
 * that size returns RELPOS_ERR_WORKSPACE before anything is launched; passing
 * a zsave buffer moves the projections out of the scratch.  Nothing in the
 * scratch needs to start at any value.  Every call on one device shares its
 * buffer, so calls that overlap on one device (concurrent streams or host
 * threads) race: the caller must order them.  Calls no allocating routine. */
#define RELPOS_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
relpos_status relpos_attn_fwd_noalloc(const relpos_problem* prob, const relpos_phi* phi,
                                      const relpos_mask* mask,
                                      const void* Q, const void* K, const void* V,
                                      const void* aQ, const void* aK, const void* b,
                                      void* O, float* lse, void* zsave, void* stream);

/* Stages of the two passes, for callers that schedule them separately (for
 * example to overlap the key-parallel pass with other work, or to time each
 * kernel).  The pipeline section of the page orders the forward as relation
 * projection, then the fused tiled attention; the backward section as the
 * query-parallel pass, the key-parallel pass, then the final contraction.
 *  FWD_PROJECT   map tables (bucket unfold) and Z^Q, Z^K of the reachable window
 *                (Eq. 3; section on the grouped reachable range); nothing with
 *                the in-block relation
 *  FWD_ATTEND    fused forward: O and LSE (with the in-block relation, the map
 *                tables first)
 *  BWD_PREPARE   map tables, projections (only when zsave is NULL) and the
 *                row terms D_i = sum_d dO_id O_id
 *  BWD_QUERY_PASS  dQ (partial when aQ is present) and dZ^Q per offset
 *  BWD_KEY_PASS    dK (partial when aK is present), dV and dZ^K per offset
 *                  (with BWD_QUERY_PASS in the same call, both passes
 *                  usually share one launch; the results are identical)
 *  BWD_CONTRACT    dQ += dZ^Q aQ, dK += dZ^K aK, daQ, daK, db, bucket fold
 * relpos_attn_fwd_stages / relpos_attn_bwd_stages take the same arguments as
 * relpos_attn_fwd / relpos_attn_bwd plus a stage mask; the stages given run
 * in the order above.  Intermediate results live in `workspace` (and
 * `zsave`), so a pass split over several calls must pass identical
 * arguments and the same buffers to every call, on the same stream.
 * relpos_attn_fwd and relpos_attn_bwd are these calls with every stage. */
enum { RELPOS_FWD_PROJECT = 1, RELPOS_FWD_ATTEND = 2, RELPOS_FWD_ALL = 3 };
enum {
  RELPOS_BWD_PREPARE = 1,
  RELPOS_BWD_QUERY_PASS = 2,
  RELPOS_BWD_KEY_PASS = 4,
  RELPOS_BWD_CONTRACT = 8,
  RELPOS_BWD_ALL = 15
};

relpos_status relpos_attn_fwd_stages(const relpos_problem* prob, const relpos_phi* phi,
                                     const relpos_mask* mask,
                                     const void* Q, const void* K, const void* V,
                                     const void* aQ, const void* aK, const void* b,
                                     void* O, float* lse, void* zsave,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     int32_t stages);

relpos_status relpos_attn_bwd_stages(const relpos_problem* prob, const relpos_phi* phi,
                                     const relpos_mask* mask,
                                     const void* Q, const void* K, const void* V,
                                     const void* aQ, const void* aK, const void* b,
                                     const void* O, const float* lse, const void* dO,
                                     const void* zsave,
                                     void* dQ, void* dK, void* dV,
                                     float* daQ, float* daK, float* db,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     int32_t stages);

/* Host-side facts about a map at length N: R (rows of the caller's tables),
 * and the truncated map the library unfolds it into, [lo_unf, hi_unf]
 * (R_unf = hi_unf - lo_unf + 1 rows).  For the bucketed maps the unfolded
 * thresholds are the first offsets beyond which the row no longer changes,
 * clipped to the offsets that exist at length N, [-(N - 1), N - 1]; bucket
 * rows that no offset reaches then have no unfolded row (their gradients
 * are zero), and every buffer grows with N, not with max_distance. */
relpos_status relpos_phi_info(const relpos_phi* phi, int64_t N, int64_t* R, int64_t* lo_unf,
                              int64_t* hi_unf);

/* Device-computed row tables (exported so they can be checked bit for bit):
 *  rows[o + N - 1]     = phi(o) for every o in [-(N-1), N-1]       (int32[2N-1])
 *  fold[u]             = original row of unfolded row u, u in [0, R_unf)  (int32[R_unf])
 * Either pointer may be NULL.  Enqueued on `stream`. */
relpos_status relpos_phi_rows(const relpos_phi* phi, int64_t N, int32_t* rows, int32_t* fold,
                              void* stream);

/* Human-readable name of a status code (static string). */
const char* relpos_status_string(int32_t status);
/* Message describing the last error on the calling thread ("" if none). */
const char* relpos_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RELPOS_ATTN_H */
