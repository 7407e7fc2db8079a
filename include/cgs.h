/*
 * cgs.h — C ABI of the cache-guided selective FFN for AMD Instinct MI355X (gfx950).
 *
 * The method is rMuscle (Zhou, Li, Chen, Gu, "rMuscle: Robotic Muscle Memory
 * for Efficient Vision-Language-Action Model Inference"):
 *   - Context Cache (§4.1, Eq. 2 and Eq. 3): rank visual tokens by the drift of
 *     their FFN input from a cached reference input, recompute the FFN only for
 *     the top ceil(rho_p P) tokens and scatter the results into the cached
 *     reference outputs;
 *   - Action Cache (§3.4 Eq. 1, §4.1 Eq. 4, §5): build a group-shared neuron
 *     mask from contribution scores, then update a dense anchor's output with
 *     the masked neurons only, reading only their weight rows;
 *   - reference rebuild (§4.2, asynchronous online reconstruction): a dense
 *     prefill that expands a compact entry into per-layer FFN inputs/outputs.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller; row-major; bf16
 *     values are passed as their uint16 bit pattern.  Nothing is freed or kept.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues kernels on it: no host synchronisation, no device allocation.
 *     Results are valid once the stream reaches that point.
 *   - `ws`/`ws_bytes` is a caller-owned device workspace of at least the size
 *     returned by the matching cgs_*_workspace() query; its contents need not
 *     be initialised and are clobbered.  Calls that run concurrently need
 *     distinct workspaces and outputs.
 *   - Errors that the host can see (null pointers, bad sizes, counts out of
 *     range, unsupported dtype/layout, workspace too small) return a status
 *     code before anything is launched.  A failed launch returns
 *     CGS_ERR_LAUNCH.  Preconditions on device data (index lists ascending
 *     and unique, value ranges of the fixed-point scores) are the caller's.
 *   - Layout of an FFN: w_gate, w_up are [ff][d]; w_down is [d][ff]
 *     (CGS_DOWN_DF, the Context Cache path and the rebuild) or neuron-major
 *     [ff][d] (CGS_DOWN_FD, the Action Cache path, so that a neuron's down
 *     weights are one contiguous row).
 *   - Size limit: the GEMM kernels move operand tiles into LDS with transfers
 *     that address their source by a 32-bit byte offset, so every matrix they
 *     read that way must span fewer than 2^32 bytes.  The FFN entry points
 *     return CGS_ERR_UNSUPPORTED (and the workspace queries 0) when one does
 *     not: ctx_ffn_recompute and ref_rebuild_dense need P*d, ff*d and
 *     rows*ff elements (rows = k, resp. P) times the element size below 2^32;
 *     the Action Cache calls need ff*d*4 < 2^32 (wc->ff*d*4 for compact weights).
 */
#ifndef CGS_H
#define CGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CGS_OK = 0,
  CGS_ERR_ARG = 1,          /* null pointer or invalid enum value */
  CGS_ERR_SHAPE = 2,        /* size or count out of range */
  CGS_ERR_WORKSPACE = 3,    /* ws too small or null while needed */
  CGS_ERR_UNSUPPORTED = 4,  /* dtype / layout / size the library does not handle */
  CGS_ERR_LAUNCH = 5,       /* a kernel launch failed */
  CGS_ERR_DATA = 6,         /* device data break a documented precondition (checked mode only) */
  CGS_ERR_TIMEOUT = 7       /* written to a status_out word: a persistent kernel's bounded wait gave up */
} cgs_status;

typedef enum { CGS_BF16 = 0, CGS_F32 = 1 } cgs_dtype;

/* Token score kind: CGS_SCORE_REL_RMS is Eq. 2 of §4.1 (relative RMS drift);
 * CGS_SCORE_COSINE ranks by cosine distance between x and x_ref instead. */
typedef enum { CGS_SCORE_REL_RMS = 0, CGS_SCORE_COSINE = 1 } cgs_score_kind;

/* Mask rule: CGS_MASK_TOPK is §5's rule (top K per step, union over the
 * group, top K of the union by summed contribution); CGS_MASK_COVERAGE keeps
 * the top-ranked neurons until `coverage` of the total contribution (§3.4). */
typedef enum { CGS_MASK_TOPK = 0, CGS_MASK_COVERAGE = 1 } cgs_mask_mode;

typedef enum { CGS_DOWN_DF = 0, CGS_DOWN_FD = 1 } cgs_down_layout;

/* One GeGLU FFN layer: y = (gelu_tanh(x W_gate^T) * (x W_up^T)) W_down. */
typedef struct {
  int32_t d;            /* model width */
  int32_t ff;           /* hidden neurons (H in §3.4) */
  int32_t dtype;        /* cgs_dtype of weights and activations */
  int32_t down_layout;  /* cgs_down_layout of w_down */
  const void* w_gate;   /* [ff][d] */
  const void* w_up;     /* [ff][d] */
  const void* w_down;   /* [d][ff] (DF) or [ff][d] (FD) */
} cgs_ffn;

/* Optional residual / RMSNorm glue applied by a finish kernel to each output
 * row y once it is final (the glue between stacked FFN layers, fused so that
 * it costs no extra pass):
 *   r[row] += round(y[row]) (+ bias),   x_next[row] = RMSNorm(r[row]),
 * with round() the rounding of y to the FFN dtype, RMSNorm(v) = v /
 * sqrt(mean(v^2) + 1e-6) (no learned scale), r fp32.  Pass NULL for none. */
typedef struct {
  float* r;              /* [rows][d] fp32 residual stream, updated in place; required */
  const float* bias;     /* [d] fp32 added to r after y, or NULL */
  void* x_next;          /* [rows][d] in the FFN dtype, or NULL */
  /* Optional fusion of the next layer's token score (§4.1, Eq. 2): with
   * score_key non-NULL (x_next and score_ref required), every row's key of
   * x_next against score_ref is written exactly as ctx_select computes it
   * (key_out), so the next selection is ctx_select_from_keys. */
  const void* score_ref; /* [rows][d] in the FFN dtype: the next layer's cached input */
  double* score_key;     /* [rows] out, or NULL */
  int32_t score_kind;    /* cgs_score_kind */
} cgs_glue;

/* ---- host helpers ------------------------------------------------------ */

/* ceil(rho * n) as in §4.1 (ceil(rho_p P) tokens) and §5 (K = ceil(rho_n H)),
 * computed as ceil(rho*n - 1e-9) and clamped to [0, n]. */
int cgs_ratio_to_count(double rho, int n);

/* Static string for a cgs_status value. */
const char* cgs_status_str(int status);

/* Checked mode, for debugging callers (initially on iff the environment
 * variable CGS_VALIDATE is set and not "0"): entry points that take index
 * lists or values with a documented range first check them on the device
 * (idx ascending, unique and in range; |x| <= 2^12 for the token score;
 * |h| < 2^24 and |w| < 2^5 for contribution scores; finite keys), wait for
 * the check on their stream and return CGS_ERR_DATA before launching
 * anything else.  The mode synchronises streams and allocates one int per
 * device on first use, so it cannot work on a stream under graph capture: a
 * checked call on a capturing stream returns CGS_ERR_UNSUPPORTED without
 * enqueuing anything (the capture stays valid).  Returns the previous
 * setting. */
int cgs_set_validate(int on);

/* ABI version (major*100 + minor). */
int cgs_version(void);

/* ---- Context Cache ----------------------------------------------------- */

/* Workspace bytes for ctx_select with P tokens. */
size_t cgs_ctx_select_workspace(int P, int d);

/* §4.1, Eq. 2 + the selected set P_l(rho_p): score every token of x against
 * x_ref and return the k highest-scoring token indices.
 *   x, x_ref : [P][d] dtype, the current FFN input after RMSNorm and the
 *              cached reference input of the same layer.
 *   k        : number of tokens to select, 0 <= k <= P (cgs_ratio_to_count).
 *   kind     : cgs_score_kind.
 *   idx_out  : [k] int32, selected token indices in ascending order; ties in
 *              score go to the lower index.
 *   key_out  : [P] double or NULL; the score key of every token (rel-RMS:
 *              d_p^2 in the fixed-point form below; cosine: 1 - cos|cos|).
 * Scores are exact functions of the inputs: per-element float64 terms are
 * rounded to int64 at 2^-24 and summed as integers, and the key is
 * fl64(Sd) / fl64(max(Sx, E)), E = max(1, ceil(d 2^24 / 10^12)).  Requires
 * |x|, |x_ref| <= 2^12 and d <= 4096.  P <= 65536. */
int ctx_select(const void* x, const void* x_ref, int P, int d, int dtype, int k, int kind,
               int32_t* idx_out, double* key_out, void* ws, size_t ws_bytes, void* stream);

/* §4.1: the set P_l(rho_p) from scores already computed (the key_out of
 * ctx_select, or the score_key of a finish kernel's glue): the k highest keys,
 * indices ascending, ties to the lower index.  keys: [P] double (device);
 * k <= P <= 65536.  No workspace. */
int ctx_select_from_keys(const double* keys, int P, int k, int32_t* idx_out, void* stream);

/* Workspace bytes for ctx_ffn_recompute with k selected rows. */
size_t cgs_ctx_ffn_recompute_workspace(int k, int P, int d, int ff, int dtype);

/* §4.1, Eq. 3: y_out[p] = F(x[p]) for p in idx, y_out[p] = y_ref[p] otherwise.
 *   w      : FFN with down_layout CGS_DOWN_DF.
 *   x      : [P][d] current FFN inputs; y_ref: [P][d] cached reference outputs.
 *   idx    : [k] int32, ascending, unique, in [0, P) (the selected visual
 *            tokens plus any always-recomputed rows the caller adds).
 *   y_out  : [P][d] dtype, must not alias y_ref or x.
 *   glue   : NULL or the residual/RMSNorm glue applied to every row of y_out
 *            (rows [P][d]); glue->r non-NULL.
 * Unselected rows are copied bit for bit.  k = 0 is a pure copy; k = P is
 * the dense FFN.  The hidden activation is rounded to dtype before the down
 * projection; products accumulate in fp32.  Row pointers must be 16-byte
 * aligned (d % 128 == 0 does it for aligned bases).  CGS_ERR_UNSUPPORTED if
 * P*d, ff*d or k*ff elements span 2^32 bytes or more (see the size limit). */
int ctx_ffn_recompute(const cgs_ffn* w, const void* x, const void* y_ref, const int32_t* idx,
                      int k, int P, void* y_out, const cgs_glue* glue, void* ws, size_t ws_bytes,
                      void* stream);

/* ---- Action Cache ------------------------------------------------------ */

/* Workspace bytes for act_build_mask. */
size_t cgs_act_build_mask_workspace(int T, int S, int ff, int d);

/* §3.4 Eq. 1 and §5: group-shared neuron mask of one layer.
 *   h_ref     : [T][ff][S] float, post-GeGLU activations of the group's T
 *               reference denoising steps (S action tokens).
 *   w         : FFN with down_layout CGS_DOWN_FD (only w_down is read).
 *   mode      : cgs_mask_mode; K (TOPK, 0 <= K <= ff) or coverage (COVERAGE,
 *               0 <= coverage <= 1).
 *   mask_out  : [ceil(ff/64)] uint64; bit n%64 of word n/64 set iff n kept.
 *   idx_out   : [ff] int32; kept neurons ascending, then -1 up to ff.
 *   count_out : [1] int32 (device), number of kept neurons.
 * Scores: A[t,n] = sum_r rint(2^24 |h|), B[n] = sum_j rint(2^40 w^2) (int64),
 * nrm = sqrt(fl64(B)), c[t,n] = fl64(A) nrm, s[n] = fl64(sum_t A) nrm.
 * TOPK: union over t of the top K of c[t,:], then the top K of the union by
 * s (ties to the lower index).  COVERAGE: with z = rint(s 2^-e), e =
 * ilogb(max s) - (61 - ceil(log2 ff)), the shortest prefix of neurons in
 * (s desc, n asc) order with fl64(sum z) >= fl64(coverage fl64(sum_all z)).
 * Requires |h| < 2^24, S*T <= 2^14, |w| < 2^5, d <= 4096, ff <= 65536. */
int act_build_mask(const float* h_ref, int T, int S, const cgs_ffn* w, int mode, int K,
                   double coverage, uint64_t* mask_out, int32_t* idx_out, int32_t* count_out,
                   void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for act_build_masks over `layers` layers (1 .. 64). */
size_t cgs_act_build_masks_workspace(int layers, int T, int S, int ff, int d);

/* act_build_mask for `layers` layers of one group in one pair of launches
 * (the layers are independent: §5 builds each layer's mask from its own
 * contributions).  h_ref: [layers][T][ff][S] float; w: host array of
 * `layers` FFNs with equal d, ff and dtype, CGS_DOWN_FD; mask_out:
 * [layers][ceil(ff/64)]; idx_out: [layers][ff]; count_out: [layers] (device).
 * Every layer's outputs are exactly act_build_mask's for that layer. */
int act_build_masks(const float* h_ref, int layers, int T, int S, const cgs_ffn* w, int mode, int K,
                    double coverage, uint64_t* mask_out, int32_t* idx_out, int32_t* count_out,
                    void* ws, size_t ws_bytes, void* stream);

/* The down-projection norms of Eq. 1 (§3.4), a property of the weights:
 * nrm_out[l][n] = sqrt(fl64(B[n])) of layer l, correctly rounded, with
 * B[n] = sum_j rint(2^40 fl64(w_nj^2)) (the exact fixed-point sum that
 * act_build_mask forms).  w: host array of `layers` (1 .. 64) FFNs with
 * equal d (<= 4096), ff (<= 65536) and dtype, CGS_DOWN_FD; only w_down is
 * read.  nrm_out: [layers][ff] double (device).  Precondition |w| < 2^5
 * (checked only in checked mode). */
int act_down_norms(const cgs_ffn* w, int layers, double* nrm_out, void* stream);

/* act_build_masks with the weight norms given (nrm: [layers][ff] as
 * act_down_norms writes them, finite and non-negative), so that only h_ref
 * is read: the group's masks, indices and counts are bit for bit those of
 * act_build_masks over the weights the norms came from.  The workspace is
 * cgs_act_build_masks_workspace(layers, T, S, ff, d) for any d.  Errors as
 * act_build_masks. */
int act_build_masks_normed(const float* h_ref, int layers, int T, int S, const double* nrm, int ff,
                           int mode, int K, double coverage, uint64_t* mask_out, int32_t* idx_out,
                           int32_t* count_out, void* ws, size_t ws_bytes, void* stream);

/* §5 keeps each cache entry's group masks with the entry (bit-packed, the
 * mask_out format above); §4.1's masked steps read a mask as its list of
 * neurons.  This turns n stored masks back into those lists.
 *   masks     : [n][ceil(ff/64)] uint64 (8-byte aligned); bit i%64 of word
 *               i/64 set iff neuron i is in the mask; bits at positions >= ff
 *               are ignored.
 *   idx_out   : [n][ff] int32; row m: the neurons of mask m ascending, then -1
 *               up to ff (act_build_mask's idx_out layout).
 *   count_out : [n] int32 (device) or NULL; the number of neurons of mask m.
 * 1 <= ff <= 65536; n = 0 is a no-op.  No workspace. */
int act_mask_indices(const uint64_t* masks, int n, int ff, int32_t* idx_out, int32_t* count_out,
                     void* stream);

/* Workspace bytes for act_ffn_masked with S tokens and K masked neurons. */
size_t cgs_act_ffn_masked_workspace(int S, int K, int d, int ff);

/* §4.1, Eq. 4: y = y_anchor + (h^M - h_anchor^M) W_down[M] for the mask M.
 *   w          : FFN with down_layout CGS_DOWN_FD.
 *   x          : [S][d] dtype, the FFN input after RMSNorm.
 *   idx        : [K] int32 mask, ascending, unique, in [0, ff).
 *   y_anchor   : [S][d] float or NULL (NULL = 0: a plain masked FFN).
 *   h_anchor   : [ff][S] float or NULL (NULL = 0); only rows idx are read.
 *   y_out      : [S][d] dtype.
 *   y_f32_out  : [S][d] float or NULL; the same result before rounding.
 *   h_out      : [ff][S] float or NULL; rows idx receive h^M, other rows
 *                are not written.
 *   glue       : NULL or the residual/RMSNorm glue applied to y (rows [S][d]).
 * With idx = 0..ff-1 and NULL anchors this is the dense anchor step; its
 * y_f32_out / h_out are the anchor state of later steps.  A list of K = ff
 * entries can only be 0..ff-1 under the precondition above, so such a call
 * reads the weight rows in order without consulting idx.  Only rows idx of
 * w_gate, w_up and w_down are read.  The delta h - h_anchor is rounded to
 * dtype before the down projection.  K = 0 gives y = y_anchor (or 0). */
int act_ffn_masked(const cgs_ffn* w, const void* x, int S, const int32_t* idx, int K,
                   const float* y_anchor, const float* h_anchor, void* y_out, float* y_f32_out,
                   float* h_out, const cgs_glue* glue, void* ws, size_t ws_bytes, void* stream);

/* §4.1 and §5: the selected neuron weights of a group prepared once, into
 * compact buffers that every masked step of the group reuses (the pages
 * gather them on a side stream while the prefill runs).  Copies rows
 * idx[0..K-1] of w_gate, w_up and the neuron-major w_down into [K][d]
 * buffers.
 *   w      : FFN with down_layout CGS_DOWN_FD.
 *   idx    : [K] int32 in [0, ff) (device).
 *   wg_out, wu_out, wd_out : [K][d] dtype each (device, caller-owned, not
 *            overlapping the weights).
 * (wg_out, wu_out, wd_out) with ff = K and CGS_DOWN_FD is the compact FFN of
 * act_ffn_masked_compact.  K = 0 is a no-op.  No workspace. */
int act_gather_rows(const cgs_ffn* w, const int32_t* idx, int K, void* wg_out, void* wu_out,
                    void* wd_out, void* stream);

/* One layer of act_gather_rows_layers. */
typedef struct {
  cgs_ffn w;              /* the full FFN, CGS_DOWN_FD */
  const int32_t* idx;     /* [K] int32 in [0, w.ff) (device) */
  int32_t K;              /* rows to copy, 0 <= K <= w.ff */
  void* wg_out;           /* [K][d] each (device, caller-owned, not overlapping the weights) */
  void* wu_out;
  void* wd_out;
} cgs_gather_layer;

/* act_gather_rows for n layers (1 .. 32, equal d and dtype) in one launch:
 * the compact weights of a whole mask group at once (§4.1, §5), e.g. when a
 * cache entry's masks enter the working set.  Each layer's results are
 * exactly act_gather_rows's.  In checked mode every idx is checked first.
 * No workspace. */
int act_gather_rows_layers(const cgs_gather_layer* layers, int n, void* stream);

/* §4.1, Eq. 4 on compact weights: as act_ffn_masked for the full FFN and the
 * mask idx, but wc holds only the mask's rows (wc->ff == K; row i is neuron
 * idx[i], as act_gather_rows writes them), so no weight address depends on
 * the index list.  idx [K] (original neuron ids) addresses only the rows of
 * h_anchor and h_out, which stay [ff][S] over the original neurons; it may be
 * NULL when both are NULL.  With K = 0 the weights may be NULL.  Results are
 * identical to act_ffn_masked's.
 * Workspace: cgs_act_ffn_masked_workspace(S, K, d, K). */
int act_ffn_masked_compact(const cgs_ffn* wc, const void* x, int S, const int32_t* idx, int K,
                           const float* y_anchor, const float* h_anchor, void* y_out,
                           float* y_f32_out, float* h_out, const cgs_glue* glue, void* ws,
                           size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * act_ffn_masked_compact without a workspace argument.  Its kernels use a
 * scratch array that the library holds in device memory, one copy per GPU,
 * kept until the process ends; the call allocates nothing.
 *   Limit: cgs_act_ffn_masked_workspace(S, K, d, K) <= CGS_NOALLOC_SCRATCH_BYTES
 *   (8 MiB: it holds e.g. S <= 64 tokens with K <= 4096 neurons at d <= 1024);
 *   larger calls return CGS_ERR_WORKSPACE before any launch.
 * The scratch's device address is looked up on the first call on each device
 * (the current device; `stream` must belong to it, else CGS_ERR_ARG);
 * CGS_ERR_LAUNCH if that lookup fails.  Nothing in the scratch has to start at
 * zero: each call writes every scratch element it reads.  All calls on one GPU
 * share its scratch, so calls that overlap in time on one GPU (on different
 * streams, or from several threads without ordering) race and give wrong
 * results.  The checked mode (cgs_set_validate) does not apply to this call.
 * Arguments, results and other errors as act_ffn_masked_compact. */
#define CGS_NOALLOC_SCRATCH_BYTES (8u << 20)
int act_ffn_masked_compact_noalloc(const cgs_ffn* wc, const void* x, int S, const int32_t* idx, int K,
                                   const float* y_anchor, const float* h_anchor, void* y_out,
                                   float* y_f32_out, float* h_out, const cgs_glue* glue, void* stream);

/* One layer of act_masked_layers: Eq. 4 (§4.1) on the compact weights of the
 * layer's mask, as one act_ffn_masked_compact call. */
typedef struct {
  cgs_ffn w;              /* the mask's compact FFN: w.ff = K rows (act_gather_rows;
                             the full FFN with K = ff for a dense anchor layer), CGS_DOWN_FD */
  const int32_t* idx;     /* [K] ascending neuron ids (rows of h_anchor / h_out), or NULL
                             when both are NULL */
  const float* y_anchor;  /* [S][d] or NULL (= 0) */
  const float* h_anchor;  /* [ff][S] over the full FFN's neurons, or NULL (= 0) */
  const float* bias;      /* [d] added to r after this layer, or NULL */
  void* y_out;            /* [S][d] dtype, or NULL */
  float* y_f32_out;       /* [S][d], or NULL */
  float* h_out;           /* [ff][S]: rows idx receive h^M, or NULL */
} cgs_masked_layer;

/* Workspace bytes for act_masked_layers with S tokens, width d and masks of
 * at most K_max neurons. */
size_t cgs_act_masked_layers_workspace(int S, int d, int K_max);

/* A chain of n stacked layers of the action expert (§4.1 Eq. 4 with the
 * residual/RMSNorm glue), enqueued by one call: for i = 0 .. n-1
 *   y_i = Eq. 4 of layers[i] on x[i],  r += round(y_i) (+ bias_i),
 *   x[i+1] = RMSNorm(r).
 * Exactly the results of n act_ffn_masked_compact calls with the glue
 * (r, bias_i, x[i+1]).  The layers of several denoising steps may be chained
 * (a dense anchor layer is its full FFN with K = ff and the list 0..ff-1), so
 * a whole denoise whose masks come from a cache entry runs without one host
 * call per layer.
 *   layers : HOST array of n layers, equal d and dtype.
 *   r      : [S][d] fp32 residual stream, updated in place.
 *   x      : [n+1][S][d] dtype; x[0] is read, x[1..n] are written.
 * n = 0 or S = 0 is a no-op.  Errors as act_ffn_masked_compact, checked for
 * every layer before anything is launched (CGS_ERR_WORKSPACE if ws is below
 * cgs_act_masked_layers_workspace(S, d, max K)).  In checked mode every
 * layer's idx is checked first. */
int act_masked_layers(const cgs_masked_layer* layers, int n, int S, float* r, void* x, void* ws,
                      size_t ws_bytes, void* stream);

/* ---- Action Cache: one whole masked denoising step in one launch -------- */

/* act_gather_rows for the persistent step below: rows idx[0..K) of w_gate and
 * w_up into [K][d] buffers, and the same neurons' down weights TRANSPOSED into
 * wdt_out [d][ldk] (wdt_out[j][i] = w_down[idx[i]][j]; columns K .. ldk-1 are
 * written as 0), so that the step kernel reads each output column's weights
 * over the mask contiguously.  idx NULL means the identity (idx[i] = i), e.g.
 * K = ff for a dense anchor step.  bf16 only; w: CGS_DOWN_FD, d % 64 == 0;
 * ldk >= K rounded up to 32, ldk % 8 == 0.  K = 0 writes only the zero
 * columns.  Issued as two kernels on `stream`; no workspace. */
int act_gather_rows_t(const cgs_ffn* w, const int32_t* idx, int K, void* wg_out, void* wu_out,
                      void* wdt_out, int ldk, void* stream);

/* One layer of act_denoise_step (§4.1, Eq. 4 with the residual/RMSNorm glue).
 * The mask M has K neurons; its weights are compact (act_gather_rows_t). */
typedef struct {
  const void* w_gate;    /* [K][d] bf16: row i is neuron idx[i]'s gate weights */
  const void* w_up;      /* [K][d] bf16 */
  const void* w_down_t;  /* [d][ldk] bf16: column i is neuron idx[i]'s down weights */
  int32_t K;             /* mask size, 0 <= K <= min(ff, 4096) */
  int32_t ldk;           /* row stride of w_down_t (>= K rounded up to 32, % 8 == 0) */
  const int32_t* idx;    /* [K] ascending neuron ids (rows of h_anchor / h_out), or NULL
                            for the identity (then K must be ff if h_anchor or h_out is set) */
  const float* y_anchor; /* [S][d] fp32 anchor output, or NULL (= 0) */
  const float* h_anchor; /* [ff][S] fp32 anchor activations (rows idx read), or NULL (= 0) */
  const float* bias;     /* [d] fp32 added to r after this layer, or NULL */
  void* y_out;           /* [S][d] bf16 output y of this layer, or NULL */
  float* y_f32_out;      /* [S][d] fp32 y before rounding, or NULL */
  float* h_out;          /* [ff][S] fp32: rows idx receive h^M, or NULL */
} cgs_step_layer;

/* Workspace bytes for act_denoise_step with masks of at most K_max neurons. */
size_t cgs_act_denoise_step_workspace(int L, int S, int d, int K_max);

/* A whole denoising step of L stacked masked FFN layers in ONE persistent
 * launch (plus a small initialising kernel), for layer l = 0 .. L-1:
 *   y_l = y_anchor_l + (h^M(x_l) - h_anchor_l^M) W_down[M]      (§4.1, Eq. 4)
 *   r  += round_bf16(y_l) (+ bias_l),   x_{l+1} = RMSNorm(r)    (eps 1e-6, no scale)
 * i.e. the same results as L calls of act_ffn_masked_compact with the glue
 * (r, bias_l, x_{l+1}), up to the fp32 summation order.  With K = ff, idx NULL
 * and no anchors a layer is the dense anchor step (y_f32_out / h_out give the
 * anchor state of the later steps).
 *   layers : HOST array of L (1 .. 24) layers.
 *   S      : action tokens, 1 .. 64;  d: 256, 512 or 1024;  ff: neurons of the
 *            full FFN (bound of idx and of the h rows).
 *   r      : [S][d] fp32 residual stream, read at the start and written at the end.
 *   x      : [L+1][S][d] bf16, 16-byte aligned: x[0] is the first layer's input
 *            (RMSNorm(r) rounded, supplied by the caller); x[1..L] receive the
 *            following layers' inputs (x[L] the next step's).  x[1..L] are
 *            also the hand-off buffers between the kernel's workgroups.
 *   status_out : device int32 or NULL; 0 on success, CGS_ERR_TIMEOUT if a
 *            wait inside the kernel gave up (then every output is invalid).
 * The kernel keeps one workgroup per CU resident for the whole step and hands
 * data between them through device-coherent stores and per-wave ready flags
 * (zeroed by the initialising kernel); every wait is bounded
 * (cgs_set_step_wait_limit).  Preconditions: no other launch of this kernel
 * may run on the device at the same time (both would need every CU); the
 * workspace is not shared with a concurrent launch.  Kernels of other
 * streams that hold CUs only delay the step (its remaining workgroups start
 * as CUs free up); a delay past the wait limit ends it with CGS_ERR_TIMEOUT.  CGS_ERR_UNSUPPORTED when
 * the device has fewer than 8 d / 32 or S CUs.  Errors as act_ffn_masked.
 * Steps of several launches (one per call) race if they overlap on a device. */
int act_denoise_step(const cgs_step_layer* layers, int L, int S, int d, int ff, float* r, void* x,
                     int32_t* status_out, void* ws, size_t ws_bytes, void* stream);

/* Time limit of act_denoise_step's waits, in ticks of the 100 MHz device
 * wall clock (default 2e7 = 0.2 s), for the launches that follow; returns the
 * previous value (a negative argument only queries).  A test aid: a limit of
 * 0 makes the first wait that is not already satisfied give up. */
long long cgs_set_step_wait_limit(long long ticks);

/* ---- Reference rebuild ------------------------------------------------- */

/* Workspace bytes for ref_rebuild_dense. */
size_t cgs_ref_rebuild_dense_workspace(int L, int P, int d, int ff, int dtype);

/* §4.2, asynchronous online reconstruction: dense prefill of a compact entry.
 *   layers    : HOST array of L FFNs (down_layout CGS_DOWN_DF), same d/ff/dtype.
 *   r0        : [P][d] dtype, the entry's compact input (residual stream).
 *   x_ref_out : [L][P][d] dtype, xbar_l = RMSNorm(r_l) (no learned scale,
 *               eps 1e-6) rounded to dtype.
 *   y_ref_out : [L][P][d] dtype, ybar_l = F_l(xbar_l).
 * r_{l+1} = r_l + ybar_l with r kept in fp32.  CGS_ERR_UNSUPPORTED if P*d,
 * ff*d or P*ff elements span 2^32 bytes or more (see the size limit). */
int ref_rebuild_dense(const cgs_ffn* layers, int L, const void* r0, int P, void* x_ref_out,
                      void* y_ref_out, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for ref_rebuild_dense_batch (0 if unsupported). */
size_t cgs_ref_rebuild_dense_batch_workspace(int L, int n, int P, int d, int ff, int dtype);

/* ref_rebuild_dense for n entries at once (§4.2: every position entering the
 * working set is reconstructed; with T candidate episodes T of them enter
 * together): one dense prefill over n P rows, so each layer's weights are
 * streamed once for all n entries and the GEMMs run n times the rows.
 *   r0        : [n][P][d] dtype (device), the entries' compact inputs.
 *   x_ref_out, y_ref_out : HOST arrays of n device pointers, entry e's
 *               [L][P][d] outputs as ref_rebuild_dense writes them (16-byte
 *               aligned, caller-owned, not overlapping each other or r0).
 * Each entry's results are those of ref_rebuild_dense on that entry alone up to
 * the fp32 summation order of the down projection's K splits (which depends on
 * the rows in the launch).  1 <= n <= 16; CGS_ERR_UNSUPPORTED if n*P*d, ff*d or
 * n*P*ff elements span 2^32 bytes or more.  Errors otherwise as
 * ref_rebuild_dense. */
int ref_rebuild_dense_batch(const cgs_ffn* layers, int L, const void* r0, int n, int P,
                            void* const* x_ref_out, void* const* y_ref_out, void* ws, size_t ws_bytes,
                            void* stream);

/* ---- Inter-layer glue (standalone) -------------------------------------- */

/* Residual add and RMSNorm between FFN layers (the glue of a layer stack,
 * not part of the selective FFN itself):
 *   r[m] = (r_in ? r_in[m] : r[m]) + (y ? y[m] : 0) + (bias ? bias : 0);
 *   x_out[m] = RMSNorm(r[m]) (eps 1e-6, no learned scale).
 *   r     : [M][d] float, written (read too when r_in is NULL); required.
 *   r_in  : [M][d] float or NULL, a separate source for the residual.
 *   y     : [M][d] y_dtype or NULL; bias: [d] float or NULL.
 *   x_out : [M][d] out_dtype or NULL.
 * Requires d % 8 == 0 and 16-byte aligned rows. */
int cgs_residual_rmsnorm(float* r, const float* r_in, const void* y, int y_dtype,
                         const float* bias, int M, int d, void* x_out, int out_dtype,
                         void* stream);

/* ---- Kernel timing (benchmarks) ----------------------------------------- */

/* Start timing every kernel launch whose site name contains `site_filter`
 * ("" = all).  Site names: "ctx.score", "ctx.topk", "ctx.glu", "ctx.down",
 * "ctx.finish", "rebuild.norm", "rebuild.glu", "rebuild.down",
 * "rebuild.finish", "act.glu.dense", "act.glu.masked", "act.down.dense",
 * "act.down.masked", "act.finish", "act.gather", "mask.contrib",
 * "mask.select", "mask.norms", "ret.dot", "ret.select", "glue.rmsnorm".  Each matching
 * launch is bracketed by two HIP events recorded on its stream; at most
 * max_launches are kept, later ones are counted as overflow.  Launches on a
 * stream that is being captured are not timed (a graph replay cannot be
 * bracketed per launch).  Process-wide host state: start, launch and query
 * from one thread. */
int cgs_profile_start(const char* site_filter, int max_launches);

/* Stop recording (the recorded launches stay queryable). */
int cgs_profile_stop(void);

/* Wait for the recorded events of the launches whose site contains `site`
 * (NULL = all) and return their summed kernel time in milliseconds and their
 * number.  Returns CGS_ERR_SHAPE if launches overflowed the buffer (the sums
 * cover the kept ones). */
int cgs_profile_result(const char* site, double* total_ms, int* launches);

/* Joint token and neuron sparsity inside the denoising loop (§6.1: for a
 * model whose visual features are concatenated with the denoising actions,
 * visual-token sparsity and neuron sparsity apply together).  Rows tok[0..k)
 * (ascending, unique, in [0, S); the caller's selection, e.g. ctx_select of
 * x against the anchor step's input) get Eq. 4 with the mask:
 *   y[p] = y_anchor[p] + (h^M(x[p]) - h_anchor^M[:, p]) W_down[M];
 * every other row keeps the anchor output, y[p] = y_anchor[p] (rounded to
 * dtype).  Weights are compact (wc->ff == K, row i is neuron idx[i]; see
 * act_gather_rows); idx [K] addresses the rows of h_anchor [ff][S].
 *   x: [S][d]; y_anchor: [S][d] float (required); h_anchor: [ff][S] float
 *   (required when k > 0 and K > 0); y_out: [S][d] dtype; y_f32_out: [S][d]
 *   float or NULL; glue: NULL or the residual/RMSNorm glue on all S rows.
 * k = S with tok = 0..S-1 equals act_ffn_masked_compact; k = 0 gives the
 * anchor output on every row.  Workspace: cgs_act_ffn_masked_workspace(max(k,
 * 1), K, d, max(K, 1)). */
int act_ffn_joint(const cgs_ffn* wc, const void* x, int S, const int32_t* tok, int k, const int32_t* idx,
                  int K, const float* y_anchor, const float* h_anchor, void* y_out, float* y_f32_out,
                  const cgs_glue* glue, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Reference retrieval over the prepared entries (§4.2 "Retrieving a Relevant
 * Reference"; §5 "Joint-History Retrieval" and "Fallback policy").
 * ------------------------------------------------------------------------ */
typedef struct {
  int hist_len;    /* L: aligned robot-state history steps */
  int joints;      /* J: joints per step, two arms of J/2 (even) */
  int arm;         /* -1: dual-arm task (larger of the two arm distances); 0 or 1: that arm */
  double min_cos;  /* below this best visual cosine, no reference is used (the paper: 0.8) */
} cgs_rerank;

/* Workspace bytes for ret_select over N entries of F features (0 if invalid). */
size_t cgs_ret_select_workspace(int N, long long F);

/* query: [F] features (dtype, device); refs: [N][F] the prepared entries'
 * features (1 <= N <= 256, 8 <= F <= 2^24, F % 8 == 0, both 16-byte aligned).
 * Precondition |feature| <= 2^7, so that the integer sums below cannot
 * overflow (every rounded product is <= 2^38, a sum of 2^24 of them < 2^63).
 * Visual match: cos_n = Sqr / sqrt(Sqq Srr) from the exact fixed-point sums
 * of the token score's cosine kind (every feature product rounded half-even
 * to an int64 at 2^-24; float64 key, 0 if a norm is 0), written to
 * cos_out[N].  top_out[T] (1 <= T <= N): the T best entries by (cos desc,
 * index asc).  Rerank: dist_out[r] = RMS over the L steps and the arm's J/2
 * joints of q_hist - r_hist[top_out[r]] (float histories [L][J] and
 * [N][L][J], device), the larger arm for arm = -1.  choice_out[0]: the
 * candidate of smallest distance (ties to the better visual rank), or -1 if
 * cos of the best match < min_cos (fallback to dense execution). */
int ret_select(const void* query, const void* refs, int N, long long F, int dtype, int T,
               const float* q_hist, const float* r_hist, const cgs_rerank* rr, double* cos_out,
               int32_t* top_out, double* dist_out, int32_t* choice_out, void* ws, size_t ws_bytes,
               void* stream);

/* ------------------------------------------------------------------------
 * Sliding GPU working set (§4.2 "Sliding Window Prefetching", Figure 12) and
 * reconstruction budget (§4.2 Eq. 5, Table 2).  Host logic only: these calls
 * touch no device memory and launch nothing; the caller rebuilds the entries
 * an advance admits (ref_rebuild_dense into the named slot).
 * ------------------------------------------------------------------------ */

/* Eq. 5: N_prep = min(N_cand, floor(M_free / M_entry), floor((T_avl - T_trans) / T_rec)),
 * clamped at 0.  Memory in bytes, times in one unit (e.g. ms); T_avl may be
 * +inf.  Returns -1 for n_cand < 0, M_entry <= 0, T_rec <= 0, M_free < 0 or a
 * NaN time. */
int cgs_prep_budget(int n_cand, double m_free, double m_entry, double t_avl, double t_trans,
                    double t_rec);

/* Table 2's parameters for one advance of the window. */
typedef struct {
  double m_free;   /* free device memory for new entries, bytes */
  double m_entry;  /* expanded footprint of one entry, bytes */
  double t_avl;    /* time available for reconstruction before the next call */
  double t_trans;  /* input-transfer time of the batch (same unit) */
  double t_rec;    /* average reconstruction time of one entry (same unit), > 0 */
} cgs_budget;

/* The working set: `slots` device slots (1 .. 2^20), initially empty. */
typedef struct cgs_window cgs_window;
cgs_window* cgs_window_create(int slots);
void cgs_window_destroy(cgs_window* w);

/* Slot holding (episode, position), or -1 if that entry is not resident. */
int cgs_window_slot(const cgs_window* w, int episode, int position);

/* Number of resident entries (-1 for a NULL window). */
int cgs_window_resident(const cgs_window* w);

/* One advance.  The window is, for each of the T candidate episodes in rank
 * order (episode[r], distinct, >= 0), the positions position[r] .. position[r]
 * + L that are below length[r].  Resident entries outside the window are
 * released: their slots, ascending, go to leave_slot[0 .. *n_leave).  The
 * window's entries that are not resident are the candidates (count in
 * *n_cand, may be NULL), ordered nearest position first (offset from
 * position[r]), then by episode rank; the first N_prep of them take the
 * lowest free slots and are listed in enter_ep/enter_pos/enter_slot[0 ..
 * *n_enter), where N_prep = min(candidates, free slots, Eq. 5 of `budget`
 * when budget is non-NULL).  Candidates beyond N_prep stay candidates at the
 * next advance.  The initial-position preload is an advance with the task's
 * reference episodes at position 0 and L = 0.  All output arrays are host
 * memory of at least `slots` elements.  Invalid arguments (a NULL pointer, a
 * negative T, L, episode, position or length, an episode listed twice, a bad
 * budget) return an error before the working set changes. */
int cgs_window_advance(cgs_window* w, int T, const int32_t* episode, const int32_t* position,
                       const int32_t* length, int L, const cgs_budget* budget, int32_t* enter_ep,
                       int32_t* enter_pos, int32_t* enter_slot, int32_t* n_enter, int32_t* leave_slot,
                       int32_t* n_leave, int32_t* n_cand);

/* The denoising schedule a cache entry's stored masks imply (§4.1 "Anchors
 * with Mask Recomputation"; §5 builds one mask per layer for every step of a
 * group).  An entry stores one mask per (layer, step): L x T masks of ff
 * bits.  A step whose masks hold every neuron in all L layers is a dense
 * anchor step, which refreshes the anchor state; every other step is an Eq. 4
 * update against the latest anchor with that step's masks.  The one-group
 * schedule is [all, G, G, G], two groups [all, G1, all, G2].
 *   counts : [L][T] neurons per mask (host); must equal the masks' bit counts.
 *   words  : [L][T][ceil(ff/64)] uint64 (host), the masks in act_build_mask's
 *            format (bits at positions >= ff ignored).
 *   kind_out   : [T] 0 = anchor, 1 = masked update.
 *   anchor_out : [T] for an anchor its ordinal among the anchors (0, 1, ..),
 *                for an update the ordinal of the latest anchor before it.
 *   mask_out   : [T] for an update the first update step whose L masks are
 *                the same bits as this step's (whose compact weights it can
 *                reuse); -1 for an anchor.
 * CGS_ERR_SHAPE if L, T or ff is out of range (1 .. 64, 1 .. 64, 1 .. 65536)
 * or step 0 is not an anchor; CGS_ERR_ARG for a NULL pointer or a count that
 * differs from its mask's bits.  Host logic only. */
int cgs_denoise_schedule(int L, int T, int ff, const int32_t* counts, const uint64_t* words,
                         int32_t* kind_out, int32_t* anchor_out, int32_t* mask_out);

#ifdef __cplusplus
}
#endif
#endif /* CGS_H */
