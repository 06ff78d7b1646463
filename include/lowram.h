/*
 * lowram.h — C ABI of the LowRAM decode path on MI355X (gfx950).
 *
 * Method: "LowRAM: Low-Rank Keys and Amortised Values for Composable KV Cache
 * Compression at Test-Time" (arXiv:2611.07025).  Sources cited below:
 *   [ABS]  the arXiv listing, Abstract;
 *   [EXPL] "LowRAM Paper: Amortised Values and Low-Rank Keys for KV
 *          Compression" (wpnews copy of an explainx.ai post), by section;
 *   [WIKI] "LowRAM: predict values from keys, store only the misses", by
 *          section.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer allocated and owned by the
 *    caller; the library never allocates, frees or synchronises.  Scratch
 *    memory is the caller's `workspace` (size from lowram_workspace_size).
 *  - Every call is asynchronous on the caller's `hip_stream` (a hipStream_t;
 *    NULL = the default stream).  Inputs must stay alive, and outputs must
 *    not be read, until the stream has reached the work.
 *  - Arrays are contiguous, row-major, in the index order written next to
 *    each argument.  bf16 is raw IEEE bfloat16 (uint16), fp16 scales are raw
 *    IEEE binary16.  int4 packs two two's-complement nibbles per byte,
 *    element 2i in the low nibble of byte i, with one fp16 scale per 32
 *    consecutive elements of the last axis (x = code * scale).
 *  - Return value: LOWRAM_OK or a negative lowram_status.  Shape and
 *    pointer arguments are checked on the host before anything is launched;
 *    on error nothing is launched and lowram_last_error() describes the
 *    problem.  A failed launch returns LOWRAM_E_HIP.  Faults inside kernels
 *    surface at the caller's next synchronisation.
 *  - Device-side preconditions (not checked by default; violating them
 *    gives unspecified results but never out-of-bounds accesses): indices
 *    are sorted ascending and unique; n_body[b] <= n_body_max;
 *    tail_len[b] <= tail_max.  Out-of-range indices are skipped.  With the
 *    environment variable LOWRAM_VALIDATE=1, lowram_decode_attn copies the
 *    call's index arrays to the host (on its stream, and waits for them),
 *    checks them with lowram_check_decode_indices and returns LOWRAM_E_ARG
 *    before any launch if one fails: a debugging aid that synchronises.
 *  - The library is stateless apart from a thread-local error string; calls
 *    on different streams may run concurrently if their outputs and
 *    workspaces do not overlap.
 *
 * Notation: B batch, G layers per group, Hq / Hkv query / KV heads (query
 * head qh reads KV head qh / (Hq/Hkv)), d head dim, r basis rank,
 * D = G*Hkv*d, N = n_body_max stored body rows, m = n_resid residual rows
 * per (sequence, layer, KV head), Te = tail_max.
 */
#ifndef LOWRAM_H
#define LOWRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LOWRAM_F32 = 0, LOWRAM_BF16 = 1 } lowram_dtype;
typedef enum { LOWRAM_STORE_NATIVE = 0, LOWRAM_STORE_INT4_G32 = 1 } lowram_store;
typedef enum {
  LOWRAM_OK = 0,
  LOWRAM_E_ARG = -1,          /* malformed shape, index or pointer          */
  LOWRAM_E_UNSUPPORTED = -2,  /* well-formed but outside the built kernels  */
  LOWRAM_E_WORKSPACE = -3,    /* workspace missing or too small             */
  LOWRAM_E_HIP = -4           /* a HIP launch or runtime call failed        */
} lowram_status;

/* Kernel choice for lowram_decode_attn and lowram_compress_prefill: AUTO
 * picks the MFMA kernels when the shape allows them (bf16, d = 128, r a
 * multiple of 64; prefill also r <= 512) and the plain kernels otherwise;
 * MFMA on a shape they do not support returns LOWRAM_E_UNSUPPORTED. */
typedef enum { LOWRAM_ALGO_AUTO = 0, LOWRAM_ALGO_PLAIN = 1, LOWRAM_ALGO_MFMA = 2 } lowram_algo;

/* Shape of one layer group's compressed cache. */
typedef struct {
  uint32_t struct_size;       /* = sizeof(lowram_shape)                      */
  int32_t batch;              /* B >= 1                                      */
  int32_t group_layers;       /* G >= 1: layers sharing one key basis        */
  int32_t n_q_heads;          /* Hq, a multiple of Hkv, Hq/Hkv <= 8          */
  int32_t n_kv_heads;         /* Hkv >= 1                                    */
  int32_t head_dim;           /* d: 64 or 128                                */
  int32_t rank;               /* r: multiple of 32, r <= D                   */
  int32_t n_body_max;         /* N: body rows allocated per sequence         */
  int32_t n_resid;            /* m: 0 <= m <= N                              */
  int32_t tail_max;           /* Te: exact tail rows allocated per sequence  */
  double rope_theta;          /* RoPE base theta > 0                         */
  int32_t dtype;              /* lowram_dtype of q, out, basis, predictor,
                                 tail, k/v and native-stored arrays          */
  int32_t coef_store;         /* lowram_store of the coefficients            */
  int32_t resid_store;        /* lowram_store of the residual values         */
  int32_t predictor_shared;   /* 1: predictor arrays have batch dim 1        */
  int32_t algo;               /* lowram_algo                                 */
  int32_t reserved;           /* must be 0                                   */
} lowram_shape;

/* The stored compressed cache of one layer group ([EXPL] "Step-by-step
 * mental model ...", item 1: what prefill leaves behind).  Read only. */
typedef struct {
  const void *coef;           /* [B,N,r] dtype, or int4 bytes [B,N,r/2]      */
  const void *coef_scale;     /* int4 only: fp16 [B,N,r/32]                  */
  const int32_t *pos;         /* [B,N] original position of body row t, or
                                 NULL meaning pos = t (no eviction)          */
  const int32_t *n_body;      /* [B] valid body rows per sequence            */
  const void *basis;          /* [B,r,D] dtype; column (l*Hkv+h)*d + j       */
  const void *w1, *b1;        /* [Bp,G,Hkv,d,d] ([out,in]) and [Bp,G,Hkv,d]  */
  const void *w2, *b2;        /* Bp = 1 if predictor_shared else B           */
  const int32_t *resid_idx;   /* [B,G,Hkv,m] ascending body rows; slots past
                                 n_body hold INT32_MAX                       */
  const void *resid_val;      /* [B,G,Hkv,m,d] dtype, or int4 [..,m,d/2]     */
  const void *resid_scale;    /* int4 only: fp16 [B,G,Hkv,m,d/32]            */
  const void *tail_k;         /* [B,G,Te,Hkv,d] exact post-RoPE keys         */
  const void *tail_v;         /* [B,G,Te,Hkv,d] exact values                 */
  const int32_t *tail_len;    /* [B] valid tail rows                         */
} lowram_cache;

/* Bytes of workspace that op (0 = lowram_compress_prefill,
 * 1 = lowram_decode_attn) needs for this shape; written to *bytes.
 * The size depends only on the shape (including its algo).  Prefill uses it
 * for the step-4 scores when err_out is NULL and, on the MFMA path with few
 * rows, for fp32 partial coefficients; lowram_compress_prefill accepts a
 * NULL workspace when it needs neither. */
int32_t lowram_workspace_size(const lowram_shape *shape, int32_t op, size_t *bytes);

/*
 * lowram_compress_prefill — compress the prompt body of one layer group.
 *
 * [EXPL] "Step-by-step mental model for one decoding session", item 1, with
 * "Asymmetric key compression with xKV" and "Value cache amortisation in
 * plain language"; [ABS] (residuals are kept only for the tokens whose
 * values the predictor regenerates worst).  Per sequence b:
 *   1. undo the rotary embedding of every key at its position pos[t];
 *   2. concatenate the pre-RoPE keys of all (layer, head) into one D-vector
 *      per row and project it on the caller's basis: c[t] = basis[b] x[t];
 *      store c (rounded to dtype, or int4 with per-32 fp16 scales);
 *   3. rebuild the keys from the STORED coefficients: k^[t] = c[t] basis[b];
 *   4. predict each value from its rebuilt pre-RoPE key with the caller's
 *      per-(layer, head) MLP f(k) = W2 gelu(W1 k + b1) + b2 (exact erf
 *      GELU) and score e = sum_j (v_j - f_j)^2 per (layer, row, head);
 *   5. per (b, layer, head) select the m rows with the largest e (ties to
 *      the lower row, NaN above +inf), listed in ascending row order;
 *   6. store the residuals v - f of the selected rows.
 * The basis and the predictor weights are inputs (fitting them is not part
 * of this call).
 * Arithmetic of the MFMA kernels: step 2 splits the fp32 pre-RoPE keys into
 * two bf16 halves so the coefficients keep fp32 accuracy before storage;
 * step 4 rounds the rebuilt keys and hidden activations to bf16 for the
 * matrix cores and evaluates GELU by a polynomial of the normal tail
 * (|error| <= 2e-4 |x|); step 6 keeps both to near fp32 (bf16 pairs) with
 * the exact erf.  The plain kernels compute in fp32 throughout.
 *
 * k_post, v  [B,G,N,Hkv,d] dtype   keys as the model produced them (post
 *                                  RoPE) and values
 * pos        [B,N] int32 or NULL   original positions (NULL: pos = t)
 * n_body     [B] int32             rows t >= n_body[b] are padding: their
 *                                  coefficients are written as 0, err 0,
 *                                  and they are never selected; when
 *                                  m > n_body[b] the trailing index slots
 *                                  hold INT32_MAX with zero residuals
 * basis, w1, b1, w2, b2            as in lowram_cache
 * coef_out, coef_scale_out         as lowram_cache.coef / coef_scale
 * resid_idx_out, resid_val_out, resid_scale_out   as in lowram_cache
 * err_out    [B,G,Hkv,N] fp32 or NULL   the step-4 scores
 * workspace  lowram_workspace_size(shape, 0) bytes (see there)
 * Errors: LOWRAM_E_ARG (shape, NULL required pointer), _UNSUPPORTED,
 * _WORKSPACE, _HIP.
 */
int32_t lowram_compress_prefill(const lowram_shape *shape,
                                const void *k_post, const void *v,
                                const int32_t *pos, const int32_t *n_body,
                                const void *basis,
                                const void *w1, const void *b1,
                                const void *w2, const void *b2,
                                void *coef_out, void *coef_scale_out,
                                int32_t *resid_idx_out, void *resid_val_out,
                                void *resid_scale_out, float *err_out,
                                void *workspace, size_t workspace_bytes,
                                void *hip_stream);

/*
 * lowram_append_body — fold exact rows into the compressed body.
 *
 * [EXPL] "Asymmetric key compression with xKV", last paragraph: newly decoded
 * tokens keep exact K/V (the exact tail).  Folding some of them into the
 * compressed body is the prefill steps 1-6 above applied to those rows with
 * the sequence's existing basis and predictor.  Per sequence b:
 *   - the n_new rows become body rows n_body[b] .. n_body[b] + n_new - 1:
 *     coefficients projected and stored as in prefill; their positions are
 *     stored in pos when the cache has positions;
 *   - per (layer, head), m_new of them are chosen by prefill's rule (largest
 *     e, ties to the lower row) among the new rows; they follow the entries
 *     already stored in resid_idx (those < n_body[b]), ascending, with their
 *     residuals v - f in the same slots;
 *   - n_body[b] grows by n_new.
 * Rows and residuals already stored are not changed.  Removing the folded
 * rows from the exact tail is the caller's (like every tail write).
 *
 * k_post_new, v_new [B,G,n_new,Hkv,d] dtype   the rows to fold: keys as the
 *                                             model produced them, values
 * pos_new    [B,n_new] int32 or NULL     their positions; NULL: n_body[b] + t
 *                                        (required when pos is not NULL)
 * basis, w1, b1, w2, b2                  as in lowram_cache
 * n_body     [B] int32, in/out
 * pos        [B,N] int32 or NULL         the cache's positions, in/out
 * coef, coef_scale, resid_idx, resid_val, resid_scale   the cache, in/out
 * err_out    [B,G,Hkv,n_new] fp32 or NULL   the new rows' step-4 scores
 * workspace  lowram_append_workspace_size(shape, n_new, m_new) bytes
 * Counts: 0 <= n_new <= n_body_max, 0 <= m_new <= min(n_new, n_resid).
 * Device-side preconditions: n_body[b] + n_new <= n_body_max, and the
 * entries stored below n_body[b] plus m_new fit in n_resid slots; rows or
 * entries that do not fit are dropped.
 * Errors: LOWRAM_E_ARG (shape, counts, NULL required pointer), _UNSUPPORTED,
 * _WORKSPACE, _HIP.
 */
int32_t lowram_append_workspace_size(const lowram_shape *shape, int32_t n_new,
                                     int32_t m_new, size_t *bytes);
int32_t lowram_append_body(const lowram_shape *shape, int32_t n_new,
                           int32_t m_new, const void *k_post_new,
                           const void *v_new, const int32_t *pos_new,
                           const void *basis, const void *w1, const void *b1,
                           const void *w2, const void *b2, int32_t *n_body,
                           int32_t *pos, void *coef, void *coef_scale,
                           int32_t *resid_idx, void *resid_val,
                           void *resid_scale, float *err_out,
                           void *workspace, size_t workspace_bytes,
                           void *hip_stream);

/* Hyperparameters of lowram_fit_predictor. */
typedef struct {
  uint32_t struct_size;       /* = sizeof(lowram_fit_params)                 */
  int32_t steps;              /* >= 0 full-batch Adam steps                  */
  double lr;                  /* step size, finite and > 0                   */
  double beta1, beta2;        /* moment decay rates, each in [0, 1)          */
  double eps;                 /* added to sqrt of the second moment, > 0     */
} lowram_fit_params;

/*
 * lowram_fit_predictor — fit the value predictors of one layer group to its
 * stored body rows, at test time.
 *
 * [EXPL] "Value cache amortisation in plain language" (during prefill a
 * small per-head MLP is fitted to map each token's key to its value) and
 * "Step-by-step mental model ...", item 1; [ABS] (predictors fitted at test
 * time, from scratch or from a meta-learned initialisation).  The pages name
 * no loss or optimiser; this call takes the plainest ones.  For every
 * predictor (b or the shared batch, layer l, KV head h):
 *   rows: t < n_body[b] of its sequence (of every sequence when
 *         predictor_shared), keys rebuilt from the STORED coefficients,
 *         k^_t = (c[t] basis[b]) restricted to the columns of (l, h), i.e.
 *         the pre-RoPE keys decode sees;
 *   loss: L = sum_t sum_j (f(k^_t)_j - v_tj)^2 / (n d), n its row count,
 *         f(k) = W2 gelu(W1 k + b1) + b2 (exact erf GELU);
 *   steps full-batch Adam steps (Kingma and Ba, "Adam: A Method for
 *   Stochastic Optimization", 2015, Algorithm 1): m = beta1 m + (1-beta1) g,
 *   s = beta2 s + (1-beta2) g^2, w -= lr m^ / (sqrt(s^) + eps) with the
 *   bias-corrected m^ = m / (1 - beta1^t), s^ = s / (1 - beta2^t).
 * A predictor with no rows keeps its weights.  The fitted weights are then
 * used by lowram_compress_prefill (which projects again and scores with them)
 * and by decode.
 * Arithmetic: fp32 weights and moments; every matrix product of a step runs
 * on the matrix cores with both operands split into bf16 pairs (x = hi + lo,
 * about 16 significant bits each) and fp32 accumulation; rebuilt keys are
 * formed once, in fp32.  The weights are rounded to dtype once, at the end.
 *
 * coef, coef_scale, n_body, basis   the stored cache (as in lowram_cache)
 * v          [B,G,N,Hkv,d] dtype    the values of the body rows
 * params     steps and Adam hyperparameters
 * w1, b1, w2, b2  in/out: [Bp,G,Hkv,d,d], [Bp,G,Hkv,d] dtype (Bp = 1 if
 *            predictor_shared else B): the initial weights on entry, the
 *            fitted ones once the stream reaches the end of the call
 * loss_out   [steps,Bp,G,Hkv] fp32 or NULL: entry s is the loss at the
 *            weights that step s + 1 starts from
 * grad_out   [Bp,G,Hkv,2d^2+2d] fp32 or NULL: the gradient of the loss at
 *            the initial weights, per predictor in the order W1 (d x d),
 *            b1, W2 (d x d), b2; written when steps >= 1
 * workspace  lowram_fit_workspace_size(shape) bytes: the rebuilt keys and
 *            transposed copies of keys and values (12 N d bytes per
 *            sequence, layer and head), fp32 weights and moments, per-split
 *            partial gradients
 * shape.algo is not used (one kernel set serves every supported shape).
 * Errors: LOWRAM_E_ARG (shape, params, NULL required pointer),
 * _UNSUPPORTED, _WORKSPACE, _HIP.
 */
int32_t lowram_fit_workspace_size(const lowram_shape *shape, size_t *bytes);
int32_t lowram_fit_predictor(const lowram_shape *shape, const void *coef,
                             const void *coef_scale, const int32_t *n_body,
                             const void *basis, const void *v,
                             const lowram_fit_params *params,
                             void *w1, void *b1, void *w2, void *b2,
                             float *loss_out, float *grad_out,
                             void *workspace, size_t workspace_bytes,
                             void *hip_stream);

/*
 * lowram_decode_attn — attention of one new query token over the compressed
 * cache of layer `layer` (0 <= layer < G) of the group.
 *
 * [EXPL] "Step-by-step mental model ...", item 2 and "Asymmetric key
 * compression with xKV" (keys rebuilt from the shared basis and re-rotated;
 * new tokens keep exact K/V), "Value cache amortisation in plain language"
 * (values regenerated from keys plus residuals); [ABS] and [WIKI]
 * flowchart (only a selected subset of KV pairs is rebuilt per step).
 * For sequence b and query head qh with KV head h = qh / (Hq/Hkv):
 *   k~_t = (c[t] basis[b]) restricted to columns of (layer, h)   pre-RoPE
 *   k_t  = RoPE(k~_t, pos[t]);   v^_t = f(k~_t) + residual_t if t is stored
 *   rows: the attended body rows A (all t < n_body[b], or the subset) and
 *   the tail rows j < tail_len[b] (exact keys and values);
 *   s = q . k / sqrt(d), p = softmax(s) over A and the tail,
 *   out = sum p v,  lse = max s + ln sum exp(s - max s).
 * With no attended row: out = 0, lse = -inf.
 *
 * q        [B,Hq,d] dtype        the new token's query, already rotated
 * cache    the stored group (lowram_cache)
 * subset_off [B+1] int32 or NULL, subset_idx [nnz] int32: CSR list of the
 *          body rows to attend per sequence (sorted, unique, shared by all
 *          heads and layers); NULL attends every body row
 * out      [B,Hq,d] dtype;  lse_out [B,Hq] fp32 or NULL
 * Errors: LOWRAM_E_ARG, _UNSUPPORTED, _WORKSPACE, _HIP.
 */
int32_t lowram_decode_attn(const lowram_shape *shape, int32_t layer,
                           const void *q, const lowram_cache *cache,
                           const int32_t *subset_off, const int32_t *subset_idx,
                           void *out, float *lse_out,
                           void *workspace, size_t workspace_bytes,
                           void *hip_stream);

/*
 * lowram_decode_attn_noalloc — lowram_decode_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without the
 * workspace, the same results, checks and errors.  Its scratch memory is a
 * device array inside the library, 64 MiB per GPU, held from the first call
 * on that GPU until the process ends; a call whose decode workspace
 * (lowram_workspace_size, op 1) exceeds 64 MiB returns LOWRAM_E_WORKSPACE
 * before any launch.  It allocates nothing and ignores LOWRAM_VALIDATE.
 * Every call on one GPU shares that array: calls that overlap on one GPU
 * (other streams, other threads) race and must be serialised by the caller.
 */
int32_t lowram_decode_attn_noalloc(const lowram_shape *shape, int32_t layer,
                                   const void *q, const lowram_cache *cache,
                                   const int32_t *subset_off, const int32_t *subset_idx,
                                   void *out, float *lse_out, void *hip_stream);

/*
 * lowram_dense_decode_attn — the uncompressed comparator: the same softmax
 * attention of one query token over an exact bf16 KV cache ([EXPL] "The
 * bottleneck LowRAM targets": the cache LowRAM compresses).
 * q [B,Hq,d] bf16, k and v [B,T,Hkv,d] bf16 (post-RoPE), ctx_len [B] int32
 * (rows t < ctx_len[b] are attended), out [B,Hq,d] bf16, lse_out [B,Hq]
 * fp32 or NULL; workspace from lowram_dense_workspace_size.
 */
int32_t lowram_dense_workspace_size(int32_t batch, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t head_dim,
                                    int32_t max_ctx, size_t *bytes);
int32_t lowram_dense_decode_attn(int32_t batch, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim,
                                 int32_t max_ctx, const void *q,
                                 const void *k, const void *v,
                                 const int32_t *ctx_len, void *out,
                                 float *lse_out, void *workspace,
                                 size_t workspace_bytes, void *hip_stream);

/*
 * lowram_check_decode_indices — the device-side preconditions of
 * lowram_decode_attn, checked on HOST copies of its index arrays (the
 * check LOWRAM_VALIDATE=1 runs; callable on its own, no GPU needed):
 *   n_body [B]: 0 <= n_body[b] <= n_body_max;
 *   tail_len [B] or NULL: 0 <= tail_len[b] <= tail_max;
 *   pos [B,N] or NULL: pos[b][t] >= 0 for t < n_body[b];
 *   resid_idx [B,G,Hkv,m] (required when m > 0): each list strictly
 *     ascending over rows in [0, n_body[b]), then INT32_MAX padding only;
 *   subset_off [B+1] or NULL with subset_idx: subset_off[0] = 0,
 *     non-decreasing; each sequence's entries strictly ascending in
 *     [0, n_body[b]).
 * Returns LOWRAM_OK, or LOWRAM_E_ARG naming the first violation in
 * lowram_last_error().
 */
int32_t lowram_check_decode_indices(const lowram_shape *shape, const int32_t *n_body,
                                    const int32_t *tail_len, const int32_t *pos,
                                    const int32_t *resid_idx, const int32_t *subset_off,
                                    const int32_t *subset_idx);

/* Static name of a status code. */
const char *lowram_status_string(int32_t status);
/* Detail of the last error raised on the calling thread ("" if none). */
const char *lowram_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LOWRAM_H */
