/*
 * ckl.h -- C ABI of libckl, a fused chunked forward-KL distillation loss for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  Given student hidden states H[T, d], the output-head
 * weights W[V, d] and, for every row t, a sparse cached teacher made of K
 * vocabulary indices idx[t, :] and their logits tlogit[t, :], the library
 * evaluates the forward KL divergence KL(p_t || q_t) between
 *   p_t = softmax over the K cached logits (temperature 1), zero elsewhere
 *         (or, with teacher_form = CKL_TEACHER_LOGPROBS, the cached
 *         log-probabilities exponentiated as given),
 *   q_t = softmax(z_t) with z_t = W h_t (full vocabulary),
 * in the sparse form given in the objective section of the README page
 * "Chunked KL loss, running Knowledge Distillation locally in less <6GB VRAM":
 *   l_t = sum_k p_tk log p_tk - sum_k p_tk z_t[idx_tk] + M_t logsumexp(z_t),
 * with M_t = sum_k p_tk (the teacher mass; 1 for renormalised logits), and
 *   loss = (1/N) sum_{t : mask_t = 1} l_t,   N = number of unmasked rows.
 * N = 0 gives loss = 0 and zero gradients.
 *
 * The backward pass (the "Full Chunked KL" paragraph of the same page: the
 * logits are recomputed chunk by chunk and the closed-form gradient is
 * applied) uses the logit gradient
 *   G[t, v] = s_t (M_t q_t[v] - p~_t[v]),   s_t = grad_loss * mask_t / N,
 * where p~_t is p_t scattered to its indices, and returns dH = G W and
 * dW = G^T H.  The T x V logit tensor is never stored: logit tiles live in
 * registers, and the backward keeps only a bounded block of G (its size is set
 * by `chunk`, see below).
 *
 * Layouts (all row-major, densely packed, no strides):
 *   H       [T, d]  in_dtype         W        [V, d]  in_dtype
 *   idx     [T, K]  int32            tlogit   [T, K]  float32
 *   mask    [T]     uint8 (nonzero = keep) or NULL (all rows kept)
 *   lse     [T]     float32          row_loss [T]     float32
 *   dH      [T, d]  dh_dtype         dW       [V, d]  dw_dtype
 *   loss, grad_loss: one float32 each.
 * Every array pointer is a DEVICE pointer (memory of the GPU current when the
 * call is made); `stream` is a hipStream_t (NULL = the legacy default stream).
 * Device arrays must be 16-byte aligned.
 *
 * Ownership.  The caller allocates every buffer, the workspace included.  The
 * library allocates no device memory at run time (its one device allocation is
 * a 64 MiB static array that comes with its code on every GPU it runs on, the
 * workspace of ckl_forward_noalloc), keeps no state between calls (apart from
 * the optional timing records, see ckl_timing_enable) and holds no pointer
 * after a call returns (apart from work queued on `stream`).
 *
 * Execution.  Calls enqueue kernels on `stream` and return without waiting
 * (no host synchronisation), except when `validate` is set (see below).
 * Results are bitwise reproducible for identical inputs, problem and
 * workspace: there are no floating-point atomics.
 *
 * Errors.  Arguments are checked on the host before anything is enqueued;
 * on error nothing is launched and outputs are untouched.  Every buffer a
 * call writes (its outputs and the used part of its workspace) must be
 * disjoint from every other buffer of the call, or the call returns
 * CKL_ERR_INVALID_ARG (the check compares address ranges; it cannot see
 * two mappings of one allocation).  HIP launch errors
 * return CKL_ERR_HIP.  ckl_last_error() returns a thread-local message that
 * describes the last non-OK status returned on the calling thread.
 */
#ifndef CKL_H_
#define CKL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CKL_OK = 0,
  CKL_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad alignment          */
  CKL_ERR_UNSUPPORTED = 2, /* valid request outside what the library handles */
  CKL_ERR_WORKSPACE = 3,   /* ws NULL or ws_bytes below ckl_workspace_size()  */
  CKL_ERR_BAD_INDEX = 4,   /* validate = 1 found idx out of [0, V) or repeated */
  CKL_ERR_HIP = 5          /* a HIP runtime call failed                      */
} ckl_status;

typedef enum { CKL_F32 = 0, CKL_BF16 = 1 } ckl_dtype;

/* What the K cached teacher values of a row are (the objective section of the
 * README page carries the teacher mass M explicitly):
 *   CKL_TEACHER_LOGITS:   logits; p = softmax over the K entries (M = 1).
 *   CKL_TEACHER_LOGPROBS: the teacher's own log-probabilities over its full
 *                         vocabulary, truncated to the top K and used as
 *                         given: p = exp(value), M = sum_k p_k (may be < 1;
 *                         -inf entries are zero-probability tokens). */
typedef enum { CKL_TEACHER_LOGITS = 0, CKL_TEACHER_LOGPROBS = 1 } ckl_teacher_form;

typedef struct {
  int64_t T;      /* rows (batch x sequence, flattened), 1 .. 4,000,000    */
  int64_t d;      /* hidden size, >= 8 and a multiple of 8                 */
  int64_t V;      /* vocabulary size, 1 .. 4,000,000                       */
  int64_t K;      /* teacher entries per row, 1 <= K <= min(V, 4096)       */
  int64_t chunk;  /* rows per chunk, >= 1: the forwards project chunk     */
                  /* rows at a time (rounded up to whole tiles); the       */
                  /* backward keeps at most about chunk*V logit gradients  */
                  /* at a time.                                            */
  int32_t in_dtype;  /* ckl_dtype of H and W                               */
  int32_t dh_dtype;  /* ckl_dtype of dH                                    */
  int32_t dw_dtype;  /* ckl_dtype of dW                                    */
  int32_t validate;  /* 1: check idx on the device (range, no repeats) and */
                     /* synchronise `stream` to report CKL_ERR_BAD_INDEX.  */
                     /* 0: no check; idx is a precondition.  Out-of-range  */
                     /* entries never cause an out-of-bounds access (they  */
                     /* match no vocabulary column) but the result is then */
                     /* undefined, as it is for repeated entries.          */
  int32_t teacher_form; /* ckl_teacher_form of tlogit (0 = logits)         */
  int64_t v_offset;  /* vocabulary shards: W holds vocabulary rows           */
  int64_t v_total;   /* [v_offset, v_offset + V) of a vocabulary of v_total */
                     /* (0 = V: W is the whole head).  idx holds ids in     */
                     /* [0, v_total); K <= v_total.  Only ckl_shard_forward,*/
                     /* ckl_shard_combine and ckl_backward accept a shard.  */
  int64_t dw_group_rows; /* ckl_forward_backward only: rows of logit       */
                     /* gradients kept for one fp32 update of dW, rounded  */
                     /* down to whole chunks (at least one chunk).  0 =    */
                     /* the default, min(16384, 8 * chunk rows).  Larger   */
                     /* groups update dW less often (faster) and hold more */
                     /* workspace (group rows x V x in_dtype).             */
  int32_t compact_mask; /* 1: when a mask is given, the kept rows are      */
                     /* gathered first (a packed copy of their H rows in   */
                     /* the workspace) and every logit tile, recompute and */
                     /* contraction runs over the kept rows only, so       */
                     /* masked rows cost no matrix work; outputs are       */
                     /* scattered back (masked rows: 0).  Teacher indices  */
                     /* of masked rows are then not validated.  0: masked  */
                     /* rows are computed and zeroed.  The workspace query */
                     /* includes the packed copies when this is 1.         */
  int32_t reserved_;  /* must be 0                                          */
} ckl_problem;

/* Workspace bytes needed by ckl_forward or ckl_shard_forward (which = 0),
 * ckl_backward (which = 1), ckl_forward_backward (which = 2) or
 * ckl_shard_combine (which = 3) for problem *p.  Writes *bytes; returns
 * CKL_OK or CKL_ERR_INVALID_ARG / CKL_ERR_UNSUPPORTED for a bad problem. */
ckl_status ckl_workspace_size(const ckl_problem* p, int which, size_t* bytes);

/* Forward pass: loss, per-row log-sum-exp and per-row KL.
 *   H, W, idx, tlogit, mask: inputs as above (mask may be NULL).
 *   loss:     [1] device float32, the masked mean of l_t.
 *   lse:      [T] device float32, logsumexp_v z_t[v] for kept rows, 0 for
 *             masked rows.  ckl_backward takes this array back.
 *   row_loss: [T] device float32 or NULL; l_t for kept rows, 0 for masked.
 *   ws:       device workspace of at least ckl_workspace_size(p, 0) bytes;
 *             its contents on entry do not matter.
 * Rows are projected one chunk at a time; the logits never leave the MFMA
 * accumulators.  The loss and its logit-gradient formula follow the
 * objective section and the Full Chunked KL paragraph of the README page
 * named above. */
ckl_status ckl_forward(const ckl_problem* p, const void* H, const void* W,
                       const int32_t* idx, const float* tlogit, const uint8_t* mask,
                       float* loss, float* lse, float* row_loss,
                       void* ws, size_t ws_bytes, void* stream);

/* ckl_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The workspace is a file-scope device array of the
 * library, 64 MiB per device, held by every device the library runs on until
 * the process ends; the call allocates nothing (no hipMalloc, no events).
 * Arguments and results as in ckl_forward.  Limits and errors:
 *   - the problem's forward workspace, ckl_workspace_size(p, 0), must fit in
 *     64 MiB (about 50,000 rows at K = 100 without packed rows), else
 *     CKL_ERR_UNSUPPORTED and nothing is launched;
 *   - validate = 1 is refused (CKL_ERR_UNSUPPORTED): the index check reads a
 *     flag back and synchronises;
 *   - `stream` must belong to the current device (CKL_ERR_INVALID_ARG).
 * Every call on one device shares that device's array, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that overlap
 * on one device race and give undefined results; calls on one stream, or
 * ordered between streams, do not overlap. */
ckl_status ckl_forward_noalloc(const ckl_problem* p, const void* H, const void* W,
                               const int32_t* idx, const float* tlogit, const uint8_t* mask,
                               float* loss, float* lse, float* row_loss, void* stream);

/* Backward pass: dH and dW of grad_loss * loss.
 *   lse:       [T] from ckl_forward on the same inputs (or from
 *              ckl_shard_combine; on a vocabulary shard dW is the shard's
 *              rows and dH its contribution to the sum over shards).
 *   grad_loss: [1] device float32 or NULL (= 1).
 *   dH, dW:    outputs, overwritten (not accumulated into).
 *   ws:        device workspace of at least ckl_workspace_size(p, 1) bytes.
 * The logit tiles are recomputed and never stored beyond a G block of about
 * chunk*V entries. */
ckl_status ckl_backward(const ckl_problem* p, const void* H, const void* W,
                        const int32_t* idx, const float* tlogit, const uint8_t* mask,
                        const float* lse, const float* grad_loss,
                        void* dH, void* dW, void* ws, size_t ws_bytes, void* stream);

/* The G-block plan ckl_backward uses for problem *p: out[0] = Tc (token rows
 * per block), out[1] = Vc (vocabulary columns per block), out[2] = number of
 * token blocks, out[3] = number of vocabulary blocks, out[4] = number of G
 * blocks held at once (each stored as G [Tc, Vc], and for fp32 also its
 * transpose; the two layouts' budget together is about chunk * V
 * elements).  dW is read-modified-
 * written once per extra token block and dH once per extra vocabulary block;
 * the vocabulary blocks are the outer loop, and W^T is staged for one block
 * at a time ([d, Vc] in the workspace).  Host-only; touches no device. */
ckl_status ckl_backward_plan(const ckl_problem* p, int64_t out[5]);

/* Forward and backward in one call, without recomputing the logits.
 *
 * The README page above lists a Forward-Chunked Loss that keeps the student
 * logits for the backward pass (the fastest variant in the article "A KL loss
 * tweak lets a single GPU distill a 120B model without melting") and the Full
 * Chunked KL that bounds memory by recomputing them.  This call keeps the
 * logits of one row chunk at a time: memory stays bounded by `chunk` and
 * nothing is recomputed.  For each chunk of rows the logit tiles are
 * multiplied once; besides the online log-sum-exp of ckl_forward the kernel
 * stores u = exp(z - m) in in_dtype, where m is a running maximum kept per
 * group of vocabulary rows (so u <= 1 and nothing overflows).  When the
 * chunk's LSE is known, u becomes G = s_t M_t u exp(m - LSE_t) in place, the
 * K teacher columns are recomputed in fp32 from the logits kept at the
 * teacher indices, and dW += G^T H_chunk, dH_chunk = G W follow (dH as a
 * split-k product summed in a fixed order).
 *
 * Arguments as in ckl_forward and ckl_backward; grad_loss ([1] device
 * float32 or NULL = 1) must hold its value when the call's kernels run.
 * loss, lse and row_loss agree with ckl_forward up to the order of the split
 * merges (float rounding); dH and dW agree with ckl_backward up to one more
 * rounding of the non-teacher entries of G to in_dtype (u is rounded before
 * it is rescaled).
 *   ws: device workspace of at least ckl_workspace_size(p, 2) bytes: with
 *   n = the number of chunks in one dW group (p->dw_group_rows, see
 *   ckl_problem), n + 1 chunk x V buffers of in_dtype (bf16: the forward's
 *   exponentials u of one chunk and G of n consecutive chunks; fp32: G of
 *   one chunk and G^T of n chunks; the fp32 update of dW runs once per n
 *   chunks), H^T and W^T, the dH split-k partials and small per-row arrays.
 * Rows per chunk: `chunk` rounded up to whole tiles (256 rows for bf16,
 * 128 for fp32), at most T rounded up. */
ckl_status ckl_forward_backward(const ckl_problem* p, const void* H, const void* W,
                                const int32_t* idx, const float* tlogit, const uint8_t* mask,
                                const float* grad_loss, float* loss, float* lse, float* row_loss,
                                void* dH, void* dW, void* ws, size_t ws_bytes, void* stream);

/* The chunk plan ckl_forward_backward uses for problem *p: out[0] = rows per
 * chunk, out[1] = number of chunks, out[2] = number of dH split-k parts,
 * out[3] = vocabulary columns per part, out[4] = chunks per dW group.
 * Host-only; touches no device. */
ckl_status ckl_fused_plan(const ckl_problem* p, int64_t out[5]);

/* Output finish for callers that keep fp32 gradients of the loss itself and
 * learn the incoming gradient later (an autograd backward of the one-call
 * path): dst[i] = scale * src[i] for i < n, rounded once to dst_dtype.
 *   src:   [n] device float32;   dst: [n] device dst_dtype (may alias src
 *          when dst_dtype is CKL_F32);
 *   scale: [1] device float32 or NULL (= 1).
 * src, dst 16-byte aligned, n a multiple of 4. */
ckl_status ckl_scale_cast(const float* src, void* dst, int64_t n, int32_t dst_dtype, const float* scale,
                          void* stream);

/* Vocabulary-parallel shards (the README usage table's tensor-parallel
 * option shards the output head; the pages do not describe the exchange).
 * With W split by rows over P devices, only the log-normaliser and the cross
 * term need the whole vocabulary, and both merge from per-shard partials:
 *   1. every shard: ckl_shard_forward(p with v_offset / v_total, its W rows)
 *      -> lse_part[t]  = log sum over the shard's rows of exp(z_t[v]),
 *         cross_part[t] = sum over the teacher entries of row t that fall in
 *                         the shard of p_tk z_t[idx_tk];
 *   2. gather the P partials of every row (an all-gather of T x 8 bytes per
 *      device) and ckl_shard_combine them into loss, lse and row_loss;
 *   3. every shard: ckl_backward(p with the same v_offset / v_total, its W
 *      rows, the combined lse) -> dW rows of the shard and that shard's
 *      contribution to dH; the sum of dH over the shards (an all-reduce) is
 *      the gradient.
 * On one device the shards can be run in turn.  Partials are fp32 (the
 * cross term summed in fp64 per shard; the merge in fp64).
 *
 * ckl_shard_forward: lse_part, cross_part are [T] device float32, written for
 * every row (masks apply in the combine).  ws: ckl_workspace_size(p, 0).
 * ckl_shard_combine: lse_parts and cross_parts are [n_shards, T] device
 * float32 (shard-major); idx and tlogit as given to the shards (the teacher
 * entropy and mass are recomputed); loss, lse, row_loss as in ckl_forward.
 * ws: ckl_workspace_size(p, 3); p->V, v_offset and v_total are not used
 * beyond argument checks. */
ckl_status ckl_shard_forward(const ckl_problem* p, const void* H, const void* W,
                             const int32_t* idx, const float* tlogit,
                             float* lse_part, float* cross_part,
                             void* ws, size_t ws_bytes, void* stream);
ckl_status ckl_shard_combine(const ckl_problem* p, int32_t n_shards,
                             const float* lse_parts, const float* cross_parts,
                             const int32_t* idx, const float* tlogit, const uint8_t* mask,
                             float* loss, float* lse, float* row_loss,
                             void* ws, size_t ws_bytes, void* stream);

/* Kernel classes for the timing records below. */
typedef enum {
  CKL_KERNEL_TEACHER_PREP = 0, /* teacher softmax + sort                      */
  CKL_KERNEL_FWD_LSE = 1,      /* forward logit tiles + online LSE + gather    */
  CKL_KERNEL_FWD_FINALIZE = 2, /* split merge, row loss, masked mean          */
  CKL_KERNEL_BWD_GRAD = 3,     /* backward logit recompute + G epilogue       */
  CKL_KERNEL_GEMM_DHDW = 4,    /* dW (+)= G^T H and dH (+)= G W, one launch   */
  CKL_KERNEL_G_PASS = 5,       /* fused call: u -> G (fp32 also G^T)        */
  CKL_KERNEL_TRANSPOSE = 6,    /* H^T and W^T staging                         */
  CKL_KERNEL_OTHER = 7,        /* counts, scales, fills, casts               */
  CKL_KERNEL_CLASSES = 8
} ckl_kernel_class;

/* Optional per-kernel timing, a measurement aid.  While enabled (on = 1),
 * every kernel the library launches is bracketed by two hipEvents recorded on
 * the launch stream; enabling (again) clears the accumulated records, on = 0
 * stops recording.  Process-wide; the records are the only state the library
 * keeps between calls, and the events are its only run-time allocations. */
ckl_status ckl_timing_enable(int on);

/* Waits for the recorded events, adds their durations to the totals of each
 * class and returns, for class `kernel_class`, the summed duration in
 * milliseconds and the number of launches since timing was enabled. */
ckl_status ckl_timing_read(int kernel_class, double* total_ms, int64_t* launches);

/* Static description of a status code. */
const char* ckl_status_string(ckl_status s);

/* Thread-local detail of the last non-OK status on this thread ("" if none). */
const char* ckl_last_error(void);

/* ABI version: (major << 16) | minor. */
int32_t ckl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CKL_H_ */
