/*
 * lce.h — C ABI of the chunked linear-cross-entropy library (gfx950 / MI355X).
 *
 * The operation (LlamaFactory PR #10762 analysis, section 4, the chunk-loss
 * autograd function; TRL "training on 1M+ tokens", section "chunking"):
 * the final hidden states h [N,H] go through the LM head W [V,H] (+ bias b [V],
 * an nn.Linear) and a per-token cross-entropy against labels y [N] with an
 * ignore label (-100 by default). Rows are independent, so the [N,V] logits
 * never need to exist at once:
 *
 *   z_ij   = h_i . W_j + b_j
 *   lse_i  = log sum_j exp(z_ij)
 *   l_i    = valid_i * (lse_i - z_{i,y_i}),      valid_i = (y_i != ignore_index)
 *   loss   = sum_i l_i  (SUM) | sum_i l_i / max(n_valid,1)  (MEAN) | l  (NONE)
 *   G_ij   = s * valid_i * (softmax_ij - [j == y_i]),  s = grad_scale (SUM)
 *                                                       or grad_scale / max(n_valid,1) (MEAN)
 *   grad_hidden = G W,   grad_weight = G^T h,   grad_bias = sum_i G_i
 *
 * grad_weight and grad_bias are accumulated in FP32 and cast to the input
 * dtype (bf16, round to nearest even) at the end (same section 4: the FP32
 * accumulators, cast once).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    allocates nothing, keeps no state between calls and is reentrant per
 *    stream. Work is enqueued on `stream` and is asynchronous: outputs are
 *    valid once the stream reaches the end of the call.
 *  - Outputs are overwritten, never accumulated into.
 *  - Argument errors are detected on the host and returned synchronously,
 *    before anything is enqueued. A label outside [0,V) that is not the
 *    ignore label is only seen on the device: that row is treated as ignored,
 *    *status is set to LCE_ERR_LABEL_RANGE and the loss is written as NaN.
 *  - Layouts are row-major. hidden: [N rows, ld_hidden elements per row],
 *    first H used; weight: [V, ld_weight], first H used (nn.Linear layout, row
 *    j is vocabulary id j); labels: int64 [N], already aligned with the rows
 *    (any causal shift happens upstream).
 *  - Reproducibility: n_valid, lse, per-row losses (NONE), grad_hidden and
 *    grad_weight (bf16 and FP32) are bit-identical from call to call on the
 *    same device and inputs (fixed summation orders). The SUM / MEAN loss and
 *    the chunk sums add rows with float64 atomics, and grad_bias adds column
 *    sums with FP32 atomics: their last bits may differ between calls. The
 *    lse of lce_forward_backward can differ from lce_forward's in the last
 *    bits: the fused call sums a labelled row's exponentials against its
 *    label logit, the forward alone against the row's maximum.
 *  - The label logit in l_i comes from the same FP32 accumulators as the
 *    row's sums, and l_i >= 0 for every row.
 */
#ifndef LCE_H
#define LCE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LCE_OK = 0,
  LCE_ERR_INVALID_ARG = 1,   /* bad sizes, strides, null required pointer, chunk_rows <= 0 */
  LCE_ERR_UNSUPPORTED = 2,   /* dtype, H % 64 != 0, misaligned pointer/stride, stride or V
                                above 2^22, NONE backward without per-row scales */
  LCE_ERR_WORKSPACE = 3,     /* workspace null or smaller than lce_workspace_bytes() */
  LCE_ERR_HIP = 4,           /* a kernel launch failed */
  LCE_ERR_LABEL_RANGE = 5,   /* device-side: a label outside [0,V) and != ignore_index */
  LCE_ERR_TOO_LARGE = 6      /* lce_forward_noalloc: the problem needs more than its fixed scratch */
} lce_status;

typedef enum {
  LCE_REDUCTION_NONE = 0,    /* loss[i] = l_i, one value per row */
  LCE_REDUCTION_SUM = 1,     /* loss[0] = sum_i l_i */
  LCE_REDUCTION_MEAN = 2     /* loss[0] = sum_i l_i / max(n_valid, 1); 0 when no row is valid */
} lce_reduction;

typedef enum { LCE_DTYPE_BF16 = 0, LCE_DTYPE_F32 = 1 } lce_dtype;   /* problems take BF16 only */

/* What lce_workspace_bytes() sizes for. */
typedef enum {
  LCE_WS_FORWARD = 0,            /* lce_forward */
  LCE_WS_BACKWARD = 1,           /* lce_forward_backward, FP32 accumulators inside the workspace */
  LCE_WS_BACKWARD_EXTERNAL_F32 = 2  /* lce_forward_backward with caller-given grad_weight_f32
                                       (and grad_bias_f32 when there is a bias) */
} lce_workspace_kind;

typedef struct {
  int64_t n_rows;        /* N >= 0: flattened token rows */
  int64_t hidden;        /* H > 0, H % 64 == 0 */
  int64_t vocab;         /* V > 0, V <= 2^22 */
  int64_t ld_hidden;     /* row stride of hidden in elements, >= H, % 8 == 0, <= 2^22 */
  int64_t ld_weight;     /* row stride of weight in elements, >= H, % 8 == 0, <= 2^22 */
  int64_t ignore_index;  /* label value that marks a row as ignored (pages: -100) */
  int64_t chunk_rows;    /* > 0: rows per loss chunk (chunk k = rows [k*c, min((k+1)c, N)));
                            LlamaFactory section 2 rejects <= 0, TRL's chunking uses 256 */
  int64_t rows_in_flight;/* backward row group: rows whose dlogits are alive at once;
                            0 = library default (16384); at most 2^20 (larger values
                            are clamped); rounded up to a multiple of 256 */
  int32_t reduction;     /* lce_reduction */
  int32_t dtype;         /* lce_dtype; only LCE_DTYPE_BF16 */
} lce_problem;

/* Bytes of device workspace the call needs (16-byte aligned start required).
 * Returns 0 when *p is invalid (the call itself then reports why). */
size_t lce_workspace_bytes(const lce_problem* p, int kind);

/* Forward: loss, per-row lse and the valid-token count.
 *   loss       [1] float (SUM/MEAN) or [N] float (NONE); required
 *   lse        [N] float, natural-log lse_i of every row (ignored rows too); nullable
 *   chunk_loss [ceil(N/chunk_rows)] float, sum of l_i over each chunk (before MEAN scaling); nullable
 *   n_valid    [1] int64, #{i : y_i != ignore_index and in range}; nullable
 *   status     [1] int32, LCE_OK or LCE_ERR_LABEL_RANGE; nullable
 * bias may be NULL (no bias). Returns an lce_status. */
int lce_forward(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                const int64_t* labels, float* loss, float* lse, float* chunk_loss, int64_t* n_valid,
                int32_t* status, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Forward and backward in one call (the pages' autograd function computes the
 * chunk gradients inside its forward pass).
 *   grad_scale      dLoss_total/dloss from the caller (1.0 for a plain loss)
 *   grad_hidden     [N, H] bf16 (row stride H); nullable: skips the G W product
 *   grad_weight     [V, H] bf16 (row stride H); nullable
 *   grad_bias       [V] bf16; nullable; requires bias
 *   grad_weight_f32 [V, H] float (row stride H); nullable: the FP32 accumulator itself
 *   grad_bias_f32   [V] float; nullable; requires bias
 * When both grad_weight and grad_weight_f32 are NULL the G^T h product is
 * skipped (the pages' needs_weight_grad == False). reduction NONE is
 * LCE_ERR_UNSUPPORTED here (lce_forward_backward_ex accepts it with per-row
 * upstream gradients). Other arguments as lce_forward. */
int lce_forward_backward(const lce_problem* p, const void* hidden, const void* weight,
                         const void* bias, const int64_t* labels, float grad_scale,
                         float* loss, float* lse, float* chunk_loss, int64_t* n_valid,
                         void* grad_hidden, void* grad_weight, void* grad_bias,
                         float* grad_weight_f32, float* grad_bias_f32, int32_t* status,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Per-launch timing for benchmarks. The caller creates the events (e.g. with
 * hipEventCreate) and owns them. When a traced entry point is given a trace,
 * it records events[2*i] just before and events[2*i+1] just after its i-th
 * kernel launch on `stream`, sets kinds[i] to the launched kernel's
 * lce_kernel_kind, and stops recording (silently) once `capacity` pairs are
 * used; `count` returns the number of pairs recorded. Results are otherwise
 * identical to the untraced call.
 * LCE_K_FWD_LSE is the logits-tile kernel with the log-sum-exp epilogue (in
 * lce_forward_backward it also stores each row group's softmax numerators
 * exp(z - r_i), r_i the row's label logit); LCE_K_BWD_DLOGITS forms the
 * group's dlogits from them (per-row scales and one patched entry per row;
 * no pass over the stored tiles); LCE_K_LABEL_LOGIT gathers each valid
 * row's label logit h_i . W_{y_i} + b_{y_i}; LCE_K_ROW_REF prepares a
 * group's row references; LCE_K_FWD_RETRY recomputes a group's stored
 * numerators against r_i = lse_i when a row's maximum lies more than 60
 * above its label logit (otherwise it returns at once); LCE_K_BIAS_SUMS
 * adds the group's grad_bias column sums (only when grad_weight is not
 * computed: otherwise grad_weight's kernel adds them);
 * LCE_K_PARTITION orders the rows with a label before the others (two
 * launches, recorded as one) and LCE_K_GATHER_ROWS copies the hidden rows
 * into that order: the backward then works on the rows with a label only.
 * LCE_K_GRAD_HIDDEN and LCE_K_GRAD_WEIGHT each cover the product kernel and,
 * when some of its tiles were split along K to fill the GPU's last round,
 * the kernel that adds the pieces (one record for both). */
typedef enum {
  LCE_K_ZERO = 0, LCE_K_PREPARE_LABELS = 1, LCE_K_FWD_LSE = 2, LCE_K_FINALIZE_ROWS = 3,
  LCE_K_FINALIZE_LOSS = 4, LCE_K_TRANSPOSE = 5, LCE_K_BWD_DLOGITS = 6, LCE_K_GRAD_HIDDEN = 7,
  LCE_K_GRAD_WEIGHT = 8, LCE_K_CAST = 9, LCE_K_LABEL_LOGIT = 10, LCE_K_ROW_REF = 11, LCE_K_FWD_RETRY = 12,
  LCE_K_BIAS_SUMS = 13, LCE_K_PARTITION = 14, LCE_K_GATHER_ROWS = 15, LCE_K_COUNT = 16
} lce_kernel_kind;

typedef struct {
  hipEvent_t* events;  /* [2 * capacity], caller-created */
  int32_t* kinds;      /* [capacity], written */
  int32_t capacity;
  int32_t count;       /* written */
  /* For each recorded launch: rows, columns and depth of the product it
   * computes, so throughput can be derived; element-wise passes over a
   * [rows, columns] block record depth 0; other kernels record zeros. */
  int64_t* dims;       /* [3 * capacity], written; nullable */
} lce_trace;

/* lce_forward / lce_forward_backward with an optional trace (NULL = untraced). */
int lce_forward_traced(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                       const int64_t* labels, float* loss, float* lse, float* chunk_loss, int64_t* n_valid,
                       int32_t* status, void* workspace, size_t workspace_bytes, hipStream_t stream,
                       lce_trace* trace);
int lce_forward_backward_traced(const lce_problem* p, const void* hidden, const void* weight,
                                const void* bias, const int64_t* labels, float grad_scale,
                                float* loss, float* lse, float* chunk_loss, int64_t* n_valid,
                                void* grad_hidden, void* grad_weight, void* grad_bias,
                                float* grad_weight_f32, float* grad_bias_f32, int32_t* status,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                lce_trace* trace);

/* Options of lce_forward_backward_ex (zero-initialised = lce_forward_backward).
 *
 * row_scale: [N] float, device, nullable. Row i's dlogits are additionally
 *   multiplied by row_scale[i]: G_i = s * row_scale[i] * valid_i *
 *   (softmax_i - onehot_i). With reduction LCE_REDUCTION_NONE this is the
 *   per-token upstream gradient dL/dl_i (the pages' autograd function
 *   multiplies its saved gradients by grad_output in backward; LlamaFactory
 *   PR #10762 analysis, section 4); NONE is accepted only with row_scale.
 * accumulate: nonzero = grad_weight_f32 and grad_bias_f32 are added to
 *   instead of overwritten (gradient accumulation across micro-batches; the
 *   trainer contract of LlamaFactory section 3). The FP32 buffers must then
 *   be given for every weight / bias gradient requested (else
 *   LCE_ERR_INVALID_ARG); grad_weight / grad_bias, if also given, receive the
 *   bf16 cast of the accumulated totals. A step-global mean over an
 *   externally all-reduced valid count n is reduction SUM with
 *   grad_scale = 1 / n. */
typedef struct {
  const float* row_scale;
  int32_t accumulate;
  int32_t reserved;      /* must be 0 */
} lce_backward_options;

/* lce_forward_backward with options (NULL = none) and an optional trace. */
int lce_forward_backward_ex(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                            const int64_t* labels, float grad_scale, float* loss, float* lse,
                            float* chunk_loss, int64_t* n_valid, void* grad_hidden, void* grad_weight,
                            void* grad_bias, float* grad_weight_f32, float* grad_bias_f32, int32_t* status,
                            void* workspace, size_t workspace_bytes, hipStream_t stream,
                            const lce_backward_options* options, lce_trace* trace);

/* data[k] *= *scale for k < n, in place, on `stream`. data: device, dtype
 * LCE_DTYPE_BF16 (round to nearest even) or LCE_DTYPE_F32; scale: one float
 * in device memory (e.g. an autograd grad_output), read by the kernel, so no
 * host synchronisation. Applies an upstream gradient to gradients computed
 * ahead of time (the pages' autograd function scales its saved gradients by
 * grad_output in backward; LlamaFactory PR #10762 analysis, section 4).
 * Returns LCE_ERR_INVALID_ARG for n < 0, a NULL pointer with n > 0 or an
 * unknown dtype. */
int lce_scale(void* data, int32_t dtype, int64_t n, const float* scale, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): lce_forward
 * without a workspace argument. Its workspace is a fixed device array of
 * LCE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the
 * first load of the library's code on that GPU until the process ends; the
 * call itself allocates nothing (no hipMalloc, no allocating library call).
 * Results are those of lce_forward (arguments and outputs the same), with
 * the forward's per-tile (max, sum-exp) partials held for as many rows at a
 * time as fit in the array. About 12 bytes per row (padded to 256 rows) plus
 * 8 per loss chunk must fit beside the partials of 256 rows
 * (32 * ceil(V / 256) * 256 bytes); a larger problem returns
 * LCE_ERR_TOO_LARGE before anything is enqueued.
 * Every call on a GPU uses that GPU's one array and leaves its contents
 * behind; each call clears what it needs zeroed itself. Calls that overlap
 * on one GPU (several streams or threads at once) race on the array: the
 * caller must order them. */
#define LCE_NOALLOC_SCRATCH_BYTES (64ull << 20)
int lce_forward_noalloc(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                        const int64_t* labels, float* loss, float* lse, float* chunk_loss, int64_t* n_valid,
                        int32_t* status, hipStream_t stream);

/* Static string for an lce_status value (never NULL). */
const char* lce_status_string(int status);

/* ABI version: 100 * major + minor. */
int lce_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LCE_H */
