/*
 * libmoe_epi — routed-expert epilogue kernels for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Callers need no HIP headers: bfloat16 tensors are passed as uint16_t
 * bit patterns, streams as void* (a hipStream_t; NULL selects the default
 * stream).
 *
 * Common contract of every compute entry point below:
 *   Memory    All tensor pointers are device-accessible memory allocated and
 *             owned by the caller; the library allocates nothing, keeps no
 *             state between calls and never synchronises. Layouts are dense
 *             row-major with no padding: one probability per row
 *             ([rows] == [rows, 1]). The call only validates its arguments and
 *             queues the kernel on `stream`; results are ready when the stream
 *             reaches that point. Calls are thread-safe. With no allocation,
 *             memset or synchronisation inside, a call can be captured into a
 *             HIP graph on `stream` and replayed; the graph then reads and
 *             writes the buffers passed at capture.
 *   Dtypes    x, y, gradients of x/y: bfloat16. probs, grad_probs: float32.
 *             All arithmetic is float32; each bfloat16 result is rounded once,
 *             to nearest with ties to even.
 *   Errors    Arguments are checked on the host before any HIP call. On a bad
 *             argument the call returns a nonzero moe_epi_status, launches
 *             nothing and leaves every output untouched. rows == 0 is valid
 *             and launches nothing. A failure reported by the HIP runtime at
 *             launch returns MOE_EPI_ERR_LAUNCH.
 *   Alignment bfloat16 pointers must be 2-byte aligned and float32 pointers
 *             4-byte aligned. When every bfloat16 pointer is 16-byte aligned
 *             and the row width (inter or hidden) is a multiple of 8, the
 *             kernels move 16 bytes per lane per access; otherwise a
 *             per-element path runs (same results, lower bandwidth).
 *   Aliasing  No output may overlap any input or another output.
 */
#ifndef MOE_EPI_H
#define MOE_EPI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_epi_status {
    MOE_EPI_SUCCESS = 0,
    MOE_EPI_ERR_NULL_POINTER = 1, /* a required pointer is NULL                              */
    MOE_EPI_ERR_BAD_SHAPE = 2,    /* rows < 0, inter/hidden <= 0, or a byte size overflows   */
    MOE_EPI_ERR_BAD_LIMIT = 3,    /* limit is not finite or not > 0                          */
    MOE_EPI_ERR_ALIAS = 4,        /* an output overlaps an input or another output           */
    MOE_EPI_ERR_LAUNCH = 5,       /* the HIP runtime reported an error at kernel launch      */
    MOE_EPI_ERR_MISALIGNED = 6,   /* a pointer is not aligned to its element size            */
    MOE_EPI_ERR_BAD_DTYPE = 7     /* a dtype code is not one of moe_epi_dtype                */
} moe_epi_status;

/* Storage types of the *_typed entry points. Arithmetic is float32 for all. */
typedef enum moe_epi_dtype {
    MOE_EPI_BF16 = 0,
    MOE_EPI_F16 = 1,
    MOE_EPI_F32 = 2
} moe_epi_dtype;

/*
 * Clamped SwiGLU times routing probability, forward.
 * Defined on the page "nemo_automodel.components.moe.swiglu_triton", module
 * description (the DeepSeek-V4-style activation used when swiglu_limit > 0):
 *   for r < rows, j < inter, with gate = x[r, j], up = x[r, inter + j], p = probs[r]:
 *     y[r, j] = bf16( silu(min(gate, limit)) * clamp(up, -limit, limit) * p )
 *   silu(z) = z / (1 + exp(-z)); math in float32, one rounding to bfloat16.
 *   The gate is clamped from above only; a NaN input propagates to y.
 *   x     [rows, 2*inter] bf16 (gate half, then up half, in each row)   in
 *   probs [rows] float32                                                in
 *   y     [rows, inter] bf16                                            out
 *   limit finite, > 0.
 * Returns a moe_epi_status.
 */
int swiglu_clamped_fwd(const uint16_t *x, const float *probs, uint16_t *y,
                       int64_t rows, int64_t inter, float limit, void *stream);

/*
 * Clamped SwiGLU times routing probability, single-pass backward.
 * Defined on the page "nemo_automodel.components.moe.swiglu_triton", module
 * description: one pass writes d_gate and d_up into the two halves of grad_x
 * and reduces the per-row probability gradient; clamp gradients follow
 * torch.clamp, i.e. inclusive masks on the input values:
 *   gc = min(gate, limit), uc = clamp(up, -limit, limit), s = sigmoid(gc),
 *   t = grad_y[r, j] * p,
 *   grad_x[r, j]         = bf16( gate <= limit          ? (t * uc) * s * (1 + gc * (1 - s)) : +0 )
 *   grad_x[r, inter + j] = bf16( -limit <= up <= limit  ? t * gc * s                        : +0 )
 *   grad_probs[r]        = sum_j grad_y[r, j] * (gc * s * uc)     (float32, any summation order)
 *   x          [rows, 2*inter] bf16     in
 *   probs      [rows] float32           in
 *   grad_y     [rows, inter] bf16       in
 *   grad_x     [rows, 2*inter] bf16     out
 *   grad_probs [rows] float32           out; may be NULL (probabilities that carry no
 *                                       gradient), then it is neither formed nor written.
 * Returns a moe_epi_status.
 */
int swiglu_clamped_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                       uint16_t *grad_x, float *grad_probs,
                       int64_t rows, int64_t inter, float limit, void *stream);

/*
 * fp32 router-weight multiply, forward.
 * Defined on the page "nemo_automodel.components.moe.optimized_ops", entries
 * _RouterWeightMulFunction (the forward equals the eager fp32 multiply bit
 * for bit) and _rw_fwd_core:
 *   out[r, k] = bf16( float32(x[r, k]) * probs[r] )      (one multiply, one rounding)
 *   x     [rows, hidden] bf16 (expert down-projection output)   in
 *   probs [rows] float32                                      in
 *   out   [rows, hidden] bf16                                 out
 * Returns a moe_epi_status.
 */
int router_weight_mul_fwd(const uint16_t *x, const float *probs, uint16_t *out,
                          int64_t rows, int64_t hidden, void *stream);

/*
 * fp32 router-weight multiply, backward (both gradients in one pass over
 * grad_out). Defined on the page "nemo_automodel.components.moe.optimized_ops",
 * entries _RouterWeightMulFunction, _rw_bwd_x_core and _rw_bwd_probs_core:
 *   grad_x[r, k]  = bf16( float32(grad_out[r, k]) * probs[r] )
 *   grad_probs[r] = sum_k float32(grad_out[r, k]) * float32(x[r, k])   (float32, any order)
 *   grad_out   [rows, hidden] bf16      in
 *   x          [rows, hidden] bf16      in; may be NULL if and only if grad_probs is NULL
 *   probs      [rows] float32           in
 *   grad_x     [rows, hidden] bf16      out
 *   grad_probs [rows] float32           out; may be NULL (the page's save_x = False case:
 *                                       probabilities without gradient, x not kept)
 * Returns a moe_epi_status.
 */
int router_weight_mul_bwd(const uint16_t *grad_out, const uint16_t *x, const float *probs,
                          uint16_t *grad_x, float *grad_probs,
                          int64_t rows, int64_t hidden, void *stream);

/*
 * The same four operations for float16 and float32 storage.
 * Page "nemo_automodel.components.moe.swiglu_triton" lists bfloat16, float16
 * and float32 as the dtypes x may have (_SUPPORTED_DTYPES); page
 * "nemo_automodel.components.moe.optimized_ops" lets the router multiply's
 * output be the activation dtype or float32, the latter for combining expert
 * outputs by scatter-add (out_dtype of _RouterWeightMulFunction.forward).
 * Contract as above, with:
 *   swiglu_clamped_*_typed: x, y, grad_y, grad_x all of `dtype`; each result
 *     is rounded once from float32 to `dtype` (float32: stored as computed).
 *   router_weight_mul_fwd_typed: x of `x_dtype`, out of `out_dtype`.
 *   router_weight_mul_bwd_typed: grad_out of `grad_out_dtype` (the output's
 *     dtype), x and grad_x of `x_dtype`; grad_probs float32.
 * Pointers are typed void* (elements of the given dtypes); alignment is the
 * element size, and the 16-byte path needs 16-byte aligned tensors and a row
 * width that is a multiple of 8. A dtype outside moe_epi_dtype returns
 * MOE_EPI_ERR_BAD_DTYPE. With every dtype MOE_EPI_BF16 these are exactly the
 * calls above.
 */
int swiglu_clamped_fwd_typed(const void *x, const float *probs, void *y, int64_t rows, int64_t inter,
                             float limit, int dtype, void *stream);
int swiglu_clamped_bwd_typed(const void *x, const float *probs, const void *grad_y, void *grad_x,
                             float *grad_probs, int64_t rows, int64_t inter, float limit, int dtype,
                             void *stream);
int router_weight_mul_fwd_typed(const void *x, int x_dtype, const float *probs, void *out, int out_dtype,
                                int64_t rows, int64_t hidden, void *stream);
int router_weight_mul_bwd_typed(const void *grad_out, int grad_out_dtype, const void *x, int x_dtype,
                                const float *probs, void *grad_x, float *grad_probs, int64_t rows,
                                int64_t hidden, void *stream);

/*
 * gate_up grouped GEMM with the clamped SwiGLU x probability epilogue fused
 * into it (the step before the epilogue above, done in one kernel).
 * Defined by three pages:
 *   "nemo_automodel.components.moe.mok_experts": the routed gate and up
 *     weights are contiguous bf16 [local_experts, expert_intermediate, hidden];
 *   "nemo_automodel.components.moe.quantized_experts",
 *     MXFP4ExpertStorageMixin._mxfp4_base_mm: the routed activations are
 *     [tokens, in_dim] grouped contiguously by local expert, offs is an int32
 *     [local_experts] tensor of cumulative token counts, and the product is
 *     [tokens, out_dim] in the activation dtype;
 *   "nemo_automodel.components.moe.swiglu_triton": the epilogue on that output.
 * Rows of expert e are [start_e, end_e): start_0 = 0, end_e = offs[e]
 * clamped to [start_e, tokens], start_{e+1} = end_e. For such a row t:
 *   gate[t, j] = bf16( sum_h a[t, h] * w_gate[e, j, h] )   (float32 accumulation)
 *   up[t, j]   = bf16( sum_h a[t, h] * w_up[e, j, h] )
 *   y[t, j]    = bf16( silu(min(gate, L)) * clamp(up, -L, L) * probs[t] )
 * i.e. swiglu_clamped_fwd of x = [gate | up]. Rows at or past the last end
 * belong to no expert: neither y nor x_out is written there.
 *   a       [tokens, hidden] bf16                  in, rows grouped by expert
 *   w_gate  [experts, inter, hidden] bf16          in
 *   w_up    [experts, inter, hidden] bf16          in
 *   offs    [experts] int32, device memory         in (read on the device only)
 *   probs   [tokens] float32                       in
 *   y       [tokens, inter] bf16                   out
 *   x_out   [tokens, 2*inter] bf16                 out, may be NULL: [gate | up] as
 *                                                  swiglu_clamped_bwd takes it
 *   limit   L, finite and > 0
 * hidden and inter must be multiples of 8 (MOE_EPI_ERR_BAD_SHAPE otherwise;
 * there is no per-element path), tokens at most INT32_MAX (offs is int32);
 * a, w_gate, w_up, y and x_out 16-byte aligned, offs and probs 4-byte
 * aligned (MOE_EPI_ERR_MISALIGNED). Outputs may not overlap any input or each
 * other (MOE_EPI_ERR_ALIAS). The caller owns every buffer; the library
 * allocates nothing and queues the work on `stream`. Returns a moe_epi_status.
 */
int grouped_gate_up_swiglu_fwd(const uint16_t *a, const uint16_t *w_gate, const uint16_t *w_up,
                               const int32_t *offs, const float *probs, uint16_t *y, uint16_t *x_out,
                               int64_t tokens, int64_t hidden, int64_t inter, int64_t experts, float limit,
                               void *stream);

/*
 * Down projection grouped GEMM with the router-weight multiply fused into it
 * (the step after the SwiGLU epilogue, and the router multiply above, in one
 * kernel). Defined by:
 *   "nemo_automodel.components.moe.mok_experts": the routed down weights are
 *     contiguous bf16 [local_experts, hidden, expert_intermediate];
 *   "nemo_automodel.components.moe.quantized_experts",
 *     MXFP4ExpertStorageMixin._mxfp4_base_mm: grouped rows and offs as for
 *     grouped_gate_up_swiglu_fwd, the product in the activation dtype;
 *   "nemo_automodel.components.moe.optimized_ops", _apply_router_weight_fp32:
 *     that product times the permuted probability in float32, cast to the
 *     output dtype (float32 when the outputs are then combined by
 *     scatter-add).
 * Rows of expert e as for grouped_gate_up_swiglu_fwd. For such a row t:
 *   out2[t, n] = bf16( sum_i h[t, i] * w_down[e, n, i] )   (float32 accumulation)
 *   out[t, n]  = out_dtype( float32(out2[t, n]) * probs[t] )
 * i.e. router_weight_mul_fwd_typed of out2. Rows at or past the last end are
 * not written.
 *   h          [tokens, inter] bf16                 in, rows grouped by expert
 *   w_down     [experts, hidden, inter] bf16        in
 *   offs       [experts] int32, device memory       in (read on the device only)
 *   probs      [tokens] float32                     in
 *   out        [tokens, hidden] of out_dtype        out
 *   out_dtype  MOE_EPI_BF16 or MOE_EPI_F32 (MOE_EPI_ERR_BAD_DTYPE otherwise)
 * inter and hidden must be multiples of 8 (MOE_EPI_ERR_BAD_SHAPE otherwise),
 * tokens at most INT32_MAX; h, w_down and out 16-byte aligned, offs and probs
 * 4-byte aligned (MOE_EPI_ERR_MISALIGNED); out may not overlap any input
 * (MOE_EPI_ERR_ALIAS). The caller owns every buffer; the library allocates
 * nothing and queues the work on `stream`. Returns a moe_epi_status.
 */
int grouped_down_router_fwd(const uint16_t *h, const uint16_t *w_down, const int32_t *offs,
                            const float *probs, void *out, int out_dtype, int64_t tokens, int64_t inter,
                            int64_t hidden, int64_t experts, void *stream);

/*
 * Combine of the routed rows back into tokens: per token, the float32 sum of
 * its top-k routed rows that this rank holds. Defined by
 * "nemo_automodel.components.moe.quantized_experts",
 * GroupedExpertsMXFP4.forward (the local experts' float32 [tokens, hidden]
 * contribution, summed over each token's top-k slots; slots routed to other
 * ranks' experts add nothing) and "nemo_automodel.components.moe
 * .optimized_ops", _apply_router_weight_fp32 (the rows are float32 for this
 * combine). For token t:
 *   out[t, :] = +0 + expert_out[row_of[t, 0], :] + ... + expert_out[row_of[t, top_k-1], :]
 * as binary32 additions in ascending slot order, skipping every slot whose
 * row index is outside [0, rows) (a slot of another rank's expert, or none).
 * The result is bit-exact: the same binary32 operations in the same order for
 * every element.
 *   expert_out [rows, hidden] of eo_dtype          in (may be NULL if rows == 0)
 *   eo_dtype   MOE_EPI_BF16, MOE_EPI_F16 or MOE_EPI_F32
 *   row_of     [tokens, top_k] int32                in, routed row of each slot
 *   out        [tokens, hidden] float32            out, every element written
 * hidden must be a multiple of 8, top_k in [1, 1024] (MOE_EPI_ERR_BAD_SHAPE
 * otherwise); expert_out and out 16-byte aligned, row_of 4-byte aligned
 * (MOE_EPI_ERR_MISALIGNED); out may not overlap an input (MOE_EPI_ERR_ALIAS).
 * tokens == 0 launches nothing. The caller owns every buffer; the library
 * allocates nothing and queues the work on `stream`. Returns a moe_epi_status.
 */
int moe_combine_fwd(const void *expert_out, int eo_dtype, const int32_t *row_of, float *out, int64_t rows,
                    int64_t tokens, int64_t top_k, int64_t hidden, void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *moe_epi_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EPI_H */
