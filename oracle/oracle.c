/*
 * CPU oracle for the routed-expert epilogue: clamped SwiGLU times routing
 * probability (forward and backward) and the fp32 router-weight multiply
 * (forward and backward).
 *
 * TEST INFRASTRUCTURE ONLY. The product library never includes, links, loads
 * or calls this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no code, header, helper or
 * table with the HIP library.
 *
 * How it computes (plain and slow on purpose):
 *   - one element at a time, in the order the definitions write the
 *     expression, in IEEE binary32 with one rounding per operation (built
 *     with -ffp-contract=off and without fast-math, so no fused
 *     multiply-add and no reassociation);
 *   - exp is the host C library's expf; division is the IEEE division;
 *   - per-row probability gradients: binary32 terms summed in binary64 in
 *     ascending column order, rounded once to binary32;
 *   - every bfloat16 result is rounded once from binary32, to nearest, ties
 *     to even.
 * Rows are independent, so rows may be handed to several OpenMP threads;
 * that changes no result.
 *
 * Sources (the pages' own words are restated, not quoted):
 *   [SW] nemo_automodel.components.moe.swiglu_triton, module description:
 *        y = silu(clamp(gate, max=L)) * clamp(up, -L, L) * probs on the
 *        grouped-GEMM output x = [gate | up] (bf16, [rows, 2*inter]) with
 *        fp32 probs [rows, 1]; fp32 math with the result rounded to x's
 *        dtype; the backward writes d_gate / d_up into the two halves of
 *        grad_x and reduces one probability gradient per row; clamp
 *        gradients follow torch.clamp: the mask is taken on the input
 *        values and includes the clamp bounds.
 *   [RW] nemo_automodel.components.moe.optimized_ops,
 *        _RouterWeightMulFunction class description and the _rw_fwd_core,
 *        _rw_bwd_x_core and _rw_bwd_probs_core entries: out = (x * probs)
 *        in fp32 cast to the output dtype; grad_x = (grad_out * probs) in
 *        fp32 cast to x's dtype; grad_probs = (grad_out * x).sum(-1) in fp32
 *        cast to probs' dtype.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---- bfloat16 <-> binary32 ------------------------------------------- */

/* Widening is exact: a bfloat16 is the upper half of a binary32. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* Round a binary32 to bfloat16, to nearest, ties to even (the rounding of
 * torch's .to(torch.bfloat16)). The kept part is the upper 16 bits; the
 * dropped lower 16 bits decide: above half -> round up, exactly half ->
 * round up only if the kept part is odd, below half -> truncate. Rounding up
 * may carry into the exponent, which is the correct result (up to +-inf).
 * NaN stays NaN: its sign and top payload bits are kept and the quiet bit
 * is set. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    uint32_t kept = bits >> 16;
    uint32_t dropped = bits & 0xFFFFu;
    if ((bits & 0x7F800000u) == 0x7F800000u && (bits & 0x007FFFFFu) != 0)
        return (uint16_t)(kept | 0x0040u);
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

/* ---- clamped SwiGLU x probs: one element ------------------------------ */

/*
 * [SW] All quantities for one element (gate g, up u, probability p, upstream
 * gradient gy, limit L), in binary32:
 *   out[0] = y before rounding        = (silu(gc) * uc) * p
 *   out[1] = d_gate before rounding   = mask_g ? (gy*p * uc) * silu'(gc) : +0
 *   out[2] = d_up before rounding     = mask_u ? (gy*p) * silu(gc)      : +0
 *   out[3] = this element's term of the probability gradient = gy * (silu(gc)*uc)
 * with gc = min(g, L) (upper clamp only), uc = clamp(u, -L, L),
 * silu(z) = z * sigma(z), sigma(z) = 1 / (1 + exp(-z)),
 * silu'(z) = sigma(z) * (1 + z * (1 - sigma(z))),
 * mask_g = (g <= L), mask_u = (-L <= u <= L): the inclusive torch.clamp
 * masks on the input values. A clamp passes NaN through (a comparison with
 * NaN is false), and a NaN input fails its mask, as torch.clamp does.
 * Masked gradients are written as +0 (a selection, not a product with the
 * mask).
 */
void oracle_swiglu_point(float g, float u, float p, float gy, float L, float out[4])
{
    float gc = (g > L) ? L : g;
    float uc = (u > L) ? L : ((u < -L) ? -L : u);
    float sig = 1.0f / (1.0f + expf(-gc));
    float a = gc * sig;                 /* silu(gc) */
    float h = a * uc;
    float t = gy * p;
    float dsilu = sig * (1.0f + gc * (1.0f - sig));
    int mask_g = (g <= L);
    int mask_u = (-L <= u) && (u <= L);
    out[0] = h * p;
    out[1] = mask_g ? (t * uc) * dsilu : 0.0f;
    out[2] = mask_u ? t * a : 0.0f;
    out[3] = gy * h;
}

/* ---- clamped SwiGLU x probs: whole tensors ---------------------------- */

/* [SW] forward. x is [rows, 2*inter] row-major (gate = columns [0, inter),
 * up = columns [inter, 2*inter)); probs is [rows]; y is [rows, inter]. */
void oracle_swiglu_clamped_fwd(const uint16_t *x, const float *probs, uint16_t *y,
                               int64_t rows, int64_t inter, float L, int nthreads)
{
    int64_t r;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * 2 * inter;
        for (int64_t j = 0; j < inter; ++j) {
            float q[4];
            oracle_swiglu_point(oracle_bf16_to_f32(xr[j]), oracle_bf16_to_f32(xr[inter + j]),
                                probs[r], 0.0f, L, q);
            y[r * inter + j] = oracle_f32_to_bf16(q[0]);
        }
    }
}

/* [SW] backward. grad_y is [rows, inter]; grad_x is [rows, 2*inter] with
 * d_gate in the first half of each row and d_up in the second; grad_probs is
 * [rows] and may be NULL, in which case no probability gradient is formed.
 * grad_probs_abs (may be NULL) receives sum_j |term_j| per row in binary64:
 * the scale against which a probability gradient summed in another order is
 * judged. */
void oracle_swiglu_clamped_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                               uint16_t *grad_x, float *grad_probs, double *grad_probs_abs,
                               int64_t rows, int64_t inter, float L, int nthreads)
{
    int64_t r;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * 2 * inter;
        const uint16_t *gyr = grad_y + r * inter;
        uint16_t *gxr = grad_x + r * 2 * inter;
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t j = 0; j < inter; ++j) {
            float q[4];
            oracle_swiglu_point(oracle_bf16_to_f32(xr[j]), oracle_bf16_to_f32(xr[inter + j]),
                                probs[r], oracle_bf16_to_f32(gyr[j]), L, q);
            gxr[j] = oracle_f32_to_bf16(q[1]);
            gxr[inter + j] = oracle_f32_to_bf16(q[2]);
            acc += (double)q[3];
            acc_abs += fabs((double)q[3]);
        }
        if (grad_probs)
            grad_probs[r] = (float)acc;
        if (grad_probs_abs)
            grad_probs_abs[r] = acc_abs;
    }
}

/* ---- fp32 router-weight multiply -------------------------------------- */

/* [RW] _rw_fwd_core: out = bf16(fp32(x) * p). x and out are [rows, hidden];
 * probs is [rows]. */
void oracle_router_weight_mul_fwd(const uint16_t *x, const float *probs, uint16_t *out,
                                  int64_t rows, int64_t hidden, int nthreads)
{
    int64_t r;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < hidden; ++k) {
            float v = oracle_bf16_to_f32(x[r * hidden + k]) * probs[r];
            out[r * hidden + k] = oracle_f32_to_bf16(v);
        }
    }
}

/* [RW] _rw_bwd_x_core and _rw_bwd_probs_core:
 *   grad_x[r,k]   = bf16(fp32(grad_out[r,k]) * p[r])
 *   grad_probs[r] = sum_k fp32(grad_out[r,k]) * fp32(x[r,k])
 * grad_probs may be NULL (probabilities that carry no gradient); x is then
 * not read and may be NULL too. grad_probs_abs (may be NULL) receives
 * sum_k |term_k| per row in binary64, the scale of the sum. */
void oracle_router_weight_mul_bwd(const uint16_t *grad_out, const uint16_t *x, const float *probs,
                                  uint16_t *grad_x, float *grad_probs, double *grad_probs_abs,
                                  int64_t rows, int64_t hidden, int nthreads)
{
    int64_t r;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; ++r) {
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t k = 0; k < hidden; ++k) {
            float g = oracle_bf16_to_f32(grad_out[r * hidden + k]);
            grad_x[r * hidden + k] = oracle_f32_to_bf16(g * probs[r]);
            if (grad_probs) {
                float term = g * oracle_bf16_to_f32(x[r * hidden + k]);
                acc += (double)term;
                acc_abs += fabs((double)term);
            }
        }
        if (grad_probs)
            grad_probs[r] = (float)acc;
        if (grad_probs && grad_probs_abs)
            grad_probs_abs[r] = acc_abs;
    }
}

/* ---- other storage dtypes: float16 and float32 ------------------------ */
/*
 * [SW] lists bfloat16, float16 and float32 as the supported dtypes of x (the
 * _SUPPORTED_DTYPES entry); [RW] lets the router multiply's output be the
 * activation dtype or float32 (the out_dtype parameter of
 * _RouterWeightMulFunction.forward, where float32 serves the path that
 * reduces expert outputs by scatter-add). The math is the same binary32 chain; only loading and the final
 * rounding depend on the dtype. Codes: 0 bfloat16, 1 float16, 2 float32.
 */
enum { ORACLE_BF16 = 0, ORACLE_F16 = 1, ORACLE_F32 = 2 };

/* float16 -> binary32, exact: sign, 5-bit exponent (bias 15), 10-bit fraction. */
float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    int ex = (h >> 10) & 0x1F;
    uint32_t frac = h & 0x3FFu;
    float mag;
    if (ex == 0) {
        mag = ldexpf((float)frac, -24);                 /* zero or subnormal: frac * 2^-24 */
    } else if (ex == 31) {
        uint32_t bits = 0x7F800000u | (frac << 13);     /* inf, or NaN keeping its payload */
        memcpy(&mag, &bits, sizeof mag);
    } else {
        mag = ldexpf((float)(1024u + frac), ex - 25);   /* (1 + frac/1024) * 2^(ex-15) */
    }
    uint32_t bits;
    memcpy(&bits, &mag, sizeof bits);
    bits |= sign;
    memcpy(&mag, &bits, sizeof mag);
    return mag;
}

/* binary32 -> float16, to nearest, ties to even, with subnormals, overflow
 * to infinity and NaN kept NaN (quiet bit set). The magnitude is written as an
 * integer multiple n of the float16 unit in the last place at its exponent,
 * and the dropped bits decide the rounding as for bfloat16. */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    int ef = (int)((bits >> 23) & 0xFFu);
    uint32_t frac = bits & 0x7FFFFFu;
    if (ef == 0xFF)
        return (uint16_t)(sign | (frac ? (0x7E00u | (frac >> 13)) : 0x7C00u));
    if (ef == 0)
        return sign;                                     /* binary32 zero/subnormal: below half of 2^-24 */
    int e = ef - 127;                                    /* value = m * 2^(e - 23), m in [2^23, 2^24) */
    uint64_t m = (uint64_t)frac | 0x800000u;
    int emin = e < -14 ? -14 : e;                        /* float16 exponent used (subnormals: -14) */
    int sh = (emin - 10) - (e - 23);                     /* value / ulp = m / 2^sh, sh >= 13 */
    uint64_t n, rem, half;
    if (sh >= 40) {
        n = 0; rem = m; half = (uint64_t)1 << 39;       /* m < 2^24: far below half an ulp */
    } else {
        n = m >> sh;
        rem = m & (((uint64_t)1 << sh) - 1);
        half = (uint64_t)1 << (sh - 1);
    }
    if (rem > half || (rem == half && (n & 1u)))
        n += 1;
    if (e < -14)
        return (uint16_t)(sign | n);                     /* subnormal (n == 1024 is the smallest normal) */
    uint32_t out = ((uint32_t)(e + 15) << 10) + (uint32_t)(n - 1024); /* n == 2048 carries into the exponent */
    if (out >= 0x7C00u)
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | out);
}

static float oracle_load(const void *p, int64_t i, int dtype)
{
    if (dtype == ORACLE_BF16)
        return oracle_bf16_to_f32(((const uint16_t *)p)[i]);
    if (dtype == ORACLE_F16)
        return oracle_f16_to_f32(((const uint16_t *)p)[i]);
    return ((const float *)p)[i];
}

static void oracle_store(void *p, int64_t i, int dtype, float v)
{
    if (dtype == ORACLE_BF16)
        ((uint16_t *)p)[i] = oracle_f32_to_bf16(v);
    else if (dtype == ORACLE_F16)
        ((uint16_t *)p)[i] = oracle_f32_to_f16(v);
    else
        ((float *)p)[i] = v;
}

/* [SW] forward with x and y of one dtype. */
void oracle_swiglu_clamped_fwd_typed(const void *x, int dtype, const float *probs, void *y,
                                     int64_t rows, int64_t inter, float L, int nthreads)
{
    int64_t r;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < inter; ++j) {
            float q[4];
            oracle_swiglu_point(oracle_load(x, r * 2 * inter + j, dtype),
                                oracle_load(x, r * 2 * inter + inter + j, dtype), probs[r], 0.0f, L, q);
            oracle_store(y, r * inter + j, dtype, q[0]);
        }
    }
}

/* [SW] backward with x, grad_y and grad_x of one dtype (grad_probs float32). */
void oracle_swiglu_clamped_bwd_typed(const void *x, int dtype, const float *probs, const void *grad_y,
                                     void *grad_x, float *grad_probs, double *grad_probs_abs,
                                     int64_t rows, int64_t inter, float L, int nthreads)
{
    int64_t r;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; ++r) {
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t j = 0; j < inter; ++j) {
            float q[4];
            oracle_swiglu_point(oracle_load(x, r * 2 * inter + j, dtype),
                                oracle_load(x, r * 2 * inter + inter + j, dtype), probs[r],
                                oracle_load(grad_y, r * inter + j, dtype), L, q);
            oracle_store(grad_x, r * 2 * inter + j, dtype, q[1]);
            oracle_store(grad_x, r * 2 * inter + inter + j, dtype, q[2]);
            acc += (double)q[3];
            acc_abs += fabs((double)q[3]);
        }
        if (grad_probs)
            grad_probs[r] = (float)acc;
        if (grad_probs_abs)
            grad_probs_abs[r] = acc_abs;
    }
}

/* [RW] forward: out (out_dtype) = round(fp32(x) * p); x of x_dtype. */
void oracle_router_weight_mul_fwd_typed(const void *x, int x_dtype, const float *probs, void *out,
                                        int out_dtype, int64_t rows, int64_t hidden, int nthreads)
{
    int64_t r;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; ++r)
        for (int64_t k = 0; k < hidden; ++k)
            oracle_store(out, r * hidden + k, out_dtype, oracle_load(x, r * hidden + k, x_dtype) * probs[r]);
}

/* [RW] backward: grad_out has the output's dtype, grad_x the dtype of x;
 * grad_probs (float32) sums the binary32 products grad_out * x in binary64. */
void oracle_router_weight_mul_bwd_typed(const void *grad_out, int go_dtype, const void *x, int x_dtype,
                                        const float *probs, void *grad_x, float *grad_probs,
                                        double *grad_probs_abs, int64_t rows, int64_t hidden, int nthreads)
{
    int64_t r;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; ++r) {
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t k = 0; k < hidden; ++k) {
            float g = oracle_load(grad_out, r * hidden + k, go_dtype);
            oracle_store(grad_x, r * hidden + k, x_dtype, g * probs[r]);
            if (grad_probs) {
                float term = g * oracle_load(x, r * hidden + k, x_dtype);
                acc += (double)term;
                acc_abs += fabs((double)term);
            }
        }
        if (grad_probs)
            grad_probs[r] = (float)acc;
        if (grad_probs && grad_probs_abs)
            grad_probs_abs[r] = acc_abs;
    }
}

/* ---- gate_up grouped GEMM with the clamped SwiGLU epilogue ------------- */
/*
 * Sources:
 *   [MK] nemo_automodel.components.moe.mok_experts, the routed expert weight
 *        parameters: routed gate and up weights are contiguous bfloat16
 *        tensors of shape [local_experts, expert_intermediate, hidden].
 *   [GM] nemo_automodel.components.moe.quantized_experts,
 *        MXFP4ExpertStorageMixin._mxfp4_base_mm: the routed activations are
 *        [tokens, in_dim], grouped contiguously by local expert; offs is an
 *        int32 [local_experts] tensor of cumulative token counts; the result is
 *        [tokens, out_dim] in the activation dtype.
 *   [SW] (above): the epilogue consumes that grouped-GEMM output, x = [gate | up].
 *
 * Rows of expert e are [start_e, end_e) with start_0 = 0, end_e = offs[e]
 * clamped to [start_e, tokens] and start_{e+1} = end_e (a count that is
 * negative, decreasing or past the end gives an empty or shortened range;
 * rows at or past the last end belong to no expert and are not written).
 * For such a row t of expert e and column j < inter:
 *   gate[t, j] = sum_h a[t, h] * w_gate[e, j, h]
 *   up[t, j]   = sum_h a[t, h] * w_up[e, j, h]
 * Each product of two bfloat16 values is exact in binary64; the products are
 * added in binary64 in ascending h, which is exact while the products of a
 * sum span fewer than about 2^37 in magnitude (true of any data the tests
 * use). The grouped GEMM's output in the activation dtype is that exact sum
 * rounded once to bfloat16.
 */

/* binary64 -> bfloat16, to nearest, ties to even, with subnormals (unit 2^-133),
 * overflow to infinity and NaN kept NaN. Same method as oracle_f32_to_f16: the
 * magnitude as an integer multiple n of the bfloat16 unit at its exponent. */
uint16_t oracle_f64_to_bf16(double v)
{
    uint64_t bits;
    memcpy(&bits, &v, sizeof bits);
    uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
    int ed = (int)((bits >> 52) & 0x7FFu);
    uint64_t frac = bits & 0xFFFFFFFFFFFFFull;
    if (ed == 0x7FF)
        return (uint16_t)(sign | (frac ? (0x7FC0u | (uint16_t)(frac >> 45)) : 0x7F80u));
    if (ed == 0)
        return sign;                                     /* binary64 zero/subnormal: far below 2^-134 */
    int e = ed - 1023;                                   /* value = m * 2^(e - 52), m in [2^52, 2^53) */
    uint64_t m = frac | (1ull << 52);
    int emin = e < -126 ? -126 : e;                      /* bfloat16 exponent used (subnormals: -126) */
    int sh = (emin - 7) - (e - 52);                      /* value / unit = m / 2^sh, sh >= 45 */
    uint64_t n, rem, half;
    if (sh >= 60) {
        n = 0; rem = m; half = 1ull << 59;               /* m < 2^53: below half a unit */
    } else {
        n = m >> sh;
        rem = m & ((1ull << sh) - 1);
        half = 1ull << (sh - 1);
    }
    if (rem > half || (rem == half && (n & 1u)))
        n += 1;
    if (e < -126)
        return (uint16_t)(sign | n);                     /* subnormal (n == 128 is the smallest normal) */
    if (e > 127)
        return (uint16_t)(sign | 0x7F80u);
    uint32_t out = ((uint32_t)(e + 127) << 7) + (uint32_t)(n - 128); /* n == 256 carries into the exponent */
    if (out >= 0x7F80u)
        return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | out);
}

/* [GM][MK] the exact grouped sums. sum is [tokens, 2*inter] (gate in columns
 * [0, inter), up in [inter, 2*inter)); abs_sum (may be NULL) receives
 * sum_h |a * w| for each output: the scale of the rounding error of a sum
 * accumulated in another order or precision. Rows of no expert are not written. */
void oracle_grouped_gate_up(const uint16_t *a, const uint16_t *w_gate, const uint16_t *w_up,
                            const int32_t *offs, double *sum, double *abs_sum,
                            int64_t tokens, int64_t hidden, int64_t inter, int64_t experts, int nthreads)
{
    int64_t start = 0;
    for (int64_t e = 0; e < experts; ++e) {
        int64_t end = offs[e];
        if (end < start) end = start;
        if (end > tokens) end = tokens;
        int64_t t;
#pragma omp parallel for schedule(static) num_threads(nthreads)
        for (t = start; t < end; ++t) {
            const uint16_t *at = a + t * hidden;
            for (int64_t half = 0; half < 2; ++half) {
                const uint16_t *w = (half == 0 ? w_gate : w_up) + e * inter * hidden;
                for (int64_t j = 0; j < inter; ++j) {
                    const uint16_t *wj = w + j * hidden;
                    double s = 0.0, s_abs = 0.0;
                    for (int64_t h = 0; h < hidden; ++h) {
                        double prod = (double)oracle_bf16_to_f32(at[h]) * (double)oracle_bf16_to_f32(wj[h]);
                        s += prod;
                        s_abs += fabs(prod);
                    }
                    sum[t * 2 * inter + half * inter + j] = s;
                    if (abs_sum)
                        abs_sum[t * 2 * inter + half * inter + j] = s_abs;
                }
            }
        }
        start = end;
    }
}

/* [GM][MK][SW] the fused forward: x = bf16(exact grouped sums) (written to
 * x_out when it is not NULL, [tokens, 2*inter]), then y = the [SW] forward of
 * that x ([tokens, inter]). sum_scratch is caller memory of tokens*2*inter
 * doubles. Rows of no expert are not written. */
void oracle_grouped_swiglu_fwd(const uint16_t *a, const uint16_t *w_gate, const uint16_t *w_up,
                               const int32_t *offs, const float *probs, uint16_t *y, uint16_t *x_out,
                               double *sum_scratch, int64_t tokens, int64_t hidden, int64_t inter,
                               int64_t experts, float L, int nthreads)
{
    oracle_grouped_gate_up(a, w_gate, w_up, offs, sum_scratch, NULL, tokens, hidden, inter, experts, nthreads);
    int64_t start = 0;
    for (int64_t e = 0; e < experts; ++e) {
        int64_t end = offs[e];
        if (end < start) end = start;
        if (end > tokens) end = tokens;
        int64_t t;
#pragma omp parallel for schedule(static) num_threads(nthreads)
        for (t = start; t < end; ++t) {
            for (int64_t j = 0; j < inter; ++j) {
                uint16_t g = oracle_f64_to_bf16(sum_scratch[t * 2 * inter + j]);
                uint16_t u = oracle_f64_to_bf16(sum_scratch[t * 2 * inter + inter + j]);
                if (x_out) {
                    x_out[t * 2 * inter + j] = g;
                    x_out[t * 2 * inter + inter + j] = u;
                }
                float q[4];
                oracle_swiglu_point(oracle_bf16_to_f32(g), oracle_bf16_to_f32(u), probs[t], 0.0f, L, q);
                y[t * inter + j] = oracle_f32_to_bf16(q[0]);
            }
        }
        start = end;
    }
}

/* ---- down projection with the router-weight multiply, and the combine --- */
/*
 * Sources:
 *   [MK] (above): the routed down weights are contiguous bfloat16
 *        [local_experts, hidden, expert_intermediate].
 *   [RW] (above), _apply_router_weight_fp32: the expert down-projection
 *        outputs [tokens, hidden] are multiplied by the permuted routing
 *        probabilities in fp32 and cast to the output dtype (the activation
 *        dtype, or fp32 where expert outputs are combined by scatter-add).
 *   [GX] nemo_automodel.components.moe.quantized_experts,
 *        GroupedExpertsMXFP4.forward: the local experts' contribution is an
 *        fp32 [tokens, hidden] tensor, formed before the expert-parallel
 *        reduction from each token's top-k routing slots.
 *
 * Down projection: for a row t of local expert e (rows grouped as in [GM],
 * offs read as above), out2[t, n] = bf16(sum_i h[t, i] * w_down[e, n, i])
 * (exact sum, rounded once: the grouped GEMM's output in the activation
 * dtype), then out[t, n] = round_out(fp32(out2[t, n]) * p[t]) as in [RW].
 *
 * Combine: out[t, :] = sum over slots j = 0 .. top_k-1 with a row r =
 * row_of[t, j] in [0, rows) of fp32(expert_out[r, :]), added in binary32 in
 * ascending j (the pages leave the order of the scatter-add open; ascending
 * slots is the reading taken, and makes the sum reproducible). A slot whose
 * row is negative or out of range contributes nothing; a token with no such
 * slot gets +0.
 */

/* [MK][GM][RW] out_dtype: ORACLE_BF16 or ORACLE_F32. Rows of no expert are not written. */
void oracle_grouped_down_router_fwd(const uint16_t *h, const uint16_t *w_down, const int32_t *offs,
                                    const float *probs, void *out, int out_dtype, int64_t tokens,
                                    int64_t inter, int64_t hidden, int64_t experts, int nthreads)
{
    int64_t start = 0;
    for (int64_t e = 0; e < experts; ++e) {
        int64_t end = offs[e];
        if (end < start) end = start;
        if (end > tokens) end = tokens;
        const uint16_t *w = w_down + e * hidden * inter;
        int64_t t;
#pragma omp parallel for schedule(static) num_threads(nthreads)
        for (t = start; t < end; ++t) {
            const uint16_t *ht = h + t * inter;
            for (int64_t n = 0; n < hidden; ++n) {
                const uint16_t *wn = w + n * inter;
                double s = 0.0;
                for (int64_t i = 0; i < inter; ++i)
                    s += (double)oracle_bf16_to_f32(ht[i]) * (double)oracle_bf16_to_f32(wn[i]);
                float out2 = oracle_bf16_to_f32(oracle_f64_to_bf16(s));
                oracle_store(out, t * hidden + n, out_dtype, out2 * probs[t]);
            }
        }
        start = end;
    }
}

/* [GX] expert_out is [rows, hidden] of eo_dtype (bfloat16 or float32); row_of
 * is [tokens, top_k]; out is float32 [tokens, hidden]. */
void oracle_moe_combine(const void *expert_out, int eo_dtype, const int32_t *row_of, float *out,
                        int64_t rows, int64_t tokens, int64_t top_k, int64_t hidden, int nthreads)
{
    int64_t t;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (t = 0; t < tokens; ++t) {
        for (int64_t n = 0; n < hidden; ++n) {
            float acc = 0.0f;
            for (int64_t j = 0; j < top_k; ++j) {
                int64_t r = row_of[t * top_k + j];
                if (r >= 0 && r < rows)
                    acc = acc + oracle_load(expert_out, r * hidden + n, eo_dtype);
            }
            out[t * hidden + n] = acc;
        }
    }
}
