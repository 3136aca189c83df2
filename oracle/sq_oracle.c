/*
 * sq_oracle.c -- CPU oracle for the SmoothQuant W8A8 quantized linear
 * Y = X W^T.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product path
 * (the HIP library and its binding) never calls it, links it or shares a
 * line of code with it.
 *
 * What it follows: the page "w8a8_smoothquant.py" (BiGRU_T_version,
 * src/bigru_t/quantization), namely
 *   - the module docstring: the transform X~ = X / s, W~ = W * s with
 *     Y = X~ W~^T, and the choice s_j = max|X_j|^alpha / max|W_j|^(1-alpha);
 *   - calibrate_smoothquant: column maxima of |X| and |W| floored at 1e-8,
 *     the power quotient, the final floor on s;
 *   - quantize_per_channel_symmetric / quantize_per_token_symmetric: one
 *     scale per row, max|row| floored at 1e-8 and divided by 127, codes
 *     round(v / scale) clamped and stored as int8;
 *   - SmoothQuantW8A8.calibrate: a running per-channel max of |X|;
 *   - SmoothQuantW8A8.freeze_quantization: s from the running max, then
 *     per-output-channel int8 of W * s;
 *   - SmoothQuantW8A8.forward (quantized branch): X / s, per-token int8,
 *     the product of the dequantised operands, then + bias. The page notes
 *     there that real hardware does INT8 x INT8 -> INT32 -> fp32; this file
 *     computes exactly that integer product.
 * and, for the per-tensor variant, the page "quantized_linear.py"
 * (quantize_tensor, QuantizedLinear); for the weight-only linear, the
 * torchao page "quantization/subclass.py" (Int8WeightOnlyQuantizedLinearWeight).
 *
 * Readings where the page is silent or garbled:
 *   R1  codes are clamped to [-128, 127]; with a max-abs scale no code
 *       below -127 can arise, so the page's [-127, 127] gives the same codes.
 *   R2  round() is round-half-to-even of the fp32 quotient.
 *   R3  every quotient is one IEEE binary32 division.
 *   R4  the powers in s are taken through binary64 (see sqo_pow below) so
 *       that the result does not depend on a math library's fp32 pow.
 *   R5  the floor 1e-8 is the binary32 number nearest to 1e-8.
 *   R6  no calibration at all means s = 1 for every channel.
 *   R9  bf16 inputs are widened exactly to fp32 by the caller; all scale
 *       and code arithmetic is fp32; the dequantised output is binary64 and
 *       a bf16 output is that value rounded once, to nearest-even, to bf16.
 *
 * Build: gcc -std=c99 -O2 -ffp-contract=off -fno-fast-math (x86-64 SSE2
 * arithmetic, never x87), optionally -fopenmp for the integer product.
 * Mutants: -DSQO_MUTANT=n plants one deliberate mistake (see the sites
 * marked MUTANT) so that the tests can show each pin catches it.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifndef SQO_MUTANT
#define SQO_MUTANT 0
#endif

/* R5: the page clamps with the Python float 1e-8 on fp32 tensors, i.e. the
 * binary32 value nearest to 1e-8. */
static const float SQO_FLOOR = 1e-8f;

/* Largest and smallest int8 codes (R1). 127 is the page's qmax. */
#define SQO_QMAX 127
#define SQO_QMIN (-128)

int sqo_mutant(void) { return SQO_MUTANT; }

static float fmax_f(float a, float b) { return a > b ? a : b; }

/* ---------------------------------------------------------------------
 * SmoothQuantW8A8.calibrate: running per-input-channel max of |X| over
 * every calibration row. `running` starts at zero (the page's buffer is
 * created with zeros) and is updated in place. No floor here: the page
 * floors only when it forms s.
 * ------------------------------------------------------------------ */
void sqo_calibrate(const float* x, int64_t rows, int64_t k, float* running)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < k; ++j) {
#if SQO_MUTANT == 13
            /* MUTANT 13: forgets the absolute value. */
            float a = x[r * k + j];
#else
            float a = fabsf(x[r * k + j]);
#endif
            if (a > running[j]) running[j] = a;
        }
}

/* ---------------------------------------------------------------------
 * calibrate_smoothquant, max_w: per input channel j the max over output
 * rows o of |W[o, j]|, floored at 1e-8 (one value per input channel).
 * ------------------------------------------------------------------ */
void sqo_weight_col_max(const float* w, int64_t n, int64_t k, float* mw)
{
    for (int64_t j = 0; j < k; ++j) mw[j] = 0.0f;
    for (int64_t o = 0; o < n; ++o)
        for (int64_t j = 0; j < k; ++j) {
#if SQO_MUTANT == 6
            /* MUTANT 6: forgets the absolute value. */
            float a = w[o * k + j];
#else
            float a = fabsf(w[o * k + j]);
#endif
            if (a > mw[j]) mw[j] = a;
        }
    for (int64_t j = 0; j < k; ++j) mw[j] = fmax_f(mw[j], SQO_FLOOR);
}

/* ---------------------------------------------------------------------
 * R4: x^a for the exponents the smoothing factor uses. The page writes
 * torch.pow in fp32, whose last bit depends on the math library. Here:
 *   a = 0    -> 1
 *   a = 1    -> x
 *   a = 1/2  -> sqrt(x)            (binary64 sqrt, correctly rounded)
 *   a = 1/4  -> sqrt(sqrt(x))      (binary64)
 *   a = 3/4  -> sqrt(x) * sqrt(sqrt(x))   (binary64 product)
 *   other a  -> pow(x, a) in binary64
 * The caller rounds the result to binary32 once.
 * ------------------------------------------------------------------ */
static double sqo_pow(double x, double a)
{
    if (a == 0.0) return 1.0;
    if (a == 1.0) return x;
    if (a == 0.5) return sqrt(x);
    if (a == 0.25) return sqrt(sqrt(x));
    if (a == 0.75) return sqrt(x) * sqrt(sqrt(x));
#if SQO_MUTANT == 20
    /* MUTANT 20: base and exponent passed the wrong way round. */
    return pow(a, x);
#elif SQO_MUTANT == 21
    /* MUTANT 21: the complementary exponent 1 - a. */
    return pow(x, 1.0 - a);
#else
    return pow(x, a);
#endif
}

/* ---------------------------------------------------------------------
 * calibrate_smoothquant: s_j = max(|X_j|)^alpha / max(|W_j|)^(1 - alpha),
 * with both maxima floored at 1e-8 first and s floored at 1e-8 last.
 *   mx : running max of |X| per channel (from sqo_calibrate), or NULL for
 *        "never calibrated" (R6: s = 1).
 *   mw : floored column max of |W| (from sqo_weight_col_max).
 * 1 - alpha is formed in binary64. The quotient is one binary32 division
 * of the two binary32-rounded powers.
 * Returns 1 when mx was NULL (the page warns in that case), else 0.
 * ------------------------------------------------------------------ */
int sqo_smoothing_factor(const float* mx, const float* mw, float alpha,
                         int64_t k, float* s)
{
    if (mx == NULL) {
        for (int64_t j = 0; j < k; ++j) s[j] = 1.0f;
        return 1;
    }
    const double a_x = (double)alpha;
#if SQO_MUTANT == 4
    /* MUTANT 4: the weight exponent uses alpha instead of 1 - alpha. */
    const double a_w = (double)alpha;
#else
    const double a_w = 1.0 - (double)alpha;
#endif
    for (int64_t j = 0; j < k; ++j) {
        float mxj = fmax_f(mx[j], SQO_FLOOR);
        float num = (float)sqo_pow((double)mxj, a_x);
        float den = (float)sqo_pow((double)mw[j], a_w);
#if SQO_MUTANT == 12
        /* MUTANT 12: multiplies the two powers instead of dividing. */
        float q = num * den;
#else
        float q = num / den;
#endif
        s[j] = fmax_f(q, SQO_FLOOR);
    }
    return 0;
}

/* ---------------------------------------------------------------------
 * freeze_quantization: W_smooth = weight * s (s broadcast over the input
 * channel, i.e. column j of every row is multiplied by s_j).
 * ------------------------------------------------------------------ */
void sqo_smooth_weight(const float* w, const float* s, int64_t n, int64_t k,
                       float* w_smooth)
{
    for (int64_t o = 0; o < n; ++o)
        for (int64_t j = 0; j < k; ++j)
            w_smooth[o * k + j] = w[o * k + j] * s[j];
}

/* ---------------------------------------------------------------------
 * forward (quantized branch): X_smooth = X / s, channel j divided by s_j.
 * ------------------------------------------------------------------ */
void sqo_smooth_act(const float* x, const float* s, int64_t m, int64_t k,
                    float* x_smooth)
{
    for (int64_t t = 0; t < m; ++t)
        for (int64_t j = 0; j < k; ++j)
#if SQO_MUTANT == 5
            /* MUTANT 5: multiplies by s instead of dividing. */
            x_smooth[t * k + j] = x[t * k + j] * s[j];
#else
            x_smooth[t * k + j] = x[t * k + j] / s[j];
#endif
}

/* Round-half-to-even of a binary32 value to an integer (R2). rintf under
 * the default rounding mode is exactly that. */
static float sqo_round_even(float v)
{
#if SQO_MUTANT == 1
    /* MUTANT 1: rounds halves away from zero. */
    return roundf(v);
#else
    return rintf(v);
#endif
}

/* ---------------------------------------------------------------------
 * quantize_per_channel_symmetric (axis 0) and quantize_per_token_symmetric
 * are the same operation on a 2-D array: one scale per row,
 *   scale[r] = max(max_j |v[r, j]|, 1e-8) / 127            (binary32)
 *   q[r, j]  = clamp(round_even(v[r, j] / scale[r]), -128, 127)
 * ------------------------------------------------------------------ */
void sqo_quantize_rows(const float* v, int64_t rows, int64_t k, int8_t* q,
                       float* scale)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float* row = v + r * k;
        float m = 0.0f;
        for (int64_t j = 0; j < k; ++j) m = fmax_f(m, fabsf(row[j]));
#if SQO_MUTANT == 2
        /* MUTANT 2: no floor; an all-zero row gets scale 1 instead. */
        float sc = m / (float)SQO_QMAX;
        if (sc == 0.0f) sc = 1.0f;
#elif SQO_MUTANT == 10
        /* MUTANT 10: divides the row max by 128 instead of 127. */
        float sc = fmax_f(m, SQO_FLOOR) / 128.0f;
#else
        float sc = fmax_f(m, SQO_FLOOR) / (float)SQO_QMAX;
#endif
        scale[r] = sc;
        for (int64_t j = 0; j < k; ++j) {
            float c = sqo_round_even(row[j] / sc);
            if (c > (float)SQO_QMAX) c = (float)SQO_QMAX;
            if (c < (float)SQO_QMIN) c = (float)SQO_QMIN;
            q[r * k + j] = (int8_t)c;
        }
    }
}

/* ---------------------------------------------------------------------
 * Per-tensor variant, page "quantized_linear.py", quantize_tensor with
 * num_bits = 8 (range [-128, 127]): one scale for the whole tensor,
 *   scale = max_i |x_i| / 127                               (binary32)
 *   scale = 1 when that value is below 1e-8 (the page's replacement)
 *   q_i   = clamp(round_even(x_i / scale), -128, 127)
 * The page returns the dequantised q * scale; its QuantizedLinear
 * multiplies the two dequantised operands and adds the bias, which is the
 * integer product (sqo_int_gemm) times the two scalars plus the bias, up to
 * rounding. bf16 tensors are widened to fp32 by the caller (R9).
 * ------------------------------------------------------------------ */
void sqo_quantize_tensor(const float* x, int64_t count, int8_t* q, float* scale_out)
{
    float m = 0.0f;
    for (int64_t i = 0; i < count; ++i) m = fmax_f(m, fabsf(x[i]));
#if SQO_MUTANT == 14
    /* MUTANT 14: the per-row floor rule instead of the replacement by 1. */
    float sc = fmax_f(m, SQO_FLOOR) / (float)SQO_QMAX;
#elif SQO_MUTANT == 15
    /* MUTANT 15: divides the tensor max by 128 instead of 127. */
    float sc = m / 128.0f;
    if (sc < SQO_FLOOR) sc = 1.0f;
#else
    float sc = m / (float)SQO_QMAX;
    if (sc < SQO_FLOOR) sc = 1.0f;
#endif
    *scale_out = sc;
    for (int64_t i = 0; i < count; ++i) {
        float c = sqo_round_even(x[i] / sc);
        if (c > (float)SQO_QMAX) c = (float)SQO_QMAX;
        if (c < (float)SQO_QMIN) c = (float)SQO_QMIN;
        q[i] = (int8_t)c;
    }
}

/* ---------------------------------------------------------------------
 * Weight-only int8 linear, the torchao page's
 * Int8WeightOnlyQuantizedLinearWeight._quantized_op: the activations stay
 * in floating point, the int8 weights are converted to the activations'
 * type, multiplied, scaled per output channel, then the bias is added:
 *   y[t][o] = (sum_j x[t][j] * wq[o][j]) * scale_w[o] + bias[o]
 * in binary64 (for bf16 activations, widened to fp32 by the caller, every
 * product is exact and the sum is nearly exact; the caller rounds once).
 * ------------------------------------------------------------------ */
void sqo_wo_linear(const float* x, const int8_t* wq, const float* scale_w,
                   const float* bias, int64_t m, int64_t n, int64_t k, double* y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < m; ++t)
        for (int64_t o = 0; o < n; ++o) {
            double sum = 0.0;
            for (int64_t j = 0; j < k; ++j)
                sum += (double)x[t * k + j] * (double)wq[o * k + j];
#if SQO_MUTANT == 16
            /* MUTANT 16: scales by the token index instead of the output
             * channel (reads scale_w[t]). */
            double v = sum * (double)scale_w[t < n ? t : n - 1];
#else
            double v = sum * (double)scale_w[o];
#endif
#if SQO_MUTANT != 17
            /* MUTANT 17 (when defined): the bias is dropped. */
            if (bias) v += (double)bias[o];
#endif
            y[t * n + o] = v;
        }
}

/* ---------------------------------------------------------------------
 * The full-precision side of quantization_error (page
 * "w8a8_smoothquant.py", SmoothQuantW8A8.quantization_error): Y_fp is the
 * plain linear layer on the unquantised input and weights, plus the bias,
 *   y_fp[t][o] = sum_j x[t][j] * w[o][j] + bias[o]
 * in binary64 (fp32 or bf16 values widened by the caller: every product is
 * exact, the sum nearly so).
 * ------------------------------------------------------------------ */
void sqo_reference_linear(const float* x, const float* w, const float* bias,
                          int64_t m, int64_t n, int64_t k, double* y)
{
#if SQO_MUTANT == 18
    /* MUTANT 18: the last term of every k sum is dropped. */
    const int64_t kk = k - 1;
#else
    const int64_t kk = k;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < m; ++t)
        for (int64_t o = 0; o < n; ++o) {
            double sum = 0.0;
            for (int64_t j = 0; j < kk; ++j)
                sum += (double)x[t * k + j] * (double)w[o * k + j];
            if (bias) sum += (double)bias[o];
            y[t * n + o] = sum;
        }
}

/* ---------------------------------------------------------------------
 * quantization_error's measure (same page and method): the Frobenius norm
 * of the difference of the two outputs over the norm of the full-precision
 * one, the latter floored at 1e-12:
 *   ratio = ||y_fp - y_q||_F / max(||y_fp||_F, 1e-12)
 * in binary64, summing in index order. norms[0] and norms[1] receive the
 * two norms; returns the ratio.
 * ------------------------------------------------------------------ */
double sqo_relative_error(const double* y_fp, const double* y_q, int64_t count,
                          double* norms)
{
    double d2 = 0.0, f2 = 0.0;
    for (int64_t i = 0; i < count; ++i) {
        const double d = y_fp[i] - y_q[i];
        d2 += d * d;
#if SQO_MUTANT == 19
        /* MUTANT 19: the denominator measures y_q instead of y_fp. */
        f2 += y_q[i] * y_q[i];
#else
        f2 += y_fp[i] * y_fp[i];
#endif
    }
    const double num = sqrt(d2), den = sqrt(f2);
    norms[0] = num;
    norms[1] = den;
    return num / (den > 1e-12 ? den : 1e-12);
}

/* ---------------------------------------------------------------------
 * The INT8 x INT8 -> INT32 product the page's forward stands in for:
 *   acc[t, o] = sum_j xq[t, j] * wq[o, j]
 * accumulated in int64. Returns the number of entries that do not fit in
 * int32 (0 for every valid input: |acc| <= 128^2 * k).
 * ------------------------------------------------------------------ */
int64_t sqo_int_gemm(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n,
                     int64_t k, int32_t* acc)
{
    int64_t overflow = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : overflow)
    for (int64_t t = 0; t < m; ++t) {
        const int8_t* xr = xq + t * k;
        for (int64_t o = 0; o < n; ++o) {
            const int8_t* wr = wq + o * k;
            int64_t sum = 0;
            for (int64_t j = 0; j < k; ++j)
#if SQO_MUTANT == 8
                /* MUTANT 8: reads the weight operand as if stored k x n. */
                sum += (int64_t)xr[j] * (int64_t)wq[j * n + o];
#else
                sum += (int64_t)xr[j] * (int64_t)wr[j];
#endif
            if (sum > INT32_MAX || sum < INT32_MIN) ++overflow;
            acc[t * n + o] = (int32_t)sum;
        }
    }
    return overflow;
}

/* ---------------------------------------------------------------------
 * Dequantisation of the integer product, in binary64:
 *   y[t, o] = acc[t, o] * scale_x[t] * scale_w[o] + bias[o]
 * (the page adds the bias after the product). bias may be NULL.
 * ------------------------------------------------------------------ */
void sqo_dequant(const int32_t* acc, const float* scale_x, const float* scale_w,
                 const float* bias, int64_t m, int64_t n, double* y)
{
    for (int64_t t = 0; t < m; ++t)
        for (int64_t o = 0; o < n; ++o) {
#if SQO_MUTANT == 3
            /* MUTANT 3: the two scales are indexed the wrong way round. */
            double v = (double)acc[t * n + o] * (double)scale_x[o % m] * (double)scale_w[t % n];
#else
            double v = (double)acc[t * n + o] * (double)scale_x[t] * (double)scale_w[o];
#endif
#if SQO_MUTANT != 9
            /* MUTANT 9 drops the bias. */
            if (bias) v += (double)bias[o];
#endif
            y[t * n + o] = v;
        }
}

/* ---------------------------------------------------------------------
 * The page's own formulation of the frozen forward ("simulation"):
 * dequantise each operand first (code * scale, exact in binary64), then
 * the product of the dequantised matrices, then + bias. It must agree with
 * sqo_dequant(sqo_int_gemm(...)) up to binary64 rounding.
 * ------------------------------------------------------------------ */
void sqo_simulated_forward(const int8_t* xq, const float* scale_x,
                           const int8_t* wq, const float* scale_w,
                           const float* bias, int64_t m, int64_t n, int64_t k,
                           double* y)
{
    for (int64_t t = 0; t < m; ++t)
        for (int64_t o = 0; o < n; ++o) {
            double sum = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                double xd = (double)xq[t * k + j] * (double)scale_x[t];
                double wd = (double)wq[o * k + j] * (double)scale_w[o];
                sum += xd * wd;
            }
            if (bias) sum += (double)bias[o];
            y[t * n + o] = sum;
        }
}

/* ---------------------------------------------------------------------
 * Round binary64 values once, to nearest-even, to bfloat16 (8 significant
 * bits, the binary32 exponent range, subnormals kept). Returns the bf16
 * bit patterns. Used for the bf16 output of the dequantised product (R9).
 * ------------------------------------------------------------------ */
void sqo_f64_to_bf16(const double* v, int64_t count, uint16_t* out)
{
    for (int64_t i = 0; i < count; ++i) {
        double x = v[i];
        uint16_t sign = signbit(x) ? 0x8000u : 0u;
        double a = fabs(x);
        if (isnan(x)) { out[i] = 0x7FC0u; continue; }
        if (a == 0.0) { out[i] = sign; continue; }
        int e;
        (void)frexp(a, &e);           /* a = f * 2^e, f in [0.5, 1) */
        int ex = e - 1;               /* a in [2^ex, 2^(ex+1)) */
        if (ex < -126) ex = -126;     /* bf16 subnormal spacing 2^-133 */
        /* quantum of bf16 at this binade: 2^(ex - 7) */
        double units = ldexp(a, 7 - ex);        /* exact scaling */
        double r = nearbyint(units);            /* ties to even */
        double rounded = ldexp(r, ex - 7);
        if (rounded >= ldexp(1.0, 128)) { out[i] = (uint16_t)(sign | 0x7F80u); continue; }
        float f = (float)rounded;               /* exact: 8 significant bits */
        uint32_t bits;
        memcpy(&bits, &f, 4);
        out[i] = (uint16_t)(sign | ((bits >> 16) & 0x7FFFu));
    }
}

/* =====================================================================
 * The learnable alpha and the straight-through backward (page
 * "w8a8_smoothquant.py": the module docstring's V5 notes, STEQuantize,
 * ste_quantize, SmoothQuantW8A8.alpha / __init__ / forward).
 *
 * alpha = sigmoid(eta) with eta a trained parameter. In the quantized
 * forward s(alpha) is recomputed from the stored maxima, X~ = X / s and
 * W~ = W * s are quantised with round / clamp, and the straight-through
 * estimator passes the gradient of the dequantised operands to X~ and W~
 * unchanged (no gradient reaches the scales: STEQuantize returns none for
 * them). With Y = Xd Wd^T + b, Xd[t][j] = xq[t][j] sx[t] and
 * Wd[o][j] = wq[o][j] sw[o]:
 *   gX[t][j] = sum_o dy[t][o] Wd[o][j]          (the gradient at X~)
 *   gW[o][j] = sum_t dy[t][o] Xd[t][j]          (the gradient at W~)
 *   dx[t][j] = gX[t][j] / s_j                   (X~ = X / s)
 *   dw[o][j] = gW[o][j] * s_j                   (W~ = W * s)
 *   db[o]    = sum_t dy[t][o]
 *   ds_j     = sum_o gW[o][j] w[o][j] - sum_t gX[t][j] x[t][j] / s_j^2
 * s = max(s_raw, 1e-8): the gradient passes the floor only where
 * s_raw >= 1e-8 (a clamp passes its gradient inside its range). With
 * s_raw = mx^alpha / mw^(1 - alpha) (both maxima floored, neither
 * differentiated: the activation maximum is a stored buffer and the weight
 * maximum is taken on detached weights),
 *   d s_raw / d alpha = s_raw (ln mx + ln mw)
 *   dalpha = sum_j [s_raw_j >= 1e-8] ds_j s_raw_j (ln mx_j + ln mw_j)
 *   deta   = dalpha alpha (1 - alpha)           (sigmoid' = a (1 - a))
 * Everything here is binary64 on binary32 inputs; s_raw is the binary32
 * quotient of sqo_smoothing_factor before its floor.
 * ===================================================================== */

/* SmoothQuantW8A8.alpha: sigmoid(eta), taken in binary64 and rounded once
 * to binary32 (the page holds eta and alpha as fp32 tensors). */
float sqo_alpha_from_eta(float eta)
{
    const double e = (double)eta;
#if SQO_MUTANT == 22
    /* MUTANT 22: the logistic function of -eta. */
    return (float)(1.0 / (1.0 + exp(e)));
#else
    return (float)(1.0 / (1.0 + exp(-e)));
#endif
}

/* SmoothQuantW8A8.__init__: eta = log(a / max(1e-6, 1 - a)) for an initial
 * alpha a, in binary64 (Python floats), stored as binary32. */
float sqo_eta_from_alpha(double a)
{
    const double d = 1.0 - a;
    return (float)log(a / (d > 1e-6 ? d : 1e-6));
}

/* The binary32 quotient s_raw_j = f32(P(mx_j, alpha)) / f32(P(mw_j,
 * 1 - alpha)) of sqo_smoothing_factor, before its floor (mx floored at
 * 1e-8 first; mw is already floored). */
static float sqo_smooth_raw(float mxj, float mwj, float alpha)
{
    const float mx = fmax_f(mxj, SQO_FLOOR);
    const float num = (float)sqo_pow((double)mx, (double)alpha);
    const float den = (float)sqo_pow((double)mwj, 1.0 - (double)alpha);
    return num / den;
}

/* ---------------------------------------------------------------------
 * The chain rule from the gradients at X~ and W~ to X, W, s, alpha, eta:
 *   gx [m][k], gw [n][k]  the gradients at X~ = X / s and W~ = W * s
 *   x, w, s, mx, mw, alpha as in sqo_ste_backward below
 * Outputs (binary64): dx [m][k], dw [n][k], ds [k], dalpha_deta [2].
 * ------------------------------------------------------------------ */
void sqo_ste_chain(const double* gx, const double* gw, const float* x, const float* w,
                   const float* s, const float* mx, const float* mw, float alpha, int64_t m,
                   int64_t n, int64_t k, double* dx, double* dw, double* ds,
                   double* dalpha_deta)
{
    /* ds from the two smoothing maps, then dx, dw through them */
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < k; ++j) {
        double from_w = 0.0, from_x = 0.0;
        for (int64_t o = 0; o < n; ++o) from_w += gw[o * k + j] * (double)w[o * k + j];
        for (int64_t t = 0; t < m; ++t) from_x += gx[t * k + j] * (double)x[t * k + j];
#if SQO_MUTANT == 24
        /* MUTANT 24: X / s differentiated as if it were X * s. */
        ds[j] = from_w + from_x;
#else
        ds[j] = from_w - from_x / ((double)s[j] * (double)s[j]);
#endif
    }
    for (int64_t t = 0; t < m; ++t)
        for (int64_t j = 0; j < k; ++j) dx[t * k + j] = gx[t * k + j] / (double)s[j];
    for (int64_t o = 0; o < n; ++o)
        for (int64_t j = 0; j < k; ++j) dw[o * k + j] = gw[o * k + j] * (double)s[j];
    /* through the floor of s, s_raw(alpha) and sigmoid(eta); no alpha
     * gradient when never calibrated (s = 1 does not depend on alpha) */
    double da = 0.0;
    for (int64_t j = 0; mx && j < k; ++j) {
        const float raw = sqo_smooth_raw(mx[j], mw[j], alpha);
#if SQO_MUTANT != 25
        /* MUTANT 25 (when defined): the floor's mask is dropped. */
        if (!(raw >= SQO_FLOOR)) continue;
#endif
        const double lnsum = log((double)fmax_f(mx[j], SQO_FLOOR)) + log((double)mw[j]);
        da += ds[j] * (double)raw * lnsum;
    }
    dalpha_deta[0] = da;
#if SQO_MUTANT == 26
    /* MUTANT 26: the sigmoid's derivative left out. */
    dalpha_deta[1] = da;
#else
    dalpha_deta[1] = da * (double)alpha * (1.0 - (double)alpha);
#endif
}

/* ---------------------------------------------------------------------
 * The straight-through backward of the quantized forward.
 *   dy   [m][n]  gradient of the loss at Y (fp32 values)
 *   x    [m][k]  the forward's activations X; w [n][k] its weights W
 *   s    [k]     the forward's smoothing factor (floored)
 *   xq, sx       per-token codes and scales of X / s (the forward's)
 *   wq, sw       per-output-channel codes and scales of W * s
 *   mx   [k]     stored activation maxima (NULL: never calibrated, no
 *                alpha gradient); mw [k] floored weight maxima
 *   alpha        the forward's alpha (binary32)
 * Outputs (binary64): dx [m][k], dw [n][k], db [n], ds [k], and
 * dalpha_deta[0] = dalpha, dalpha_deta[1] = deta. gx, gw [m][k], [n][k]
 * receive the gradients at X~ and W~.
 * ------------------------------------------------------------------ */
void sqo_ste_backward(const float* dy, const float* x, const float* w, const float* s,
                      const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                      const float* mx, const float* mw, float alpha, int64_t m, int64_t n,
                      int64_t k, double* gx, double* gw, double* dx, double* dw, double* db,
                      double* ds, double* dalpha_deta)
{
    /* the gradients at X~ and W~: the estimator passes the gradient of the
     * dequantised operand straight through round and clamp. Each sum runs
     * over its index in increasing order; the loops are nested so that the
     * innermost one walks a row (j) of the output. */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < m; ++t) {
        double* acc = gx + t * k;
        for (int64_t j = 0; j < k; ++j) acc[j] = 0.0;
        for (int64_t o = 0; o < n; ++o) {
            const double d = (double)dy[t * n + o];
            const double so = (double)sw[o];
            const int8_t* q = wq + o * k;
            for (int64_t j = 0; j < k; ++j) acc[j] += d * ((double)q[j] * so);
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < n; ++o) {
        double* acc = gw + o * k;
        for (int64_t j = 0; j < k; ++j) acc[j] = 0.0;
        for (int64_t t = 0; t < m; ++t) {
            const double d = (double)dy[t * n + o];
#if SQO_MUTANT == 23
            /* MUTANT 23: the activation scale of the wrong token. */
            const double st = (double)sx[(t + 1) % m];
#else
            const double st = (double)sx[t];
#endif
            const int8_t* q = xq + t * k;
            for (int64_t j = 0; j < k; ++j) acc[j] += d * ((double)q[j] * st);
        }
    }
    for (int64_t o = 0; o < n; ++o) {
        double acc = 0.0;
        for (int64_t t = 0; t < m; ++t) acc += (double)dy[t * n + o];
        db[o] = acc;
    }
    sqo_ste_chain(gx, gw, x, w, s, mx, mw, alpha, m, n, k, dx, dw, ds, dalpha_deta);
}

/* ---------------------------------------------------------------------
 * The auxiliary loss of the module docstring: the relative squared error
 *   L = ||y_fp - y_q||_F^2 / ||y_fp||_F^2       (denominator floored at 1e-24)
 * and its gradient at y_q, dL/dy_q = 2 (y_q - y_fp) / ||y_fp||_F^2, the
 * part of it that reaches eta (y_fp, the unquantised linear, does not
 * depend on alpha). binary64. Returns L.
 * ------------------------------------------------------------------ */
double sqo_aux_loss_grad(const double* y_fp, const double* y_q, int64_t count, double* dy_q)
{
    double d2 = 0.0, f2 = 0.0;
    for (int64_t i = 0; i < count; ++i) {
        const double d = y_q[i] - y_fp[i];
        d2 += d * d;
        f2 += y_fp[i] * y_fp[i];
    }
    const double den = f2 > 1e-24 ? f2 : 1e-24;
    for (int64_t i = 0; i < count; ++i)
#if SQO_MUTANT == 27
        /* MUTANT 27: the factor 2 of the square left out. */
        dy_q[i] = (y_q[i] - y_fp[i]) / den;
#else
        dy_q[i] = 2.0 * (y_q[i] - y_fp[i]) / den;
#endif
    return d2 / den;
}
