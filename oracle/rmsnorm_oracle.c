/*
 * rmsnorm_oracle.c -- plain, slow fp64 CPU oracle for RMSNorm.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library and includes nothing from it.
 *
 * Sources (three web pages, cited by title and section):
 *   [PR]  MLX pull request "RMSNormVJP backward writes a full {n_rows, D}
 *         gw_temp intermediate" -- sections "Proposed changes" and "POC".
 *         The POC's correctness guard differentiates the reference
 *         expression  (rsqrt(mean(x^2 over the last axis) + eps) * x) * w
 *         computed in fp32, with gradients returned for x and w.
 *   [FA]  mlxcel issue "Fused residual-add RMSNorm and fused RoPE +
 *         KV-append decode kernels" -- the FusedAddRMSNorm bullet of the
 *         candidate-fusion list (new residual = input + residual, output =
 *         rmsnorm(new residual) * (weight_bias + weight), rsqrt(mean + eps),
 *         fp32 sum kept once), "Regression guard" (Gemma 1+w case), and the
 *         gated-activation bullet (silu of the first half of a row times its
 *         second half).
 *
 * Every routine computes in IEEE fp64 with plain loops in row order; there is
 * no blocking, fusion or reordering beyond the definition.  Inputs are the
 * storage-dtype values widened exactly to fp64 by the caller.
 *
 * Readings where the pages leave a step open:
 *   - the mean divides by D and eps sits inside the square root ([PR] POC
 *     reference expression);
 *   - the fused form normalises the unrounded sum x + residual ([FA]);
 *   - the VJP recomputes r from x (the POC times a grad call as forward
 *     recompute plus VJP) -- no saved statistics are an input;
 *   - dx is not printed on the pages; it is the derivative of the POC
 *     expression:  with g = weight_bias + w, r = (mean(x^2) + eps)^(-1/2),
 *     S = sum_j dy_j g_j x_j:   dx_j = r g_j dy_j - x_j r^3 S / D ;
 *   - dw is the sum over rows of each row's dy_j x_j r  ([PR] "Proposed
 *     changes": gw is a per-row contribution summed over rows), and does not
 *     depend on w or weight_bias.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* [PR] POC reference expression, with the weight_bias offset of [FA]:
 *   ms_i = (1/D) sum_j x_ij^2,  r_i = 1/sqrt(ms_i + eps),
 *   y_ij = x_ij * r_i * (weight_bias + w_j).
 * rstd (may be NULL) receives r_i. */
void orc_rmsnorm_fwd(int64_t rows, int64_t D, const double *x, const double *w,
                     double eps, double weight_bias, double *y, double *rstd)
{
    for (int64_t i = 0; i < rows; ++i) {
        const double *xi = x + i * D;
        double *yi = y + i * D;
        double ss = 0.0;
        for (int64_t j = 0; j < D; ++j)
            ss += xi[j] * xi[j];
        double ms = ss / (double)D;
        double r = 1.0 / sqrt(ms + eps);
        if (rstd)
            rstd[i] = r;
        for (int64_t j = 0; j < D; ++j)
            yi[j] = xi[j] * r * (weight_bias + w[j]);
    }
}

/* [FA] FusedAddRMSNorm: h = x + residual (the new residual, returned
 * unrounded so the caller rounds it to the storage dtype), and
 * normed = rmsnorm(h) * (weight_bias + w) computed from the unrounded h. */
void orc_fused_add_rmsnorm_fwd(int64_t rows, int64_t D, const double *x,
                               const double *residual, const double *w,
                               double eps, double weight_bias, double *normed,
                               double *new_residual)
{
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < D; ++j)
            new_residual[i * D + j] = x[i * D + j] + residual[i * D + j];
    }
    orc_rmsnorm_fwd(rows, D, new_residual, w, eps, weight_bias, normed, NULL);
}

/* Backward (VJP) of the [PR] POC expression for an upstream gradient dy.
 *   dx_ij = r_i g_j dy_ij - x_ij r_i^3 S_i / D,   S_i = sum_j dy_ij g_j x_ij
 *   dw_j  = sum_i dy_ij x_ij r_i              (summed over all rows here)
 * dw is overwritten (an empty row set gives dw = 0). */
void orc_rmsnorm_vjp(int64_t rows, int64_t D, const double *x, const double *w,
                     const double *dy, double eps, double weight_bias,
                     double *dx, double *dw)
{
    for (int64_t j = 0; j < D; ++j)
        dw[j] = 0.0;
    for (int64_t i = 0; i < rows; ++i) {
        const double *xi = x + i * D;
        const double *dyi = dy + i * D;
        double *dxi = dx + i * D;
        double ss = 0.0;
        for (int64_t j = 0; j < D; ++j)
            ss += xi[j] * xi[j];
        double ms = ss / (double)D;
        double r = 1.0 / sqrt(ms + eps);
        double S = 0.0;
        for (int64_t j = 0; j < D; ++j)
            S += dyi[j] * (weight_bias + w[j]) * xi[j];
        double r3 = r * r * r;
        for (int64_t j = 0; j < D; ++j) {
            double g = weight_bias + w[j];
            dxi[j] = r * g * dyi[j] - xi[j] * r3 * S / (double)D;
            dw[j] += dyi[j] * xi[j] * r;
        }
    }
}

/* Backward of [FA]'s fused form for training: with h = x + residual (the
 * saved new_residual) feeding both normed = rmsnorm(h) * g and the next
 * residual stream, the gradient reaching h -- and through the sum both x
 * and residual -- is the RMSNorm VJP for dy plus the residual-stream
 * gradient d_new_residual.  dw is the VJP's.  The row statistic is
 * recomputed from h as given. */
void orc_fused_add_rmsnorm_vjp(int64_t rows, int64_t D, const double *h, const double *w,
                               const double *dy, const double *d_new_residual, double eps,
                               double weight_bias, double *dh, double *dw)
{
    orc_rmsnorm_vjp(rows, D, h, w, dy, eps, weight_bias, dh, dw);
    for (int64_t i = 0; i < rows * D; ++i)
        dh[i] += d_new_residual[i];
}

/* [FA] gated activation: x is [rows, 2d]; with a = x[:, :d], b = x[:, d:2d],
 *   y = silu(a) * b,   silu(a) = a * sigmoid(a) = a / (1 + exp(-a)).
 * y is [rows, d]. */
void orc_silu_gate(int64_t rows, int64_t d, const double *x, double *y)
{
    for (int64_t i = 0; i < rows; ++i) {
        const double *a = x + i * 2 * d;
        const double *b = a + d;
        for (int64_t j = 0; j < d; ++j)
            y[i * d + j] = a[j] / (1.0 + exp(-a[j])) * b[j];
    }
}

/* Backward of the gated activation for an upstream gradient dy [rows, d]:
 * with s = sigmoid(a) = 1 / (1 + exp(-a)),
 *   d/db = dy * a * s,   d/da = dy * b * s * (1 + a * (1 - s))
 * (the derivative of a * s is s + a * s * (1 - s)).  dx is [rows, 2d]: the
 * gradient of the first half, then of the second. */
void orc_silu_gate_vjp(int64_t rows, int64_t d, const double *x, const double *dy, double *dx)
{
    for (int64_t i = 0; i < rows; ++i) {
        const double *a = x + i * 2 * d;
        const double *b = a + d;
        double *da = dx + i * 2 * d;
        double *db = da + d;
        for (int64_t j = 0; j < d; ++j) {
            const double g = dy[i * d + j];
            const double sg = 1.0 / (1.0 + exp(-a[j]));
            db[j] = g * a[j] * sg;
            da[j] = g * b[j] * sg * (1.0 + a[j] * (1.0 - sg));
        }
    }
}

/* ------------------------------------------------------------------------
 * Round-to-nearest-even from fp64 straight to a binary format with
 * `mant` stored mantissa bits and exponent range [emin, emax], returning the
 * rounded value as fp64 (no double rounding through fp32).  IEEE 754 rule:
 * scale by the quantum of the value's binade (or of the subnormal range),
 * round to an integer with ties to even, scale back; results at or beyond
 * 2^(emax+1) overflow to infinity.
 * ------------------------------------------------------------------------ */
static double rne_to_format(double v, int mant, int emin, int emax)
{
    if (isnan(v) || isinf(v) || v == 0.0)
        return v;
    int e;
    (void)frexp(fabs(v), &e);      /* |v| = m * 2^e, m in [0.5, 1) */
    int binade = e - 1;            /* |v| in [2^binade, 2^(binade+1)) */
    if (binade < emin)
        binade = emin;             /* subnormal range: fixed quantum */
    int qexp = binade - mant;
    double q = ldexp(v, -qexp);    /* exact: power-of-two scaling */
    double n = nearbyint(q);       /* default mode: ties to even */
    double out = ldexp(n, qexp);
    if (fabs(out) >= ldexp(1.0, emax + 1))
        return copysign(INFINITY, v);
    return out;
}

double orc_round_f16(double v)  { return rne_to_format(v, 10, -14, 15); }
double orc_round_bf16(double v) { return rne_to_format(v, 7, -126, 127); }
double orc_round_f32(double v)  { return rne_to_format(v, 23, -126, 127); }

/* Array forms: kind 0 = fp32, 1 = fp16, 2 = bf16. */
void orc_round_array(int kind, int64_t n, const double *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) {
        if (kind == 1)
            out[i] = orc_round_f16(in[i]);
        else if (kind == 2)
            out[i] = orc_round_bf16(in[i]);
        else
            out[i] = orc_round_f32(in[i]);
    }
}
