/*
 * gla_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU reference for the forward pass of key-only gated
 * linear attention as defined in "GTR: Gated Token Recurrence for Efficient
 * Dense Prediction" (paper, Section 2.1).  Only tests/, the smoke check and
 * the CPU-baseline leg of the benchmark may load this file's library.  It
 * shares no code, header or table with the HIP implementation.
 *
 * What it computes, per (batch b, head h), token by token along the scan:
 *   gamma_t = sigmoid(z_t)^(1/tau)                  (Sec. 2.1, retention gate)
 *   S_t     = Diag(gamma_t) S_{t-1} + k_t^T v_t,  S_0 = 0   (Sec. 2.1)
 *   o_t     = scale * q_t S_t,   scale = d_k^(-1/2) by default (Sec. 2.1)
 *   optional output gate (Sec. 2.1, output-gate paragraph):
 *   u_t     = SiLU(r_t) (.) w (.) o_t / sqrt(mean(o_t^2) + eps)
 * The scan visits the H x W patch grid in one of four directions and the
 * result is written back at each token's original grid position (Sec. 2.1,
 * scan-direction paragraph and Figure 2).
 *
 * Readings taken where the pages are silent (each is listed in the design doc):
 *   - token t = h*W + w (row-major grid); left-to-right is raster order,
 *     right-to-left is that order reversed, top-to-bottom is column-major
 *     order, bottom-to-top is column-major order reversed;
 *   - one continuous scan of L = H*W tokens, decay applied before the add,
 *     o_t uses the updated S_t;
 *   - r is the pre-activation x W_r, the SiLU is applied here;
 *   - RMSNorm is over d_v per head, eps inside the square root, one weight
 *     vector of length d_v shared by all heads (NULL means ones).
 *
 * Layouts: q, k, z are [B, L, NH, dk]; v, r, out are [B, L, NH, dv];
 * all contiguous row-major.  q, k, v, r are binary16 or binary32 (dtype),
 * z is binary32 (gla_oracle_fwd) or binary64 (gla_oracle_fwd_zd), w is
 * binary32, out is binary64.
 *
 * The gate logits themselves come from a low-rank projection of the block
 * input x (Sec. 2.1, retention gate, rank r = 16):
 *   z_t = (x_t W1) W2 + b,  W1: d_model x rank,  W2: rank x (NH*dk)
 * computed by gla_oracle_gate_logits in binary64.  Reading taken where the
 * pages are silent: the first factor is shared by all heads and the second
 * factor and bias hold every head's d_k columns side by side (head h owns
 * columns h*dk .. h*dk + dk - 1), as in GLA's low-rank gate.  Both factors
 * are stored transposed, as the weights of linear layers: w1 is
 * [rank][d_model], w2 is [NH*dk][rank].
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_F16 0
#define ORACLE_F32 1
#define ORACLE_F64 2

/* IEEE 754 binary16 -> double, from the format's definition: 1 sign bit,
 * 5 exponent bits with bias 15, 10 fraction bits. */
double gla_oracle_half_to_double(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 31;
    int frac = bits & 1023;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);              /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
    return sign ? -mag : mag;
}

static double load_elem(const void *base, int dtype, size_t idx)
{
    if (dtype == ORACLE_F16)
        return gla_oracle_half_to_double(((const uint16_t *)base)[idx]);
    if (dtype == ORACLE_F64)
        return ((const double *)base)[idx];
    return (double)((const float *)base)[idx];
}

/* log(sigmoid(x)), evaluated without overflow: for x >= 0 it is
 * -log(1 + e^-x); for x < 0 it is x - log(1 + e^x). */
static double log_sigmoid(double x)
{
    if (x >= 0.0)
        return -log1p(exp(-x));
    return x - log1p(exp(x));
}

/* SiLU(x) = x * sigmoid(x). */
static double silu(double x)
{
    return x / (1.0 + exp(-x));
}

/* Scan position i -> original token index, for the four directions. */
long gla_oracle_scan_token(int dir, long i, long H, long W)
{
    long L = H * W;
    long j;
    switch (dir) {
    case 0: return i;                               /* left-to-right */
    case 1: return L - 1 - i;                       /* right-to-left */
    case 2: return (i % H) * W + i / H;             /* top-to-bottom */
    case 3: j = L - 1 - i; return (j % H) * W + j / H; /* bottom-to-top */
    default: return -1;
    }
}

/*
 * Forward pass over the (b, h) units [unit_begin, unit_end) of the B*NH
 * units (unit = b*NH + h); output rows of other units are left untouched.
 * r == NULL: out = o.  w == NULL: RMSNorm weight of ones.
 * Returns 0 on success, 1 on a bad argument, 2 on allocation failure.
 */
static int fwd_impl(const void *q, const void *k, const void *v, const void *z, int zdtype,
                    const void *r, const float *w, int dtype,
                    int B, int NH, int H, int W, int dk, int dv, int dir,
                    double tau, double scale, double eps,
                    long unit_begin, long unit_end, double *out)
{
    if (!q || !k || !v || !z || !out || B < 1 || NH < 1 || H < 1 || W < 1 ||
        dk < 1 || dv < 1 || dir < 0 || dir > 3 || !(tau > 0.0) ||
        (dtype != ORACLE_F16 && dtype != ORACLE_F32))
        return 1;
    if (unit_begin < 0) unit_begin = 0;
    if (unit_end > (long)B * NH) unit_end = (long)B * NH;
    const long L = (long)H * W;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long unit = unit_begin; unit < unit_end; ++unit) {
        const long b = unit / NH, h = unit % NH;
        double *S = calloc((size_t)dk * dv, sizeof(double));
        double *qt = malloc(sizeof(double) * dk), *kt = malloc(sizeof(double) * dk);
        double *gt = malloc(sizeof(double) * dk), *vt = malloc(sizeof(double) * dv);
        double *ot = malloc(sizeof(double) * dv);
        if (!S || !qt || !kt || !gt || !vt || !ot) {
            failed = 1;
            free(S); free(qt); free(kt); free(gt); free(vt); free(ot);
            continue;
        }
        for (long i = 0; i < L; ++i) {
            const long t = gla_oracle_scan_token(dir, i, H, W);
            const size_t rk = ((size_t)(b * L + t) * NH + h) * dk;
            const size_t rv = ((size_t)(b * L + t) * NH + h) * dv;
            for (int c = 0; c < dk; ++c) {
                qt[c] = load_elem(q, dtype, rk + c);
                kt[c] = load_elem(k, dtype, rk + c);
                gt[c] = exp(log_sigmoid(load_elem(z, zdtype, rk + c)) / tau);
            }
            for (int j = 0; j < dv; ++j)
                vt[j] = load_elem(v, dtype, rv + j);
            /* S_t = Diag(gamma_t) S_{t-1} + k_t^T v_t */
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j)
                    S[(size_t)c * dv + j] = gt[c] * S[(size_t)c * dv + j] + kt[c] * vt[j];
            /* o_t = scale * q_t S_t */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int c = 0; c < dk; ++c)
                    acc += qt[c] * S[(size_t)c * dv + j];
                ot[j] = scale * acc;
            }
            if (r) {
                double ms = 0.0;
                for (int j = 0; j < dv; ++j)
                    ms += ot[j] * ot[j];
                ms /= (double)dv;
                const double inv = 1.0 / sqrt(ms + eps);
                for (int j = 0; j < dv; ++j) {
                    const double wj = w ? (double)w[j] : 1.0;
                    out[rv + j] = silu(load_elem(r, dtype, rv + j)) * wj * ot[j] * inv;
                }
            } else {
                for (int j = 0; j < dv; ++j)
                    out[rv + j] = ot[j];
            }
        }
        free(S); free(qt); free(kt); free(gt); free(vt); free(ot);
    }
    return failed ? 2 : 0;
}

/* Forward pass with binary32 gate logits z. */
int gla_oracle_fwd(const void *q, const void *k, const void *v, const float *z,
                   const void *r, const float *w, int dtype,
                   int B, int NH, int H, int W, int dk, int dv, int dir,
                   double tau, double scale, double eps,
                   long unit_begin, long unit_end, double *out)
{
    return fwd_impl(q, k, v, z, ORACLE_F32, r, w, dtype, B, NH, H, W, dk, dv, dir,
                    tau, scale, eps, unit_begin, unit_end, out);
}

/* Forward pass with binary64 gate logits z (for logits computed by
 * gla_oracle_gate_logits, used without rounding). */
int gla_oracle_fwd_zd(const void *q, const void *k, const void *v, const double *z,
                      const void *r, const float *w, int dtype,
                      int B, int NH, int H, int W, int dk, int dv, int dir,
                      double tau, double scale, double eps,
                      long unit_begin, long unit_end, double *out)
{
    return fwd_impl(q, k, v, z, ORACLE_F64, r, w, dtype, B, NH, H, W, dk, dv, dir,
                    tau, scale, eps, unit_begin, unit_end, out);
}

/*
 * Gate logits of `tokens` tokens from the low-rank projection (Sec. 2.1,
 * retention gate):
 *   hproj = x_t W1            (rank values;  W1[m][j] = w1[j * d_model + m])
 *   z_t   = hproj W2 + b      (nout values;  W2[j][o] = w2[o * rank + j])
 * x: [tokens][d_model] and w1 in `dtype` (binary16 or binary32), w2 and bias
 * binary32 (bias NULL means zeros), z: [tokens][nout] binary64.  With
 * nout = NH * dk, z read as [B, L, NH, dk] gives every head its columns.
 * Returns 0 on success, 1 on a bad argument, 2 on allocation failure.
 */
int gla_oracle_gate_logits(const void *x, const void *w1, const float *w2, const float *bias,
                           int dtype, long tokens, int d_model, int rank, int nout, double *z)
{
    if (!x || !w1 || !w2 || !z || tokens < 0 || d_model < 1 || rank < 1 || nout < 1 ||
        (dtype != ORACLE_F16 && dtype != ORACLE_F32))
        return 1;
    int failed = 0;
#pragma omp parallel for schedule(static) reduction(| : failed)
    for (long t = 0; t < tokens; ++t) {
        double *hp = malloc(sizeof(double) * rank);
        if (!hp) {
            failed = 1;
            continue;
        }
        for (int j = 0; j < rank; ++j) {
            double acc = 0.0;
            for (int m = 0; m < d_model; ++m)
                acc += load_elem(x, dtype, (size_t)t * d_model + m) *
                       load_elem(w1, dtype, (size_t)j * d_model + m);
            hp[j] = acc;
        }
        for (int o = 0; o < nout; ++o) {
            double acc = bias ? (double)bias[o] : 0.0;
            for (int j = 0; j < rank; ++j)
                acc += hp[j] * (double)w2[(size_t)o * rank + j];
            z[(size_t)t * nout + o] = acc;
        }
        free(hp);
    }
    return failed ? 2 : 0;
}
