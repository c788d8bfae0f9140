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
 * Readings taken where the pages are silent:
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
 * all contiguous row-major.  q, k, v, r are binary16, binary32 or binary64
 * (dtype; binary64 serves the finite-difference pins of the backward),
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
#include <string.h>

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
        (dtype != ORACLE_F16 && dtype != ORACLE_F32 && dtype != ORACLE_F64))
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

/*
 * Backward pass of the ungated forward (r == NULL): given the gradient dO of
 * the outputs o, the gradients of q, k, v and of the gate logits z.  With
 * S_t as in the forward (S_0 = 0) and dS the gradient with respect to S_t,
 * taken along the scan from its last token back to its first:
 *     dS    <- dS + scale * q_t^T dO_t          (o_t = scale * q_t S_t)
 *     dq_t   = scale * dO_t S_t^T
 *     dk_t   = dS v_t^T ,   dv_t = k_t dS        (S_t = ... + k_t^T v_t)
 *     dgamma_t[c] = sum_j dS[c][j] S_{t-1}[c][j]  (S_t = Diag(gamma_t) S_{t-1} + ...)
 *     dz_t   = dgamma_t * gamma_t * (1 - sigmoid(z_t)) / tau
 *     dS    <- Diag(gamma_t) dS                  (on to S_{t-1})
 * (gamma = sigmoid(z)^(1/tau), so dgamma/dz = gamma (1 - sigmoid(z)) / tau.)
 * The states S_{t-1}, S_t of a block of 64 scan positions are recomputed
 * from a checkpoint taken every 64 positions in a first forward sweep.
 * dO is [B, L, NH, dv] in `dtype`; the four outputs are binary64 in the
 * layouts of q, k, v and z.  Returns 0, 1 (bad argument) or 2 (allocation).
 */
int gla_oracle_bwd(const void *q, const void *k, const void *v, const void *z, int zdtype,
                   const void *dout, int dtype, int B, int NH, int H, int W, int dk, int dv,
                   int dir, double tau, double scale, long unit_begin, long unit_end,
                   double *dq, double *dkk, double *dvv, double *dz)
{
    if (!q || !k || !v || !z || !dout || !dq || !dkk || !dvv || !dz || B < 1 || NH < 1 ||
        H < 1 || W < 1 || dk < 1 || dv < 1 || dir < 0 || dir > 3 || !(tau > 0.0) ||
        (dtype != ORACLE_F16 && dtype != ORACLE_F32 && dtype != ORACLE_F64) ||
        (zdtype != ORACLE_F32 && zdtype != ORACLE_F64))
        return 1;
    if (unit_begin < 0) unit_begin = 0;
    if (unit_end > (long)B * NH) unit_end = (long)B * NH;
    const long L = (long)H * W;
    const long BLK = 64;
    const long nblk = (L + BLK - 1) / BLK;
    const size_t SS = (size_t)dk * dv;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long unit = unit_begin; unit < unit_end; ++unit) {
        const long b = unit / NH, h = unit % NH;
        double *ck = calloc((size_t)(nblk + 1) * SS, sizeof(double)); /* ck[m]: state before block m */
        double *st = malloc(sizeof(double) * (size_t)(BLK + 1) * SS);  /* states of one block */
        double *dS = calloc(SS, sizeof(double));
        double *gm = malloc(sizeof(double) * (size_t)L * dk);          /* gamma, scan order */
        double *sg = malloc(sizeof(double) * (size_t)L * dk);          /* sigmoid(z), scan order */
        double *dot = malloc(sizeof(double) * dv);
        if (!ck || !st || !dS || !gm || !sg || !dot) {
            failed = 1;
            free(ck); free(st); free(dS); free(gm); free(sg); free(dot);
            continue;
        }
        /* forward sweep: gates and one checkpoint per block */
        double *S = ck; /* running state, copied into ck[m] at block starts */
        double *run = calloc(SS, sizeof(double));
        if (!run) { failed = 1; free(ck); free(st); free(dS); free(gm); free(sg); free(dot); continue; }
        for (long i = 0; i < L; ++i) {
            const long t = gla_oracle_scan_token(dir, i, H, W);
            const size_t rk = ((size_t)(b * L + t) * NH + h) * dk;
            const size_t rv = ((size_t)(b * L + t) * NH + h) * dv;
            if (i % BLK == 0) memcpy(S + (size_t)(i / BLK) * SS, run, sizeof(double) * SS);
            for (int c = 0; c < dk; ++c) {
                const double zc = load_elem(z, zdtype, rk + c);
                gm[i * dk + c] = exp(log_sigmoid(zc) / tau);
                sg[i * dk + c] = 1.0 / (1.0 + exp(-zc));
            }
            for (int c = 0; c < dk; ++c) {
                const double kc = load_elem(k, dtype, rk + c);
                for (int j = 0; j < dv; ++j)
                    run[(size_t)c * dv + j] = gm[i * dk + c] * run[(size_t)c * dv + j] +
                                              kc * load_elem(v, dtype, rv + j);
            }
        }
        free(run);
        /* backward sweep, block by block */
        for (long m = nblk - 1; m >= 0; --m) {
            const long i0 = m * BLK, i1 = (i0 + BLK < L) ? i0 + BLK : L;
            /* st[0] = state before i0; st[1 + (i - i0)] = S_i */
            memcpy(st, ck + (size_t)m * SS, sizeof(double) * SS);
            for (long i = i0; i < i1; ++i) {
                const long t = gla_oracle_scan_token(dir, i, H, W);
                const size_t rk = ((size_t)(b * L + t) * NH + h) * dk;
                const size_t rv = ((size_t)(b * L + t) * NH + h) * dv;
                const double *prev = st + (size_t)(i - i0) * SS;
                double *cur = st + (size_t)(i - i0 + 1) * SS;
                for (int c = 0; c < dk; ++c) {
                    const double kc = load_elem(k, dtype, rk + c);
                    for (int j = 0; j < dv; ++j)
                        cur[(size_t)c * dv + j] = gm[i * dk + c] * prev[(size_t)c * dv + j] +
                                                  kc * load_elem(v, dtype, rv + j);
                }
            }
            for (long i = i1 - 1; i >= i0; --i) {
                const long t = gla_oracle_scan_token(dir, i, H, W);
                const size_t rk = ((size_t)(b * L + t) * NH + h) * dk;
                const size_t rv = ((size_t)(b * L + t) * NH + h) * dv;
                const double *prev = st + (size_t)(i - i0) * SS;
                const double *cur = st + (size_t)(i - i0 + 1) * SS;
                for (int j = 0; j < dv; ++j) dot[j] = load_elem(dout, dtype, rv + j);
                /* dS += scale q^T dO */
                for (int c = 0; c < dk; ++c) {
                    const double qc = scale * load_elem(q, dtype, rk + c);
                    for (int j = 0; j < dv; ++j) dS[(size_t)c * dv + j] += qc * dot[j];
                }
                /* dq = scale dO S^T ; dk = dS v^T ; dgamma = rowsum(dS .* S_prev) */
                for (int c = 0; c < dk; ++c) {
                    double aq = 0.0, ak = 0.0, ag = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        aq += dot[j] * cur[(size_t)c * dv + j];
                        ak += dS[(size_t)c * dv + j] * load_elem(v, dtype, rv + j);
                        ag += dS[(size_t)c * dv + j] * prev[(size_t)c * dv + j];
                    }
                    dq[rk + c] = scale * aq;
                    dkk[rk + c] = ak;
                    dz[rk + c] = ag * gm[i * dk + c] * (1.0 - sg[i * dk + c]) / tau;
                }
                /* dv = k dS */
                for (int j = 0; j < dv; ++j) {
                    double a = 0.0;
                    for (int c = 0; c < dk; ++c)
                        a += load_elem(k, dtype, rk + c) * dS[(size_t)c * dv + j];
                    dvv[rv + j] = a;
                }
                /* on to S_{t-1} */
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j) dS[(size_t)c * dv + j] *= gm[i * dk + c];
            }
        }
        free(ck); free(st); free(dS); free(gm); free(sg); free(dot);
    }
    return failed ? 2 : 0;
}
