/*
 * dgrad_oracle.c -- plain, slow, fp64 CPU oracle for conv2d backward-data.
 *
 * TEST INFRASTRUCTURE. Only tests/, the smoke check and the CPU-baseline leg
 * of bench.py may load this library. The product path (convolution_backward_amd)
 * never calls it, shares no code, header, table or helper with it, and this
 * file includes nothing from the product.
 *
 * What it computes (the plain definition of dgrad, the operation named by
 * "[CUTLASS] Conv2d dgrad", apache/tvm PR #10110, and by cuDNN's
 * ConvolutionBackwardData in "Performance improvements by calling cuDNN API",
 * JuliaGPU/CUDA.jl PR #321):
 *
 *   The forward layer is a cross-correlation (no filter flip) with one
 *   stride s and one symmetric zero padding `pad` in both spatial dims:
 *     y[n,p,q,k] = sum_{r,t,c} x[n, p*s - pad + r, q*s - pad + t, c] * w[k,r,t,c]
 *   with P = floor((H + 2 pad - R)/s) + 1 and Q likewise from W and S.
 *   dgrad is its adjoint with respect to x:
 *     dx[n,h,w,c] = sum_{k,r,t} dy[n,p,q,k] * w[k,r,t,c]
 *   over the taps (r,t) for which h = p*s - pad + r and w = q*s - pad + t
 *   have an integer solution (p,q) with 0 <= p < P and 0 <= q < Q.
 *   Taps without such a solution contribute nothing; positions that no tap
 *   reaches are exactly 0.
 *
 *   Optional fused epilogue: out = acc * g(z[n,h,w,c]), where z is the saved
 *   pre-activation. g = relu'(z) = [z > 0], or g = hardswish'(z) with
 *   hardswish(z) = z * min(max(z + 3, 0), 6) / 6 (the activation named in the
 *   Bolt paper notes, KuangjuX/Paper-reading #28, "Insights"), whose
 *   derivative is 0 below -3, z/3 + 1/2 on the closed interval [-3, 3], and 1
 *   above 3. The closed interval (values -1/2 and 3/2 at the kinks) is a
 *   reading: the pages print no formula.
 *
 * Arithmetic: inputs are fp16 bit patterns decoded exactly to fp64; the sum
 * and the epilogue are evaluated in fp64 and returned unrounded. A separate
 * round-to-nearest-even fp64 -> fp16 encoder serves the bit-exact tests.
 *
 * Layouts: dy [N][P][Q][K], w [K][R][S][C], z and dx [N][H][W][C], all
 * C-contiguous. Output rows are linear pixel indices (n*H + h)*W + w.
 *
 * The file also holds the filter gradient (wgrad) of the same layer and the
 * forward layer with its bias + hardswish epilogue, below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_EPI_NONE 0
#define ORACLE_EPI_DRELU 1
#define ORACLE_EPI_DHARDSWISH 2

/* ---- fp16 <-> fp64, written from the IEEE 754 binary16 format ---------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_half_to_double(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(frac + 1024), expo - 25);  /* (1 + frac/1024) * 2^(expo-15) */
    return sign ? -mag : mag;
}

/* Round an fp64 value to the nearest binary16 value, ties to even. */
uint16_t oracle_double_to_half_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7e00;
    /* 65520 is halfway between the largest finite half (65504) and 2^16;
     * the tie goes to the even neighbour 2^16, which overflows to infinity. */
    if (a >= 65520.0)
        return sign | 0x7c00;
    /* spacing of binary16 values around a */
    double quantum;
    if (a < ldexp(1.0, -14)) {
        quantum = ldexp(1.0, -24);
    } else {
        int e;
        frexp(a, &e);                   /* a = f * 2^e, f in [0.5, 1) */
        quantum = ldexp(1.0, e - 11);   /* 2^(e-1) has 10 fraction bits below it */
    }
    double n = nearbyint(a / quantum); /* exact division by a power of two; ties to even */
    double v = n * quantum;
    if (v < ldexp(1.0, -14))
        return sign | (uint16_t)n;      /* subnormal (n == 1024 encodes 2^-14 itself) */
    int e;
    double f = frexp(v, &e);            /* v = f * 2^e */
    int biased = e - 1 + 15;
    if (biased >= 31)
        return sign | 0x7c00;
    int frac = (int)(f * 2048.0) - 1024;
    return sign | (uint16_t)(biased << 10) | (uint16_t)frac;
}

/* ---- the epilogue factor g(z) ------------------------------------------ */

double oracle_relu_grad(double z)
{
    return z > 0.0 ? 1.0 : 0.0;
}

double oracle_hardswish_grad(double z)
{
    if (z < -3.0)
        return 0.0;
    if (z > 3.0)
        return 1.0;
    return z / 3.0 + 0.5;
}

static double epilogue_factor(int epi, double z)
{
    if (epi == ORACLE_EPI_DRELU)
        return oracle_relu_grad(z);
    if (epi == ORACLE_EPI_DHARDSWISH)
        return oracle_hardswish_grad(z);
    return 1.0;
}

/* ---- shapes ------------------------------------------------------------- */

/* Forward output extent along one spatial dim; < 1 means no valid output. */
int oracle_out_extent(int in, int filt, int stride, int pad)
{
    if (stride < 1)
        return 0;
    int span = in + 2 * pad - filt;
    if (span < 0)
        return 0;
    return span / stride + 1;
}

static int check_args(int N, int H, int W, int C, int K, int R, int S,
                      int stride, int pad, int epi, const void* z)
{
    if (N < 1 || H < 1 || W < 1 || C < 1 || K < 1 || R < 1 || S < 1)
        return 1;
    if (stride < 1 || pad < 0)
        return 1;
    if (oracle_out_extent(H, R, stride, pad) < 1 || oracle_out_extent(W, S, stride, pad) < 1)
        return 1;
    if (epi < 0 || epi > 2 || (epi != ORACLE_EPI_NONE && z == NULL))
        return 1;
    return 0;
}

/* ---- dgrad, one output pixel at a time ---------------------------------- */

/*
 * For each requested pixel (n,h,w): walk every filter tap (r,t), keep it when
 * h + pad - r and w + pad - t are non-negative multiples of the stride whose
 * quotients p, q fall inside [0,P) x [0,Q), and accumulate
 * dy[n,p,q,k] * w[k,r,t,c] over k for all c. Then apply the epilogue.
 *
 * rows: linear pixel indices (n*H + h)*W + w; out: [nrows][C] fp64.
 * Returns 0 on success, 1 on invalid arguments, 2 on allocation failure.
 */
int oracle_dgrad_rows(const uint16_t* dy, const uint16_t* wt, const uint16_t* z,
                      int N, int H, int W, int C, int K, int R, int S,
                      int stride, int pad, int epi,
                      const int64_t* rows, int64_t nrows, double* out, int nthreads)
{
    if (check_args(N, H, W, C, K, R, S, stride, pad, epi, z))
        return 1;
    if (nrows < 0 || (nrows > 0 && (rows == NULL || out == NULL)) || dy == NULL || wt == NULL)
        return 1;
    const int P = oracle_out_extent(H, R, stride, pad);
    const int Q = oracle_out_extent(W, S, stride, pad);
    const int64_t npix = (int64_t)N * H * W;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= npix)
            return 1;

    /* decode table for every fp16 pattern, and the filter decoded once */
    double* lut = (double*)malloc(sizeof(double) * 65536);
    const int64_t wcount = (int64_t)K * R * S * C;
    double* wd = (double*)malloc(sizeof(double) * (size_t)wcount);
    if (!lut || !wd) {
        free(lut);
        free(wd);
        return 2;
    }
    for (int b = 0; b < 65536; ++b)
        lut[b] = oracle_half_to_double((uint16_t)b);
    for (int64_t i = 0; i < wcount; ++i)
        wd[i] = lut[wt[i]];

    if (nthreads < 1)
        nthreads = omp_get_max_threads();
    int failed = 0;

#pragma omp parallel num_threads(nthreads)
    {
        double* acc = (double*)malloc(sizeof(double) * (size_t)C);
        if (!acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int64_t it = 0; it < nrows; ++it) {
            if (!acc)
                continue;
            const int64_t pix = rows[it];
            const int n = (int)(pix / ((int64_t)H * W));
            const int h = (int)((pix / W) % H);
            const int x = (int)(pix % W);
            for (int c = 0; c < C; ++c)
                acc[c] = 0.0;
            for (int r = 0; r < R; ++r) {
                const int a = h + pad - r;          /* = p * stride */
                if (a < 0 || a % stride != 0)
                    continue;
                const int p = a / stride;
                if (p >= P)
                    continue;
                for (int t = 0; t < S; ++t) {
                    const int b = x + pad - t;      /* = q * stride */
                    if (b < 0 || b % stride != 0)
                        continue;
                    const int q = b / stride;
                    if (q >= Q)
                        continue;
                    const uint16_t* dyrow = dy + (((int64_t)n * P + p) * Q + q) * K;
                    for (int k = 0; k < K; ++k) {
                        const double d = lut[dyrow[k]];
                        const double* wrow = wd + (((int64_t)k * R + r) * S + t) * C;
                        for (int c = 0; c < C; ++c)
                            acc[c] += d * wrow[c];
                    }
                }
            }
            double* o = out + it * (int64_t)C;
            if (epi == ORACLE_EPI_NONE) {
                for (int c = 0; c < C; ++c)
                    o[c] = acc[c];
            } else {
                const uint16_t* zrow = z + pix * (int64_t)C;
                for (int c = 0; c < C; ++c)
                    o[c] = acc[c] * epilogue_factor(epi, lut[zrow[c]]);
            }
        }
        free(acc);
    }
    free(lut);
    free(wd);
    return failed ? 2 : 0;
}

/* Every pixel, in order: out is [N][H][W][C] fp64. */
int oracle_dgrad_full(const uint16_t* dy, const uint16_t* wt, const uint16_t* z,
                      int N, int H, int W, int C, int K, int R, int S,
                      int stride, int pad, int epi, double* out, int nthreads)
{
    const int64_t npix = (int64_t)N * H * W;
    if (npix < 1)
        return 1;
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)npix);
    if (!rows)
        return 2;
    for (int64_t i = 0; i < npix; ++i)
        rows[i] = i;
    int rc = oracle_dgrad_rows(dy, wt, z, N, H, W, C, K, R, S, stride, pad, epi,
                               rows, npix, out, nthreads);
    free(rows);
    return rc;
}

/* ---- wgrad, one filter row at a time ------------------------------------ */

/*
 * The gradient of the same forward layer with respect to its filter (the
 * "wgrad" that "[CUTLASS] Conv2d dgrad", apache/tvm PR #10110, defers):
 *   dw[k,r,t,c] = sum over n,p,q of dy[n,p,q,k] * x[n, p*s - pad + r, q*s - pad + t, c],
 * where an input position outside the image (padding) contributes zero.
 *
 * For each requested filter row (k,r,t): walk every dy position (n,p,q),
 * keep it when the input position is inside the image, and accumulate
 * dy[n,p,q,k] * x[n,h,w,c] over all c. When abs_out is not NULL it receives
 * the sum of |dy * x| (the scale of the rounding error a float sum can make).
 *
 * rows: linear filter-row indices (k*R + r)*S + t; out, abs_out: [nrows][C].
 * Returns 0 on success, 1 on invalid arguments, 2 on allocation failure.
 */
int oracle_wgrad_rows(const uint16_t* dy, const uint16_t* x,
                      int N, int H, int W, int C, int K, int R, int S,
                      int stride, int pad,
                      const int64_t* rows, int64_t nrows, double* out, double* abs_out, int nthreads)
{
    if (check_args(N, H, W, C, K, R, S, stride, pad, ORACLE_EPI_NONE, NULL))
        return 1;
    if (nrows < 0 || (nrows > 0 && (rows == NULL || out == NULL)) || dy == NULL || x == NULL)
        return 1;
    const int P = oracle_out_extent(H, R, stride, pad);
    const int Q = oracle_out_extent(W, S, stride, pad);
    const int64_t nfrows = (int64_t)K * R * S;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= nfrows)
            return 1;
    double* lut = (double*)malloc(sizeof(double) * 65536);
    if (!lut)
        return 2;
    for (int b = 0; b < 65536; ++b)
        lut[b] = oracle_half_to_double((uint16_t)b);
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
    int failed = 0;

#pragma omp parallel num_threads(nthreads)
    {
        double* acc = (double*)malloc(sizeof(double) * (size_t)C * 2);
        if (!acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < nrows; ++it) {
            if (!acc)
                continue;
            const int64_t fr = rows[it];
            const int k = (int)(fr / ((int64_t)R * S));
            const int r = (int)((fr / S) % R);
            const int t = (int)(fr % S);
            double* sum = acc;
            double* mag = acc + C;
            for (int c = 0; c < C; ++c)
                sum[c] = mag[c] = 0.0;
            for (int n = 0; n < N; ++n)
                for (int p = 0; p < P; ++p) {
                    const int h = p * stride - pad + r;
                    if (h < 0 || h >= H)
                        continue;
                    for (int q = 0; q < Q; ++q) {
                        const int w = q * stride - pad + t;
                        if (w < 0 || w >= W)
                            continue;
                        const double d = lut[dy[(((int64_t)n * P + p) * Q + q) * K + k]];
                        const uint16_t* xrow = x + (((int64_t)n * H + h) * W + w) * C;
                        for (int c = 0; c < C; ++c) {
                            const double v = d * lut[xrow[c]];
                            sum[c] += v;
                            mag[c] += fabs(v);
                        }
                    }
                }
            for (int c = 0; c < C; ++c) {
                out[it * (int64_t)C + c] = sum[c];
                if (abs_out)
                    abs_out[it * (int64_t)C + c] = mag[c];
            }
        }
        free(acc);
    }
    free(lut);
    return failed ? 2 : 0;
}

/* ---- forward conv + bias + hardswish, one output pixel at a time --------- */

/* hardswish(z) = z * min(max(z + 3, 0), 6) / 6, the activation of the Bolt
 * paper notes' Conv2D + BiasAdd + Hardswish fusion. */
double oracle_hardswish(double z)
{
    double g = z + 3.0;
    if (g < 0.0)
        g = 0.0;
    if (g > 6.0)
        g = 6.0;
    return z * g / 6.0;
}

/*
 * The forward layer itself with the fused bias + activation epilogue that
 * the Bolt notes describe (Conv2D + BiasAdd + Hardswish):
 *   z[n,p,q,k] = bias[k] + sum over r,t,c of x[n, p*s - pad + r, q*s - pad + t, c] * w[k,r,t,c]
 *   y = hardswish(z) (act = 1) or y = z (act = 0),
 * where input positions in the padding contribute zero.
 *
 * rows: linear output pixel indices (n*P + p)*Q + q; z_out, y_out: [nrows][K]
 * (either may be NULL). Returns 0 on success, 1 on invalid arguments, 2 on
 * allocation failure.
 */
int oracle_forward_rows(const uint16_t* x, const uint16_t* wt, const uint16_t* bias,
                        int N, int H, int W, int C, int K, int R, int S,
                        int stride, int pad, int act,
                        const int64_t* rows, int64_t nrows, double* z_out, double* y_out, int nthreads)
{
    if (check_args(N, H, W, C, K, R, S, stride, pad, ORACLE_EPI_NONE, NULL) || act < 0 || act > 1)
        return 1;
    if (nrows < 0 || (nrows > 0 && rows == NULL) || x == NULL || wt == NULL || bias == NULL)
        return 1;
    const int P = oracle_out_extent(H, R, stride, pad);
    const int Q = oracle_out_extent(W, S, stride, pad);
    const int64_t nout = (int64_t)N * P * Q;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= nout)
            return 1;
    double* lut = (double*)malloc(sizeof(double) * 65536);
    if (!lut)
        return 2;
    for (int b = 0; b < 65536; ++b)
        lut[b] = oracle_half_to_double((uint16_t)b);
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
    int failed = 0;

#pragma omp parallel num_threads(nthreads)
    {
        double* acc = (double*)malloc(sizeof(double) * (size_t)K);
        if (!acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int64_t it = 0; it < nrows; ++it) {
            if (!acc)
                continue;
            const int64_t pix = rows[it];
            const int n = (int)(pix / ((int64_t)P * Q));
            const int p = (int)((pix / Q) % P);
            const int q = (int)(pix % Q);
            for (int k = 0; k < K; ++k)
                acc[k] = lut[bias[k]];
            for (int r = 0; r < R; ++r) {
                const int h = p * stride - pad + r;
                if (h < 0 || h >= H)
                    continue;
                for (int t = 0; t < S; ++t) {
                    const int w = q * stride - pad + t;
                    if (w < 0 || w >= W)
                        continue;
                    const uint16_t* xrow = x + (((int64_t)n * H + h) * W + w) * C;
                    for (int k = 0; k < K; ++k) {
                        const uint16_t* wrow = wt + (((int64_t)k * R + r) * S + t) * C;
                        double sum = 0.0;
                        for (int c = 0; c < C; ++c)
                            sum += lut[xrow[c]] * lut[wrow[c]];
                        acc[k] += sum;
                    }
                }
            }
            for (int k = 0; k < K; ++k) {
                if (z_out)
                    z_out[it * (int64_t)K + k] = acc[k];
                if (y_out)
                    y_out[it * (int64_t)K + k] = act ? oracle_hardswish(acc[k]) : acc[k];
            }
        }
        free(acc);
    }
    free(lut);
    return failed ? 2 : 0;
}

/*
 * Two dgrad steps of a bottleneck, one after the other: the chain that the
 * persistent kernel fusion of the Bolt paper notes (KuangjuX/Paper-reading
 * #28, "Persistent kernel (GEMM/Conv) fusion") runs as one kernel. Its
 * arithmetic is that of the two separate calls:
 *
 *   t[c]   = fp16_RNE( dgrad(dy, w1; stride 1, pad)[pixel, c] * g(z[pixel, c]) )
 *   dx[ci] = sum over c < Cm of t[c] * w2[c][ci]        (fp64, unrounded)
 *
 * w1 [K][R][S][Cm] is the RxS filter, w2 [Cm][C] the 1x1 filter of the
 * convolution in front of it (its dgrad is a plain product over channels).
 * t is rounded once to fp16 because the unfused pair stores it in fp16
 * between the calls (a reading: the notes fuse without saying what the
 * intermediate precision is). mag (may be NULL): sum over c of
 * |t[c]| * |w2[c][ci]|, the scale of the rounding error of dx.
 *
 * rows: linear pixel indices (n*H + h)*W + w; out, mag: [nrows][C].
 * Returns 0 on success, 1 on invalid arguments, 2 on allocation failure.
 */
int oracle_chain_rows(const uint16_t* dy, const uint16_t* w1, const uint16_t* z, const uint16_t* w2,
                      int N, int H, int W, int Cm, int K, int R, int S, int pad, int C, int epi,
                      const int64_t* rows, int64_t nrows, double* out, double* mag, int nthreads)
{
    if (C < 1 || Cm < 1 || w2 == NULL || nrows < 0 || (nrows > 0 && out == NULL))
        return 1;
    double* t = (double*)malloc(sizeof(double) * (size_t)(nrows * Cm + 1));
    double* w2d = (double*)malloc(sizeof(double) * (size_t)Cm * (size_t)C);
    if (!t || !w2d) {
        free(t);
        free(w2d);
        return 2;
    }
    const int rc = oracle_dgrad_rows(dy, w1, z, N, H, W, Cm, K, R, S, 1, pad, epi, rows, nrows, t, nthreads);
    if (rc != 0) {
        free(t);
        free(w2d);
        return rc;
    }
    for (int64_t i = 0; i < (int64_t)Cm * C; ++i)
        w2d[i] = oracle_half_to_double(w2[i]);
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 8)
    for (int64_t it = 0; it < nrows; ++it) {
        double* o = out + it * (int64_t)C;
        double* m = mag ? mag + it * (int64_t)C : NULL;
        for (int ci = 0; ci < C; ++ci) {
            o[ci] = 0.0;
            if (m)
                m[ci] = 0.0;
        }
        for (int c = 0; c < Cm; ++c) {
            const double tc = oracle_half_to_double(oracle_double_to_half_rne(t[it * (int64_t)Cm + c]));
            const double* wrow = w2d + (int64_t)c * C;
            for (int ci = 0; ci < C; ++ci) {
                o[ci] += tc * wrow[ci];
                if (m)
                    m[ci] += fabs(tc) * fabs(wrow[ci]);
            }
        }
    }
    free(t);
    free(w2d);
    return 0;
}

/* RNE fp16 encoding of an fp64 array (bit-exact comparisons). */
void oracle_round_to_half(const double* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_double_to_half_rne(in[i]);
}

int oracle_max_threads(void)
{
    return omp_get_max_threads();
}
