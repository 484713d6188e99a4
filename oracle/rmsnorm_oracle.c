/*
 * Plain fp64 CPU reference for RMSNorm forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the GPU library, and neither includes the other.
 *
 * What it computes (the plain definition; every stored input is widened
 * exactly to double, eps and offset arrive as float and are widened exactly):
 *
 *   forward   (RMSNorm; Liger-Kernel PR #1388 "Summary" and FlyDSL PR #855
 *              "Implementation": per-row two-pass RMS math with eps and offset
 *              as runtime scalars)
 *       ms_i   = (1/N) sum_j v_ij^2
 *       rstd_i = 1 / sqrt(ms_i + eps)
 *       y_ij   = v_ij * rstd_i * (gamma_j + offset)
 *     One rounding to the storage type happens after the gamma multiply
 *     ("llama mode" of Liger-Kernel PR #1388 "Results", read as fp32 compute
 *     and a single cast of the final product).
 *
 *   fused residual add (FlyDSL PR #855 "Hybrid atomic / two-stage backward":
 *              fused-add is a specialization of the same op)
 *       h_ij = round_T(x_ij + r_ij);  (y, rstd) = forward(h)
 *
 *   backward  (chain rule of the forward; rstd recomputed here from v)
 *       w_j   = gamma_j + offset,  g_ij = dy_ij * w_j,  xhat_ij = v_ij * rstd_i
 *       c_i   = (1/N) sum_j g_ij * xhat_ij
 *       dx_ij = rstd_i * (g_ij - xhat_ij * c_i)      [+ dh_ij, fused-add]
 *       dgamma_j = sum_i dy_ij * xhat_ij              (fp32 accumulation and a
 *                  write in the parameter dtype: FlyDSL PR #855
 *                  "512-thread vec8 fast path" and "Hybrid ... backward")
 *     The fused-add backward adds the gradient flowing into the residual
 *     output, dh, to dx; dx is the residual gradient (FlyDSL PR #855,
 *     "Hybrid atomic / two-stage backward" and "Fused-add RMSNorm backward").
 *
 * Non-affine RMSNorm (no gamma; Liger-Kernel PR #1388 "Validation" tests the
 * affine and non-affine ops): gamma == NULL means w_j = 1, and offset must be 0.
 *
 * fp8 output (TransformerEngine PR #583: the normalization kernel's output
 * type may be float8 E4M3, used by its fp8 training runs).  The page fixes
 * only the type; the readings taken, after the usual delayed-scaling use of
 * such an output:
 *     t_ij   = y_ij * scale              (scale: the caller's float32 factor)
 *     code_ij = E4M3(t_ij)               nearest, ties to even, saturating
 *     amax   = max_ij |y_ij|             (before scaling; NaN if any y_ij is NaN)
 * E4M3 is the OCP "FN" format: 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, largest finite 448 = 1.75 * 2^8, smallest
 * normal 2^-6, subnormals m * 2^-9 (m = 1..7); codes 0x7F / 0xFF are NaN.
 *
 * LayerNorm on the same machinery (TransformerEngine PR #583: matching tuned
 * configurations are registered for LayerNorm).  The page gives no formula;
 * the standard LayerNorm is taken, with the same eps, offset and fused-add
 * conventions as RMSNorm above and an optional bias beta:
 *       mu_i   = (1/N) sum_j v_ij
 *       var_i  = (1/N) sum_j (v_ij - mu_i)^2
 *       rstd_i = 1 / sqrt(var_i + eps)
 *       xhat_ij = (v_ij - mu_i) * rstd_i
 *       y_ij   = xhat_ij * (gamma_j + offset) + beta_j
 *   backward (chain rule), g = dy * w:
 *       dx_ij  = rstd_i * (g_ij - mean_j(g) - xhat_ij * mean_j(g * xhat))  [+ dh_ij]
 *       dgamma_j = sum_i dy_ij * xhat_ij,   dbeta_j = sum_i dy_ij
 *
 * Rounding to a storage type is round-to-nearest, ties to even (FlyDSL PR #855,
 * "512-thread vec8 fast path": software RNE / hardware conversion).
 * Storage types: float32, bfloat16, float64 and IEEE binary16 (FlyDSL PR #855
 * "512-thread vec8 fast path": the 128-bit path serves FP16 and BF16, and the
 * validation coverage there lists FP32, FP16 and BF16; binary16 takes the same
 * single nearest-even rounding of each output).
 *
 * Parallelism: OpenMP over independent rows (forward, dx) and over independent
 * column ranges (dgamma, each column summed over rows in row order).  No sum is
 * reordered.
 *
 * Pins (tests/test_oracle_pins.py; the fp8 encoder also against a
 * brute-force nearest-code search and torch's float8_e4m3fn cast): finite differences, the RMS invariant, the
 * sum_j v_j dx_j identity, closed forms (N = 1, constant rows, eps = 0 scale
 * invariance, gamma/offset equivalence, fused-add reductions), the fp64
 * torch.nn.functional.rms_norm with autograd, hand-worked fixtures under
 * tests/golden/, and brute-force nearest-value rounding.
 */

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2, ORACLE_F16 = 3 };
enum { ORACLE_OK = 0, ORACLE_EINVAL = 1, ORACLE_ENOMEM = 2 };

static int dtype_ok(int dt) { return dt == ORACLE_F32 || dt == ORACLE_BF16 || dt == ORACLE_F64 || dt == ORACLE_F16; }

/* Value of an IEEE binary16 bit pattern: 1 sign bit, 5 exponent bits with
 * bias 15, 10 fraction bits; exponent field 0 holds the subnormals
 * f * 2^-24, field 31 infinity (f = 0) and NaN. */
static double f16_value(uint16_t b)
{
    const double sign = (b & 0x8000u) ? -1.0 : 1.0;
    const int field = (b >> 10) & 0x1F;
    const int frac = b & 0x3FF;
    if (field == 0x1F)
        return frac ? NAN : sign * INFINITY;
    if (field == 0)
        return sign * ldexp((double)frac, -24);
    return sign * ldexp((double)(1024 + frac), field - 25);
}

/* Widen one stored element to double (exact for every storage type). */
static double load_elem(int dt, const void *base, int64_t i)
{
    if (dt == ORACLE_F64)
        return ((const double *)base)[i];
    if (dt == ORACLE_F32)
        return (double)((const float *)base)[i];
    if (dt == ORACLE_F16)
        return f16_value(((const uint16_t *)base)[i]);
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Nearest bf16 to v, ties to even, as a bit pattern.
 * bf16 keeps 8 significant bits and float32's exponent range; below 2^-126 the
 * spacing is fixed at 2^-133.  v / spacing is an exact power-of-two scaling,
 * so nearbyint (ties to even in the default rounding mode) gives the answer. */
static uint16_t bf16_bits_from_double(double v)
{
    if (isnan(v))
        return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    if (isinf(v) || v == 0.0) {
        float f = (float)v;
        uint32_t b;
        memcpy(&b, &f, sizeof b);
        return (uint16_t)(b >> 16);
    }
    int e;
    frexp(fabs(v), &e); /* |v| = m * 2^e with m in [0.5, 1), so floor(log2|v|) = e - 1 */
    int q = e - 1;
    if (q < -126)
        q = -126;
    double spacing = ldexp(1.0, q - 7);
    double r = nearbyint(v / spacing) * spacing;
    if (fabs(r) >= 0x1p128) /* rounded past the largest finite bf16 */
        return (uint16_t)(r < 0 ? 0xFF80u : 0x7F80u);
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    return (uint16_t)(b >> 16);
}

/* Nearest binary16 to v, ties to even, as a bit pattern.
 * 11 significant bits; at and below 2^-14 the spacing is fixed at 2^-24.  The
 * largest finite value is 65504 = (2 - 2^-10) * 2^15; a value that rounds on
 * this grid to 2^16 or beyond becomes infinity (so 65520, the midpoint between
 * 65504 and 2^16, goes to infinity by the ties-to-even rule). */
static uint16_t f16_bits_from_double(double v)
{
    const uint16_t sign = signbit(v) ? 0x8000u : 0;
    if (isnan(v))
        return (uint16_t)(sign | 0x7E00u);
    const double a = fabs(v);
    if (isinf(v))
        return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);
    int lg = e2 - 1; /* floor(log2 a) */
    if (lg < -14)
        lg = -14;
    const double step = ldexp(1.0, lg - 10);
    const double rounded = nearbyint(a / step) * step;
    if (rounded >= 65536.0)
        return (uint16_t)(sign | 0x7C00u);
    if (rounded < 0x1p-14) /* subnormal or zero: the fraction counts units of 2^-24 */
        return (uint16_t)(sign | (uint16_t)(rounded * 0x1p24));
    int er;
    frexp(rounded, &er); /* rounding may have carried into the next binade */
    const int lr = er - 1;
    const int frac = (int)(ldexp(rounded, 10 - lr)) - 1024;
    return (uint16_t)(sign | (uint16_t)((lr + 15) << 10) | (uint16_t)frac);
}

/* Store v rounded (nearest, ties to even) into element i of a storage array. */
static void store_elem(int dt, void *base, int64_t i, double v)
{
    if (dt == ORACLE_F64)
        ((double *)base)[i] = v;
    else if (dt == ORACLE_F32)
        ((float *)base)[i] = (float)v; /* C conversion: nearest, ties to even */
    else if (dt == ORACLE_F16)
        ((uint16_t *)base)[i] = f16_bits_from_double(v);
    else
        ((uint16_t *)base)[i] = bf16_bits_from_double(v);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Round n doubles to the storage type dt. */
int oracle_round(int dt, const double *src, int64_t n, void *dst)
{
    if (!dtype_ok(dt) || !src || !dst || n < 0)
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        store_elem(dt, dst, i, src[i]);
    return ORACLE_OK;
}

/* w_j = gamma_j + offset, or 1 without gamma */
static double scale_w(int dt, const void *gamma, int64_t j, double off)
{
    return gamma ? load_elem(dt, gamma, j) + off : 1.0;
}

/* rstd_i = 1 / sqrt((1/N) sum_j v_ij^2 + eps) */
static double row_rstd(int dt, const void *v, int64_t row, int64_t N, double eps)
{
    double ss = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        double a = load_elem(dt, v, row * N + j);
        ss += a * a;
    }
    double ms = ss / (double)N;
    return 1.0 / sqrt(ms + eps);
}

/* Forward.  y64 [M, N] (may be NULL), rstd64 [M] (may be NULL). */
int oracle_fwd(int dt, const void *v, const void *gamma, int64_t M, int64_t N,
               float eps, float offset, double *y64, double *rstd64)
{
    if (!dtype_ok(dt) || !v || M < 0 || N <= 0 || (!gamma && offset != 0.0f))
        return ORACLE_EINVAL;
    const double e = (double)eps, off = (double)offset;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double rstd = row_rstd(dt, v, i, N, e);
        if (rstd64)
            rstd64[i] = rstd;
        if (y64) {
            for (int64_t j = 0; j < N; ++j) {
                double w = scale_w(dt, gamma, j, off);
                y64[i * N + j] = load_elem(dt, v, i * N + j) * rstd * w;
            }
        }
    }
    return ORACLE_OK;
}

/* Fused residual add then forward.  h_out [M, N] in storage type dt receives
 * round_T(x + r); the forward normalises that stored h. */
int oracle_fused_add_fwd(int dt, const void *x, const void *r, const void *gamma,
                         int64_t M, int64_t N, float eps, float offset,
                         void *h_out, double *y64, double *rstd64)
{
    if (!dtype_ok(dt) || !x || !r || !h_out || M < 0 || N <= 0 || (!gamma && offset != 0.0f))
        return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            store_elem(dt, h_out, i * N + j,
                       load_elem(dt, x, i * N + j) + load_elem(dt, r, i * N + j));
    return oracle_fwd(dt, h_out, gamma, M, N, eps, offset, y64, rstd64);
}

/* Backward.  v is the forward's input (h for the fused-add variant); dh, when
 * not NULL, is added to dx; gamma NULL is the non-affine op (no dgamma).
 * Outputs (each may be NULL):
 *   dx64 [M, N]; dgamma64 [N];
 *   c64 [M]     = (1/N) sum_j g_ij xhat_ij;
 *   sabs64 [M]  = (1/N) sum_j |g_ij xhat_ij|  (the size of the terms that
 *                 cancel in dx, used by the tests' tolerance floor). */
int oracle_bwd(int dt, const void *dy, const void *v, const void *gamma, const void *dh,
               int64_t M, int64_t N, float eps, float offset,
               double *dx64, double *dgamma64, double *c64, double *sabs64)
{
    if (!dtype_ok(dt) || !dy || !v || M < 0 || N <= 0 || (!gamma && (offset != 0.0f || dgamma64)))
        return ORACLE_EINVAL;
    const double e = (double)eps, off = (double)offset;

    double *rstd = (double *)malloc((size_t)(M > 0 ? M : 1) * sizeof(double));
    if (!rstd)
        return ORACLE_ENOMEM;

    /* rows: rstd, c, sabs, dx */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        rstd[i] = row_rstd(dt, v, i, N, e);
        double dot = 0.0, dabs = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double w = scale_w(dt, gamma, j, off);
            double g = load_elem(dt, dy, i * N + j) * w;
            double xhat = load_elem(dt, v, i * N + j) * rstd[i];
            dot += g * xhat;
            dabs += fabs(g * xhat);
        }
        double c = dot / (double)N;
        if (c64)
            c64[i] = c;
        if (sabs64)
            sabs64[i] = dabs / (double)N;
        if (dx64) {
            for (int64_t j = 0; j < N; ++j) {
                double w = scale_w(dt, gamma, j, off);
                double g = load_elem(dt, dy, i * N + j) * w;
                double xhat = load_elem(dt, v, i * N + j) * rstd[i];
                double d = rstd[i] * (g - xhat * c);
                if (dh)
                    d += load_elem(dt, dh, i * N + j);
                dx64[i * N + j] = d;
            }
        }
    }

    /* columns: dgamma_j = sum_i dy_ij * xhat_ij, each column summed over the
     * rows in row order; threads own disjoint column ranges */
    if (dgamma64) {
#pragma omp parallel
        {
            int64_t nt = 1, t = 0;
#ifdef _OPENMP
            nt = omp_get_num_threads();
            t = omp_get_thread_num();
#endif
            int64_t j0 = N * t / nt, j1 = N * (t + 1) / nt;
            for (int64_t j = j0; j < j1; ++j)
                dgamma64[j] = 0.0;
            for (int64_t i = 0; i < M; ++i)
                for (int64_t j = j0; j < j1; ++j)
                    dgamma64[j] += load_elem(dt, dy, i * N + j) * (load_elem(dt, v, i * N + j) * rstd[i]);
        }
    }
    free(rstd);
    return ORACLE_OK;
}

/* ---- fp8 E4M3 (OCP FN) -------------------------------------------------- */

/* Nearest E4M3 code to t, ties to even, saturating at +-448.  As for bf16:
 * below 2^-6 the spacing is fixed at 2^-9, above it is 2^(floor(log2|t|) - 3),
 * and nearbyint of the exact quotient gives ties to even. */
static uint8_t e4m3_from_double(double t)
{
    const uint8_t sign = signbit(t) ? 0x80 : 0x00;
    double a = fabs(t);
    if (isnan(t))
        return (uint8_t)(sign | 0x7F);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);
    int q = e - 1; /* floor(log2 a) */
    if (q < -6)
        q = -6;
    const double spacing = ldexp(1.0, q - 3);
    const double r = nearbyint(a / spacing) * spacing; /* at most 448: a < 448 = 14 * 32 */
    if (r == 0.0)
        return sign;
    if (r < 0x1p-6) /* subnormal: r = m * 2^-9 */
        return (uint8_t)(sign | (uint8_t)(r / 0x1p-9));
    frexp(r, &e);
    const int E = e - 1;                               /* r = (1 + m/8) * 2^E */
    const int m = (int)(r / ldexp(1.0, E - 3)) - 8;    /* exact: 0..7 */
    return (uint8_t)(sign | (uint8_t)(((E + 7) << 3) | m));
}

static double e4m3_to_double(uint8_t c)
{
    const double s = (c & 0x80) ? -1.0 : 1.0;
    const int e = (c >> 3) & 0xF, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        return s * ldexp((double)m, -9);
    return s * ldexp(1.0 + m / 8.0, e - 7);
}

int oracle_e4m3_encode(const double *src, int64_t n, uint8_t *dst)
{
    if (!src || !dst || n < 0)
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = e4m3_from_double(src[i]);
    return ORACLE_OK;
}

int oracle_e4m3_decode(const uint8_t *src, int64_t n, double *dst)
{
    if (!src || !dst || n < 0)
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = e4m3_to_double(src[i]);
    return ORACLE_OK;
}

/* fp8-output forward of v (h for the fused-add op: the caller forms h first).
 * code [M, N] = E4M3(y64 * scale).  With tol > 0, code_lo / code_hi [M, N]
 * (each may be NULL) are the codes of t * (1 - tol) and t * (1 + tol): since
 * the encoding is monotone, every value within a relative tol of t encodes
 * to a code between them.  rstd64 [M] and amax64 (one value) may be NULL. */
int oracle_fwd_fp8(int dt, const void *v, const void *gamma, int64_t M, int64_t N, float eps, float offset,
                   float scale, double tol, uint8_t *code, uint8_t *code_lo, uint8_t *code_hi, double *rstd64,
                   double *amax64)
{
    if (!dtype_ok(dt) || !v || !code || M < 0 || N <= 0 || tol < 0.0 || (!gamma && offset != 0.0f))
        return ORACLE_EINVAL;
    const double e = (double)eps, off = (double)offset, sc = (double)scale;
    double amax = 0.0;
    int any_nan = 0; /* a NaN y makes amax NaN: the window saw a non-number */
#pragma omp parallel for schedule(static) reduction(max : amax) reduction(|| : any_nan)
    for (int64_t i = 0; i < M; ++i) {
        const double rstd = row_rstd(dt, v, i, N, e);
        if (rstd64)
            rstd64[i] = rstd;
        for (int64_t j = 0; j < N; ++j) {
            const double y = load_elem(dt, v, i * N + j) * rstd * scale_w(dt, gamma, j, off);
            const double t = y * sc;
            if (isnan(y))
                any_nan = 1;
            else if (fabs(y) > amax)
                amax = fabs(y);
            code[i * N + j] = e4m3_from_double(t);
            /* t * (1 -+ tol) toward / away from zero: the lower and upper ends
             * of the interval in value order */
            const double lo = t < 0 ? t * (1.0 + tol) : t * (1.0 - tol);
            const double hi = t < 0 ? t * (1.0 - tol) : t * (1.0 + tol);
            if (code_lo)
                code_lo[i * N + j] = e4m3_from_double(lo);
            if (code_hi)
                code_hi[i * N + j] = e4m3_from_double(hi);
        }
    }
    if (amax64)
        *amax64 = any_nan ? NAN : amax;
    return ORACLE_OK;
}

/* ---- LayerNorm ------------------------------------------------------------ */

/* mu_i and rstd_i = 1 / sqrt(var_i + eps) of row i (two passes over the row) */
static void ln_row_stats(int dt, const void *v, int64_t row, int64_t N, double eps, double *mu, double *rstd)
{
    double s = 0.0;
    for (int64_t j = 0; j < N; ++j)
        s += load_elem(dt, v, row * N + j);
    const double m = s / (double)N;
    double q = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        const double d = load_elem(dt, v, row * N + j) - m;
        q += d * d;
    }
    *mu = m;
    *rstd = 1.0 / sqrt(q / (double)N + eps);
}

/* LayerNorm forward.  beta NULL means no bias; gamma NULL means w = 1 (offset
 * 0).  y64 [M, N], mean64 [M], rstd64 [M] may each be NULL. */
int oracle_ln_fwd(int dt, const void *v, const void *gamma, const void *beta, int64_t M, int64_t N, float eps,
                  float offset, double *y64, double *mean64, double *rstd64)
{
    if (!dtype_ok(dt) || !v || M < 0 || N <= 0 || (!gamma && offset != 0.0f))
        return ORACLE_EINVAL;
    const double e = (double)eps, off = (double)offset;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double mu, rstd;
        ln_row_stats(dt, v, i, N, e, &mu, &rstd);
        if (mean64)
            mean64[i] = mu;
        if (rstd64)
            rstd64[i] = rstd;
        if (y64) {
            for (int64_t j = 0; j < N; ++j) {
                const double xhat = (load_elem(dt, v, i * N + j) - mu) * rstd;
                y64[i * N + j] = xhat * scale_w(dt, gamma, j, off) + (beta ? load_elem(dt, beta, j) : 0.0);
            }
        }
    }
    return ORACLE_OK;
}

/* LayerNorm backward of the forward of v (h for fused-add; dh is then added
 * to dx).  Outputs (each may be NULL): dx64 [M, N]; dgamma64 [N] (needs
 * gamma); dbeta64 [N]; and per row, for the tests' tolerance floor,
 * c1 = mean_j(g), c2 = mean_j(g * xhat), s1 = mean_j |g|, s2 = mean_j |g * xhat|
 * (stats64 [M, 4]). */
int oracle_ln_bwd(int dt, const void *dy, const void *v, const void *gamma, const void *dh, int64_t M, int64_t N,
                  float eps, float offset, double *dx64, double *dgamma64, double *dbeta64, double *stats64)
{
    if (!dtype_ok(dt) || !dy || !v || M < 0 || N <= 0 || (!gamma && (offset != 0.0f || dgamma64)))
        return ORACLE_EINVAL;
    const double e = (double)eps, off = (double)offset;
    double *mu = (double *)malloc((size_t)(M > 0 ? M : 1) * sizeof(double));
    double *rs = (double *)malloc((size_t)(M > 0 ? M : 1) * sizeof(double));
    if (!mu || !rs) {
        free(mu);
        free(rs);
        return ORACLE_ENOMEM;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        ln_row_stats(dt, v, i, N, e, &mu[i], &rs[i]);
        double sg = 0.0, sgx = 0.0, ag = 0.0, agx = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            const double g = load_elem(dt, dy, i * N + j) * scale_w(dt, gamma, j, off);
            const double xhat = (load_elem(dt, v, i * N + j) - mu[i]) * rs[i];
            sg += g;
            sgx += g * xhat;
            ag += fabs(g);
            agx += fabs(g * xhat);
        }
        const double c1 = sg / (double)N, c2 = sgx / (double)N;
        if (stats64) {
            stats64[4 * i + 0] = c1;
            stats64[4 * i + 1] = c2;
            stats64[4 * i + 2] = ag / (double)N;
            stats64[4 * i + 3] = agx / (double)N;
        }
        if (dx64) {
            for (int64_t j = 0; j < N; ++j) {
                const double g = load_elem(dt, dy, i * N + j) * scale_w(dt, gamma, j, off);
                const double xhat = (load_elem(dt, v, i * N + j) - mu[i]) * rs[i];
                double d = rs[i] * (g - c1 - xhat * c2);
                if (dh)
                    d += load_elem(dt, dh, i * N + j);
                dx64[i * N + j] = d;
            }
        }
    }
    /* columns, each summed over the rows in row order */
    if (dgamma64 || dbeta64) {
#pragma omp parallel
        {
            int64_t nt = 1, t = 0;
#ifdef _OPENMP
            nt = omp_get_num_threads();
            t = omp_get_thread_num();
#endif
            int64_t j0 = N * t / nt, j1 = N * (t + 1) / nt;
            for (int64_t j = j0; j < j1; ++j) {
                if (dgamma64)
                    dgamma64[j] = 0.0;
                if (dbeta64)
                    dbeta64[j] = 0.0;
            }
            for (int64_t i = 0; i < M; ++i)
                for (int64_t j = j0; j < j1; ++j) {
                    const double d = load_elem(dt, dy, i * N + j);
                    if (dgamma64)
                        dgamma64[j] += d * ((load_elem(dt, v, i * N + j) - mu[i]) * rs[i]);
                    if (dbeta64)
                        dbeta64[j] += d;
                }
        }
    }
    free(mu);
    free(rs);
    return ORACLE_OK;
}
