/*
 * qlinear_oracle.c -- plain, slow CPU oracle for the quantized linear GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP library; the two meet only at the byte level of the seeded
 * synthetic inputs.
 *
 * What it computes (restated from the pages, never copied):
 *
 *   "Building a High-Performance and Portable vLLM Linear Backend with Helion"
 *   (PyTorch blog post; English body mirrored on wqu.guru), section
 *   "Helion Linear Backend / Scope", defines the three 8-bit formats:
 *     FP8_Dynamic -- FP8 operands, one scale per activation token (row of A)
 *                    and one per weight output channel (row of B);
 *     W8A8_INT8   -- the same scaling with INT8 operands;
 *     Block_FP8   -- FP8 with one activation scale per 1x128 group along K
 *                    and one weight scale per 128x128 block.
 *   The same post, section "Kernel Implementation", says the quantized
 *   kernels are a plain tiled matrix product plus scaling; the techfeed.io
 *   summary of it (section on the single kernel covering several variants)
 *   shows the product as a sum over K tiles into one accumulator.
 *
 * Readings taken where the pages are silent (each is listed in the design doc):
 *   - Y = A * B^T: A is [M,K] (tokens x reduction), B is [N,K] (output
 *     channels x reduction); both rows are K-contiguous.
 *   - Dequantisation is x = q * s, so the scales multiply the exact integer
 *     (or exact FP8) dot product; for Block_FP8 each 128-wide K group is
 *     scaled before the groups are summed.
 *   - FP8 is OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF are NaN, max 448).
 *   - The output is bfloat16, rounded to nearest-even straight from the
 *     double-precision value (one rounding, no detour through fp32).
 *
 * Precision: int8 dot products are summed in int64 (exact).  Each e4m3 value
 * is an integer multiple of 2^-9 with magnitude <= 448, so every product is a
 * multiple of 2^-18 below 2^17.62 and any running sum of fewer than 171196 of
 * them is exact in double: the FP8 dot products below are exact regardless
 * of summation order.  Scales are applied in double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FMT_E4M3 0
#define ORC_FMT_INT8 1

/* ---------------------------------------------------------------------- */
/* Decoding: OCP 8-bit floating point E4M3FN and two's-complement int8.    */
/* ---------------------------------------------------------------------- */

/* OCP "8-bit Floating Point Specification", E4M3 encoding: 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 * subnormals m * 2^-9; S.1111.111 is NaN; there are no infinities. */
double orc_e4m3_to_double(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);               /* m/8 * 2^(1-7) */
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

double orc_int8_to_double(uint8_t code)
{
    return (double)(int8_t)code;
}

/* ---------------------------------------------------------------------- */
/* Rounding: double -> bfloat16 bits, round to nearest, ties to even.      */
/* ---------------------------------------------------------------------- */

/* bfloat16: 1 sign, 8 exponent bits (bias 127), 7 fraction bits.  Normal
 * numbers are >= 2^-126 and have a spacing (ulp) of 2^(e-7) in the binade
 * [2^e, 2^(e+1)); below 2^-126 the spacing stays 2^-133 (gradual underflow).
 * The value |x|/ulp is formed exactly (scaling by a power of two), rounded to
 * an integer with ties to even (rint under the default rounding mode), and
 * scaled back.  The rounded value is exactly representable in bf16, hence in
 * fp32, so its top 16 fp32 bits are the bf16 encoding.  Results at or above
 * 2^128 are infinities. */
uint16_t orc_double_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;
    int e;
    if (a >= ldexp(1.0, -126)) {
        int ex;
        frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
        e = ex - 1;                    /* a in [2^e, 2^(e+1)) */
    } else {
        e = -126;
    }
    double ulp_exp = (double)(e - 7);
    double q = ldexp(a, -(int)ulp_exp);           /* exact */
    double r = rint(q);                           /* ties to even */
    double v = ldexp(r, (int)ulp_exp);
    if (v >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)v;                           /* exact by construction */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | ((bits >> 16) & 0x7FFFu));
}

/* ---------------------------------------------------------------------- */
/* The GEMMs.                                                              */
/* ---------------------------------------------------------------------- */

typedef struct {
    int fmt;           /* ORC_FMT_E4M3 or ORC_FMT_INT8 */
    int block;         /* 0: per-token x per-channel scales; 1: Block_FP8 */
    int64_t M, N, K;
    const uint8_t *A; int64_t lda;
    const float *sA;
    const uint8_t *B; int64_t ldb;
    const float *sB;
    uint16_t *Y; int64_t ldy;
    double *ydbl;      /* [M][N] value before rounding, or NULL */
    double *bound;     /* [M][N] sum of |products| times scales, or NULL */
    int64_t *acc_i;    /* [M][N] exact int8 dot product, or NULL */
    double *acc_f;     /* [M][N] exact fp8 dot product, or NULL */
    /* point mode: evaluate only the listed (m, n) pairs */
    int64_t npts;
    const int64_t *pm, *pn;
    /* work split */
    int64_t first, last;   /* range of flat output indices (or point indices) */
} orc_job;

static double dec(int fmt, uint8_t c)
{
    return fmt == ORC_FMT_INT8 ? orc_int8_to_double(c) : orc_e4m3_to_double(c);
}

/* One output element (m, n).  Writes slot `slot` of the optional outputs. */
static void orc_one(const orc_job *j, int64_t m, int64_t n, int64_t slot)
{
    const uint8_t *a = j->A + m * j->lda;
    const uint8_t *b = j->B + n * j->ldb;
    double y, s_abs;
    if (!j->block) {
        /* FP8_Dynamic / W8A8_INT8: y = sA[m] * sB[n] * sum_k a[m,k] b[n,k] */
        double abssum = 0.0;
        if (j->fmt == ORC_FMT_INT8) {
            int64_t acc = 0, aacc = 0;
            for (int64_t k = 0; k < j->K; ++k) {
                int64_t p = (int64_t)(int8_t)a[k] * (int64_t)(int8_t)b[k];
                acc += p;
                aacc += p < 0 ? -p : p;
            }
            if (j->acc_i) j->acc_i[slot] = acc;
            y = ((double)acc * (double)j->sA[m]) * (double)j->sB[n];
            abssum = (double)aacc;
        } else {
            double acc = 0.0;
            for (int64_t k = 0; k < j->K; ++k) {
                double p = orc_e4m3_to_double(a[k]) * orc_e4m3_to_double(b[k]);
                acc += p;
                abssum += fabs(p);
            }
            if (j->acc_f) j->acc_f[slot] = acc;
            y = (acc * (double)j->sA[m]) * (double)j->sB[n];
        }
        s_abs = (abssum * fabs((double)j->sA[m])) * fabs((double)j->sB[n]);
    } else {
        /* Block_FP8: y = sum_g sA[m,g] * sB[n/128,g] * sum_{k in group g} a b */
        int64_t G = j->K / 128;
        int64_t nb = n / 128;
        double total_exact = 0.0;
        y = 0.0;
        s_abs = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            double p = 0.0, pa = 0.0;
            for (int64_t k = g * 128; k < g * 128 + 128; ++k) {
                double t = dec(j->fmt, a[k]) * dec(j->fmt, b[k]);
                p += t;
                pa += fabs(t);
            }
            double sa = (double)j->sA[m * G + g];
            double sb = (double)j->sB[nb * G + g];
            y += (p * sa) * sb;
            s_abs += (pa * fabs(sa)) * fabs(sb);
            total_exact += p;
        }
        if (j->acc_f) j->acc_f[slot] = total_exact;
    }
    if (j->ydbl) j->ydbl[slot] = y;
    if (j->bound) j->bound[slot] = s_abs;
    if (j->Y) {
        if (j->npts)
            j->Y[slot] = orc_double_to_bf16(y);
        else
            j->Y[m * j->ldy + n] = orc_double_to_bf16(y);
    }
}

static void *orc_worker(void *arg)
{
    const orc_job *j = (const orc_job *)arg;
    for (int64_t i = j->first; i < j->last; ++i) {
        if (j->npts) {
            orc_one(j, j->pm[i], j->pn[i], i);
        } else {
            int64_t m = i / j->N, n = i % j->N;
            orc_one(j, m, n, i);
        }
    }
    return NULL;
}

static int orc_run(orc_job base, int64_t total, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (total <= 0) return 0;
    if ((int64_t)nthreads > total) nthreads = (int)total;
    pthread_t tid[256];
    orc_job jobs[256];
    int64_t chunk = (total + nthreads - 1) / nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].first = (int64_t)t * chunk;
        jobs[t].last = jobs[t].first + chunk < total ? jobs[t].first + chunk : total;
        if (jobs[t].first >= jobs[t].last) break;
        if (t == 0) continue;               /* the caller's thread runs job 0 */
        if (pthread_create(&tid[t], NULL, orc_worker, &jobs[t]) != 0)
            return -1;
        started = t;
    }
    orc_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    return 0;
}

/* Full product.  Returns 0 on success, -1 on bad arguments.  Optional
 * outputs are dense [M][N]; Y uses row stride ldy. */
int orc_scaled_mm(int fmt, int block, int64_t M, int64_t N, int64_t K,
                  const uint8_t *A, int64_t lda, const float *sA,
                  const uint8_t *B, int64_t ldb, const float *sB,
                  uint16_t *Y, int64_t ldy,
                  double *ydbl, double *bound, int64_t *acc_i, double *acc_f,
                  int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || (Y && ldy < N))
        return -1;
    if (block && (K % 128 != 0))
        return -1;
    orc_job j;
    memset(&j, 0, sizeof j);
    j.fmt = fmt; j.block = block; j.M = M; j.N = N; j.K = K;
    j.A = A; j.lda = lda; j.sA = sA; j.B = B; j.ldb = ldb; j.sB = sB;
    j.Y = Y; j.ldy = ldy; j.ydbl = ydbl; j.bound = bound;
    j.acc_i = acc_i; j.acc_f = acc_f;
    return orc_run(j, M * N, nthreads);
}

/* The same, evaluated only at the npts listed (pm[i], pn[i]) positions; all
 * outputs are dense [npts] arrays (Y included). */
int orc_scaled_mm_points(int fmt, int block, int64_t M, int64_t N, int64_t K,
                         const uint8_t *A, int64_t lda, const float *sA,
                         const uint8_t *B, int64_t ldb, const float *sB,
                         int64_t npts, const int64_t *pm, const int64_t *pn,
                         uint16_t *Y, double *ydbl, double *bound,
                         int64_t *acc_i, double *acc_f, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || npts < 0)
        return -1;
    if (block && (K % 128 != 0))
        return -1;
    for (int64_t i = 0; i < npts; ++i)
        if (pm[i] < 0 || pm[i] >= M || pn[i] < 0 || pn[i] >= N)
            return -1;
    orc_job j;
    memset(&j, 0, sizeof j);
    j.fmt = fmt; j.block = block; j.M = M; j.N = N; j.K = K;
    j.A = A; j.lda = lda; j.sA = sA; j.B = B; j.ldb = ldb; j.sB = sB;
    j.Y = Y; j.ldy = 0; j.ydbl = ydbl; j.bound = bound;
    j.acc_i = acc_i; j.acc_f = acc_f;
    j.npts = npts; j.pm = pm; j.pn = pn;
    if (npts == 0) return 0;
    return orc_run(j, npts, nthreads);
}

/* Vector helpers so the decode and rounding rules can be pinned in bulk. */
void orc_e4m3_decode_n(const uint8_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_to_double(in[i]);
}

void orc_double_to_bf16_n(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_double_to_bf16(in[i]);
}

/* ---------------------------------------------------------------------- */
/* Activation quantization (the step upstream of the GEMM).               */
/* ---------------------------------------------------------------------- */
/*
 * "HelionがvLLMに統合 ..." (24-ai.news), section "vLLMに統合されたカーネル"
 * (kernels integrated into vLLM), items 1 and 5: dynamic per-token FP8
 * quantization and per-token-group FP8 quantization of the activations
 * feeding scaled_mm / scaled_mm_blockwise.  The pages give names only.
 * Readings (listed in the design doc): the input is bfloat16; a row (or 1x128
 * group) gets scale s = amax / 448 (e4m3) or amax / 127 (int8), computed in
 * fp32 with one correctly rounded division; an all-zero row or group gets
 * s = 1; each code is the quotient x / s (fp32, correctly rounded) clamped
 * to +-448 and rounded to the nearest e4m3 value, ties to the even code
 * (int8: rounded to the nearest integer, ties to even, clamped to +-127).
 *
 * The fp32 steps are taken in C float arithmetic (x86-64 SSE: every float
 * operation is rounded once to fp32; built with -ffp-contract=off).  The
 * e4m3 rounding is done by exhaustive search over the 127 non-negative
 * finite codes, decoded by orc_e4m3_to_double: the nearest value wins and
 * a tie goes to the code whose last mantissa bit is 0.
 */

static float orc_bf16_to_float(uint16_t h)
{
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, sizeof f);
    return f;
}

/* Nearest e4m3 code to v (|v| <= 448), ties to the even code; the sign of
 * v (including -0) is kept. */
uint8_t orc_e4m3_nearest(float v)
{
    double a = fabs((double)v);
    int best = 0;
    double best_d = a;                     /* distance to code 0 (+0) */
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(orc_e4m3_to_double((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 0x80 : 0));
}

/* Round half to even on a float holding a value of magnitude < 2^23. */
static float orc_rint_even(float x)
{
    float f = floorf(x);
    float r = x - f;                       /* exact: x and f share the binade scale */
    if (r > 0.5f || (r == 0.5f && fmodf(f, 2.0f) != 0.0f))
        f += 1.0f;
    return f;
}

static void orc_quant_span(int fmt, const uint16_t *x, int64_t n, uint8_t *q, float *s_out)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(orc_bf16_to_float(x[i]));
        if (a > amax) amax = a;
    }
    const float qmax = fmt == ORC_FMT_INT8 ? 127.0f : 448.0f;
    float s = amax / qmax;
    if (amax == 0.0f) s = 1.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = orc_bf16_to_float(x[i]) / s;
        if (fmt == ORC_FMT_INT8) {
            float r = orc_rint_even(v);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[i] = (uint8_t)(int8_t)r;
        } else {
            if (v > 448.0f) v = 448.0f;
            if (v < -448.0f) v = -448.0f;
            q[i] = orc_e4m3_nearest(v);
        }
    }
    *s_out = s;
}

/* Per-token: x [M, ldx] bf16 bits -> q [M, ldq] codes, s [M]. */
int orc_quant_per_token(int fmt, int64_t M, int64_t K, const uint16_t *x, int64_t ldx,
                        uint8_t *q, int64_t ldq, float *s)
{
    if ((fmt != ORC_FMT_E4M3 && fmt != ORC_FMT_INT8) || M < 0 || K < 0 || ldx < K || ldq < K)
        return 1;
    for (int64_t m = 0; m < M; ++m)
        orc_quant_span(fmt, x + m * ldx, K, q + m * ldq, s + m);
    return 0;
}

/* Per 1 x group along K (e4m3): s [M, K/group] row-major. */
int orc_quant_per_group(int64_t M, int64_t K, int64_t group, const uint16_t *x, int64_t ldx,
                        uint8_t *q, int64_t ldq, float *s)
{
    if (M < 0 || K < 0 || group <= 0 || K % group || ldx < K || ldq < K)
        return 1;
    const int64_t G = K / group;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < G; ++g)
            orc_quant_span(ORC_FMT_E4M3, x + m * ldx + g * group, group,
                           q + m * ldq + g * group, s + m * G + g);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Fused producers: RMS norm and SiLU-and-mul ahead of the quantizer.      */
/* ---------------------------------------------------------------------- */
/*
 * "HelionがvLLMに統合 ..." (24-ai.news), section "vLLMに統合されたカーネル",
 * items 2, 3, 6 and 7 (rms_norm_dynamic_per_token_quant,
 * silu_and_mul_dynamic_per_token_quant, rms_norm_per_block_quant,
 * silu_and_mul_per_block_quant), and the section on per-kernel performance
 * that reports their speed-ups: a normalisation or gated activation fused
 * with the dynamic quantizer above.  The pages give names only.  Readings
 * (listed in the design doc):
 *   - a fused kernel returns exactly what the unfused pair returns: the
 *     producer's output is a bfloat16 activation, which the quantizer above
 *     (per token, or per 1x128 group) then reads;
 *   - the producer's bf16 value is its real-number result rounded once to
 *     nearest-even, evaluated here in double:
 *       RMS norm over a row of K:  h_k = x_k, or with a residual
 *         h_k = bf16(x_k + r_k) (and the residual row is replaced by h);
 *         ms = (sum_k h_k^2) / K,  inv = 1 / sqrt(ms + eps),
 *         y_k = bf16((h_k * w_k) * inv)        (w: bf16 weight of length K);
 *       SiLU-and-mul over a row of 2K (gate | up):
 *         y_k = bf16((g_k / (1 + exp(-g_k))) * u_k).
 *   Each square h_k^2 and product h_k * w_k of bf16 values is exact in
 *   double; the sum of squares is taken for k increasing.  x_k + r_k is
 *   exact in double unless the exponents differ by more than 45, and then
 *   the sum lies far inside one bf16 rounding interval, so rounding it
 *   first to double does not change its bf16 rounding.
 */

static double orc_bf16_to_double(uint16_t h) { return (double)orc_bf16_to_float(h); }

/* x [M, ldx], optional residual r [M, ldr] (replaced by h), weight w [K],
 * output y [M, ldy]; all bf16 bits.  Returns 0, or 1 on bad arguments. */
int orc_rms_norm(int64_t M, int64_t K, const uint16_t *x, int64_t ldx, uint16_t *r, int64_t ldr,
                 const uint16_t *w, float eps, uint16_t *y, int64_t ldy)
{
    if (M < 0 || K <= 0 || ldx < K || ldy < K || (r && ldr < K) || !(eps >= 0.0f))
        return 1;
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * ldx;
        uint16_t *rr = r ? r + m * ldr : NULL;
        uint16_t *yr = y + m * ldy;
        double sum = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double h = orc_bf16_to_double(xr[k]);
            if (rr) {
                rr[k] = orc_double_to_bf16(h + orc_bf16_to_double(rr[k]));
                h = orc_bf16_to_double(rr[k]);
            }
            sum += h * h;
        }
        const double ms = sum / (double)K;
        const double inv = 1.0 / sqrt(ms + (double)eps);
        for (int64_t k = 0; k < K; ++k) {
            const double h = orc_bf16_to_double(rr ? rr[k] : xr[k]);
            yr[k] = orc_double_to_bf16((h * orc_bf16_to_double(w[k])) * inv);
        }
    }
    return 0;
}

/* x [M, ldx] holding gate columns 0..K-1 and up columns K..2K-1; y [M, ldy]. */
int orc_silu_and_mul(int64_t M, int64_t K, const uint16_t *x, int64_t ldx, uint16_t *y,
                     int64_t ldy)
{
    if (M < 0 || K <= 0 || ldx < 2 * K || ldy < K)
        return 1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            const double g = orc_bf16_to_double(x[m * ldx + k]);
            const double u = orc_bf16_to_double(x[m * ldx + K + k]);
            y[m * ldy + k] = orc_double_to_bf16((g / (1.0 + exp(-g))) * u);
        }
    return 0;
}
