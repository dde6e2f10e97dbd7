/*
 * CPU oracle for the output-centric MoE decode expert layer -- TEST
 * INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
 * baseline call it; the product path never does.
 *
 * Plain, slow, obviously correct: every value is decoded to float64 and every
 * sum is taken in float64, in the order the definition states it. It shares
 * no code, header or table with the HIP library.
 *
 * What it computes (the ordinary routed SwiGLU expert layer; the warp-decode
 * post reorganises its parallelism but does not approximate it -- "Warp
 * decode", section "How the two kernels work"):
 *
 *   for each token b and routed slot j, with expert e = ids[b][j]:
 *     g[i] = sum_h Wg^[e][i][h] * x[b][h]        (gate projection)
 *     u[i] = sum_h Wu^[e][i][h] * x[b][h]        (up projection)
 *     a[b][j][i] = SiLU(g[i]) * u[i],  SiLU(t) = t / (1 + exp(-t))
 *   out[b][h] = sum_j w[b][j] * sum_i Wd^[e_j][h][i] * a[b][j][i]
 *
 * where W^ is the block-scaled weight decoded exactly, in one of two formats
 * (fmt argument of the *_fmt functions; the plain functions are MXFP8):
 *   MXFP8 (fmt 0): W^[e][n][c] = E4M3(q[e][n][c]) * UE8M0(s[e][n][c / 32])
 *     (FP8 E4M3 codes with one UE8M0 scale per 32 values along the
 *     reduction axis, as the GC-MoE summary's section "How to use" names the
 *     block format);
 *   MXFP4 (fmt 1): W^[e][n][c] = E2M1(nibble c of row n) * UE8M0(s[e][n][c / 32])
 *     (the FP4 E2M1 routed weights with the same K32 UE8M0 granularity that
 *     the same section describes), two codes per byte: element c is the low
 *     nibble of byte c/2 when c is even and the high nibble when c is odd, so
 *     a row of K codes is K/2 bytes.
 * Element formats per the OCP Microscaling v1.0 definition.
 *
 * Conventions the definition leaves open, and the reading taken here:
 *  - duplicate expert ids in a token's row are legal and their terms add;
 *  - an expert id outside [0, E) makes that token's outputs NaN;
 *  - NaN codes (E4M3 0x7F/0xFF, UE8M0 0xFF) propagate as NaN.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math: sums stay in the
 * written order).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* OCP FP8 E4M3 ("E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (2^-6 * m/8); exponent 15 with mantissa 7 is
 * NaN; there are no infinities. */
double oracle_e4m3_value(unsigned code)
{
    code &= 0xFFu;
    const int sign = (code >> 7) & 1;
    const int ex = (code >> 3) & 0xF;
    const int man = code & 0x7;
    double mag;
    if (ex == 0xF && man == 0x7)
        return NAN;
    if (ex == 0)
        mag = ldexp((double)man / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)man / 8.0, ex - 7);
    return sign ? -mag : mag;
}

/* OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit. Exponent field
 * 0 is subnormal (m/2); there are no NaN and no infinities, so the values are
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives. */
double oracle_e2m1_value(unsigned code)
{
    code &= 0xFu;
    const int sign = (code >> 3) & 1;
    const int ex = (code >> 1) & 0x3;
    const int man = code & 0x1;
    double mag;
    if (ex == 0)
        mag = (double)man * 0.5;
    else
        mag = ldexp(1.0 + (double)man / 2.0, ex - 1);
    return sign ? -mag : mag;
}

/* UE8M0: an unsigned 8-bit exponent, value 2^(code - 127); code 0xFF is NaN. */
double oracle_ue8m0_value(unsigned code)
{
    code &= 0xFFu;
    if (code == 0xFF)
        return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* bfloat16 bit pattern -> float64: the pattern is the top half of a float32. */
double oracle_bf16_value(unsigned bits)
{
    uint32_t u = (uint32_t)(bits & 0xFFFFu) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void fill_e4m3_table(double t[256])
{
    for (unsigned c = 0; c < 256; ++c)
        t[c] = oracle_e4m3_value(c);
}

static int bad_shape(int B, int E, int k, int H, int I)
{
    return B < 0 || E < 1 || k < 1 || k > E || H < 32 || I < 32 || (H % 32) || (I % 32);
}

enum { FMT_MXFP8 = 0, FMT_MXFP4 = 1 };

/* Bytes of codes in a row of n values. */
static long row_bytes(long n, int fmt)
{
    return fmt == FMT_MXFP4 ? n / 2 : n;
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* SiLU(gate) * up, in float64. t / (1 + exp(-t)) gives -0 rather than NaN
 * when exp(-t) overflows. */
static double swiglu(double g, double u)
{
    return g / (1.0 + exp(-g)) * u;
}

/* One row dot: sum_c W^[c] * v[c] over a row of n values with n/32 scales.
 * MXFP8: code c is byte c. MXFP4: code c is nibble c (low nibble first). */
static double mx_row_dot(const double tab[256], const uint8_t *q, const uint8_t *s,
                         const double *v, long n, int fmt)
{
    double acc = 0.0;
    for (long c = 0; c < n; ++c) {
        double wv;
        if (fmt == FMT_MXFP4)
            wv = oracle_e2m1_value((c % 2) ? (unsigned)(q[c / 2] >> 4) : (unsigned)(q[c / 2] & 0xFu));
        else
            wv = tab[q[c]];
        acc += wv * oracle_ue8m0_value(s[c / 32]) * v[c];
    }
    return acc;
}

/*
 * Gate/up half of the layer: a[b][j][i] = SiLU(g) * u, float64 [B][k][I].
 * x: bf16 bits [B][H]; ids: int32 [B][k]; w*_q: uint8 [E][I][H] (MXFP8) or
 * [E][I][H/2] (MXFP4); w*_s: uint8 [E][I][H/32]. Returns 0, or -2 on a bad
 * shape or format.
 */
int oracle_gate_up_fmt(const uint16_t *x, const int32_t *ids,
                       const uint8_t *wg_q, const uint8_t *wg_s,
                       const uint8_t *wu_q, const uint8_t *wu_s,
                       int B, int E, int k, int H, int I, double *a, int nthreads, int fmt)
{
    if (bad_shape(B, E, k, H, I) || (fmt != FMT_MXFP8 && fmt != FMT_MXFP4))
        return -2;
    const long rb = row_bytes(H, fmt);
    double tab[256];
    fill_e4m3_table(tab);
    set_threads(nthreads);
    double *xd = (double *)malloc(sizeof(double) * (size_t)(B > 0 ? B : 1) * (size_t)H);
    if (!xd)
        return -1;
    for (long t = 0; t < (long)B * H; ++t)
        xd[t] = oracle_bf16_value(x[t]);

    const long nrow = (long)B * k * I;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < nrow; ++r) {
        const long i = r % I;
        const long bj = r / I;
        const long b = bj / k;
        const int e = ids[bj];
        if (e < 0 || e >= E) {
            a[r] = NAN;
            continue;
        }
        const size_t row = (size_t)e * (size_t)I + (size_t)i;
        const double g = mx_row_dot(tab, wg_q + row * (size_t)rb, wg_s + row * (size_t)(H / 32),
                                    xd + b * H, H, fmt);
        const double u = mx_row_dot(tab, wu_q + row * (size_t)rb, wu_s + row * (size_t)(H / 32),
                                    xd + b * H, H, fmt);
        a[r] = swiglu(g, u);
    }
    free(xd);
    return 0;
}

int oracle_gate_up(const uint16_t *x, const int32_t *ids,
                   const uint8_t *wg_q, const uint8_t *wg_s,
                   const uint8_t *wu_q, const uint8_t *wu_s,
                   int B, int E, int k, int H, int I, double *a, int nthreads)
{
    return oracle_gate_up_fmt(x, ids, wg_q, wg_s, wu_q, wu_s, B, E, k, H, I, a, nthreads, FMT_MXFP8);
}

/*
 * Down half: out[b][h] = sum_j w[b][j] * sum_i Wd^[e_j][h][i] * a[b][j][i].
 * a: float64 [B][k][I]; w: float32 [B][k]; wd_q: uint8 [E][H][I] (MXFP8) or
 * [E][H][I/2] (MXFP4); wd_s: uint8 [E][H][I/32]; out: float64 [B][H].
 */
int oracle_down_fmt(const double *a, const int32_t *ids, const float *w,
                    const uint8_t *wd_q, const uint8_t *wd_s,
                    int B, int E, int k, int H, int I, double *out, int nthreads, int fmt)
{
    if (bad_shape(B, E, k, H, I) || (fmt != FMT_MXFP8 && fmt != FMT_MXFP4))
        return -2;
    const long rb = row_bytes(I, fmt);
    double tab[256];
    fill_e4m3_table(tab);
    set_threads(nthreads);
    const long nout = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long o = 0; o < nout; ++o) {
        const long h = o % H;
        const long b = o / H;
        double acc = 0.0;
        for (long j = 0; j < k; ++j) {
            const int e = ids[b * k + j];
            if (e < 0 || e >= E) {
                acc = NAN;
                break;
            }
            const size_t row = (size_t)e * (size_t)H + (size_t)h;
            const double d = mx_row_dot(tab, wd_q + row * (size_t)rb, wd_s + row * (size_t)(I / 32),
                                        a + (b * k + j) * I, I, fmt);
            acc += (double)w[b * k + j] * d;
        }
        out[o] = acc;
    }
    return 0;
}

int oracle_down(const double *a, const int32_t *ids, const float *w,
                const uint8_t *wd_q, const uint8_t *wd_s,
                int B, int E, int k, int H, int I, double *out, int nthreads)
{
    return oracle_down_fmt(a, ids, w, wd_q, wd_s, B, E, k, H, I, out, nthreads, FMT_MXFP8);
}

/* The whole layer. `a` may be NULL (scratch is then allocated here); when
 * given it receives the float64 intermediate [B][k][I]. */
int oracle_moe_decode_fmt(const uint16_t *x, const int32_t *ids, const float *w,
                          const uint8_t *wg_q, const uint8_t *wg_s,
                          const uint8_t *wu_q, const uint8_t *wu_s,
                          const uint8_t *wd_q, const uint8_t *wd_s,
                          int B, int E, int k, int H, int I,
                          double *out, double *a, int nthreads, int fmt)
{
    if (bad_shape(B, E, k, H, I) || (fmt != FMT_MXFP8 && fmt != FMT_MXFP4))
        return -2;
    double *scratch = NULL;
    if (!a) {
        scratch = (double *)malloc(sizeof(double) * (size_t)(B > 0 ? B : 1) * (size_t)k * (size_t)I);
        if (!scratch)
            return -1;
        a = scratch;
    }
    int rc = oracle_gate_up_fmt(x, ids, wg_q, wg_s, wu_q, wu_s, B, E, k, H, I, a, nthreads, fmt);
    if (rc == 0)
        rc = oracle_down_fmt(a, ids, w, wd_q, wd_s, B, E, k, H, I, out, nthreads, fmt);
    free(scratch);
    return rc;
}

int oracle_moe_decode(const uint16_t *x, const int32_t *ids, const float *w,
                      const uint8_t *wg_q, const uint8_t *wg_s,
                      const uint8_t *wu_q, const uint8_t *wu_s,
                      const uint8_t *wd_q, const uint8_t *wd_s,
                      int B, int E, int k, int H, int I,
                      double *out, double *a, int nthreads)
{
    return oracle_moe_decode_fmt(x, ids, w, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, B, E, k, H, I, out, a,
                                 nthreads, FMT_MXFP8);
}

/*
 * Router front-end: per token b, from float32 logits l[b][0..E):
 *   ids[b][0..k) = the k experts with the largest logits, in descending
 *     order, ties to the lower expert id (softmax is strictly increasing, so
 *     this is the top-k of the routing probabilities p = softmax(l));
 *   w[b][j] = p[ids[b][j]] / sum_{j'<k} p[ids[b][j']] * routed_scale
 *     = exp(l_j - m) / sum_{j'} exp(l_j' - m) * routed_scale, m = the largest
 *     logit (the renormalised top-k probabilities);
 *   then n_shared shared-expert slots: ids[b][k + s] = E + s, w = 1.
 * Output rows have k + n_shared entries. A NaN logit is never selected; when
 * fewer than k logits can be selected the remaining ids are -1 with weight
 * NaN. Weights computed in float64, stored as float32 (round to nearest).
 * Returns 0, or -2 on bad sizes (k < 1, k > E, n_shared < 0).
 */
int oracle_route(const float *logits, int B, int E, int k, int n_shared, double routed_scale,
                 int32_t *ids, float *w)
{
    if (B < 0 || E < 1 || k < 1 || k > E || n_shared < 0)
        return -2;
    const int kt = k + n_shared;
    char *taken = (char *)malloc((size_t)E);
    double *sel = (double *)malloc(sizeof(double) * (size_t)k);
    if (!taken || !sel) {
        free(taken);
        free(sel);
        return -1;
    }
    for (int b = 0; b < B; ++b) {
        const float *l = logits + (size_t)b * E;
        memset(taken, 0, (size_t)E);
        int nsel = 0;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e] || isnan(l[e]))
                    continue;
                if (best < 0 || l[e] > l[best])      /* strict: ties keep the lower id */
                    best = e;
            }
            ids[(size_t)b * kt + j] = best;
            if (best >= 0) {
                taken[best] = 1;
                sel[nsel++] = (double)l[best];
            }
        }
        double sum = 0.0;
        for (int j = 0; j < nsel; ++j)
            sum += exp(sel[j] - sel[0]);
        for (int j = 0; j < k; ++j)
            w[(size_t)b * kt + j] = j < nsel ? (float)(exp(sel[j] - sel[0]) / sum * routed_scale) : NAN;
        for (int s = 0; s < n_shared; ++s) {
            ids[(size_t)b * kt + k + s] = E + s;
            w[(size_t)b * kt + k + s] = 1.0f;
        }
    }
    free(taken);
    free(sel);
    return 0;
}

/* Threads an OpenMP region in this library will use for a given request. */
int oracle_threads(int nthreads)
{
    return set_threads(nthreads);
}
