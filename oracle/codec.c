/*
 * ORACLE -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow CPU reference for the FP8 parts of the packed QKV projection.
 * Only tests/, the smoke check and the CPU-baseline leg of bench.py load this
 * library.  It shares no source, header, table or constant generator with the
 * GPU library; nothing in the product path may link or call it.
 *
 * What it computes (sources: the "96 is enough" page, section "The change",
 * and the PR #344 page, section "Changes"):
 *   - the projection runs in FP8.  The pages never name the FP8 format; the
 *     reading taken here is OCP FP8 E4M3 ("e4m3fn": bias 7, 3 mantissa bits,
 *     no infinities, 0x7F/0xFF are NaN, largest finite 448);
 *   - one per-tensor scale derived from the tensor's absolute maximum
 *     (amax), covering the whole logical W_packed = [W_q | W_k | W_v] without
 *     materialising the concatenation (PR #344, "Changes").
 *
 * Readings where the pages are silent:
 *   - encode = round to nearest, ties to the code with an even last bit,
 *     saturating at +-448, sign kept (so -0 and negative underflow give 0x80);
 *   - scale s = fl32(amax / 448), inverse inv = fl32(448 / amax), codes are
 *     enc(fl32(v * inv)) (a product, not a quotient);
 *   - amax == 0, or 448/amax not finite  ->  s = inv = 1;
 *   - a NaN or infinite amax is reported as an error (return value 1).
 *
 * Two independent encoders are provided on purpose: one by exponent /
 * mantissa arithmetic, one by searching the sorted table of finite values.
 * The tests require them to agree on every fp32 bit pattern.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math: IEEE behaviour of
 * float multiply/divide and of nearbyint() is part of the definition).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------- decode */

/* Value of an e4m3 code.  sign s (bit 7), exponent e (bits 6..3, bias 7),
 * mantissa m (bits 2..0).  e == 0: subnormal, 2^-6 * m/8.  Otherwise
 * 2^(e-7) * (1 + m/8).  e == 15 and m == 7 is NaN (0x7F, 0xFF). */
double orc_e4m3_decode(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

void orc_e4m3_decode_table(double out[256])
{
    for (int c = 0; c < 256; ++c)
        out[c] = orc_e4m3_decode((uint8_t)c);
}

/* ------------------------------------------------- encode, by arithmetic */

/* Nearest e4m3 code to v; ties to the even code; saturating; sign kept.
 * Works on the exact double value of v and uses nearbyint(), which rounds
 * half to even in the default rounding mode. */
uint8_t orc_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    if (a < ldexp(1.0, -6)) {
        /* subnormal grid: multiples of 2^-9.  A result of 8 is the smallest
         * normal, 2^-6, whose code is also 8 (e = 1, m = 0). */
        double r = nearbyint(a / ldexp(1.0, -9));
        return (uint8_t)(sign | (uint8_t)r);
    }
    int ex;
    (void)frexp(a, &ex);         /* a = f * 2^ex with f in [0.5, 1) */
    int e = ex - 1;              /* a = (2f) * 2^e with 2f in [1, 2) */
    double r = nearbyint(ldexp(a, 3 - e)); /* significand in eighths: [8, 16] */
    if (r == 16.0) {             /* rounding carried into the next binade */
        r = 8.0;
        e += 1;
    }
    int efield = e + 7;          /* 1..15; a < 448 keeps (15, 7) unreachable */
    return (uint8_t)(sign | (efield << 3) | ((int)r - 8));
}

/* ------------------------------------------- encode, by searching a table */

static double g_pos_values[127]; /* finite non-negative values, codes 0..126 */
static int g_table_ready = 0;

static void build_pos_table(void)
{
    if (g_table_ready)
        return;
    for (int c = 0; c < 127; ++c)
        g_pos_values[c] = orc_e4m3_decode((uint8_t)c);
    g_table_ready = 1;
}

/* The table is increasing in the code for non-negative codes (checked by the
 * tests).  Find the two neighbours of |v| by bisection and keep the nearer;
 * on a tie keep the even code.  Beyond 448 the nearest finite code is 126. */
uint8_t orc_e4m3_encode_search(float v)
{
    build_pos_table();
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    if (a >= g_pos_values[126])
        return (uint8_t)(sign | 126);
    int lo = 0, hi = 126;        /* invariant: table[lo] <= a < table[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g_pos_values[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - g_pos_values[lo];
    double dhi = g_pos_values[hi] - a;
    int pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | pick);
}

/* Compare the two encoders over fp32 bit patterns [begin, end).  NaN
 * patterns are skipped.  Returns the number of disagreements; the first one
 * found is stored in *first_bad (if any). */
int64_t orc_e4m3_encoders_disagree(uint64_t begin, uint64_t end, uint32_t* first_bad)
{
    build_pos_table();
    int64_t bad = 0;
    uint64_t first = UINT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : first)
    for (int64_t i = (int64_t)begin; i < (int64_t)end; ++i) {
        uint32_t bits = (uint32_t)i;
        float v;
        memcpy(&v, &bits, 4);
        if (isnan(v))
            continue;
        if (orc_e4m3_encode(v) != orc_e4m3_encode_search(v)) {
            bad += 1;
            if ((uint64_t)i < first)
                first = (uint64_t)i;
        }
    }
    if (first_bad)
        *first_bad = (first == UINT64_MAX) ? 0u : (uint32_t)first;
    return bad;
}

void orc_e4m3_encode_array(const float* v, int64_t n, uint8_t* codes)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        codes[i] = orc_e4m3_encode(v[i]);
}

/* ------------------------------------------------ per-tensor quantizer */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float bf16_bits_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* scale and inverse scale from an amax; returns 1 when amax is not finite */
static int scales_from_amax(float amax, float* s, float* inv)
{
    if (!isfinite(amax)) {
        *s = 1.0f;
        *inv = 1.0f;
        return 1;
    }
    float i = 448.0f / amax;     /* IEEE fp32 division */
    if (amax == 0.0f || !isfinite(i)) {
        *s = 1.0f;
        *inv = 1.0f;
        return 0;
    }
    *s = amax / 448.0f;
    *inv = i;
    return 0;
}

static float amax_f32(const float* v, int64_t n)
{
    float m = 0.0f;
    int nan_seen = 0;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (isnan(a))
            nan_seen = 1;
        else if (a > m)
            m = a;
    }
    return nan_seen ? NAN : m;
}

/* Quantize n fp32 values with one per-tensor scale.
 * scales_out[0] = s, scales_out[1] = inv.  Returns 0, or 1 for a non-finite
 * amax (codes are still written with s = inv = 1). */
int orc_quantize_f32(const float* v, int64_t n, uint8_t* codes, float* scales_out)
{
    float amax = amax_f32(v, n);
    float s, inv;
    int rc = scales_from_amax(amax, &s, &inv);
    for (int64_t i = 0; i < n; ++i) {
        float scaled = v[i] * inv;  /* fp32 product */
        codes[i] = orc_e4m3_encode(scaled);
    }
    scales_out[0] = s;
    scales_out[1] = inv;
    return rc;
}

/* Same, for bf16 input given as raw 16-bit patterns. */
int orc_quantize_bf16(const uint16_t* v, int64_t n, uint8_t* codes, float* scales_out)
{
    float amax = 0.0f;
    int nan_seen = 0;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(bf16_bits_to_f32(v[i]));
        if (isnan(a))
            nan_seen = 1;
        else if (a > amax)
            amax = a;
    }
    if (nan_seen)
        amax = NAN;
    float s, inv;
    int rc = scales_from_amax(amax, &s, &inv);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float scaled = bf16_bits_to_f32(v[i]) * inv;
        codes[i] = orc_e4m3_encode(scaled);
    }
    scales_out[0] = s;
    scales_out[1] = inv;
    return rc;
}

/* The logical packed weight W_packed[d][n], n over [Q heads | K heads |
 * V heads], read from three separate row-major pieces without building the
 * concatenation ("96 is enough", "The change"; PR #344, "Changes").  One
 * scale for the whole pack.  The same codes are written twice:
 * w_packed[d][n] (D rows of N) and w_packed_t[n][d] (N rows of D). */
int orc_pack_quantize(int32_t D, int32_t H, int32_t d_qk, int32_t d_v,
                      const float* wq, int64_t ldq, const float* wk, int64_t ldk,
                      const float* wv, int64_t ldv,
                      uint8_t* w_packed, uint8_t* w_packed_t, float* scales_out)
{
    int64_t nq = (int64_t)H * d_qk;
    int64_t nv = (int64_t)H * d_v;
    int64_t N = 2 * nq + nv;
    float amax = 0.0f;
    int nan_seen = 0;
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t n = 0; n < N; ++n) {
            float w = (n < nq) ? wq[d * ldq + n]
                    : (n < 2 * nq) ? wk[d * ldk + (n - nq)]
                    : wv[d * ldv + (n - 2 * nq)];
            float a = fabsf(w);
            if (isnan(a))
                nan_seen = 1;
            else if (a > amax)
                amax = a;
        }
    }
    if (nan_seen)
        amax = NAN;
    float s, inv;
    int rc = scales_from_amax(amax, &s, &inv);
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t n = 0; n < N; ++n) {
            float w = (n < nq) ? wq[d * ldq + n]
                    : (n < 2 * nq) ? wk[d * ldk + (n - nq)]
                    : wv[d * ldv + (n - 2 * nq)];
            uint8_t c = orc_e4m3_encode(w * inv);
            w_packed[d * N + n] = c;
            w_packed_t[n * D + d] = c;
        }
    }
    scales_out[0] = s;
    scales_out[1] = inv;
    return rc;
}

/* ------------------------------------------------------ bf16 rounding */

/* Round a double to the nearest bf16 (8 significant bits), ties to even,
 * directly from the double (no intermediate fp32 rounding, which could
 * round twice).  Overflow gives +-inf; NaN gives a quiet NaN. */
uint16_t orc_round_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    double a = fabs(x);
    double r;
    if (a == 0.0) {
        r = 0.0;
    } else if (a < ldexp(1.0, -126)) {
        r = nearbyint(a / ldexp(1.0, -133)) * ldexp(1.0, -133); /* subnormal grid */
    } else {
        int ex;
        frexp(a, &ex);                                   /* a in [2^(ex-1), 2^ex) */
        double q = ldexp(1.0, ex - 8);                   /* spacing of 8-bit significands */
        r = nearbyint(a / q) * q;
    }
    float f = (r >= ldexp(1.0, 128)) ? INFINITY : (float)r; /* exact when finite */
    if (signbit(x))
        f = -f;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

void orc_round_bf16_array(const double* x, int64_t n, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_round_bf16(x[i]);
}

/* Round a double to fp32 (the C conversion rounds to nearest even). */
void orc_round_f32_array(const double* x, int64_t n, float* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)x[i];
}

/* ================================================================ e5m2
 *
 * Optional gradient format (the attention-ready variants: FP8 gradients in
 * OCP FP8 E5M2, whose wider exponent range suits gradients).  OCP E5M2:
 * sign bit 7, exponent bits 6..2 (bias 15), mantissa bits 1..0; exponent 0
 * is subnormal (2^-14 * m/4); exponent 31 holds infinity (m = 0) and NaN
 * (m != 0); the largest finite value is 1.75 * 2^15 = 57344.
 *
 * Readings, as for e4m3: round to nearest, ties to even, saturating at
 * +-57344 (never infinity), sign kept; per-tensor scale
 * s = fl32(amax / 57344), inv = fl32(57344 / amax), codes enc(fl32(v * inv)).
 */

double orc_e5m2_decode(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 2) & 31;
    int m = code & 3;
    double mag;
    if (e == 31)
        mag = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        mag = ldexp((double)m / 4.0, -14);
    else
        mag = ldexp(1.0 + (double)m / 4.0, e - 15);
    if (isnan(mag))
        return NAN;
    return s ? -mag : mag;
}

void orc_e5m2_decode_table(double out[256])
{
    for (int c = 0; c < 256; ++c)
        out[c] = orc_e5m2_decode((uint8_t)c);
}

/* Nearest e5m2 code by exponent / mantissa arithmetic (see orc_e4m3_encode). */
uint8_t orc_e5m2_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    if (a >= 57344.0)
        return (uint8_t)(sign | 0x7B);
    if (a < ldexp(1.0, -14)) {
        /* subnormal grid: multiples of 2^-16; 4 is the smallest normal */
        double r = nearbyint(a / ldexp(1.0, -16));
        return (uint8_t)(sign | (uint8_t)r);
    }
    int ex;
    (void)frexp(a, &ex);
    int e = ex - 1;                          /* a = (2f) * 2^e, 2f in [1, 2) */
    double r = nearbyint(ldexp(a, 2 - e));   /* significand in quarters: [4, 8] */
    if (r == 8.0) {
        r = 4.0;
        e += 1;
    }
    int efield = e + 15;                     /* 1..30 below 57344 */
    return (uint8_t)(sign | (efield << 2) | ((int)r - 4));
}

static double g_pos5[124];                   /* finite non-negative values, codes 0..0x7B */
static int g_pos5_ready = 0;

static void build_pos5(void)
{
    if (g_pos5_ready)
        return;
    for (int c = 0; c < 124; ++c)
        g_pos5[c] = orc_e5m2_decode((uint8_t)c);
    g_pos5_ready = 1;
}

/* Nearest e5m2 code by bisection over the sorted finite values. */
uint8_t orc_e5m2_encode_search(float v)
{
    build_pos5();
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    if (a >= g_pos5[123])
        return (uint8_t)(sign | 123);
    int lo = 0, hi = 123;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g_pos5[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - g_pos5[lo];
    double dhi = g_pos5[hi] - a;
    int pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | pick);
}

int64_t orc_e5m2_encoders_disagree(uint64_t begin, uint64_t end, uint32_t* first_bad)
{
    build_pos5();
    int64_t bad = 0;
    uint64_t first = UINT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : first)
    for (int64_t i = (int64_t)begin; i < (int64_t)end; ++i) {
        uint32_t bits = (uint32_t)i;
        float v;
        memcpy(&v, &bits, 4);
        if (isnan(v))
            continue;
        if (orc_e5m2_encode(v) != orc_e5m2_encode_search(v)) {
            bad += 1;
            if ((uint64_t)i < first)
                first = (uint64_t)i;
        }
    }
    if (first_bad)
        *first_bad = (first == UINT64_MAX) ? 0u : (uint32_t)first;
    return bad;
}

void orc_e5m2_encode_array(const float* v, int64_t n, uint8_t* codes)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        codes[i] = orc_e5m2_encode(v[i]);
}

/* Per-tensor e5m2 quantisation of bf16 patterns; as orc_quantize_bf16 with
 * 57344 in place of 448. */
int orc_quantize_bf16_e5m2(const uint16_t* v, int64_t n, uint8_t* codes, float* scales_out)
{
    float amax = 0.0f;
    int nan_seen = 0;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(bf16_bits_to_f32(v[i]));
        if (isnan(a))
            nan_seen = 1;
        else if (a > amax)
            amax = a;
    }
    if (nan_seen)
        amax = NAN;
    float s = 1.0f, inv = 1.0f;
    int rc = 0;
    if (!isfinite(amax)) {
        rc = 1;
    } else {
        float i = 57344.0f / amax;
        if (amax != 0.0f && isfinite(i)) {
            s = amax / 57344.0f;
            inv = i;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        codes[i] = orc_e5m2_encode(bf16_bits_to_f32(v[i]) * inv);
    scales_out[0] = s;
    scales_out[1] = inv;
    return rc;
}
