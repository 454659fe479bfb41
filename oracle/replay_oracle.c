/*
 * replay_oracle.c -- plain, slow, float64 CPU oracle for the ReplaySSM decode
 * path.  TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
 * CPU-baseline leg of the benchmark load it; the HIP library never does, and
 * this file shares no code, header or table with it.
 *
 * What it computes is the plain definition.  The pages state that the
 * checkpoint-plus-buffer ("history") rewriting gives exactly the eager
 * result (page "ReplaySSM: Cachear Inputs, No Estado", section "La solucion",
 * last paragraph; page "ReplaySSM: Cache SSM Inputs, Not State" (arXiv
 * 2610.13778 abstract page), Abstract), so the oracle simply runs the eager
 * recurrence, token after token, in float64:
 *
 *   S_t = a_t S_{t-1} + dt_t (v_t k_t^T)          eq. "Forma resumen"
 *   y_t = S_t q_t                                  section "Los dos caminos"
 *
 * with S a P x N matrix per (sequence, head), v in R^P, k, q in R^N shared by
 * the heads of a group (section "Los dos caminos", last paragraph), and the
 * group of head h taken as floor(h*G/H) (contiguous groups; the pages do not
 * say how heads map to groups).
 *
 * The quantisers give the expected storage codes of a low-precision copy of
 * the state (Abstract: a low-precision copy serves outputs while a higher
 * precision one takes the updates).  Their rounding decisions are taken in
 * float32, the precision the copy is produced from:
 *   bf16     : 1 sign, 8 exponent, 7 mantissa bits; round to nearest, ties
 *              to an even mantissa.
 *   e4m3fn   : the OCP 8-bit float E4M3 (bias 7, 3 mantissa bits, no
 *              infinities, S.1111.111 is NaN, largest finite 448); round to
 *              nearest, ties to even, saturating to +-448.
 *   per-head : sigma = amax|x| / 448 in float32 (1 when amax is 0), and
 *              code = e4m3(x / sigma) with a correctly rounded float32 divide.
 *   e2m1     : the OCP 4-bit float E2M1 (bias 1, 1 mantissa bit, no
 *              infinities or NaN, largest 6); round to nearest, ties to even,
 *              saturating to +-6.
 *   MX blocks: 32 consecutive values of a head's row-major tile share a
 *              power-of-two scale X = 2^(floor(log2 amax) - 2) (2 = exponent
 *              of E2M1's largest value; X = 2^-127 when amax is 0, exponent
 *              clamped to -127..127), stored as its biased exponent byte
 *              (E8M0); code = e2m1(x / X), exact division.  Two codes per
 *              byte, the first in the low nibble.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Eager recurrence                                                           */
/* ------------------------------------------------------------------------ */

/*
 * Runs T eager steps for every (sequence, head).
 *   q, k : [T][B][G][N]   v : [T][B][H][P]   dt, a : [T][B][H]
 *   S    : [B][H][P][N]   in: the state before the first token; out: after
 *   y    : [T][B][H][P]   outputs
 */
void oracle_eager(int64_t T, int64_t B, int64_t H, int64_t G, int64_t P, int64_t N,
                  const double *q, const double *k, const double *v,
                  const double *dt, const double *a, double *S, double *y)
{
    int64_t bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < B * H; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        const int64_t g = (h * G) / H;
        double *St = S + bh * P * N;
        for (int64_t t = 0; t < T; ++t) {
            const double at = a[(t * B + b) * H + h];
            const double dtt = dt[(t * B + b) * H + h];
            const double *vt = v + ((t * B + b) * H + h) * P;
            const double *kt = k + ((t * B + b) * G + g) * N;
            const double *qt = q + ((t * B + b) * G + g) * N;
            double *yt = y + ((t * B + b) * H + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                double *row = St + p * N;
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    row[n] = at * row[n] + dtt * (vt[p] * kt[n]);
                    acc += row[n] * qt[n];
                }
                yt[p] = acc;
            }
        }
    }
}

/*
 * Gated DeltaNet layers (the second layer type the pages name beside Mamba-2:
 * page "ReplaySSM: Cache SSM Inputs, Not State", Abstract; page "ReplaySSM:
 * que cambia en los modelos hibridos de IA", section "Una integracion
 * concreta no cubre todas las opciones").  The pages print no equation for
 * it; this is the published gated delta rule (Yang, Kautz, Hatamizadeh,
 * "Gated Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025), with
 * S a P x N (value x key) matrix per (sequence, head):
 *
 *   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   y_t = S_t q_t
 *
 * Row p of S (s, in R^N) therefore takes
 *   s <- alpha_t (s - beta_t (s . k_t) k_t) + beta_t v_t[p] k_t
 * with (s . k_t) taken on the row before the update.  Layout as
 * oracle_eager; the dt slot carries beta_t and the a slot alpha_t.
 */
void oracle_eager_gdn(int64_t T, int64_t B, int64_t H, int64_t G, int64_t P, int64_t N,
                      const double *q, const double *k, const double *v,
                      const double *beta, const double *alpha, double *S, double *y)
{
    int64_t bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < B * H; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        const int64_t g = (h * G) / H;
        double *St = S + bh * P * N;
        for (int64_t t = 0; t < T; ++t) {
            const double al = alpha[(t * B + b) * H + h];
            const double be = beta[(t * B + b) * H + h];
            const double *vt = v + ((t * B + b) * H + h) * P;
            const double *kt = k + ((t * B + b) * G + g) * N;
            const double *qt = q + ((t * B + b) * G + g) * N;
            double *yt = y + ((t * B + b) * H + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                double *row = St + p * N;
                double sk = 0.0;
                for (int64_t n = 0; n < N; ++n) sk += row[n] * kt[n];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    row[n] = al * (row[n] - be * sk * kt[n]) + be * vt[p] * kt[n];
                    acc += row[n] * qt[n];
                }
                yt[p] = acc;
            }
        }
    }
}

/* Threads the OpenMP runtime will use for oracle_eager. */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the number of threads later oracle calls use (timing on one core). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* bf16                                                                      */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 pattern -> float32 value: the 16 bits are the top half of a float32. */
float oracle_bf16_decode(uint16_t c) { return f32_from_bits((uint32_t)c << 16); }

/* float32 -> bf16, nearest value, ties to the even pattern.  Candidates are
   the pattern toward zero and the next one away from zero; past the largest
   finite bf16 the next "value" is 2^128, which encodes as infinity. */
uint16_t oracle_bf16_encode(float x)
{
    uint32_t u = bits_from_f32(x);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);          /* quiet NaN, sign kept */
    uint16_t lo = (uint16_t)(u >> 16);                              /* toward zero */
    if ((u & 0xFFFFu) == 0) return lo;                              /* exact (incl. inf) */
    uint16_t hi = (uint16_t)(lo + 1);                               /* away from zero */
    double al = fabs((double)oracle_bf16_decode(lo));
    double ah = ((hi & 0x7FFFu) == 0x7F80u) ? ldexp(1.0, 128)
                                             : fabs((double)oracle_bf16_decode(hi));
    double ax = fabs((double)x);
    double dl = ax - al, dh = ah - ax;
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo & 1u) ? hi : lo;                                     /* tie: even pattern */
}

void oracle_bf16_encode_n(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_encode(x[i]);
}

void oracle_bf16_decode_n(const uint16_t *c, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_decode(c[i]);
}

/* ------------------------------------------------------------------------ */
/* OCP E4M3 (e4m3fn)                                                          */
/* ------------------------------------------------------------------------ */

/* code -> value, from the format: exponent field e (4 bits, bias 7), mantissa
   m (3 bits).  e == 0 is subnormal: m/8 * 2^-6.  0x7F / 0xFF are NaN. */
float oracle_e4m3_decode(uint8_t c)
{
    const int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    double mag;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(s ? -mag : mag);
}

/* Values of the non-negative finite codes 0x00..0x7E, increasing; filled
   once when the library is loaded. */
static float e4m3_table[127];

__attribute__((constructor)) static void e4m3_table_init(void)
{
    for (int c = 0; c < 127; ++c) e4m3_table[c] = oracle_e4m3_decode((uint8_t)c);
}

/* float32 -> e4m3fn: nearest finite value, ties to the even code, magnitudes
   above the largest finite value saturate to it; NaN -> 0x7F (sign kept). */
uint8_t oracle_e4m3_encode(float x)
{
    const float *table = e4m3_table;
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x)) return (uint8_t)(sign | 0x7F);
    double ax = fabs((double)x);
    if (ax >= (double)table[126]) return (uint8_t)(sign | 126);
    /* largest code with value <= ax (binary search over the sorted table) */
    int lo = 0, hi = 126;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if ((double)table[mid] <= ax) lo = mid; else hi = mid;
    }
    double dl = ax - (double)table[lo], dh = (double)table[hi] - ax;
    int c;
    if (dl < dh) c = lo;
    else if (dh < dl) c = hi;
    else c = (lo & 1) ? hi : lo;
    return (uint8_t)(sign | c);
}

void oracle_e4m3_encode_n(const float *x, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}

void oracle_e4m3_decode_n(const uint8_t *c, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}

/* Per-head quantisation of `heads` blocks of `n` float32 values each.
   scale[i] = amax_i / 448 (float32 divide), or 1 when amax_i == 0;
   codes    = e4m3(x / scale[i]) (float32 divide). */
void oracle_quant_heads_e4m3(const float *x, int64_t heads, int64_t n,
                             uint8_t *codes, float *scale)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < heads; ++i) {
        const float *xi = x + i * n;
        float amax = 0.0f;
        for (int64_t j = 0; j < n; ++j) {
            float m = fabsf(xi[j]);
            if (m > amax) amax = m;
        }
        const float s = (amax > 0.0f) ? amax / 448.0f : 1.0f;
        scale[i] = s;
        for (int64_t j = 0; j < n; ++j) codes[i * n + j] = oracle_e4m3_encode(xi[j] / s);
    }
}

/* ------------------------------------------------------------------------ */
/* OCP E2M1 (FP4) and MX block scaling                                       */
/* ------------------------------------------------------------------------ */

/* code (low 4 bits) -> value, from the format: sign, exponent e (2 bits,
   bias 1), mantissa m (1 bit); e == 0 is subnormal: m/2. */
float oracle_e2m1_decode(uint8_t c)
{
    const int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    const double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (float)(s ? -mag : mag);
}

/* value -> code: nearest of the eight magnitudes, ties to the even code,
   magnitudes above 6 saturate to 6.  The comparison is exact (double). */
uint8_t oracle_e2m1_encode(double x)
{
    const uint8_t sign = signbit(x) ? 0x8 : 0x0;
    const double ax = fabs(x);
    if (!(ax < 6.0)) return (uint8_t)(sign | 7);   /* saturate (NaN too) */
    int lo = 0;
    while (lo < 7 && (double)oracle_e2m1_decode((uint8_t)(lo + 1)) <= ax) ++lo;
    const double vl = oracle_e2m1_decode((uint8_t)lo), vh = oracle_e2m1_decode((uint8_t)(lo + 1));
    int c;
    if (ax - vl < vh - ax) c = lo;
    else if (vh - ax < ax - vl) c = lo + 1;
    else c = (lo & 1) ? lo + 1 : lo;
    return (uint8_t)(sign | c);
}

void oracle_e2m1_decode_n(const uint8_t *c, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e2m1_decode(c[i]);
}

void oracle_e2m1_encode_n(const double *x, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e2m1_encode(x[i]);
}

/* MX FP4 quantisation of nblk blocks of 32 float32 values:
   packed[16 * i + j] holds the codes of x[32 i + 2 j] (low nibble) and
   x[32 i + 2 j + 1] (high nibble); scale[i] = biased exponent of X_i. */
void oracle_quant_blocks_mxfp4(const float *x, int64_t nblk, uint8_t *packed, uint8_t *scale)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < nblk; ++i) {
        const float *xi = x + 32 * i;
        float amax = 0.0f;
        for (int j = 0; j < 32; ++j) {
            const float m = fabsf(xi[j]);
            if (m > amax) amax = m;
        }
        int se = -127;
        if (amax > 0.0f) {
            int e;
            (void)frexp((double)amax, &e);   /* amax = f 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
            se = (e - 1) - 2;
            if (se < -127) se = -127;
            if (se > 127) se = 127;
        }
        scale[i] = (uint8_t)(se + 127);
        const double X = ldexp(1.0, se);
        for (int j = 0; j < 16; ++j) {
            const uint8_t c0 = oracle_e2m1_encode((double)xi[2 * j] / X);
            const uint8_t c1 = oracle_e2m1_encode((double)xi[2 * j + 1] / X);
            packed[16 * i + j] = (uint8_t)(c0 | (c1 << 4));
        }
    }
}

/* values of MX FP4 blocks: out[32 i + k] = e2m1(code) * 2^(scale[i] - 127) */
void oracle_dequant_blocks_mxfp4(const uint8_t *packed, const uint8_t *scale, int64_t nblk, float *out)
{
    for (int64_t i = 0; i < nblk; ++i) {
        const double X = ldexp(1.0, (int)scale[i] - 127);
        for (int j = 0; j < 16; ++j) {
            const uint8_t b = packed[16 * i + j];
            out[32 * i + 2 * j] = (float)(oracle_e2m1_decode(b & 0xF) * X);
            out[32 * i + 2 * j + 1] = (float)(oracle_e2m1_decode(b >> 4) * X);
        }
    }
}
