/*
 * nvfp4_oracle.c -- plain, slow CPU definition of every result the NVFP4 hot path computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or call this file:
 * only the test-suite, the smoke check and the CPU-baseline leg of the benchmark do.  It shares
 * no code, header, table or constant generator with the HIP library, and it includes nothing
 * but libc.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared (fp32 steps must be
 * single IEEE binary32 operations with round-to-nearest-even; no FMA contraction, no flush).
 *
 * Citation keys (the three web pages this follows):
 *   [P1] "Entrenamiento de Modelos de Lenguaje con 4 Bits de Precision" (focoia.com.mx)
 *   [P2] "FP4 All the Way: Formacion totalmente cuantificada de LLM" (slashpage.com summary of
 *        Chmiel, Fishman, Banner, Soudry)
 *   [P3] "I ricercatori di Nvidia sbloccano il tutorial LLM a 8 bit che corrisponde alle
 *        prestazioni a 4 bit" (massacarraranews.com)
 * Where the pages are silent the reading taken is named in the comment ("reading: ...").
 *
 * Pinned within rounding rather than bit for bit (the orders are readings; their results equal
 * the exact-arithmetic definitions except within a few fp32 roundings of a rounding midpoint):
 *   - the fp32 operation order of the block scale step (t = amax_b * k1, enc = s_enc / scale);
 *     the tensor scales themselves ARE pinned as single correctly rounded divisions;
 *   - the butterfly order of the 16-point Hadamard transform (its matrix IS pinned exactly).
 * The Philox generator is pinned by its published known answers, and the two maps that draw
 * from it are pinned by the properties a random draw must have (balanced, pairwise independent
 * Hadamard signs; an injective, pairwise independent element -> SR draw map).  WHICH output
 * bits each map takes is a convention with no observable consequence beyond those properties.
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>
#include <float.h>
#include <string.h>
#include <stdlib.h>

#define OR_OK 0
#define OR_ERR_SHAPE (-2)
#define OR_ERR_NONFINITE (-3)
#define OR_ERR_ARG (-4)

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_RNE = 0, OR_SR = 1 };
enum { OR_1x16 = 0, OR_16x16 = 1 };

/* ------------------------------------------------------------------------------------------ */
/* Element format E2M1 [P1 Caracteristicas del Formato NVFP4]: 1 sign, 2 exponent, 1 mantissa   */
/* bit.  Exponent bias 1 (the standard minifloat rule that puts 1.0 at exponent field 1).        */
/* A zero exponent field is the subnormal row: value = mantissa * 2^(1-bias) * 1/2.              */
/* ------------------------------------------------------------------------------------------ */
double or_e2m1_value(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag;
    if (e == 0)
        mag = 0.5 * (double)m;                     /* 2^(1-1) * (0 + m/2) */
    else
        mag = ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* Round-to-nearest onto the E2M1 grid, the forward-pass rounding [P2 Describir].  Reading:
 * ties go to the even code (mantissa bit 0), |z| beyond 6 saturates to 6, and the sign is kept
 * (a negative value that rounds to zero gives code 0x8).  Written as the plain definition:
 * the nearest of the eight magnitudes. */
unsigned or_e2m1_rne(float z)
{
    double a = fabs((double)z);
    if (a > 6.0) a = 6.0;            /* beyond the grid the nearest value is its end point */
    unsigned best = 0;
    double bestd = INFINITY;
    for (unsigned c = 0; c < 8; ++c) {
        double d = fabs(a - or_e2m1_value(c));
        if (d < bestd || (d == bestd && (c & 1u) == 0)) {
            bestd = d;
            best = c;
        }
    }
    return (signbit(z) ? 8u : 0u) | best;
}

/* Stochastic rounding onto the E2M1 grid [P2 Describir: backward and update passes;
 * P1 Metodologia: stochastic rounding on gradients].  Reading: with lo <= |z| < hi the two
 * neighbouring grid magnitudes, round up with probability p = (|z|-lo)/(hi-lo); the event is
 * u < p with u = r16 / 2^16 drawn from a 16-bit uniform.  |z| >= 6 gives 6; sign kept. */
unsigned or_e2m1_sr(float z, unsigned r16)
{
    double a = fabs((double)z);
    unsigned idx;
    if (a >= 6.0) {
        idx = 7;
    } else {
        unsigned lo = 0;
        for (unsigned c = 0; c < 8; ++c)
            if (or_e2m1_value(c) <= a) lo = c;
        double vlo = or_e2m1_value(lo), vhi = or_e2m1_value(lo + 1);
        double p = (a - vlo) / (vhi - vlo);
        double u = (double)(r16 & 0xFFFFu) / 65536.0;
        idx = (u < p) ? lo + 1 : lo;
    }
    return (signbit(z) ? 8u : 0u) | idx;
}

/* ------------------------------------------------------------------------------------------ */
/* Scale format E4M3 [P1 Caracteristicas: one E4M3 factor per 16-element block].  Reading: the */
/* OCP "E4M3FN" variant: bias 7, no infinities, 0x7F/0xFF NaN, largest finite 448.  Block     */
/* scales are non-negative, so only bytes 0x00..0x7E are ever produced.                        */
/* ------------------------------------------------------------------------------------------ */
double or_e4m3_value(unsigned b)
{
    unsigned s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);          /* subnormal: 2^(1-7) * m/8 */
    else
        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* Round-to-nearest-even, saturating, of a non-negative fp32 onto E4M3: the nearest of the 127
 * finite non-negative values, ties to the even byte; anything above 448 becomes 448. */
unsigned or_e4m3_rne_sat(float t)
{
    double a = (double)t;
    if (a > 448.0) a = 448.0;        /* beyond the grid the nearest value is its end point */
    unsigned best = 0;
    double bestd = INFINITY;
    for (unsigned b = 0; b <= 0x7E; ++b) {
        double d = fabs(a - or_e4m3_value(b));
        if (d < bestd || (d == bestd && (b & 1u) == 0)) {
            bestd = d;
            best = b;
        }
    }
    return best;
}

/* ------------------------------------------------------------------------------------------ */
/* Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: */
/* as easy as 1, 2, 3", SC'11).  The pages name no generator; reading: Philox keyed by the      */
/* caller's 64-bit seed, counter = element index / 8, so results are reproducible.             */
/* ------------------------------------------------------------------------------------------ */
void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;     /* round multipliers */
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;     /* Weyl key increments */
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* 16-bit uniform for element idx of an output tensor (idx = row * K + k in the quantized
 * tensor's own coordinates).  Reading: key = seed, counter = (idx >> 3, 0, 0); the eight
 * elements sharing a counter take the 16-bit halves of the four output words in order. */
unsigned or_sr_bits(uint64_t seed, uint64_t idx)
{
    uint64_t j = idx >> 3;
    uint32_t ctr[4] = { (uint32_t)j, (uint32_t)(j >> 32), 0u, 0u };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t out[4];
    or_philox4x32_10(ctr, key, out);
    uint32_t w = out[(idx & 7u) >> 1];
    return (idx & 1u) ? (w >> 16) : (w & 0xFFFFu);
}

/* Array forms of the scalar codecs above (each element is one call of the scalar function). */
void or_e2m1_rne_n(const float *z, int64_t n, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)or_e2m1_rne(z[i]);
}

void or_e2m1_sr_n(const float *z, const uint32_t *r16, int64_t n, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)or_e2m1_sr(z[i], r16[i]);
}

void or_e4m3_rne_sat_n(const float *t, int64_t n, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)or_e4m3_rne_sat(t[i]);
}

void or_sr_bits_n(uint64_t seed, const uint64_t *idx, int64_t n, uint32_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = or_sr_bits(seed, idx[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* Input access and bf16 rounding.                                                             */
/* ------------------------------------------------------------------------------------------ */
static float bf16_bits_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float load_elem(const void *x, int dtype, int64_t i)
{
    if (dtype == OR_BF16) return bf16_bits_to_f32(((const uint16_t *)x)[i]);
    return ((const float *)x)[i];
}

/* fp32 -> bf16, round to nearest with ties to the even 16-bit pattern (the conversion the GPU
 * uses for bf16 outputs).  Finite inputs only. */
uint16_t or_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t keep = u >> 16, rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1;
    return (uint16_t)keep;
}

/* ------------------------------------------------------------------------------------------ */
/* Two-level scaling [P3 Come funziona NVFP4?: a multi-level scaling copes with outliers].     */
/* Reading: a per-tensor fp32 level maps the tensor amax A onto the largest product of the two */
/* formats, 6 * 448 = 2688, so the block holding A gets scale 448 and a code of 6.             */
/*   k1 = 448 / A   (turns a block amax into its E4M3 scale target)                            */
/*   s_enc = 2688 / A, s_dec = A / 2688 (the stored per-tensor decode scale)                   */
/* each a single correctly rounded fp32 division.  A below 2^-100 (zero included) is treated   */
/* as zero: k1 = 448, s_enc = s_dec = 1, which sends every block scale to 0 and every code to  */
/* +-0, and keeps all later steps finite.                                                      */
/* ------------------------------------------------------------------------------------------ */
void or_tensor_scales(float A, float out3[3])
{
    const float tiny = 0x1p-100f;
    if (!(A >= tiny)) {
        out3[0] = 448.0f; out3[1] = 1.0f; out3[2] = 1.0f;
        return;
    }
    out3[0] = 448.0f / A;
    out3[1] = 2688.0f / A;
    out3[2] = A / 2688.0f;
}

/* Block step for one block with amax ab: returns the scale byte and the element encode
 * factor.  Reading: t = fl(ab * k1) rounded RNE-saturating to E4M3; the encode factor is
 * fl(s_enc / scale) (0 for a zero scale, which sends the block to +-0). */
static void block_scale(float ab, const float ts[3], unsigned *scale_byte, float *enc)
{
    float t = ab * ts[0];
    unsigned sb = or_e4m3_rne_sat(t);
    *scale_byte = sb;
    if (sb == 0) {
        *enc = 0.0f;
    } else {
        float dec = (float)or_e4m3_value(sb);      /* exact: every E4M3 value is an fp32 */
        *enc = ts[1] / dec;
    }
}

static void put_nibble(uint8_t *codes, int64_t row_bytes, int64_t r, int64_t c, unsigned v)
{
    uint8_t *p = codes + r * row_bytes + (c >> 1);
    if (c & 1) *p = (uint8_t)((*p & 0x0Fu) | ((v & 0xFu) << 4));
    else       *p = (uint8_t)((*p & 0xF0u) | (v & 0xFu));
}

static unsigned get_nibble(const uint8_t *codes, int64_t row_bytes, int64_t r, int64_t c)
{
    uint8_t b = codes[r * row_bytes + (c >> 1)];
    return (c & 1) ? (b >> 4) : (b & 0xFu);
}

/* ------------------------------------------------------------------------------------------ */
/* Per-tensor amax: exact max |x| over [rows x cols] with row stride ld (elements).            */
/* ------------------------------------------------------------------------------------------ */
int or_amax(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld, float *amax)
{
    float A = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float v = load_elem(x, dtype, r * ld + c);
            if (!isfinite(v)) return OR_ERR_NONFINITE;
            float a = fabsf(v);
            if (a > A) A = a;
        }
    *amax = A;
    return OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* 1D NVFP4 quantize [P1 Caracteristicas: 16 contiguous elements share one E4M3 scale;         */
/* P2 Describir: round-to-nearest forward, stochastic rounding on gradients].                  */
/* x: [rows x cols], cols % 16 == 0, row stride ld.  Out: codes [rows x cols/2] (element 2j in  */
/* the low nibble), scales [rows x cols/16], amax and s_dec.  amax_in != NULL supplies A.       */
/* ------------------------------------------------------------------------------------------ */
int or_quantize_1d(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                   const float *amax_in, int rounding, uint64_t seed,
                   uint8_t *codes, uint8_t *scales, float *amax_out, float *s_dec_out)
{
    if (cols % 16 != 0 || rows < 0 || cols < 0 || ld < cols) return OR_ERR_SHAPE;
    float A;
    if (amax_in) A = *amax_in;
    else {
        int rc = or_amax(x, dtype, rows, cols, ld, &A);
        if (rc) return rc;
    }
    float ts[3];
    or_tensor_scales(A, ts);
    int64_t nb = cols / 16;
    int err = 0;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            float y[16], ab = 0.0f;
            for (int i = 0; i < 16; ++i) {
                y[i] = load_elem(x, dtype, r * ld + b * 16 + i);
                if (!isfinite(y[i])) err = 1;
                if (fabsf(y[i]) > ab) ab = fabsf(y[i]);
            }
            unsigned sb;
            float enc;
            block_scale(ab, ts, &sb, &enc);
            scales[r * nb + b] = (uint8_t)sb;
            for (int i = 0; i < 16; ++i) {
                float z = y[i] * enc;
                int64_t k = b * 16 + i;
                unsigned code = (rounding == OR_SR)
                    ? or_e2m1_sr(z, or_sr_bits(seed, (uint64_t)(r * cols + k)))
                    : or_e2m1_rne(z);
                put_nibble(codes, cols / 2, r, k, code);
            }
        }
    }
    if (err) return OR_ERR_NONFINITE;
    if (amax_out) *amax_out = A;
    if (s_dec_out) *s_dec_out = ts[2];
    return OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* 2D NVFP4 quantize for weights [P1 Metodologia: two-dimensional block scaling for weights].  */
/* Reading: one E4M3 scale per 16x16 tile anchored at (0,0); rounding RNE (weights are forward */
/* operands).  codes [rows x cols/2], scales [rows/16 x cols/16]; optionally the transposed    */
/* copy: codes_t [cols x rows/2] holding the same codes at transposed positions and scales_t   */
/* [cols/16 x rows/16].                                                                        */
/* ------------------------------------------------------------------------------------------ */
int or_quantize_2d(const void *w, int dtype, int64_t rows, int64_t cols, int64_t ld,
                   const float *amax_in, uint8_t *codes, uint8_t *scales,
                   uint8_t *codes_t, uint8_t *scales_t, float *amax_out, float *s_dec_out)
{
    if (rows % 16 != 0 || cols % 16 != 0 || rows < 0 || cols < 0 || ld < cols) return OR_ERR_SHAPE;
    float A;
    if (amax_in) A = *amax_in;
    else {
        int rc = or_amax(w, dtype, rows, cols, ld, &A);
        if (rc) return rc;
    }
    float ts[3];
    or_tensor_scales(A, ts);
    int64_t tr = rows / 16, tc = cols / 16;
    int err = 0;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < tr; ++i) {
        for (int64_t j = 0; j < tc; ++j) {
            float ab = 0.0f;
            for (int a = 0; a < 16; ++a)
                for (int b = 0; b < 16; ++b) {
                    float v = load_elem(w, dtype, (i * 16 + a) * ld + j * 16 + b);
                    if (!isfinite(v)) err = 1;
                    if (fabsf(v) > ab) ab = fabsf(v);
                }
            unsigned sb;
            float enc;
            block_scale(ab, ts, &sb, &enc);
            scales[i * tc + j] = (uint8_t)sb;
            if (scales_t) scales_t[j * tr + i] = (uint8_t)sb;
            for (int a = 0; a < 16; ++a)
                for (int b = 0; b < 16; ++b) {
                    int64_t r = i * 16 + a, c = j * 16 + b;
                    float z = load_elem(w, dtype, r * ld + c) * enc;
                    unsigned code = or_e2m1_rne(z);
                    put_nibble(codes, cols / 2, r, c, code);
                    if (codes_t) put_nibble(codes_t, rows / 2, c, r, code);
                }
        }
    }
    if (err) return OR_ERR_NONFINITE;
    if (amax_out) *amax_out = A;
    if (s_dec_out) *s_dec_out = ts[2];
    return OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Random Hadamard transform [P1 Metodologia: random Hadamard transforms].  Reading: size 16,  */
/* Sylvester matrix H16 (H[i][j] = (-1)^popcount(i & j)), a random diagonal sign matrix D      */
/* applied first, normalisation 1/4 so that (H D / 4) is orthogonal; applied to the two wgrad  */
/* operands along the token (reduction) dimension, in 16-token chunks that coincide with the   */
/* NVFP4 blocks.  Signs: d_j = -1 iff bit j of word 0 of Philox(key = sign_seed, counter 0).   */
/* ------------------------------------------------------------------------------------------ */
void or_rht_signs(uint64_t sign_seed, int d[16])
{
    uint32_t ctr[4] = {0u, 0u, 0u, 0u};
    uint32_t key[2] = { (uint32_t)sign_seed, (uint32_t)(sign_seed >> 32) };
    uint32_t out[4];
    or_philox4x32_10(ctr, key, out);
    for (int j = 0; j < 16; ++j) d[j] = ((out[0] >> j) & 1u) ? -1 : 1;
}

/* In place: x <- (1/4) H16 D x, computed with the fast Walsh-Hadamard butterflies in the
 * fixed order h = 1, 2, 4, 8 (each a single fp32 add or subtract), then one multiply by 1/4. */
void or_rht16(float x[16], const int d[16])
{
    for (int i = 0; i < 16; ++i)
        if (d[i] < 0) x[i] = -x[i];
    for (int h = 1; h < 16; h <<= 1)
        for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
                float a = x[i], b = x[i + h];
                x[i] = a + b;
                x[i + h] = a - b;
            }
    for (int i = 0; i < 16; ++i) x[i] = 0.25f * x[i];
}

/* amax of the transformed tensor (reading: the amax of what is actually encoded). */
int or_hadamard_amax(const void *x, int dtype, int64_t T, int64_t F, int64_t ld,
                     uint64_t sign_seed, float *amax)
{
    if (T % 16 != 0 || ld < F) return OR_ERR_SHAPE;
    int d[16];
    or_rht_signs(sign_seed, d);
    float A = 0.0f;
    for (int64_t f = 0; f < F; ++f)
        for (int64_t c = 0; c < T / 16; ++c) {
            float y[16];
            for (int i = 0; i < 16; ++i) {
                y[i] = load_elem(x, dtype, (c * 16 + i) * ld + f);
                if (!isfinite(y[i])) return OR_ERR_NONFINITE;
            }
            or_rht16(y, d);
            for (int i = 0; i < 16; ++i)
                if (fabsf(y[i]) > A) A = fabsf(y[i]);
        }
    *amax = A;
    return OR_OK;
}

/* The transformed tensor itself, transposed: y [F x T] fp32 with y[f][16c .. 16c + 15] =
 * (1/4) H16 D x[16c .. 16c + 15][f] (or_rht16).  This is the tensor the Hadamard quantizer
 * encodes; the quantization-noise diagnostic of that quantizer compares against it. */
int or_hadamard_transform(const void *x, int dtype, int64_t T, int64_t F, int64_t ld,
                          uint64_t sign_seed, float *y_out)
{
    if (T % 16 != 0 || T < 0 || F < 0 || ld < F) return OR_ERR_SHAPE;
    int d[16];
    or_rht_signs(sign_seed, d);
    for (int64_t f = 0; f < F; ++f)
        for (int64_t c = 0; c < T / 16; ++c) {
            float y[16];
            for (int i = 0; i < 16; ++i) {
                y[i] = load_elem(x, dtype, (c * 16 + i) * ld + f);
                if (!isfinite(y[i])) return OR_ERR_NONFINITE;
            }
            or_rht16(y, d);
            for (int i = 0; i < 16; ++i) y_out[f * T + c * 16 + i] = y[i];
        }
    return OR_OK;
}

/* Hadamard + transpose + 1D quantize of one wgrad operand x [T tokens x F features] (row
 * stride ld).  Output is feature-major so that the reduction dimension (tokens) is contiguous:
 * codes [F x T/2], scales [F x T/16]; element (f, t) has SR index f * T + t. */
int or_hadamard_quantize(const void *x, int dtype, int64_t T, int64_t F, int64_t ld,
                         uint64_t sign_seed, const float *amax_in, int rounding, uint64_t seed,
                         uint8_t *codes, uint8_t *scales, float *amax_out, float *s_dec_out)
{
    if (T % 16 != 0 || T < 0 || F < 0 || ld < F) return OR_ERR_SHAPE;
    float A;
    if (amax_in) A = *amax_in;
    else {
        int rc = or_hadamard_amax(x, dtype, T, F, ld, sign_seed, &A);
        if (rc) return rc;
    }
    float ts[3];
    or_tensor_scales(A, ts);
    int d[16];
    or_rht_signs(sign_seed, d);
    int64_t nb = T / 16;
    int err = 0;
#pragma omp parallel for schedule(static)
    for (int64_t f = 0; f < F; ++f) {
        for (int64_t c = 0; c < nb; ++c) {
            float y[16], ab = 0.0f;
            for (int i = 0; i < 16; ++i) {
                y[i] = load_elem(x, dtype, (c * 16 + i) * ld + f);
                if (!isfinite(y[i])) err = 1;
            }
            or_rht16(y, d);
            for (int i = 0; i < 16; ++i)
                if (fabsf(y[i]) > ab) ab = fabsf(y[i]);
            unsigned sb;
            float enc;
            block_scale(ab, ts, &sb, &enc);
            scales[f * nb + c] = (uint8_t)sb;
            for (int i = 0; i < 16; ++i) {
                float z = y[i] * enc;
                int64_t t = c * 16 + i;
                unsigned code = (rounding == OR_SR)
                    ? or_e2m1_sr(z, or_sr_bits(seed, (uint64_t)(f * T + t)))
                    : or_e2m1_rne(z);
                put_nibble(codes, T / 2, f, t, code);
            }
        }
    }
    if (err) return OR_ERR_NONFINITE;
    if (amax_out) *amax_out = A;
    if (s_dec_out) *s_dec_out = ts[2];
    return OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Dequantize: x_hat = fl(fl(v * scale_b) * s_dec) in fp32 (the first product is exact).       */
/* layout OR_1x16: scales [rows x cols/16]; OR_16x16: scales [rows/16 x cols/16].              */
/* out_dtype OR_F32 writes float, OR_BF16 writes the RNE bf16 of that float.                   */
/* ------------------------------------------------------------------------------------------ */
static unsigned scale_at(const uint8_t *scales, int layout, int64_t rows, int64_t cols,
                         int64_t r, int64_t k)
{
    (void)rows;
    if (layout == OR_16x16) return scales[(r / 16) * (cols / 16) + k / 16];
    return scales[r * (cols / 16) + k / 16];
}

int or_dequantize(const uint8_t *codes, const uint8_t *scales, int layout, float s_dec,
                  int64_t rows, int64_t cols, int out_dtype, void *out, int64_t ld)
{
    if (cols % 16 != 0 || (layout == OR_16x16 && rows % 16 != 0) || ld < cols) return OR_ERR_SHAPE;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            float v = (float)or_e2m1_value(get_nibble(codes, cols / 2, r, k));
            float s = (float)or_e4m3_value(scale_at(scales, layout, rows, cols, r, k));
            float xh = (v * s) * s_dec;
            if (out_dtype == OR_BF16) ((uint16_t *)out)[r * ld + k] = or_f32_to_bf16(xh);
            else ((float *)out)[r * ld + k] = xh;
        }
    return OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* NVFP4 x NVFP4 GEMM reference [P2 Describir: weights, activations and gradients all in FP4,  */
/* i.e. all three training GEMMs take FP4 operands].  C = A * B^T with A [M x K], B [N x K],   */
/* both K-contiguous NVFP4:                                                                    */
/*   C[m,n] = s_dA * s_dB * sum_kb ( sA[m,kb] * sB[n,kb] * sum_{k in kb} vA[m,k] * vB[n,k] )    */
/* accumulated in float64 over blocks in ascending kb (every block term is exact in float64).  */
/* rows: NULL for all M rows, else nrows indices of A rows to evaluate; out [nrows x N].       */
/* ------------------------------------------------------------------------------------------ */
int or_gemm_f64(const uint8_t *a_codes, const uint8_t *a_scales, int a_layout, float a_sdec,
                const uint8_t *b_codes, const uint8_t *b_scales, int b_layout, float b_sdec,
                int64_t M, int64_t N, int64_t K, const int64_t *rows, int64_t nrows, double *out)
{
    if (K % 16 != 0) return OR_ERR_SHAPE;
    if (!rows) nrows = M;
    int64_t nb = K / 16;
    double sd = (double)a_sdec * (double)b_sdec;
    /* decode B once (values and block scales); a cache of or_e2m1_value / or_e4m3_value */
    double lut[16];
    for (unsigned c = 0; c < 16; ++c) lut[c] = or_e2m1_value(c);
    double *vb = (double *)malloc((size_t)(N * K) * sizeof(double));
    double *sbv = (double *)malloc((size_t)(N * nb) * sizeof(double));
    if (!vb || !sbv) { free(vb); free(sbv); return OR_ERR_ARG; }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) vb[n * K + k] = lut[get_nibble(b_codes, K / 2, n, k)];
        for (int64_t kb = 0; kb < nb; ++kb)
            sbv[n * nb + kb] = or_e4m3_value(scale_at(b_scales, b_layout, N, K, n, kb * 16));
    }
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ii = 0; ii < nrows; ++ii) {
        int64_t m = rows ? rows[ii] : ii;
        if (m < 0 || m >= M) { err = 1; continue; }
        double *va = (double *)malloc((size_t)K * sizeof(double));
        double *sa = (double *)malloc((size_t)nb * sizeof(double));
        if (!va || !sa) { free(va); free(sa); err = 1; continue; }
        for (int64_t k = 0; k < K; ++k) va[k] = lut[get_nibble(a_codes, K / 2, m, k)];
        for (int64_t kb = 0; kb < nb; ++kb)
            sa[kb] = or_e4m3_value(scale_at(a_scales, a_layout, M, K, m, kb * 16));
        for (int64_t n = 0; n < N; ++n) {
            const double *vbn = vb + n * K;
            double acc = 0.0;
            for (int64_t kb = 0; kb < nb; ++kb) {
                double p = 0.0;
                for (int i = 0; i < 16; ++i) p += va[kb * 16 + i] * vbn[kb * 16 + i];
                acc += sa[kb] * sbv[n * nb + kb] * p;
            }
            out[ii * N + n] = sd * acc;
        }
        free(va);
        free(sa);
    }
    free(vb);
    free(sbv);
    return err ? OR_ERR_ARG : OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* MXFP4, the rival 4-bit format [P3 NVFP4 in pratica; Difficolta di quantificazione].          */
/* Reading (OCP MX v1.0): 32-element blocks along K, E8M0 power-of-two scale                  */
/* 2^(floor(log2 amax_b) - 2) (2 = the largest E2M1 exponent), byte = exponent + 127, clamped */
/* to [-127, 127]; amax_b = 0 gives exponent 0; no per-tensor scale; z = x * 2^-e exactly.    */
/* ------------------------------------------------------------------------------------------ */
int or_mx_quantize_1d(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                      int rounding, uint64_t seed, uint8_t *codes, uint8_t *scales)
{
    if (cols % 32 != 0 || ld < cols) return OR_ERR_SHAPE;
    int64_t nb = cols / 32;
    int err = 0;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float y[32], ab = 0.0f;
            for (int i = 0; i < 32; ++i) {
                y[i] = load_elem(x, dtype, r * ld + b * 32 + i);
                if (!isfinite(y[i])) err = 1;
                if (fabsf(y[i]) > ab) ab = fabsf(y[i]);
            }
            int e = 0;
            if (ab > 0.0f) {
                int E;
                frexp((double)ab, &E);             /* ab = f * 2^E, f in [0.5, 1) */
                e = (E - 1) - 2;
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            scales[r * nb + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; ++i) {
                float z = ldexpf(y[i], -e);
                int64_t k = b * 32 + i;
                unsigned code = (rounding == OR_SR)
                    ? or_e2m1_sr(z, or_sr_bits(seed, (uint64_t)(r * cols + k)))
                    : or_e2m1_rne(z);
                put_nibble(codes, cols / 2, r, k, code);
            }
        }
    return err ? OR_ERR_NONFINITE : OR_OK;
}

/* Format sweep ("FP4 All the Way", Describir: block size, scale format and rounding method are
 * the FP4 design choices the authors explore).  Quantize x with `block` elements per scale along
 * the row and the scale format `scale_fmt`, then dequantize into y [rows x cols] (fp32, dense):
 *   scale_fmt 0: E4M3 block scale under the per-tensor fp32 scale, the NVFP4 steps of
 *                or_quantize_1d with the block size as a parameter; y = (v * scale) * s_dec;
 *   scale_fmt 1: E8M0 scale 2^(floor(log2 amax_b) - 2), no tensor scale, the steps of
 *                or_mx_quantize_1d with the block size as a parameter; y = v * 2^e.
 * Rounding RNE or SR (element index r * cols + k).  amax_out receives the tensor amax used
 * (E4M3) or 0 (E8M0). */
int or_qdq(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld, int block,
           int scale_fmt, const float *amax_in, int rounding, uint64_t seed, float *y,
           float *amax_out)
{
    if (block != 8 && block != 16 && block != 32) return OR_ERR_SHAPE;
    if (scale_fmt != 0 && scale_fmt != 1) return OR_ERR_SHAPE;
    if (cols % block != 0 || rows < 0 || cols < 0 || ld < cols) return OR_ERR_SHAPE;
    float A = 0.0f, ts[3] = {1.0f, 1.0f, 1.0f};
    if (scale_fmt == 0) {
        if (amax_in) A = *amax_in;
        else {
            int rc = or_amax(x, dtype, rows, cols, ld, &A);
            if (rc) return rc;
        }
        or_tensor_scales(A, ts);
    }
    int64_t nb = cols / block;
    int err = 0;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float v[32], ab = 0.0f;
            for (int i = 0; i < block; ++i) {
                v[i] = load_elem(x, dtype, r * ld + b * block + i);
                if (!isfinite(v[i])) err = 1;
                if (fabsf(v[i]) > ab) ab = fabsf(v[i]);
            }
            unsigned sb = 0;
            float enc = 0.0f;
            int e = 0;
            if (scale_fmt == 0) {
                block_scale(ab, ts, &sb, &enc);
            } else if (ab > 0.0f) {
                int E;
                frexp((double)ab, &E);
                e = (E - 1) - 2;
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            for (int i = 0; i < block; ++i) {
                int64_t k = b * block + i;
                float z = scale_fmt == 0 ? v[i] * enc : ldexpf(v[i], -e);
                unsigned code = (rounding == OR_SR)
                    ? or_e2m1_sr(z, or_sr_bits(seed, (uint64_t)(r * cols + k)))
                    : or_e2m1_rne(z);
                float q = (float)or_e2m1_value(code);
                if (scale_fmt == 0) {
                    float sc = (float)or_e4m3_value(sb);
                    float t = q * sc;
                    y[r * cols + k] = t * ts[2];
                } else {
                    y[r * cols + k] = ldexpf(q, e);
                }
            }
        }
    if (err) return OR_ERR_NONFINITE;
    if (amax_out) *amax_out = A;
    return OR_OK;
}

int or_mx_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                     float *out, int64_t ld)
{
    if (cols % 32 != 0 || ld < cols) return OR_ERR_SHAPE;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            double v = or_e2m1_value(get_nibble(codes, cols / 2, r, k));
            int e = (int)scales[r * (cols / 32) + k / 32] - 127;
            out[r * ld + k] = (float)ldexp(v, e);
        }
    return OR_OK;
}

/* C[m,n] = sum_kb 2^(eA[m,kb] + eB[n,kb]) * sum_{k in kb} vA * vB over 32-blocks, float64. */
int or_mx_gemm_f64(const uint8_t *a_codes, const uint8_t *a_scales,
                   const uint8_t *b_codes, const uint8_t *b_scales,
                   int64_t M, int64_t N, int64_t K, const int64_t *rows, int64_t nrows, double *out)
{
    if (K % 32 != 0) return OR_ERR_SHAPE;
    if (!rows) nrows = M;
    int64_t nb = K / 32;
    double lut[16];
    for (unsigned c = 0; c < 16; ++c) lut[c] = or_e2m1_value(c);
    double *vb = (double *)malloc((size_t)(N * K) * sizeof(double));
    if (!vb) return OR_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) vb[n * K + k] = lut[get_nibble(b_codes, K / 2, n, k)];
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ii = 0; ii < nrows; ++ii) {
        int64_t m = rows ? rows[ii] : ii;
        if (m < 0 || m >= M) { err = 1; continue; }
        double *va = (double *)malloc((size_t)K * sizeof(double));
        if (!va) { err = 1; continue; }
        for (int64_t k = 0; k < K; ++k) va[k] = lut[get_nibble(a_codes, K / 2, m, k)];
        for (int64_t n = 0; n < N; ++n) {
            const double *vbn = vb + n * K;
            double acc = 0.0;
            for (int64_t kb = 0; kb < nb; ++kb) {
                double p = 0.0;
                for (int i = 0; i < 32; ++i) p += va[kb * 32 + i] * vbn[kb * 32 + i];
                int e = ((int)a_scales[m * nb + kb] - 127) + ((int)b_scales[n * nb + kb] - 127);
                acc += ldexp(p, e);
            }
            out[ii * N + n] = acc;
        }
        free(va);
    }
    free(vb);
    return err ? OR_ERR_ARG : OR_OK;
}
