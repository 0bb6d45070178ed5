/*
 * synth.c -- seeded synthetic inputs for the routed-MoE layer workloads.
 *
 * Serves both the CPU oracle and the GPU library, so it holds none of the
 * layer's arithmetic: only counter-based random streams, rounding to the
 * storage encodings (fp32, bf16, fp16), int4 nibble packing and the Zipf
 * ranking of the router bias.
 *
 * Random numbers: every value is a pure function of (key, row, attempt,
 * element index), so any row can be regenerated alone and threads never share
 * state.  The mixing function is the SplitMix64 finaliser (Steele, Lea and
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014);
 *   stream(key, row, attempt) = mix(key ^ mix(row*G + attempt*H + 1))
 *   draw(stream, i)           = mix(stream + (i+1)*G)
 *   uniform                   = (draw >> 11) * 2^-53            in [0, 1)
 *   normal pair (Box-Muller, in fp32 with 24-bit uniforms v = (draw >> 40) * 2^-24)
 *                             = sqrt(-2 ln(1-v1)) * (cos, sin)(2 pi v2)
 * with G = 0x9E3779B97F4A7C15 and H = 0xD1B54A32D192ED03.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SYN_G 0x9E3779B97F4A7C15ULL
#define SYN_H 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t cfg, uint64_t layer, uint64_t tensor)
{
    uint64_t k = mix64(seed + SYN_G);
    k = mix64(k ^ mix64(cfg + 0x1000));
    k = mix64(k ^ mix64(layer + 0x2000));
    k = mix64(k ^ mix64(tensor + 0x3000));
    return k;
}

static inline uint64_t stream_of(uint64_t key, uint64_t row, uint64_t attempt)
{
    return mix64(key ^ mix64(row * SYN_G + attempt * SYN_H + 1));
}

static inline uint64_t draw(uint64_t stream, uint64_t i)
{
    return mix64(stream + (i + 1) * SYN_G);
}

static inline double unif(uint64_t stream, uint64_t i)
{
    return (double)(draw(stream, i) >> 11) * 0x1.0p-53;
}

static inline float unif24(uint64_t stream, uint64_t i)
{
    return (float)(draw(stream, i) >> 40) * 0x1.0p-24f;
}

/* Normal pair number p of a stream (elements 2p and 2p+1). */
static inline void normal_pair(uint64_t stream, uint64_t p, float *n0, float *n1)
{
    float v1 = unif24(stream, 2 * p), v2 = unif24(stream, 2 * p + 1);
    float r = sqrtf(-2.0f * logf(1.0f - v1));
    float sn, cs;
    sincosf(6.28318530717958647692f * v2, &sn, &cs);
    *n0 = r * cs;
    *n1 = r * sn;
}

/* ---- storage rounding (round to nearest, ties to even, from double) ---- */

static uint16_t round_to_bits(double v, int frac_bits, int bias, int max_exp_field)
{
    /* generic IEEE-style small float: returns sign|exp|frac with frac_bits bits */
    uint16_t sign = signbit(v) ? (uint16_t)0x8000 : 0;
    int exp_bits = frac_bits == 7 ? 8 : 5;
    uint32_t inf = ((1u << exp_bits) - 1) << frac_bits;
    if (isnan(v)) return (uint16_t)(inf | (1u << (frac_bits - 1)));
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | inf);
    int min_exp = 1 - bias;                  /* exponent of the smallest normal */
    int e;
    if (a == 0.0) return sign;
    frexp(a, &e);                             /* a in [2^(e-1), 2^e) */
    int qexp = (e - 1) - frac_bits;           /* quantum at this binade */
    if (e - 1 < min_exp) qexp = min_exp - frac_bits;
    double q = nearbyint(ldexp(a, -qexp));    /* integer count of quanta, RNE */
    /* rebuild the encoding from q * 2^qexp */
    double r = ldexp(q, qexp);
    if (r == 0.0) return sign;
    frexp(r, &e);
    if (e - 1 > max_exp_field - 1 - bias) return (uint16_t)(sign | inf);
    uint32_t field;
    if (e - 1 < min_exp) {
        field = (uint32_t)ldexp(r, -(min_exp - frac_bits));                 /* subnormal */
    } else {
        uint32_t frac = (uint32_t)(ldexp(r, frac_bits - (e - 1)) - ldexp(1.0, frac_bits));
        field = ((uint32_t)(e - 1 + bias) << frac_bits) | frac;
    }
    return (uint16_t)(sign | field);
}

/* Fast path for values in the normal range of the target: drop the low
 * mantissa bits of the double with round-half-even (a carry into the exponent
 * field is the correct result, including overflow to infinity). */
static inline uint16_t round_fast(double v, int frac_bits, int bias, int max_field)
{
    uint64_t b;
    memcpy(&b, &v, sizeof b);
    int eb = (int)((b >> 52) & 0x7ff) - 1023 + bias;
    if (eb < 1 || eb > max_field - 1)
        return round_to_bits(v, frac_bits, bias, max_field);
    int drop = 52 - frac_bits;
    uint64_t m = b & 0xFFFFFFFFFFFFFULL;
    uint64_t keep = m >> drop, rest = m & ((1ULL << drop) - 1), half = 1ULL << (drop - 1);
    uint32_t r = ((uint32_t)eb << frac_bits) | (uint32_t)keep;
    if (rest > half || (rest == half && (keep & 1))) r += 1;
    return (uint16_t)(((b >> 63) << 15) | r);
}

static inline uint16_t to_bf16(double v) { return round_fast(v, 7, 127, 255); }
static inline uint16_t to_fp16(double v) { return round_fast(v, 10, 15, 31); }

uint16_t synth_bf16(double v) { return to_bf16(v); }
uint16_t synth_fp16(double v) { return to_fp16(v); }

enum { SYN_F32 = 0, SYN_BF16 = 1 };

static inline void store(int kind, void *out, int64_t idx, double v)
{
    if (kind == SYN_F32)
        ((float *)out)[idx] = (float)v;
    else
        ((uint16_t *)out)[idx] = to_bf16(v);
}

/* rows x cols normals * scale; row r uses stream (key, row0 + r, attempt 0). */
void synth_normal(uint64_t key, int64_t rows, int64_t cols, int64_t row0, double scale,
                  int kind, void *out)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        uint64_t s = stream_of(key, (uint64_t)(row0 + r), 0);
        for (int64_t c = 0; c < cols; c += 2) {
            float n0, n1;
            normal_pair(s, (uint64_t)(c >> 1), &n0, &n1);
            store(kind, out, r * cols + c, (double)n0 * scale);
            if (c + 1 < cols) store(kind, out, r * cols + c + 1, (double)n1 * scale);
        }
    }
}

/* Token rows of N(0,1) values; token t draws from attempt attempts[t] (NULL: all 0). */
void synth_x_rows(uint64_t key, int64_t T, int64_t D, const int32_t *attempts, int kind,
                  void *out)
{
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        uint64_t s = stream_of(key, (uint64_t)t, attempts ? (uint64_t)attempts[t] : 0);
        for (int64_t d = 0; d < D; d += 2) {
            float n0, n1;
            normal_pair(s, (uint64_t)(d >> 1), &n0, &n1);
            store(kind, out, t * D + d, (double)n0);
            if (d + 1 < D) store(kind, out, t * D + d + 1, (double)n1);
        }
    }
}

/* n uniform values in [lo, hi) stored as fp32. */
void synth_uniform_f32(uint64_t key, int64_t n, double lo, double hi, float *out)
{
    uint64_t s = stream_of(key, 0, 0);
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(lo + (hi - lo) * unif(s, (uint64_t)i));
}

/* rows x cols uniform values in [lo, hi) stored as fp16 bits (row streams). */
void synth_uniform_fp16(uint64_t key, int64_t rows, int64_t cols, double lo, double hi,
                        uint16_t *out)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        uint64_t s = stream_of(key, (uint64_t)r, 0);
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = to_fp16(lo + (hi - lo) * unif(s, (uint64_t)c));
    }
}

/* rows x cols nibbles uniform on 0..15, packed two per byte: element 2i in the
 * low nibble of byte i, element 2i+1 in the high nibble.  cols must be even. */
void synth_nibbles(uint64_t key, int64_t rows, int64_t cols, uint8_t *out)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        uint64_t s = stream_of(key, (uint64_t)r, 0);
        for (int64_t c = 0; c < cols / 2; ++c) {
            uint64_t b = draw(s, (uint64_t)c);
            out[r * (cols / 2) + c] = (uint8_t)((b >> 60) | (((b >> 56) & 0xF) << 4));
        }
    }
}

/* Router bias with Zipf-shaped popularity: a seeded random ranking r_e of
 * 1..E (Fisher-Yates), bias_e = -s * ln(r_e), so the rank-1 expert has bias 0. */
void synth_zipf_bias(uint64_t key, int64_t E, double s, float *out)
{
    int64_t *rank = (int64_t *)malloc((size_t)E * sizeof(int64_t));
    if (!rank) return;
    for (int64_t e = 0; e < E; ++e) rank[e] = e + 1;
    uint64_t st = stream_of(key, 0, 0);
    for (int64_t i = E - 1; i > 0; --i) {
        int64_t j = (int64_t)(unif(st, (uint64_t)i) * (double)(i + 1));
        int64_t tmp = rank[i]; rank[i] = rank[j]; rank[j] = tmp;
    }
    for (int64_t e = 0; e < E; ++e) out[e] = (float)(-s * log((double)rank[e]));
    free(rank);
}

int synth_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
