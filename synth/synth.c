/*
 * Seeded synthetic input generator (host, plain C + OpenMP).
 *
 * This file holds no arithmetic of the decode step itself: it only draws
 * random numbers and encodes them into the storage formats the step reads
 * (IEEE binary16, and the 32-weight Q8_0 / Q4_0 / int8-asymmetric blocks).
 * Both the GPU library and the CPU oracle consume its output; neither is
 * imported here.
 *
 * Random stream: SplitMix64 used as a counter-based generator (Steele, Lea,
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014; the
 * finaliser constants are Vigna's published SplitMix64).  Draw c of stream s
 * is mix64(s + (c + 1) * 0x9E3779B97F4A7C15).  Normal variates 2p and 2p+1
 * of a stream are the cosine and sine outputs of the Box-Muller transform of
 * draws 2p and 2p+1, so every element is independent of thread count and
 * chunking.
 *
 * Canonical block layouts (little-endian, blocks run along the input
 * dimension k of each output row, row-major over blocks):
 *   Q8_0    34 B: fp16 d, int8 q[32]             w_i = d * q_i
 *   Q4_0    18 B: fp16 d, uint8 b[16]            byte j: low nibble = q_j,
 *                                                high nibble = q_{j+16},
 *                                                w_i = d * (q_i - 8)
 *   U8A_G32 36 B: fp16 s, fp16 z, uint8 q[32]    w_i = s * (q_i - z)
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t stream, uint64_t c) {
    return mix64(stream + (c + 1) * GOLDEN);
}

/* Standard normal numbers 2p and 2p+1 of a stream. */
static inline void normal_pair(uint64_t stream, uint64_t p, double* z0, double* z1) {
    const double two_pi = 6.283185307179586476925286766559;
    uint64_t a = draw(stream, 2 * p), b = draw(stream, 2 * p + 1);
    double u1 = (double)((a >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
    double u2 = (double)(b >> 11) * 0x1.0p-53;       /* [0, 1) */
    double r = sqrt(-2.0 * log(u1));
    *z0 = r * cos(two_pi * u2);
    *z1 = r * sin(two_pi * u2);
}

static inline double normal_at(uint64_t stream, uint64_t i) {
    double z0, z1;
    normal_pair(stream, i >> 1, &z0, &z1);
    return (i & 1) ? z1 : z0;
}

/* 32 consecutive normals starting at an even index, scaled by std. */
static inline void normal_block(uint64_t stream, uint64_t first, double std, double* w) {
    for (int i = 0; i < 32; i += 2) {
        double z0, z1;
        normal_pair(stream, (first >> 1) + (uint64_t)(i >> 1), &z0, &z1);
        w[i] = std * z0;
        w[i + 1] = std * z1;
    }
}

/* double -> binary16, round to nearest even, subnormals kept, overflow to inf. */
static uint16_t d2h(double x) {
    uint64_t bits;
    memcpy(&bits, &x, 8);
    uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
    double a = fabs(x);
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u); /* rounds past the largest finite */
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                       /* a = m * 2^e, m in [0.5, 1) */
    int qe = e - 11;                    /* quantum for 11 significant bits */
    if (qe < -24) qe = -24;             /* subnormal quantum 2^-24 */
    double r = nearbyint(ldexp(a, -qe)); /* default rounding mode: ties to even */
    double v = ldexp(r, qe);
    if (v < 0x1.0p-14) {                /* subnormal, or exactly 2^-14 via carry */
        return (uint16_t)(sign | (uint16_t)ldexp(v, 24));
    }
    int e2;
    double m2 = frexp(v, &e2);          /* v = m2 * 2^e2 */
    uint16_t exp_field = (uint16_t)(e2 - 1 + 15);
    uint16_t mant = (uint16_t)ldexp(m2 * 2.0 - 1.0, 10);
    return (uint16_t)(sign | (exp_field << 10) | mant);
}

static double h2d(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m + 1024), e - 25);
    return s ? -v : v;
}

static inline void put_u16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 255); p[1] = (uint8_t)(v >> 8); }

/* ---- exported ---------------------------------------------------------- */

uint16_t synth_d2h(double x) { return d2h(x); }
double synth_h2d(uint16_t h) { return h2d(h); }
uint64_t synth_draw(uint64_t stream, uint64_t c) { return draw(stream, c); }
double synth_normal_at(uint64_t stream, uint64_t i) { return normal_at(stream, i); }

/* out[i] = mean + std * N_i, as doubles. */
void synth_normal_f64(uint64_t stream, int64_t n, double mean, double std, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < (n + 1) / 2; ++p) {
        double z0, z1;
        normal_pair(stream, (uint64_t)p, &z0, &z1);
        out[2 * p] = mean + std * z0;
        if (2 * p + 1 < n) out[2 * p + 1] = mean + std * z1;
    }
}

/* out[i] = fp16(mean + std * N_i). */
void synth_normal_f16(uint64_t stream, int64_t n, double mean, double std, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < (n + 1) / 2; ++p) {
        double z0, z1;
        normal_pair(stream, (uint64_t)p, &z0, &z1);
        out[2 * p] = d2h(mean + std * z0);
        if (2 * p + 1 < n) out[2 * p + 1] = d2h(mean + std * z1);
    }
}

/* out[i] uniform in [lo, hi) (hi - lo < 2^31). */
void synth_uniform_i32(uint64_t stream, int64_t n, int32_t lo, int32_t hi, int32_t* out) {
    uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = draw(stream, (uint64_t)i) >> 11;
        out[i] = lo + (int32_t)((r * span) >> 53);
    }
}

/* Weight matrix [n][k] drawn as std * N, quantised to Q8_0 blocks.
 * d = fp16(amax / 127); q = clamp(round_half_away(w / d), -127, 127). */
void synth_q8_0(uint64_t stream, int64_t n, int64_t k, double std, uint8_t* out) {
    int64_t nb = k / 32, total = n * nb;
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < total; ++blk) {
        double w[32], amax = 0.0;
        int64_t row = blk / nb, b = blk % nb;
        normal_block(stream, (uint64_t)(row * k + b * 32), std, w);
        for (int i = 0; i < 32; ++i)
            if (fabs(w[i]) > amax) amax = fabs(w[i]);
        uint16_t dh = d2h(amax / 127.0);
        double d = h2d(dh);
        uint8_t* p = out + blk * 34;
        put_u16(p, dh);
        for (int i = 0; i < 32; ++i) {
            double q = (d == 0.0) ? 0.0 : round(w[i] / d);
            if (q > 127) q = 127;
            if (q < -127) q = -127;
            p[2 + i] = (uint8_t)(int8_t)q;
        }
    }
}

/* Weight matrix [n][k] drawn as std * N, quantised to Q4_0 blocks.
 * d = fp16(amax / 7); q = clamp(round_half_away(w / d), -8, 7) + 8. */
void synth_q4_0(uint64_t stream, int64_t n, int64_t k, double std, uint8_t* out) {
    int64_t nb = k / 32, total = n * nb;
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < total; ++blk) {
        double w[32], amax = 0.0;
        int64_t row = blk / nb, b = blk % nb;
        normal_block(stream, (uint64_t)(row * k + b * 32), std, w);
        for (int i = 0; i < 32; ++i)
            if (fabs(w[i]) > amax) amax = fabs(w[i]);
        uint16_t dh = d2h(amax / 7.0);
        double d = h2d(dh);
        int q[32];
        for (int i = 0; i < 32; ++i) {
            double v = (d == 0.0) ? 0.0 : round(w[i] / d);
            if (v > 7) v = 7;
            if (v < -8) v = -8;
            q[i] = (int)v + 8;
        }
        uint8_t* p = out + blk * 18;
        put_u16(p, dh);
        for (int j = 0; j < 16; ++j) p[2 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
    }
}

/* Weight matrix [n][k] drawn as std * N, quantised to int8-asymmetric
 * groups of 32: s = fp16((max - min) / 255), z = fp16(round(-min / s)),
 * q = clamp(round(w / s) + z, 0, 255). */
void synth_u8a_g32(uint64_t stream, int64_t n, int64_t k, double std, uint8_t* out) {
    int64_t nb = k / 32, total = n * nb;
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < total; ++blk) {
        double w[32], mn = INFINITY, mx = -INFINITY;
        int64_t row = blk / nb, b = blk % nb;
        normal_block(stream, (uint64_t)(row * k + b * 32), std, w);
        for (int i = 0; i < 32; ++i) {
            if (w[i] < mn) mn = w[i];
            if (w[i] > mx) mx = w[i];
        }
        uint16_t sh = d2h((mx - mn) / 255.0);
        double s = h2d(sh);
        uint16_t zh = 0;
        double z = 0.0;
        if (s != 0.0) {
            zh = d2h(round(-mn / s));
            z = h2d(zh);
        }
        uint8_t* p = out + blk * 36;
        put_u16(p, sh);
        put_u16(p + 2, zh);
        for (int i = 0; i < 32; ++i) {
            double q = (s == 0.0) ? 0.0 : round(w[i] / s) + z;
            if (q > 255) q = 255;
            if (q < 0) q = 0;
            p[4 + i] = (uint8_t)q;
        }
    }
}
