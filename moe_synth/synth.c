/*
 * Seeded synthetic inputs for the quantized routed-MoE layer.
 *
 * This module only draws random numbers and lays them out in the canonical
 * storage formats; it contains none of the layer's arithmetic.  Both the CPU
 * oracle and the GPU path consume what it produces.
 *
 * Generator: xoshiro256** (Blackman & Vigna, "Scrambled linear pseudorandom
 * number generators", 2018), each substream seeded through SplitMix64 from
 * (seed, tensor tag, substream index).  Every substream is a pure function of
 * that triple, so results do not depend on the number of threads.
 *
 * Distributions:
 *   uniform double  u in [0,1): top 53 bits of one draw times 2^-53
 *   normal          Box-Muller in double, rounded once to fp32
 *   bounded int     Lemire's multiply-shift with rejection (unbiased)
 *   fp16 values     drawn in double, rounded to fp16 round-to-nearest-even
 *
 * Canonical storage formats (little-endian):
 *   Q8_32 block, 34 bytes: fp16 scale d, then 32 int8 codes; value = d * q.
 *   Q2_256 superblock, 84 bytes: fp16 d, fp16 dmin, 16 bytes sm (subblock j of
 *     16 weights: scale s_j = low nibble, min m_j = high nibble), 64 bytes qs
 *     (weight i has its 2-bit code in byte i/4 at bit 2*(i%4));
 *     value_i = d * s_{i/16} * q_i - dmin * m_{i/16}.
 *   A matrix [rows][cols] is stored row by row, each row as cols/32 (Q8) or
 *   cols/256 (Q2) consecutive blocks; a bank of n matrices is n matrices back
 *   to back.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef struct { uint64_t s[4]; } xo256;

static uint64_t splitmix64(uint64_t *state) {
    uint64_t z = (*state += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static void xo_seed(xo256 *r, uint64_t seed, uint64_t tag, uint64_t index) {
    uint64_t st = seed;
    uint64_t a = splitmix64(&st);
    st = a ^ (tag * 0xD6E8FEB86659FD93ULL);
    uint64_t b = splitmix64(&st);
    st = b ^ (index * 0xA0761D6478BD642FULL + 0xE7037ED1A0B428DBULL);
    for (int i = 0; i < 4; ++i) r->s[i] = splitmix64(&st);
}

static inline uint64_t rotl64(uint64_t x, int k) { return (x << k) | (x >> (64 - k)); }

static inline uint64_t xo_next(xo256 *r) {
    uint64_t *s = r->s;
    uint64_t result = rotl64(s[1] * 5, 7) * 9;
    uint64_t t = s[1] << 17;
    s[2] ^= s[0];
    s[3] ^= s[1];
    s[1] ^= s[2];
    s[0] ^= s[3];
    s[2] ^= t;
    s[3] = rotl64(s[3], 45);
    return result;
}

static inline double xo_u53(xo256 *r) { return (double)(xo_next(r) >> 11) * 0x1.0p-53; }

/* Lemire, "Fast random integer generation in an interval" (2019). */
static uint32_t xo_bounded(xo256 *r, uint32_t n) {
    uint32_t x = (uint32_t)(xo_next(r) >> 32);
    uint64_t m = (uint64_t)x * n;
    uint32_t l = (uint32_t)m;
    if (l < n) {
        uint32_t t = (uint32_t)(-n) % n;
        while (l < t) {
            x = (uint32_t)(xo_next(r) >> 32);
            m = (uint64_t)x * n;
            l = (uint32_t)m;
        }
    }
    return (uint32_t)(m >> 32);
}

/* double -> IEEE binary16, round to nearest even (finite inputs). */
uint16_t synth_f16_from_double(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a != a) return sign | 0x7e00;
    if (a >= 65520.0) return sign | 0x7c00;
    if (a < 0x1p-14) {
        double q = nearbyint(a * 0x1p24);   /* subnormal quantum 2^-24; 1024 encodes 2^-14 */
        return sign | (uint16_t)q;
    }
    int e;
    double m = frexp(a, &e);                /* a = m * 2^e, m in [0.5, 1) */
    double sig = nearbyint(ldexp(m, 11));   /* 11-bit significand in [1024, 2048] */
    int E = e - 1 + 15;
    if (sig == 2048.0) { sig = 1024.0; E += 1; }
    if (E >= 31) return sign | 0x7c00;
    return sign | (uint16_t)(E << 10) | (uint16_t)((int)sig - 1024);
}

#define CHUNK 4096

/* n values ~ N(mean, std) in fp32; substream per chunk of CHUNK values. */
void synth_normal_f32(float *out, int64_t n, double mean, double std, uint64_t seed, uint64_t tag) {
    int64_t nchunks = (n + CHUNK - 1) / CHUNK;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < nchunks; ++c) {
        xo256 r;
        xo_seed(&r, seed, tag, (uint64_t)c);
        int64_t lo = c * CHUNK, hi = lo + CHUNK < n ? lo + CHUNK : n;
        for (int64_t i = lo; i < hi; i += 2) {
            double u1 = 1.0 - xo_u53(&r); /* (0, 1] */
            double u2 = xo_u53(&r);
            double rad = sqrt(-2.0 * log(u1));
            double ang = 2.0 * M_PI * u2;
            out[i] = (float)(mean + std * rad * cos(ang));
            if (i + 1 < hi) out[i + 1] = (float)(mean + std * rad * sin(ang));
        }
    }
}

/* n integers uniform in [lo, hi] (inclusive). */
void synth_uniform_i32(int32_t *out, int64_t n, int32_t lo, int32_t hi, uint64_t seed, uint64_t tag) {
    uint32_t span = (uint32_t)((int64_t)hi - (int64_t)lo + 1);
    int64_t nchunks = (n + CHUNK - 1) / CHUNK;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < nchunks; ++c) {
        xo256 r;
        xo_seed(&r, seed, tag, (uint64_t)c);
        int64_t a = c * CHUNK, b = a + CHUNK < n ? a + CHUNK : n;
        for (int64_t i = a; i < b; ++i) out[i] = (int32_t)((int64_t)lo + xo_bounded(&r, span));
    }
}

/* Table [rows][k]: each row holds k distinct values of [0, n_values), drawn by a
 * partial Fisher-Yates shuffle in draw order.  Requires k <= n_values <= 4096. */
int synth_distinct_rows(int32_t *out, int64_t rows, int32_t k, int32_t n_values, uint64_t seed, uint64_t tag) {
    if (k < 0 || n_values <= 0 || k > n_values || n_values > 4096) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        int32_t perm[4096];
        xo256 r;
        xo_seed(&r, seed, tag, (uint64_t)row);
        for (int32_t i = 0; i < n_values; ++i) perm[i] = i;
        for (int32_t j = 0; j < k; ++j) {
            int32_t pick = j + (int32_t)xo_bounded(&r, (uint32_t)(n_values - j));
            int32_t tmp = perm[j];
            perm[j] = perm[pick];
            perm[pick] = tmp;
            out[row * k + j] = perm[j];
        }
    }
    return 0;
}

static inline void put_f16(uint8_t *p, uint16_t h) {
    p[0] = (uint8_t)(h & 0xff);
    p[1] = (uint8_t)(h >> 8);
}

/* Bank of n_mats Q8_32 matrices [rows][cols]: codes uniform over [-127, 127]
 * (bytes of the stream with the value -128 skipped), scales U(smin, smax) in
 * fp16.  One substream per matrix row. */
int synth_q8_bank(uint8_t *out, int64_t n_mats, int64_t rows, int64_t cols, double smin, double smax,
                  uint64_t seed, uint64_t tag) {
    if (cols % 32 != 0) return -1;
    int64_t nb = cols / 32;
    int64_t total_rows = n_mats * rows;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < total_rows; ++row) {
        xo256 r;
        xo_seed(&r, seed, tag, (uint64_t)row);
        uint8_t *p = out + row * nb * 34;
        uint64_t word = 0;
        int left = 0;
        for (int64_t b = 0; b < nb; ++b) {
            double u = xo_u53(&r);
            put_f16(p + b * 34, synth_f16_from_double(smin + (smax - smin) * u));
            for (int j = 0; j < 32;) {
                if (left == 0) { word = xo_next(&r); left = 8; }
                uint8_t byte = (uint8_t)(word & 0xff);
                word >>= 8;
                --left;
                if (byte == 0x80) continue;
                p[b * 34 + 2 + j] = byte;
                ++j;
            }
        }
    }
    return 0;
}

/* Bank of n_mats Q2_256 matrices [rows][cols]: every 2-bit code and every
 * 4-bit scale/min uniform (whole random bytes), d and dmin U(smin, smax) fp16. */
int synth_q2_bank(uint8_t *out, int64_t n_mats, int64_t rows, int64_t cols, double smin, double smax,
                  uint64_t seed, uint64_t tag) {
    if (cols % 256 != 0) return -1;
    int64_t nsb = cols / 256;
    int64_t total_rows = n_mats * rows;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < total_rows; ++row) {
        xo256 r;
        xo_seed(&r, seed, tag, (uint64_t)row);
        uint8_t *p = out + row * nsb * 84;
        for (int64_t s = 0; s < nsb; ++s) {
            uint8_t *sb = p + s * 84;
            put_f16(sb, synth_f16_from_double(smin + (smax - smin) * xo_u53(&r)));
            put_f16(sb + 2, synth_f16_from_double(smin + (smax - smin) * xo_u53(&r)));
            for (int j = 0; j < 80; j += 8) {
                uint64_t w = xo_next(&r);
                memcpy(sb + 4 + j, &w, 8);
            }
        }
    }
    return 0;
}
