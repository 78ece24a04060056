/*
 * Seeded synthetic inputs for the routed MoE layer: bf16 activations and
 * router weights, and MXFP4 (or FP8 block-scaled) expert weights, all drawn
 * from scaled normals.
 *
 * This is input synthesis only.  It implements none of the layer's
 * arithmetic: the layer decodes MXFP4 and quantises activations; this file
 * only *encodes* normals into MXFP4 once, to produce weights to decode.
 *
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC'11), a counter-based generator:
 * element i of stream s under seed S uses counter (i/4, S_hi, s_hi) and key
 * (S_lo, s_lo); each 4x32-bit output gives four normals by the Box-Muller
 * transform.  Any element can be generated independently, so generation
 * parallelises over rows with no shared state.
 *
 * Weight encoding (input synthesis rule): for each run of 32 values, the
 * smallest power of two 2^e with amax / 2^e <= 6 becomes the e8m0 scale
 * (byte e + 127) and each value / 2^e is rounded to the nearest e2m1 grid
 * point {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even code.  Element 2i of a
 * row goes to the low nibble of byte i.
 *
 * Built with gcc (-O2 -fopenmp -ffp-contract=off); deterministic for a given
 * libm.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void syn_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += PHILOX_W0; k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Four standard normals for counter block `blk` of (seed, stream). */
static void normals4(uint64_t seed, uint64_t stream, uint64_t blk, float z[4]) {
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)(seed >> 32), (uint32_t)(stream >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)stream};
    uint32_t r[4];
    syn_philox4x32_10(ctr, key, r);
    const float two_m24 = 5.9604644775390625e-08f; /* 2^-24 */
    for (int p = 0; p < 2; ++p) {
        float u1 = (float)((r[2 * p] >> 8) + 1u) * two_m24;   /* (0, 1] */
        float u2 = (float)(r[2 * p + 1] >> 8) * two_m24;      /* [0, 1) */
        float rad = sqrtf(-2.0f * logf(u1));
        float ang = 6.2831853071795864769f * u2;
        float sn, cs;
        sincosf(ang, &sn, &cs);
        z[2 * p] = rad * cs;
        z[2 * p + 1] = rad * sn;
    }
}

/* out[i] = scale * N_i for i in [first, first + n) of the stream. */
static void normal_range(uint64_t seed, uint64_t stream, int64_t first, int64_t n, float scale, float* out) {
    int64_t i = first, end = first + n, o = 0;
    float z[4];
    while (i < end) {
        uint64_t blk = (uint64_t)i >> 2;
        int lane = (int)(i & 3);
        normals4(seed, stream, blk, z);
        for (; lane < 4 && i < end; ++lane, ++i, ++o) out[o] = scale * z[lane];
    }
}

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)((u + bias) >> 16);
}

void syn_normal_f32(uint64_t seed, uint64_t stream, int64_t n, float scale, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < (n + 4095) / 4096; ++c) {
        int64_t first = c * 4096, cnt = (n - first < 4096) ? n - first : 4096;
        normal_range(seed, stream, first, cnt, scale, out + first);
    }
}

void syn_bf16_normal(uint64_t seed, uint64_t stream, int64_t n, float scale, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < (n + 4095) / 4096; ++c) {
        float buf[4096];
        int64_t first = c * 4096, cnt = (n - first < 4096) ? n - first : 4096;
        normal_range(seed, stream, first, cnt, scale, buf);
        for (int64_t i = 0; i < cnt; ++i) out[first + i] = f32_to_bf16_rne(buf[i]);
    }
}

static inline uint8_t e2m1_nearest_even(float a) {
    /* a >= 0 and a <= 6; grid 0, .5, 1, 1.5, 2, 3, 4, 6 = codes 0..7.  A value
       exactly between two grid points goes to the even code (0, 2, 4, 6). */
    return (uint8_t)((a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
                     (a > 2.5f) + (a >= 3.5f) + (a > 5.0f));
}

/* Encode one row of K floats (K % 32 == 0) into K/2 code bytes and K/32 scale bytes. */
static void encode_row_mxfp4(const float* v, int64_t K, uint8_t* codes, uint8_t* scales) {
    for (int64_t b = 0; b < K / 32; ++b) {
        const float* blk = v + b * 32;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(blk[i]));
        int e;
        if (amax == 0.0f) {
            e = -127;
        } else {
            int ex;
            float mant = frexpf(amax, &ex);   /* amax = mant * 2^ex, mant in [0.5, 1) */
            float f = 2.0f * mant;
            int q = ex - 1;
            e = (f <= 1.5f) ? q - 2 : q - 1;
            if (e < -127) e = -127;
            if (e > 127) e = 127;
        }
        scales[b] = (uint8_t)(e + 127);
        const float inv = ldexpf(1.0f, -e);   /* exact power of two; |x| * inv is exact */
        uint8_t n[32];
        for (int i = 0; i < 32; ++i) {
            float x = blk[i];
            n[i] = e2m1_nearest_even(fabsf(x) * inv) | (signbit(x) ? 8 : 0);
        }
        for (int i = 0; i < 16; ++i) codes[b * 16 + i] = (uint8_t)(n[2 * i] | (n[2 * i + 1] << 4));
    }
}

/* rows x K matrix of scale * N_{r*K + c}, MXFP4-encoded. */
void syn_mxfp4_normal(uint64_t seed, uint64_t stream, int64_t rows, int64_t K, float scale,
                      uint8_t* codes, uint8_t* scales) {
    #pragma omp parallel
    {
        float buf[16384];
        #pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            for (int64_t c0 = 0; c0 < K; c0 += 16384) {
                int64_t cnt = (K - c0 < 16384) ? K - c0 : 16384;
                normal_range(seed, stream, r * K + c0, cnt, scale, buf);
                encode_row_mxfp4(buf, cnt, codes + r * (K / 2) + c0 / 2, scales + r * (K / 32) + c0 / 32);
            }
        }
    }
}

/* E matrices (one stream per matrix: stream_base + e), each rows x K. */
void syn_mxfp4_normal_batched(uint64_t seed, uint64_t stream_base, int64_t E, int64_t rows, int64_t K,
                              float scale, uint8_t* codes, uint8_t* scales) {
    #pragma omp parallel
    {
        float buf[16384];
        #pragma omp for schedule(static) collapse(2)
        for (int64_t e = 0; e < E; ++e) {
            for (int64_t r = 0; r < rows; ++r) {
                uint8_t* cb = codes + (e * rows + r) * (K / 2);
                uint8_t* sb = scales + (e * rows + r) * (K / 32);
                for (int64_t c0 = 0; c0 < K; c0 += 16384) {
                    int64_t cnt = (K - c0 < 16384) ? K - c0 : 16384;
                    normal_range(seed, stream_base + (uint64_t)e, r * K + c0, cnt, scale, buf);
                    encode_row_mxfp4(buf, cnt, cb + c0 / 2, sb + c0 / 32);
                }
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * FP8 block-scaled weights (input synthesis rule for the e4m3 / 128 x 128
 * format): for each 128 x 128 block, s = amax / 448 in binary32 (0 for an
 * all-zero block) and each value goes to the e4m3 grid point nearest v / s
 * (v / 1 when s == 0), ties to the even code.
 * ------------------------------------------------------------------------- */

/* |x| <= 448 (larger magnitudes are clamped) -> e4m3 FN byte, round to nearest even. */
static uint8_t e4m3_nearest_even(float x) {
    const uint8_t sign = signbit(x) ? 0x80 : 0;
    float a = fabsf(x);
    if (a > 448.0f) a = 448.0f;
    int ex;
    frexpf(a, &ex);                        /* a = m * 2^ex, m in [0.5, 1) */
    int binade = ex - 1;
    if (binade < -6) binade = -6;          /* subnormals share the spacing of binade -6 */
    const float quantum = ldexpf(1.0f, binade - 3);
    const float r = rintf(a / quantum) * quantum;   /* exact division by a power of two; rintf ties to even */
    if (r == 0.0f) return sign;
    int ex2;
    frexpf(r, &ex2);
    const int e = ex2 - 1;
    if (e < -6) return sign | (uint8_t)(r * 512.0f);              /* subnormal: r = m * 2^-9 */
    const int m = (int)((ldexpf(r, -e) - 1.0f) * 8.0f);           /* exact */
    return sign | (uint8_t)(((e + 7) << 3) | m);
}

/* E matrices of rows x K (rows and K multiples of 128), the same normals as
 * syn_mxfp4_normal_batched, encoded as e4m3 codes [E][rows][K] and binary32
 * block scales [E][rows/128][K/128]. */
void syn_fp8block_normal_batched(uint64_t seed, uint64_t stream_base, int64_t E, int64_t rows, int64_t K,
                                 float scale, uint8_t* codes, float* scales) {
    const int64_t bands = rows / 128, KB = K / 128;
    #pragma omp parallel
    {
        float* buf = (float*)malloc(sizeof(float) * 128 * (size_t)K);
        #pragma omp for schedule(static) collapse(2)
        for (int64_t e = 0; e < E; ++e) {
            for (int64_t b = 0; b < bands; ++b) {
                for (int64_t i = 0; i < 128; ++i)
                    normal_range(seed, stream_base + (uint64_t)e, (b * 128 + i) * K, K, scale, buf + i * K);
                for (int64_t c = 0; c < KB; ++c) {
                    float amax = 0.0f;
                    for (int64_t i = 0; i < 128; ++i)
                        for (int64_t j = 0; j < 128; ++j) amax = fmaxf(amax, fabsf(buf[i * K + c * 128 + j]));
                    const float s = amax / 448.0f;
                    const float d = amax > 0.0f ? s : 1.0f;
                    scales[(e * bands + b) * KB + c] = s;
                    for (int64_t i = 0; i < 128; ++i) {
                        uint8_t* row = codes + ((e * rows) + b * 128 + i) * K + c * 128;
                        for (int64_t j = 0; j < 128; ++j) row[j] = e4m3_nearest_even(buf[i * K + c * 128 + j] / d);
                    }
                }
            }
        }
        free(buf);
    }
}

int syn_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
