/*
 * pq2_oracle.c -- plain, slow CPU oracle for the packed-ternary x INT8
 * activation matmul ("PQ2" weights).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or helper with the HIP
 * library; both sides meet only at the seeded input generators.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no FMA contraction, no fast-math: the FP32 quantiser steps are single
 * IEEE-754 operations in round-to-nearest-even, exactly as written).
 *
 * Sources (the web pages the method is described on):
 *  [KE]  "Kernel experiments: recorded evidence" (companion guide to
 *        "Making a ternary reasoning model fast in vLLM").
 *  [BIB] "Baseline and the integer breakthrough" (same series).
 *
 * Format facts used here, restated:
 *  - A raw PQ2 block holds 128 weights in 34 bytes: bytes 0-1 are an IEEE
 *    binary16 scale (little-endian), bytes 2..33 are 32 code bytes
 *    ([KE] section A, Diagram 1 and Test 1's preparation code; [BIB]
 *    "Separate the codes from their scales", interleaved address formula).
 *  - Weight 4b+s of the block sits in bits 2s..2s+1 of code byte b, lowest
 *    bits first; code c in 0..3 stands for the value c-1, so 0,1,2,3 mean
 *    -1,0,+1,+2 ([KE] Test 1 byte expansion, slow path; Test 2 expansion
 *    of four planes; [BIB] "Unpack four weights with fewer instructions").
 *  - The prepared layout is one allocation: all code bytes first as
 *    [N][K/4] (row*K/4 + block*32 + byte), then all fp16 scales as
 *    [N][K/128] ([KE] Test 4; [BIB] "Separate the codes from their scales").
 *  - Activations are quantised per 128-element group: scale = max|x|/127 in
 *    FP32, x/scale correctly rounded, rounded half-to-even, clamped to
 *    +-127; an all-zero group divides by 1 ([BIB] "Calculate with small
 *    integers" step 1; [KE] Test 6 quantizer).
 *  - Each group's integer dot product is multiplied by activation scale x
 *    weight scale and the groups are summed ([BIB] "Calculate with small
 *    integers" steps 3-4; [KE] Test 8 FP64 reconstruction).
 *
 * Every function is the plain definition: no blocking, no fusion, no
 * reordering beyond what the definition states.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GROUP 128
#define BLOCK_BYTES 34

enum { ORACLE_BF16 = 0, ORACLE_F16 = 1, ORACLE_F32 = 2 };

/* IEEE binary16 bit pattern -> double (exact: every binary16 is a double). */
static double half_bits_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)mant, -24);               /* subnormal / zero */
    } else if (expo == 31) {
        v = mant ? NAN : INFINITY;
    } else {
        v = ldexp((double)(mant | 0x400), expo - 25); /* 1.mant * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 bit pattern -> float: the upper half of a binary32 (exact). */
static float bf16_bits_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* One activation element as FP32 (exact for bf16, f16 and f32 inputs). */
static float load_activation(const void* x, int dtype, int64_t idx) {
    if (dtype == ORACLE_BF16) return bf16_bits_to_float(((const uint16_t*)x)[idx]);
    if (dtype == ORACLE_F16) return (float)half_bits_to_double(((const uint16_t*)x)[idx]);
    return ((const float*)x)[idx];
}

/* Signed weight value of weight i (0..127) of a block whose 32 code bytes
 * start at `codes`: code bits 2s..2s+1 of byte i/4, s = i%4, value code-1. */
int oracle_decode_weight(const uint8_t* codes, int i) {
    int byte = codes[i / 4];
    int code = (byte >> (2 * (i % 4))) & 3;
    return code - 1;
}

/* Decode one code byte into its four weight values, weight 4b+s -> out[s]. */
void oracle_decode_byte(uint8_t byte, int8_t out[4]) {
    for (int s = 0; s < 4; ++s) out[s] = (int8_t)(((byte >> (2 * s)) & 3) - 1);
}

/* Raw blocks -> prepared planes.  raw row n starts at raw + n*row_stride;
 * block g of that row at byte 34*g.  planes: codes [n][k/4] then scales
 * [n][k/128] (two bytes each).  Values are copied unchanged. */
int oracle_prepare_planes(const uint8_t* raw, int64_t row_stride, int64_t n, int64_t k,
                          uint8_t* planes) {
    if (k <= 0 || k % GROUP || n <= 0 || row_stride < (k / GROUP) * BLOCK_BYTES) return 1;
    int64_t groups = k / GROUP;
    uint8_t* code_plane = planes;
    uint8_t* scale_plane = planes + n * (k / 4);
    for (int64_t row = 0; row < n; ++row) {
        for (int64_t g = 0; g < groups; ++g) {
            const uint8_t* block = raw + row * row_stride + g * BLOCK_BYTES;
            for (int b = 0; b < 32; ++b) code_plane[row * (k / 4) + g * 32 + b] = block[2 + b];
            scale_plane[(row * groups + g) * 2 + 0] = block[0];
            scale_plane[(row * groups + g) * 2 + 1] = block[1];
        }
    }
    return 0;
}

/* Tile layout of the weights for the decode GEMV (the layout's definition
 * is stated with the library's pq2_prepare_tiles; the pages motivate it in
 * [KE] section H, Tests 24 and 25: the bytes one wave loads sit next to each
 * other).  Same values, other addresses.  T = ceil(n/16) tiles of 16 rows,
 * S8 = ceil(G/8) segments of 8 groups, one 4352-byte unit per (tile,
 * segment) at (t*S8 + sb)*4352:
 *  - code byte 1024*b + 16*l + 4*u + v of the unit, bits 2s..2s+1, with
 *    l = j + 16*kb, holds the code of weight k0 + 4s + v of row 16t + j,
 *    k0 = 128*(8sb + 2b + u/2) + 64*(u%2) + 16*kb;
 *  - the fp16 scale of row 16t + j, group 8*sb + e sits at unit byte
 *    4096 + 16*j + 2*e (little-endian);
 *  - padding (rows >= n, groups >= G): code 1 (weight 0), scale 0.
 * Written as a scatter over every (row, weight) and (row, group) of the
 * padded matrix, one field at a time. */
int64_t oracle_tiles_bytes(int64_t n, int64_t k) {
    if (k <= 0 || k % GROUP || n <= 0) return -1;
    return ((n + 15) / 16) * ((k / GROUP + 7) / 8) * 4352;
}

int oracle_prepare_tiles(const uint8_t* raw, int64_t row_stride, int64_t n, int64_t k, uint8_t* out) {
    if (k <= 0 || k % GROUP || n <= 0 || row_stride < (k / GROUP) * BLOCK_BYTES) return 1;
    int64_t groups = k / GROUP, tiles = (n + 15) / 16, s8 = (groups + 7) / 8;
    for (int64_t i = 0; i < oracle_tiles_bytes(n, k); ++i) out[i] = 0;
    for (int64_t t = 0; t < tiles; ++t) {
        for (int64_t sb = 0; sb < s8; ++sb) {
            uint8_t* unit = out + (t * s8 + sb) * 4352;
            for (int b = 0; b < 4; ++b) {
                for (int l = 0; l < 64; ++l) {
                    int j = l % 16, kb = l / 16;
                    int64_t row = 16 * t + j;
                    for (int u = 0; u < 4; ++u) {
                        int64_t g = 8 * sb + 2 * b + u / 2;
                        int64_t k0 = 128 * g + 64 * (u % 2) + 16 * kb;
                        for (int v = 0; v < 4; ++v) {
                            for (int s = 0; s < 4; ++s) {
                                int64_t w = k0 + 4 * s + v;   /* weight index within the row */
                                unsigned code = 1;
                                if (row < n && g < groups) {
                                    int64_t i = w % GROUP;    /* weight index within its block */
                                    uint8_t byte = raw[row * row_stride + g * BLOCK_BYTES + 2 + i / 4];
                                    code = (byte >> (2 * (i % 4))) & 3u;
                                }
                                unit[1024 * b + 16 * l + 4 * u + v] |= (uint8_t)(code << (2 * s));
                            }
                        }
                    }
                }
            }
            for (int j = 0; j < 16; ++j) {
                int64_t row = 16 * t + j;
                for (int e = 0; e < 8; ++e) {
                    int64_t g = 8 * sb + e;
                    if (row < n && g < groups) {
                        unit[4096 + 16 * j + 2 * e] = raw[row * row_stride + g * BLOCK_BYTES + 0];
                        unit[4096 + 16 * j + 2 * e + 1] = raw[row * row_stride + g * BLOCK_BYTES + 1];
                    }
                }
            }
        }
    }
    return 0;
}

/* Group-128 INT8 activation quantisation.  x is [m][k] with row stride
 * `row_stride` elements; q is [m][k] int8; xs is [m][k/128] float. */
int oracle_quantize_act_i8(const void* x, int dtype, int64_t row_stride, int64_t m, int64_t k,
                           int8_t* q, float* xs) {
    if (k <= 0 || k % GROUP || m <= 0 || row_stride < k) return 1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F16 && dtype != ORACLE_F32) return 1;
    int64_t groups = k / GROUP;
    for (int64_t row = 0; row < m; ++row) {
        for (int64_t g = 0; g < groups; ++g) {
            int64_t base = row * row_stride + g * GROUP;
            float amax = 0.0f;
            for (int i = 0; i < GROUP; ++i) {
                float a = fabsf(load_activation(x, dtype, base + i));
                if (a > amax) amax = a;
            }
            float scale = amax / 127.0f;               /* one IEEE FP32 division */
            float divisor = scale > 0.0f ? scale : 1.0f;
            for (int i = 0; i < GROUP; ++i) {
                float a = load_activation(x, dtype, base + i);
                float r = nearbyintf(a / divisor);     /* ties to even (FE_TONEAREST) */
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                q[row * k + g * GROUP + i] = (int8_t)r;
            }
            xs[row * groups + g] = scale;
        }
    }
    return 0;
}

/* One output y[mi][ni] from raw blocks, plus its acceptance bound. */
static void one_output(const int8_t* q, const float* xs, const uint8_t* raw, int64_t row_stride,
                       int64_t k, int64_t mi, int64_t ni, double* y, double* bound) {
    int64_t groups = k / GROUP;
    double acc = 0.0, mag = 0.0;
    for (int64_t g = 0; g < groups; ++g) {
        const uint8_t* block = raw + ni * row_stride + g * BLOCK_BYTES;
        int32_t dot = 0;                                   /* exact integer group dot */
        for (int i = 0; i < GROUP; ++i)
            dot += (int32_t)q[mi * k + g * GROUP + i] * oracle_decode_weight(block + 2, i);
        double ws = half_bits_to_double((uint16_t)(block[0] | (block[1] << 8)));
        /* |dot| < 2^15, xs has 24 significant bits, ws 11: the product is exact. */
        double term = (double)dot * (double)xs[mi * groups + g] * ws;
        acc += term;
        mag += fabs(term);
    }
    *y = acc;
    *bound = 1e-5 * mag + 1e-6;
}

/* Full output y[m][n] (double) and bound[m][n]. */
int oracle_matmul_raw(const int8_t* q, const float* xs, const uint8_t* raw, int64_t row_stride,
                      int64_t m, int64_t n, int64_t k, double* y, double* bound) {
    if (k <= 0 || k % GROUP || m <= 0 || n <= 0 || row_stride < (k / GROUP) * BLOCK_BYTES) return 1;
    for (int64_t mi = 0; mi < m; ++mi)
        for (int64_t ni = 0; ni < n; ++ni)
            one_output(q, xs, raw, row_stride, k, mi, ni, &y[mi * n + ni], &bound[mi * n + ni]);
    return 0;
}

/* Selected outputs (mi[c], ni[c]) for c < count: for full-size shapes that
 * the complete product would take too long for. */
int oracle_matmul_raw_sample(const int8_t* q, const float* xs, const uint8_t* raw,
                             int64_t row_stride, int64_t m, int64_t n, int64_t k,
                             const int64_t* mi, const int64_t* ni, int64_t count,
                             double* y, double* bound) {
    if (k <= 0 || k % GROUP || m <= 0 || n <= 0 || row_stride < (k / GROUP) * BLOCK_BYTES) return 1;
    for (int64_t c = 0; c < count; ++c) {
        if (mi[c] < 0 || mi[c] >= m || ni[c] < 0 || ni[c] >= n) return 1;
        one_output(q, xs, raw, row_stride, k, mi[c], ni[c], &y[c], &bound[c]);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Smaller activation groups ([KE] section C, Diagram 3, Tests 8 and 9): the
 * weights keep their 128-weight blocks and one fp16 scale per block, while
 * each activation row is quantised in groups of `agroup` = 128, 64 or 32
 * elements, every group with its own scale max|x|/127 (the same steps as
 * above, on the smaller group).  A weight block then spans 128/agroup
 * activation groups; the integer dot of each activation group against the
 * block's codes is scaled by that group's xs and the block's ws, and all
 * these terms are summed.  agroup = 128 is the group-128 definition above.
 */
static int valid_agroup(int64_t agroup) { return agroup == 128 || agroup == 64 || agroup == 32; }

/* q is [m][k] int8; xs is [m][k/agroup] float. */
int oracle_quantize_act_i8_g(const void* x, int dtype, int64_t row_stride, int64_t m, int64_t k,
                             int64_t agroup, int8_t* q, float* xs) {
    if (k <= 0 || k % GROUP || m <= 0 || row_stride < k || !valid_agroup(agroup)) return 1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F16 && dtype != ORACLE_F32) return 1;
    int64_t ngroups = k / agroup;
    for (int64_t row = 0; row < m; ++row) {
        for (int64_t a = 0; a < ngroups; ++a) {
            int64_t base = row * row_stride + a * agroup;
            float amax = 0.0f;
            for (int64_t i = 0; i < agroup; ++i) {
                float v = fabsf(load_activation(x, dtype, base + i));
                if (v > amax) amax = v;
            }
            float scale = amax / 127.0f;               /* one IEEE FP32 division */
            float divisor = scale > 0.0f ? scale : 1.0f;
            for (int64_t i = 0; i < agroup; ++i) {
                float v = load_activation(x, dtype, base + i);
                float r = nearbyintf(v / divisor);     /* ties to even (FE_TONEAREST) */
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                q[row * k + a * agroup + i] = (int8_t)r;
            }
            xs[row * ngroups + a] = scale;
        }
    }
    return 0;
}

/* One output with activation groups of `agroup`, plus its acceptance bound
 * (the same form as the group-128 bound, over every scaled term). */
static void one_output_g(const int8_t* q, const float* xs, const uint8_t* raw, int64_t row_stride,
                         int64_t k, int64_t agroup, int64_t mi, int64_t ni, double* y, double* bound) {
    int64_t blocks = k / GROUP, per_block = GROUP / agroup, ngroups = k / agroup;
    double acc = 0.0, mag = 0.0;
    for (int64_t g = 0; g < blocks; ++g) {
        const uint8_t* block = raw + ni * row_stride + g * BLOCK_BYTES;
        double ws = half_bits_to_double((uint16_t)(block[0] | (block[1] << 8)));
        for (int64_t s = 0; s < per_block; ++s) {
            int64_t a = g * per_block + s;             /* activation group */
            int32_t dot = 0;                           /* exact integer dot over that group */
            for (int64_t i = 0; i < agroup; ++i)
                dot += (int32_t)q[mi * k + a * agroup + i] * oracle_decode_weight(block + 2, (int)(s * agroup + i));
            /* |dot| < 2^15, xs has 24 significant bits, ws 11: exact in double. */
            double term = (double)dot * (double)xs[mi * ngroups + a] * ws;
            acc += term;
            mag += fabs(term);
        }
    }
    *y = acc;
    *bound = 1e-5 * mag + 1e-6;
}

int oracle_matmul_raw_g(const int8_t* q, const float* xs, const uint8_t* raw, int64_t row_stride,
                        int64_t m, int64_t n, int64_t k, int64_t agroup, double* y, double* bound) {
    if (k <= 0 || k % GROUP || m <= 0 || n <= 0 || row_stride < (k / GROUP) * BLOCK_BYTES || !valid_agroup(agroup))
        return 1;
    for (int64_t mi = 0; mi < m; ++mi)
        for (int64_t ni = 0; ni < n; ++ni)
            one_output_g(q, xs, raw, row_stride, k, agroup, mi, ni, &y[mi * n + ni], &bound[mi * n + ni]);
    return 0;
}

int oracle_matmul_raw_sample_g(const int8_t* q, const float* xs, const uint8_t* raw, int64_t row_stride,
                               int64_t m, int64_t n, int64_t k, int64_t agroup, const int64_t* mi,
                               const int64_t* ni, int64_t count, double* y, double* bound) {
    if (k <= 0 || k % GROUP || m <= 0 || n <= 0 || row_stride < (k / GROUP) * BLOCK_BYTES || !valid_agroup(agroup))
        return 1;
    for (int64_t c = 0; c < count; ++c) {
        if (mi[c] < 0 || mi[c] >= m || ni[c] < 0 || ni[c] >= n) return 1;
        one_output_g(q, xs, raw, row_stride, k, agroup, mi[c], ni[c], &y[c], &bound[c]);
    }
    return 0;
}
