// small_m_common.h -- pieces shared by the small-m (decode / verification)
// kernels of libpq2: the per-wave activation staging geometry, the kinds of
// activation source, and the exact in-kernel group-128 quantiser used by the
// fused (quantise + matmul) entry points.
#pragma once

#include "pq2_device.h"
#include "pq2_internal.h"

#include <hip/hip_fp16.h>

namespace pq2 {

constexpr int kGroupLanes = 8;   // lanes per row slot
constexpr int kRowSlots = 8;     // row slots per wave
constexpr int kBlockPitch = 9;   // LDS quads per group (8 + 1 pad; pad dword 0 = sum(q))
constexpr int kSegQuads = kGroupLanes * kBlockPitch;  // LDS quads per (segment, column)

// Bytes 0 of a, b, c, d packed into one dword (byte i from the i-th argument).
__device__ __forceinline__ uint32_t low_bytes4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
    return ab | (cd << 16);
}

// INT8 quantisation (page "Baseline and the integer breakthrough",
// "Calculate with small integers" step 1) of one activation group of 16 * GL
// elements held 16 per lane by GL aligned lanes (GL = 8: a 128-element group;
// 4 and 2: the 64- and 32-element groups of page "Kernel experiments: recorded
// evidence", section C): lane j of the group holds elements 16j..16j+15 in v.
// Returns the lane's 16 codes in plane order (dword s = codes 16j + s, +4,
// +8, +12), or with PLANE false in natural order (dword s = codes 16j + 4s ..
// 16j + 4s + 3), and sets gsum (group sum of q, all GL lanes) and scale
// (max|x| / 127, correctly rounded).  The codes equal the
// definition q = clamp(rint(RN(x / d)), +-127), d = scale or 1 for an
// all-zero group, bit for bit:
//  * RN(x / d) is computed as the double product x * fl64(1 / d) rounded to
//    fp32.  The quotient of two fp32 values is either an fp32 value or at
//    least 2^-49 (relative) away from every fp32 rounding midpoint (24-bit
//    significands, 25-bit midpoints), and the product is within 2^-52 of
//    the quotient, so both round to the same fp32 value, for subnormal d too;
//  * the clamp to +-127 comes before the rounding: adding 1.5 * 2^23 rounds
//    the clamped value half to even in the low mantissa bits, whose low byte
//    is the two's-complement code.
template <bool PLANE = true, int GL = 8>
__device__ __forceinline__ uint4 quantize_lane16(const float (&v)[16], int& gsum, float& scale) {
#pragma clang fp contract(off)
    static_assert(GL == 8 || GL == 4 || GL == 2, "lanes per activation group");
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
    if constexpr (GL == 8) {
        amax = max8_f(amax);
    } else {
        amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
        if constexpr (GL == 4) amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
    }
    scale = amax / 127.0f;
    const float d = scale > 0.0f ? scale : 1.0f;
    // The IEEE quotient v / d without a division per element.  v / d of two
    // fp32 values is either an fp32 value or at least 2^-49 (relative) away
    // from every fp32 rounding midpoint (its numerator and denominator have
    // 24-bit significands, a midpoint 25 bits), while the double product
    // v * fl64(1 / d) is within 2^-52 of it; so rounding that product to fp32
    // gives exactly the IEEE quotient, ties and subnormal scales included.
    const double r = 1.0 / (double)d;
    constexpr float kRound = 12582912.0f;  // 1.5 * 2^23: t + kRound rounds t half to even
    uint32_t bits[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float t = fminf(127.0f, fmaxf(-127.0f, (float)((double)v[e] * r)));
        bits[e] = __float_as_uint(t + kRound);  // low byte: the two's-complement code
    }
    uint4 out;
    if constexpr (PLANE) {
        out.x = low_bytes4(bits[0], bits[4], bits[8], bits[12]);
        out.y = low_bytes4(bits[1], bits[5], bits[9], bits[13]);
        out.z = low_bytes4(bits[2], bits[6], bits[10], bits[14]);
        out.w = low_bytes4(bits[3], bits[7], bits[11], bits[15]);
    } else {
        out.x = low_bytes4(bits[0], bits[1], bits[2], bits[3]);
        out.y = low_bytes4(bits[4], bits[5], bits[6], bits[7]);
        out.z = low_bytes4(bits[8], bits[9], bits[10], bits[11]);
        out.w = low_bytes4(bits[12], bits[13], bits[14], bits[15]);
    }
    int s = dot4(out.x, 0x01010101u, 0);
    s = dot4(out.y, 0x01010101u, s);
    s = dot4(out.z, 0x01010101u, s);
    s = dot4(out.w, 0x01010101u, s);
    if constexpr (GL == 8) {
        gsum = sum8_i(s);
    } else {
        s += dpp_i<kDppXor1>(s);
        if constexpr (GL == 4) s += dpp_i<kDppXor2>(s);
        gsum = s;
    }
    return out;
}

// The 16 elements of x a lane quantises, from its SRC-typed 16-byte loads.
template <int SRC>
__device__ __forceinline__ void x_to_float16(const uint4 (&w)[src_xloads(SRC)], float (&v)[16]) {
    if constexpr (SRC == kSrcF32) {
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            v[4 * l + 0] = __uint_as_float(w[l].x);
            v[4 * l + 1] = __uint_as_float(w[l].y);
            v[4 * l + 2] = __uint_as_float(w[l].z);
            v[4 * l + 3] = __uint_as_float(w[l].w);
        }
    } else {
#pragma unroll
        for (int l = 0; l < 2; ++l) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t d = word_of(w[l], i);
                if constexpr (SRC == kSrcBf16) {
                    v[8 * l + 2 * i] = __uint_as_float(d << 16);
                    v[8 * l + 2 * i + 1] = __uint_as_float(d & 0xFFFF0000u);
                } else {
                    v[8 * l + 2 * i] = __half2float(__ushort_as_half((unsigned short)(d & 0xFFFFu)));
                    v[8 * l + 2 * i + 1] = __half2float(__ushort_as_half((unsigned short)(d >> 16)));
                }
            }
        }
    }
}

}  // namespace pq2
