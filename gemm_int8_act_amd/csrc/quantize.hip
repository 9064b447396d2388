// quantize.hip -- group-128 INT8 activation quantisation and raw-block ->
// prepared-plane preparation for gfx950.
//
// Quantiser (page "Baseline and the integer breakthrough", "Calculate with
// small integers" step 1; page "Kernel experiments: recorded evidence",
// Test 6): per group of 128 elements, scale = max|x| / 127 as one correctly
// rounded FP32 division, each element divided by the scale (or by 1 for an
// all-zero group) with the FP32 quotient correctly rounded, rounded half to
// even, clamped to +-127.  The scale is that one IEEE division; each
// element's quotient is the double product x * fl64(1 / divisor) rounded to
// FP32, which equals the IEEE quotient (the argument is beside the code), so
// q and xs are bit-identical to the definition, subnormal scales included.
//
// Geometry: 16 lanes (one DPP row) per group, 8 consecutive elements per lane
// (one 16-byte load for 2-byte types), 16 groups per 256-thread workgroup.
// The group max is a 4-step DPP reduction inside the row.
#include "pq2_device.h"
#include "pq2_internal.h"

#include <hip/hip_fp16.h>

namespace pq2 {

template <int DT>
__device__ __forceinline__ float elem_to_float(uint32_t bits16_or_32) {
    if constexpr (DT == 0) return __uint_as_float(bits16_or_32 << 16);        // bf16
    if constexpr (DT == 1) return __half2float(__ushort_as_half((unsigned short)bits16_or_32));
    return __uint_as_float(bits16_or_32);                                        // f32
}

// Max over each aligned group of LPG = 16, 8 or 4 lanes; all lanes agree.
template <int LPG>
__device__ __forceinline__ float max_lanes_f(float v) {
    if constexpr (LPG == 16) return max16_f(v);
    if constexpr (LPG == 8) return max8_f(v);
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    return fmaxf(v, dpp_f<kDppXor2>(v));
}

// DT: 0 bf16, 1 f16, 2 f32.  VEC: row bases are 16-byte aligned (2-byte types)
// or 16-byte aligned (f32), so each lane's 8 elements load as whole vectors.
// LPG lanes per activation group of 8 * LPG elements: 16 for the group-128
// quantiser; 8 and 4 for activation groups of 64 and 32 (page "Kernel
// experiments: recorded evidence", section C, Tests 8 and 9), the same
// steps on the smaller group.
template <int DT, bool VEC, int LPG = 16>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ x, int64_t row_stride,
                                                       int64_t k, int64_t total_groups,
                                                       int8_t* __restrict__ q, float* __restrict__ xs) {
    constexpr int AG = 8 * LPG;     // elements per activation group
    constexpr int GPB = 256 / LPG;  // groups per workgroup
    const int64_t gid = (int64_t)blockIdx.x * GPB + (threadIdx.x / LPG);
    const int l = threadIdx.x % LPG;
    if (gid >= total_groups) return;  // whole LPG-lane groups leave together
    const int64_t groups = k / AG;
    const int64_t row = gid / groups;
    const int64_t g = gid - row * groups;
    const int64_t base = row * row_stride + g * AG + l * 8;

    float v[8];
    if constexpr (DT == 2) {
        const float* xp = static_cast<const float*>(x) + base;
        if constexpr (VEC) {
            const float4 a = *reinterpret_cast<const float4*>(xp);
            const float4 b = *reinterpret_cast<const float4*>(xp + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = xp[e];
        }
    } else {
        const uint16_t* xp = static_cast<const uint16_t*>(x) + base;
        if constexpr (VEC) {
            const uint4 w = *reinterpret_cast<const uint4*>(xp);
            const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = elem_to_float<DT>(words[e] & 0xFFFFu);
                v[2 * e + 1] = elem_to_float<DT>(words[e] >> 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = elem_to_float<DT>(xp[e]);
        }
    }

    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    amax = max_lanes_f<LPG>(amax);

    const float scale = amax / 127.0f;                 // one IEEE division
    const float divisor = scale > 0.0f ? scale : 1.0f;
    // v / divisor as the IEEE quotient without a division per element: the
    // double product v * fl64(1 / divisor), rounded to fp32, is that quotient
    // (two fp32 values' quotient is an fp32 value or at least 2^-49 relative
    // from every fp32 rounding midpoint; the product is within 2^-52 of it).
    const double inv = 1.0 / (double)divisor;
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float r = rintf((float)((double)v[e] * inv));  // ties to even
        r = fminf(127.0f, fmaxf(-127.0f, r));
        packed[e >> 2] |= ((uint32_t)(int)r & 0xFFu) << (8 * (e & 3));
    }
    *reinterpret_cast<uint2*>(q + row * k + g * AG + l * 8) = make_uint2(packed[0], packed[1]);
    if (l == 0) xs[row * groups + g] = scale;
}

template <int DT, bool VEC, int LPG = 16>
static hipError_t launch_q(const void* x, int64_t row_stride, int64_t m, int64_t k, int8_t* q,
                           float* xs, hipStream_t stream) {
    constexpr int GPB = 256 / LPG;
    const int64_t total = m * (k / (8 * LPG));
    const int64_t blocks = (total + GPB - 1) / GPB;
    clear_stale_error();
    hipLaunchKernelGGL((quantize_kernel<DT, VEC, LPG>), dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       row_stride, k, total, q, xs);
    return hipGetLastError();
}

template <int LPG>
static hipError_t launch_q_lpg(const void* x, int dtype, int64_t row_stride, int64_t m, int64_t k, int8_t* q,
                               float* xs, hipStream_t stream) {
    const int esize = dtype == 2 ? 4 : 2;
    const bool vec = ((uintptr_t)x % 16 == 0) && ((row_stride * esize) % 16 == 0);
    if (dtype == 0) return vec ? launch_q<0, true, LPG>(x, row_stride, m, k, q, xs, stream)
                               : launch_q<0, false, LPG>(x, row_stride, m, k, q, xs, stream);
    if (dtype == 1) return vec ? launch_q<1, true, LPG>(x, row_stride, m, k, q, xs, stream)
                               : launch_q<1, false, LPG>(x, row_stride, m, k, q, xs, stream);
    return vec ? launch_q<2, true, LPG>(x, row_stride, m, k, q, xs, stream)
               : launch_q<2, false, LPG>(x, row_stride, m, k, q, xs, stream);
}

hipError_t launch_quantize_g(const void* x, int dtype, int64_t row_stride, int64_t m, int64_t k, int agroup,
                             int8_t* q, float* xs, hipStream_t stream) {
    if (agroup == 128) return launch_q_lpg<16>(x, dtype, row_stride, m, k, q, xs, stream);
    if (agroup == 64) return launch_q_lpg<8>(x, dtype, row_stride, m, k, q, xs, stream);
    if (agroup == 32) return launch_q_lpg<4>(x, dtype, row_stride, m, k, q, xs, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_quantize(const void* x, int dtype, int64_t row_stride, int64_t m, int64_t k,
                           int8_t* q, float* xs, hipStream_t stream) {
    const int esize = dtype == 2 ? 4 : 2;
    const bool vec = ((uintptr_t)x % 16 == 0) && ((row_stride * esize) % 16 == 0);
    if (dtype == 0) return vec ? launch_q<0, true>(x, row_stride, m, k, q, xs, stream)
                               : launch_q<0, false>(x, row_stride, m, k, q, xs, stream);
    if (dtype == 1) return vec ? launch_q<1, true>(x, row_stride, m, k, q, xs, stream)
                               : launch_q<1, false>(x, row_stride, m, k, q, xs, stream);
    return vec ? launch_q<2, true>(x, row_stride, m, k, q, xs, stream)
               : launch_q<2, false>(x, row_stride, m, k, q, xs, stream);
}

// ------------------------------------------------------------------ plane order
// The same quantiser, writing each 16-byte block of q (the activations that
// meet one code dword, weights 16t..16t+15) as a 4x4 byte transpose:
// qp[16t + 4s + j] = q[16t + 4j + s], so dword s of the block is the plane-s
// partner of the code dword (page "Kernel experiments", Test 21 / Diagram 7:
// plane-order activations), plus qsum[row][group] = the group's sum of q for
// the -1 code offset.  8 lanes per group, 16 elements (two 16-byte loads for
// 2-byte types) per lane, 8 groups per wave, 32 groups per 256-thread block.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void quantize_planes_kernel(const void* __restrict__ x, int64_t row_stride,
                                                              int64_t k, int64_t total_groups,
                                                              int8_t* __restrict__ qp, float* __restrict__ xs,
                                                              int32_t* __restrict__ qsum) {
    const int64_t gid = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int t = threadIdx.x & 7;
    if (gid >= total_groups) return;  // whole 8-lane groups leave together
    const int64_t groups = k / 128;
    const int64_t row = gid / groups;
    const int64_t g = gid - row * groups;
    const int64_t base = row * row_stride + g * 128 + t * 16;

    float v[16];
    if constexpr (DT == 2) {
        const float* xp = static_cast<const float*>(x) + base;
        if constexpr (VEC) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float4 a = *reinterpret_cast<const float4*>(xp + 4 * h);
                v[4 * h] = a.x; v[4 * h + 1] = a.y; v[4 * h + 2] = a.z; v[4 * h + 3] = a.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = xp[e];
        }
    } else {
        const uint16_t* xp = static_cast<const uint16_t*>(x) + base;
        if constexpr (VEC) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint4 w = *reinterpret_cast<const uint4*>(xp + 8 * h);
                const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[8 * h + 2 * e] = elem_to_float<DT>(words[e] & 0xFFFFu);
                    v[8 * h + 2 * e + 1] = elem_to_float<DT>(words[e] >> 16);
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = elem_to_float<DT>(xp[e]);
        }
    }

    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
    amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
    amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
    amax = fmaxf(amax, dpp_f<kDppHalfMirror>(amax));  // max over the group's 8 lanes

    const float scale = amax / 127.0f;                 // one IEEE division
    const float divisor = scale > 0.0f ? scale : 1.0f;
    uint32_t nat[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float r = rintf(v[e] / divisor);               // IEEE division, ties to even
        r = fminf(127.0f, fmaxf(-127.0f, r));
        nat[e >> 2] |= ((uint32_t)(int)r & 0xFFu) << (8 * (e & 3));
    }
    const uint4 Q = make_uint4(nat[0], nat[1], nat[2], nat[3]);
    int s = dot4(Q.x, 0x01010101u, 0);
    s = dot4(Q.y, 0x01010101u, s);
    s = dot4(Q.z, 0x01010101u, s);
    s = dot4(Q.w, 0x01010101u, s);
    s = sum8_i(s);
    *reinterpret_cast<uint4*>(qp + row * k + g * 128 + t * 16) = to_plane_order(Q);
    if (t == 0) {
        xs[row * groups + g] = scale;
        qsum[row * groups + g] = s;
    }
}

template <int DT, bool VEC>
static hipError_t launch_qp(const void* x, int64_t row_stride, int64_t m, int64_t k, int8_t* qp,
                            float* xs, int32_t* qsum, hipStream_t stream) {
    const int64_t total = m * (k / 128);
    const int64_t blocks = (total + 31) / 32;
    clear_stale_error();
    hipLaunchKernelGGL((quantize_planes_kernel<DT, VEC>), dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       row_stride, k, total, qp, xs, qsum);
    return hipGetLastError();
}

hipError_t launch_quantize_planes(const void* x, int dtype, int64_t row_stride, int64_t m, int64_t k,
                                  int8_t* qp, float* xs, int32_t* qsum, hipStream_t stream) {
    const int esize = dtype == 2 ? 4 : 2;
    const bool vec = ((uintptr_t)x % 16 == 0) && ((row_stride * esize) % 16 == 0);
    if (dtype == 0) return vec ? launch_qp<0, true>(x, row_stride, m, k, qp, xs, qsum, stream)
                               : launch_qp<0, false>(x, row_stride, m, k, qp, xs, qsum, stream);
    if (dtype == 1) return vec ? launch_qp<1, true>(x, row_stride, m, k, qp, xs, qsum, stream)
                               : launch_qp<1, false>(x, row_stride, m, k, qp, xs, qsum, stream);
    return vec ? launch_qp<2, true>(x, row_stride, m, k, qp, xs, qsum, stream)
               : launch_qp<2, false>(x, row_stride, m, k, qp, xs, qsum, stream);
}

// ------------------------------------------------------------------ prepare
// One thread per 34-byte raw block: byte loads (raw rows may sit at any
// alignment), two 16-byte stores into the code plane, one 2-byte store into
// the scale plane.  Values are copied unchanged (page "Baseline and the
// integer breakthrough", "Separate the codes from their scales").
__global__ __launch_bounds__(256) void prepare_kernel(const uint8_t* __restrict__ raw, int64_t stride,
                                                      int64_t n, int64_t groups, int64_t total,
                                                      uint8_t* __restrict__ planes) {
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= total) return;
    const int64_t row = id / groups;
    const int64_t g = id - row * groups;
    const uint8_t* b = raw + row * stride + g * 34;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        w[i] = (uint32_t)b[2 + 4 * i] | ((uint32_t)b[3 + 4 * i] << 8) | ((uint32_t)b[4 + 4 * i] << 16) |
               ((uint32_t)b[5 + 4 * i] << 24);
    }
    uint4* dst = reinterpret_cast<uint4*>(planes + row * groups * 32 + g * 32);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    uint16_t* scale_plane = reinterpret_cast<uint16_t*>(planes + n * groups * 32);
    scale_plane[row * groups + g] = (uint16_t)(b[0] | (b[1] << 8));
}

hipError_t launch_prepare(const uint8_t* raw, int64_t stride, int64_t n, int64_t k, uint8_t* planes,
                          hipStream_t stream) {
    const int64_t groups = k / 128;
    const int64_t total = n * groups;
    const int64_t blocks = (total + 255) / 256;
    clear_stale_error();
    hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, raw, stride, n,
                       groups, total, planes);
    return hipGetLastError();
}

}  // namespace pq2
