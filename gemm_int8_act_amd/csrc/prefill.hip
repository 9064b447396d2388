// prefill.hip -- prefill matmul (many activation rows) on the gfx950 INT8
// matrix cores.
//
// What it computes is the same definition as the small-m path (page
// "Baseline and the integer breakthrough", "Use matrix hardware for
// prefill"; page "Kernel experiments: recorded evidence", Tests 2 and 7):
// per group of 128 weights an exact INT32 matrix product of INT8 activations
// and decoded codes, then a per-element FP32 rescale by xs[m][g] * ws[n][g]
// accumulated over groups.
//
// Design:
//  * Workgroup tile BM x BN = 128 x 128 outputs, 4 waves as 2 x 2, each wave
//    64 x 64 = 2 x 2 tiles of v_mfma_i32_32x32x32_i8.  One group (k = 128) =
//    four MFMA k-steps of 32.
//  * Operand order inside a k-step is free as long as A and B agree: lane l
//    of an MFMA supplies 16 bytes of row (l % 32) of A and of column (l % 32)
//    of B for the same 16 k positions.  We give lane half h = l / 32 in
//    k-step kk the 16 weights of code dword t = 2kk + h, in the order the
//    add/XOR decode produces them (plane s, byte j <-> weight 16t + 4j + s),
//    and stage A in LDS already byte-transposed to that order.  So B needs
//    no re-shuffle after decoding: one code dword -> one 16-byte operand.
//  * Both tiles live in LDS with a quad-level XOR swizzle (slot t ^ (row & 7))
//    so the 32 rows a fragment read touches spread over all banks.
//  * After the four MFMA k-steps of a group, each lane rescales its 16 INT32
//    results per tile: acc += float(dot) * xs[m] * ws[n].
#include "pq2_device.h"
#include "pq2_internal.h"

#include <hip/hip_fp16.h>

namespace pq2 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;
constexpr int kBN = 128;

__global__ __launch_bounds__(256) void prefill_kernel(const int8_t* __restrict__ q,
                                                      const float* __restrict__ xs,
                                                      const uint8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales,
                                                      float* __restrict__ y, int m, int n, int k,
                                                      int groups) {
    __shared__ uint4 As[kBM * 8];  // [row m][quad slot]: plane-ordered activations
    __shared__ uint4 Bs[kBN * 8];  // [row n][quad slot]: decoded signed weights
    __shared__ float xsS[kBM];
    __shared__ float wsS[kBN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int nb = blockIdx.x * kBN;
    const int mb = blockIdx.y * kBM;
    const int k4 = k >> 2;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    float acc[2][2][16];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    for (int g = 0; g < groups; ++g) {
        // Stage A: 128 rows x 8 quads, four quads per thread.
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int it = tid + 256 * p;
            const int i = it >> 3;
            const int t = it & 7;
            const int row = mb + i;
            uint4 Q = make_uint4(0u, 0u, 0u, 0u);
            if (row < m) Q = *reinterpret_cast<const uint4*>(q + (size_t)row * k + (size_t)g * 128 + t * 16);
            As[i * 8 + (t ^ (i & 7))] = to_plane_order(Q);
        }
        // Stage B: 128 rows x 32 code bytes; thread = (row, half), 4 code dwords each.
        {
            const int i = tid >> 1;
            const int h = tid & 1;
            const int row = nb + i;
            uint4 C = make_uint4(0u, 0u, 0u, 0u);
            if (row < n) C = *reinterpret_cast<const uint4*>(codes + (size_t)row * k4 + (size_t)g * 32 + h * 16);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t d = word_of(C, c);
                const int t = 4 * h + c;
                Bs[i * 8 + (t ^ (i & 7))] =
                    make_uint4(expand_plane<0>(d), expand_plane<1>(d), expand_plane<2>(d), expand_plane<3>(d));
            }
        }
        if (tid < kBM) {
            const int row = mb + tid;
            xsS[tid] = row < m ? xs[(size_t)row * groups + g] : 0.0f;
        } else {
            const int i = tid - kBM;
            const int row = nb + i;
            wsS[i] = row < n ? __half2float(__ushort_as_half(scales[(size_t)row * groups + g])) : 0.0f;
        }
        __syncthreads();

        v16i D[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) D[a][b][r] = 0;

#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int t = 2 * kk + hi;
            v4i af[2], bf[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int i = wm * 64 + mt * 32 + l32;
                const uint4 v = As[i * 8 + (t ^ (i & 7))];
                af[mt] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int i = wn * 64 + nt * 32 + l32;
                const uint4 v = Bs[i * 8 + (t ^ (i & 7))];
                bf[nt] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    D[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mt], bf[nt], D[mt][nt], 0, 0, 0);
        }

        // Rescale: lane holds column n = l32 of each 32x32 tile and rows
        // 8*(r/4) + 4*hi + (r%4), r = 0..15.
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const float wsv = wsS[wn * 64 + nt * 32 + l32];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const float4 xv = *reinterpret_cast<const float4*>(&xsS[wm * 64 + mt * 32 + rb * 8 + hi * 4]);
                    const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = rb * 4 + e;
                        acc[mt][nt][r] += ((float)D[mt][nt][r] * xa[e]) * wsv;
                    }
                }
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int col = nb + wn * 64 + nt * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = mb + wm * 64 + mt * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
                if (row < m && col < n) y[(size_t)row * n + col] = acc[mt][nt][r];
            }
        }
}

hipError_t launch_prefill(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m,
                          int64_t n, int64_t k, float* y, hipStream_t stream) {
    const uint8_t* codes = planes;
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(planes + n * (k / 4));
    const dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
    clear_stale_error();
    hipLaunchKernelGGL(prefill_kernel, grid, dim3(256), 0, stream, q, xs, codes, scales, y, (int)m,
                       (int)n, (int)k, (int)(k / 128));
    return hipGetLastError();
}

}  // namespace pq2
