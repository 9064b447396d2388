// small_m_planes.hip -- the small-m matmul reading activations that are
// already in code-plane order, with their per-group sums.
//
// Same definition as small_m.hip (page "Baseline and the integer
// breakthrough", the integer hot loop; page "Kernel experiments: recorded
// evidence", Tests 2 and 7): per group of 128 weights an exact INT32 dot of
// INT8 activations and signed codes, scaled in FP32 by xs * ws and summed over
// groups lane by lane.  The activation operand arrives from the plane-order
// quantiser (Test 21 on the same page: the quantiser feeds a layout the
// matmul can use without a re-shuffle), so:
//  * no workgroup-wide staging or transposition: every wave copies the 16-byte
//    activation blocks of its own k segments into a private LDS region and
//    reads them back 16 bytes at a time, so all lanes of a row slot share them;
//  * decode is the masked-plane form for every M: code dword D gives the four
//    byte planes D & 0x03.., D & 0x0C.., D & 0x30.., (D >> 2) & 0x30..; plane s
//    holds (c << 2s) per byte, so three INT32 accumulators (planes 0, 1 and
//    2+3 scaled by 1, 4 and 16) recombine exactly as a0 + (a1 >> 2) + (a23 >> 4)
//    and the "code - 1" offset is one subtraction of sum(q) per group;
//  * the per-group sums arrive precomputed next to xs.
// Layout of work: as in small_m.hip -- a wave is 8 row slots x 8 group lanes,
// each lane owns R weight rows and walks groups j, j+8, ... of the wave's
// k segments; waves of a workgroup split k and are summed in index order.
#include "pq2_device.h"
#include "pq2_internal.h"

#include <hip/hip_fp16.h>

namespace pq2 {

constexpr int kGroupLanes = 8;   // lanes per row slot (one group each)
constexpr int kRowSlots = 8;     // row slots per wave

template <int MC, int R, int SEGS>
__global__ __launch_bounds__(512) void small_m_planes_kernel(
    const int8_t* __restrict__ qp, const float* __restrict__ xs, const int32_t* __restrict__ qsum,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, float* __restrict__ y, int n,
    int k, int groups, int nseg, int segs_per_wave, int mtotal) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int RB = kRowSlots * R;
    constexpr int QUADS = SEGS * MC * 64;  // private activation quads per wave
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int slot = lane >> 3;
    const int j = lane & 7;
    const int m0 = blockIdx.y * MC;
    const int mcount = min(MC, mtotal - m0);
    const int row_base = blockIdx.x * RB;
    const int rows_here = min(RB, n - row_base);
    const int seg_begin = wave * segs_per_wave;
    const int seg_end = min(seg_begin + segs_per_wave, nseg);
    const uint32_t k4 = (uint32_t)k >> 2;
    uint4* qw = reinterpret_cast<uint4*>(smem) + (size_t)wave * QUADS;
    float* red = reinterpret_cast<float*>(reinterpret_cast<uint4*>(smem) + (size_t)nwaves * QUADS);

    const auto code_rs = make_rsrc(codes + (size_t)row_base * k4, (uint32_t)rows_here * k4);
    const auto scale_rs = make_rsrc(scales + (size_t)row_base * groups, (uint32_t)(rows_here * groups * 2));
    const auto q_rs = make_rsrc(qp + (size_t)m0 * k, (uint32_t)(mcount * k));
    const auto xs_rs = make_rsrc(xs + (size_t)m0 * groups, (uint32_t)(mcount * groups * 4));
    const auto qs_rs = make_rsrc(qsum + (size_t)m0 * groups, (uint32_t)(mcount * groups * 4));

    // Per-lane LDS byte offsets of the 8 activation quads of its group in a
    // (segment, column) block: quad t of group-lane j sits at slot t ^ j.
    uint32_t rd_off[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) rd_off[t] = (uint32_t)(j * 8 + (t ^ j)) * 16u;
    const uint32_t wr_off = (uint32_t)(slot * 8 + (j ^ slot)) * 16u;  // this lane copies quad j of group-lane slot

    float acc[MC][R];
#pragma unroll
    for (int m = 0; m < MC; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

    for (int base = seg_begin; base < seg_end; base += SEGS) {
        // 1. Activation blocks of this step (L2-resident, short latency) ...
        uint4 qv[SEGS][MC];
        uint32_t xsv[SEGS][MC], tv[SEGS][MC];
#pragma unroll
        for (int si = 0; si < SEGS; ++si) {
            const bool sok = base + si < seg_end;
            const int gq = (base + si) * kGroupLanes + slot;  // group this lane copies a quad of
            const int g = (base + si) * kGroupLanes + j;      // group this lane computes
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const bool qok = sok && gq < groups && m < mcount;
                const bool gok = sok && g < groups && m < mcount;
                qv[si][m] = buf_load16(q_rs, qok ? (uint32_t)(m * k + gq * 128 + j * 16) : kBufferOOB);
                xsv[si][m] = buf_load4(xs_rs, gok ? (uint32_t)((m * groups + g) * 4) : kBufferOOB);
                tv[si][m] = buf_load4(qs_rs, gok ? (uint32_t)((m * groups + g) * 4) : kBufferOOB);
            }
        }
        // 2. ... then every code load of the step (HBM), all in flight together.
        uint4 cw[SEGS][R][2];
        uint32_t wsraw[SEGS][R];
#pragma unroll
        for (int si = 0; si < SEGS; ++si) {
            const int g = (base + si) * kGroupLanes + j;
            const bool gok = (base + si < seg_end) && (g < groups);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t rl = (uint32_t)(slot + kRowSlots * r);
                const uint32_t off = gok ? rl * k4 + (uint32_t)g * 32u : kBufferOOB;
                cw[si][r][0] = buf_load16<kAuxNonTemporal>(code_rs, off);
                cw[si][r][1] = buf_load16<kAuxNonTemporal>(code_rs, off + 16u);
                wsraw[si][r] = buf_load2(scale_rs, gok ? (rl * groups + g) * 2u : kBufferOOB);
            }
        }
        // 3. Private LDS copy of the activation blocks.  One wave writes and
        //    reads its own region; LDS operations of a wave complete in order.
#pragma unroll
        for (int si = 0; si < SEGS; ++si)
#pragma unroll
            for (int m = 0; m < MC; ++m)
                *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(qw + (si * MC + m) * 64) + wr_off) = qv[si][m];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // 4. Integer group dots, FP32 scaling, lane-serial accumulation.
#pragma unroll
        for (int si = 0; si < SEGS; ++si) {
            if (base + si < seg_end) {
                int a0[MC][R], a1[MC][R], a2[MC][R];
#pragma unroll
                for (int m = 0; m < MC; ++m)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        a0[m][r] = -(int)tv[si][m];
                        a1[m][r] = 0;
                        a2[m][r] = 0;
                    }
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    uint4 P[MC];
#pragma unroll
                    for (int m = 0; m < MC; ++m)
                        P[m] = *reinterpret_cast<const uint4*>(
                            reinterpret_cast<const unsigned char*>(qw + (si * MC + m) * 64) + rd_off[t]);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t d = word_of(cw[si][r][t >> 2], t & 3);
                        const uint32_t c0 = mask_plane<0>(d), c1 = mask_plane<1>(d);
                        const uint32_t c2 = mask_plane<2>(d), c3 = mask_plane<3>(d);
#pragma unroll
                        for (int m = 0; m < MC; ++m) {
                            a0[m][r] = dot4(P[m].x, c0, a0[m][r]);
                            a1[m][r] = dot4(P[m].y, c1, a1[m][r]);
                            a2[m][r] = dot4(P[m].z, c2, a2[m][r]);
                            a2[m][r] = dot4(P[m].w, c3, a2[m][r]);
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float wsf = __half2float(__ushort_as_half((unsigned short)wsraw[si][r]));
#pragma unroll
                    for (int m = 0; m < MC; ++m) {
                        const int dot = a0[m][r] + (a1[m][r] >> 2) + (a2[m][r] >> 4);
                        acc[m][r] += ((float)dot * __uint_as_float(xsv[si][m])) * wsf;
                    }
                }
            }
        }
    }

    // 5. Reduce over the 8 group lanes, then over waves in index order.
#pragma unroll
    for (int m = 0; m < MC; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = sum8_f(acc[m][r]);

    if (nwaves == 1) {
#pragma unroll
        for (int m = 0; m < MC; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int rl = slot + kRowSlots * r;
                if (j == (m & 7) && m < mcount && rl < rows_here) y[(size_t)(m0 + m) * n + row_base + rl] = acc[m][r];
            }
        return;
    }
    if (j == 0) {
#pragma unroll
        for (int m = 0; m < MC; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) red[(wave * MC + m) * RB + slot + kRowSlots * r] = acc[m][r];
    }
    __syncthreads();
    for (int o = threadIdx.x; o < MC * RB; o += nthreads) {
        const int m = o / RB;
        const int rl = o - m * RB;
        float sum = red[m * RB + rl];
        for (int w = 1; w < nwaves; ++w) sum += red[(w * MC + m) * RB + rl];
        if (m < mcount && rl < rows_here) y[(size_t)(m0 + m) * n + row_base + rl] = sum;
    }
}


// ------------------------------------------------------------------ plane-order host side
namespace {

size_t planes_lds_bytes(int mc, int segs, int waves, int rows_per_wg) {
    return (size_t)waves * segs * mc * 1024 + (size_t)waves * mc * rows_per_wg * 4;
}

template <int MC, int R, int SEGS>
hipError_t launch_planes_one(const int8_t* qp, const float* xs, const int32_t* qsum, const uint8_t* planes,
                             int64_t m, int64_t n, int64_t k, float* y, int waves, int nseg,
                             int segs_per_wave, int chunks, hipStream_t stream) {
    auto kern = small_m_planes_kernel<MC, R, SEGS>;
    const size_t lds = planes_lds_bytes(MC, SEGS, waves, kRowSlots * R);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(planes + n * (k / 4));
    const dim3 grid((unsigned)((n + kRowSlots * R - 1) / (kRowSlots * R)), (unsigned)chunks);
    clear_stale_error();
    hipLaunchKernelGGL(kern, grid, dim3(64 * waves), lds, stream, qp, xs, qsum, planes, scales, y, (int)n,
                       (int)k, (int)(k / 128), nseg, segs_per_wave, (int)m);
    return hipGetLastError();
}

template <int MC, int R>
hipError_t planes_pick_segs(const int8_t* qp, const float* xs, const int32_t* qsum, const uint8_t* planes,
                            int64_t m, int64_t n, int64_t k, float* y, int segs, int waves, int nseg,
                            int per_wave, int chunks, hipStream_t stream) {
    switch (segs) {
        case 1: return launch_planes_one<MC, R, 1>(qp, xs, qsum, planes, m, n, k, y, waves, nseg, per_wave, chunks, stream);
        case 2: return launch_planes_one<MC, R, 2>(qp, xs, qsum, planes, m, n, k, y, waves, nseg, per_wave, chunks, stream);
        case 3: return launch_planes_one<MC, R, 3>(qp, xs, qsum, planes, m, n, k, y, waves, nseg, per_wave, chunks, stream);
        default: return launch_planes_one<MC, R, 4>(qp, xs, qsum, planes, m, n, k, y, waves, nseg, per_wave, chunks, stream);
    }
}

template <int MC>
hipError_t planes_pick_rows(const int8_t* qp, const float* xs, const int32_t* qsum, const uint8_t* planes,
                            int64_t m, int64_t n, int64_t k, float* y, int rows, int segs, int waves,
                            int nseg, int per_wave, int chunks, hipStream_t stream) {
    switch (rows) {
        case 1: return planes_pick_segs<MC, 1>(qp, xs, qsum, planes, m, n, k, y, segs, waves, nseg, per_wave, chunks, stream);
        case 2: return planes_pick_segs<MC, 2>(qp, xs, qsum, planes, m, n, k, y, segs, waves, nseg, per_wave, chunks, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

SmallMConfig default_planes_config(int64_t m, int64_t n, int64_t k) {
    (void)n;
    (void)k;
    SmallMConfig c;
    c.rows_per_lane = m <= 2 ? 1 : 2;
    c.max_waves = 8;
    c.decode = 2;
    return c;
}

hipError_t launch_small_m_planes(const int8_t* qp, const float* xs, const int32_t* qsum, const uint8_t* planes,
                                 int64_t m, int64_t n, int64_t k, float* y, const SmallMConfig& cfg,
                                 hipStream_t stream) {
    const int rows = cfg.rows_per_lane;
    if (rows != 1 && rows != 2) return hipErrorInvalidValue;
    if (cfg.max_waves < 1 || cfg.max_waves > 8) return hipErrorInvalidValue;
    const int groups = (int)(k / 128);
    const int nseg = (groups + kGroupLanes - 1) / kGroupLanes;
    const int per_wave = (nseg + cfg.max_waves - 1) / cfg.max_waves;
    const int waves = (nseg + per_wave - 1) / per_wave;
    int segs = per_wave < 4 ? per_wave : 4;
    int mc = (int)(m < 8 ? m : 8);
    // Private activation blocks of all waves plus the reduction buffer must fit LDS.
    while (mc > 1 && planes_lds_bytes(mc, segs, waves, kRowSlots * rows) > 144 * 1024) --mc;
    while (segs > 1 && planes_lds_bytes(mc, segs, waves, kRowSlots * rows) > 144 * 1024) --segs;
    const int chunks = (int)((m + mc - 1) / mc);
    mc = (int)((m + chunks - 1) / chunks);
#define PQ2_PMC(C) \
    case C: return planes_pick_rows<C>(qp, xs, qsum, planes, m, n, k, y, rows, segs, waves, nseg, per_wave, chunks, stream);
    switch (mc) {
        PQ2_PMC(1) PQ2_PMC(2) PQ2_PMC(3) PQ2_PMC(4) PQ2_PMC(5) PQ2_PMC(6) PQ2_PMC(7) PQ2_PMC(8)
        default: return hipErrorInvalidValue;
    }
#undef PQ2_PMC
}


}  // namespace pq2
