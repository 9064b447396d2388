// small_m.hip -- decode / small-batch matmul (1..16 activation columns) of
// prepared PQ2 planes x group-128 INT8 activations on gfx950.
//
// What it computes (page "Baseline and the integer breakthrough",
// "Calculate with small integers"; page "Kernel experiments: recorded
// evidence", section B, Test 6): for every output row n and column m,
//   y[m][n] = sum_g float(dot[m][n][g]) * xs[m][g] * ws[n][g],
//   dot[m][n][g] = sum_{i in group g} q[m][i] * (c[n][i] - 1)   (exact int32).
//
// Design (MI355X-first, not a translation of the pages' Triton/CUDA):
//  * HBM is the bound: every code byte is read once, with 16-byte loads that
//    a wave issues for ALL of its work before anything else (one-shot), so
//    the whole matrix is in flight while activations are staged.
//  * Work unit = one lane x one 128-weight group x R rows.  A wave is 8 row
//    slots x 8 group lanes: the 8 lanes of a slot read 8 consecutive groups
//    (256 contiguous bytes) of one row.  The lane loops over its segments of
//    8 groups and keeps FP32 partial sums in registers, so the cross-lane
//    reduction happens once per output (3 DPP adds), not once per group.
//  * Activations: the workgroup stages its columns' q into LDS once, in
//    code-plane order (each 16-byte quad byte-transposed so a code dword's
//    plane s meets q[16t+4j+s]), XOR-swizzled so the 8 group lanes hit 8
//    different bank groups.  Each q quad read from LDS serves R rows.
//  * k is split over W waves of the workgroup (each takes consecutive
//    segments); the W wave partials are summed through LDS in fixed order.
//  * Two exact decodes (template DEC): 1 = the pages' add/XOR expansion
//    (four signed planes, 15 ALU ops per code dword), 2 = masked planes
//    d & (3 << 2s) paired with plane-ordered q, three integer accumulators
//    re-weighted by shifts and the -1 offset applied once per group as
//    -sum(q) (page "Kernel experiments", Test 21 / Diagram 7); 5 ALU ops
//    per code dword.  Both give the identical int32 dot.
//  * Determinism and batch invariance: per output, the sum is lane-serial
//    over segments, a fixed DPP tree over the 8 group lanes, then waves in
//    index order.  None of it depends on the number of columns.
#include "pq2_device.h"
#include "pq2_internal.h"

#include <hip/hip_fp16.h>

namespace pq2 {

constexpr int kGroupLanes = 8;   // lanes per row slot (one group each)
constexpr int kRowSlots = 8;     // row slots per wave

template <int MC, int R, int SEGS, int DEC>
__global__ __launch_bounds__(512) void small_m_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ xs, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int n, int k, int groups, int nseg,
    int segs_per_wave, int mtotal) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int gpad = nseg * kGroupLanes;
    uint4* qlds = reinterpret_cast<uint4*>(smem);                                   // [gpad][MC][8 quads]
    float2* slds = reinterpret_cast<float2*>(smem + (size_t)gpad * MC * 128);       // [gpad][MC] {xs, sum q}
    float* red = reinterpret_cast<float*>(smem + (size_t)gpad * MC * 136);          // [W][MC][8R]

    constexpr int RB = kRowSlots * R;  // rows per workgroup
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

    // Buffer resources over exactly the bytes this workgroup may read: a row
    // past n, a group past k or a column past m reads as zero.
    const auto code_rs = make_rsrc(codes + (size_t)row_base * k4, (uint32_t)rows_here * k4);
    const auto scale_rs = make_rsrc(scales + (size_t)row_base * groups, (uint32_t)(rows_here * groups * 2));
    const auto q_rs = make_rsrc(q + (size_t)m0 * k, (uint32_t)(mcount * k));
    const auto xs_rs = make_rsrc(xs + (size_t)m0 * groups, (uint32_t)(mcount * groups * 4));

    // Staging items = (group, column, quad t); 8 consecutive threads take the
    // 8 quads of one (group, column) so its sum of q is an 8-lane reduction.
    constexpr int QB = 4;  // staging items per thread per batch
    const int nitems = gpad * MC * 8;
    uint4 qv[QB];
    uint32_t xv[QB];
    auto stage_load = [&](int base_it) {
#pragma unroll
        for (int i = 0; i < QB; ++i) {
            const int it = base_it + i * nthreads;
            const int t = it & 7;
            const int gm = it >> 3;
            const int m = gm % MC;
            const int g = gm / MC;
            const bool ok = it < nitems && m < mcount && g < groups;
            qv[i] = buf_load16(q_rs, ok ? (uint32_t)(m * k + g * 128 + t * 16) : kBufferOOB);
            xv[i] = buf_load4(xs_rs, ok ? (uint32_t)((m * groups + g) * 4) : kBufferOOB);
        }
    };
    auto stage_store = [&](int base_it) {
#pragma unroll
        for (int i = 0; i < QB; ++i) {
            const int it = base_it + i * nthreads;
            if (it < nitems) {  // uniform over each aligned group of 8 lanes
                const int t = it & 7;
                const int gm = it >> 3;
                const int g = gm / MC;
                const uint4 Q = qv[i];
                int tsum = dot4(Q.x, 0x01010101u, 0);
                tsum = dot4(Q.y, 0x01010101u, tsum);
                tsum = dot4(Q.z, 0x01010101u, tsum);
                tsum = dot4(Q.w, 0x01010101u, tsum);
                tsum = sum8_i(tsum);
                qlds[(size_t)gm * 8 + (t ^ (g & 7))] = to_plane_order(Q);
                if (t == 0) slds[gm] = make_float2(__uint_as_float(xv[i]), __int_as_float(tsum));
            }
        }
    };

    // Codes and raw fp16 scales of up to SEGS segments of this wave's rows.
    uint4 cw[SEGS][R][2];
    uint32_t wsraw[SEGS][R];
    auto load_step = [&](int base) {
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
    };

    // 1. First batch of activation loads (short L2 latency), then every code
    //    load of this wave's first step (HBM), so both are in flight together
    //    and staging does not wait for the codes.
    stage_load(threadIdx.x);
    load_step(seg_begin);
    // 2. Stage q in plane order, plus {xs, sum q} per (group, column).
    stage_store(threadIdx.x);
    for (int b = threadIdx.x + QB * nthreads; b < nitems; b += QB * nthreads) {
        stage_load(b);
        stage_store(b);
    }
    __syncthreads();

    // 3. Integer group dots, FP32 scaling, lane-serial accumulation.
    float acc[MC][R];
#pragma unroll
    for (int m = 0; m < MC; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

    for (int base = seg_begin; base < seg_end; base += SEGS) {
        if (base != seg_begin) load_step(base);
#pragma unroll
        for (int si = 0; si < SEGS; ++si) {
            if (base + si < seg_end) {
                const int g = (base + si) * kGroupLanes + j;  // g & 7 == j
                const int gm0 = g * MC;
                float xsv[MC];
                int a0[MC][R], a1[MC][R], a2[MC][R];
#pragma unroll
                for (int m = 0; m < MC; ++m) {
                    const float2 v = slds[gm0 + m];
                    xsv[m] = v.x;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        a0[m][r] = DEC == 2 ? -__float_as_int(v.y) : 0;
                        a1[m][r] = 0;
                        a2[m][r] = 0;
                    }
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    uint4 P[MC];
#pragma unroll
                    for (int m = 0; m < MC; ++m) P[m] = qlds[(size_t)(gm0 + m) * 8 + (t ^ j)];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t d = word_of(cw[si][r][t >> 2], t & 3);
                        if constexpr (DEC == 2) {
                            const uint32_t c0 = mask_plane<0>(d), c1 = mask_plane<1>(d);
                            const uint32_t c2 = mask_plane<2>(d), c3 = mask_plane<3>(d);
#pragma unroll
                            for (int m = 0; m < MC; ++m) {
                                a0[m][r] = dot4(P[m].x, c0, a0[m][r]);
                                a1[m][r] = dot4(P[m].y, c1, a1[m][r]);
                                a2[m][r] = dot4(P[m].z, c2, a2[m][r]);
                                a2[m][r] = dot4(P[m].w, c3, a2[m][r]);
                            }
                        } else {
                            const uint32_t e0 = expand_plane<0>(d), e1 = expand_plane<1>(d);
                            const uint32_t e2 = expand_plane<2>(d), e3 = expand_plane<3>(d);
#pragma unroll
                            for (int m = 0; m < MC; ++m) {
                                a0[m][r] = dot4(P[m].x, e0, a0[m][r]);
                                a0[m][r] = dot4(P[m].y, e1, a0[m][r]);
                                a0[m][r] = dot4(P[m].z, e2, a0[m][r]);
                                a0[m][r] = dot4(P[m].w, e3, a0[m][r]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float wsf = __half2float(__ushort_as_half((unsigned short)wsraw[si][r]));
#pragma unroll
                    for (int m = 0; m < MC; ++m) {
                        // a1 = 4 * (plane-1 sum), a2 = 16 * (plane-2 + plane-3 sums): exact shifts.
                        const int dot = DEC == 2 ? a0[m][r] + (a1[m][r] >> 2) + (a2[m][r] >> 4) : a0[m][r];
                        acc[m][r] += ((float)dot * xsv[m]) * wsf;
                    }
                }
            }
        }
    }

    // 4. Reduce over the 8 group lanes, then over waves in index order.
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

// ------------------------------------------------------------------ host side
namespace {

constexpr size_t kLdsBudget = 80 * 1024;  // keeps two workgroups per CU

size_t lds_bytes(int mc, int gpad, int waves, int rows_per_wg) {
    return (size_t)gpad * mc * 136 + (size_t)waves * mc * rows_per_wg * 4;
}

template <int MC, int R, int SEGS, int DEC>
hipError_t launch_one(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m, int64_t n,
                      int64_t k, float* y, int waves, int nseg, int segs_per_wave, int chunks,
                      hipStream_t stream) {
    auto kern = small_m_kernel<MC, R, SEGS, DEC>;
    const int groups = (int)(k / 128);
    const size_t lds = lds_bytes(MC, nseg * kGroupLanes, waves, kRowSlots * R);
    static bool attr_set = false;  // one instantiation = one static
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const uint8_t* codes = planes;
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(planes + n * (k / 4));
    const dim3 grid((unsigned)((n + kRowSlots * R - 1) / (kRowSlots * R)), (unsigned)chunks);
    clear_stale_error();
    hipLaunchKernelGGL(kern, grid, dim3(64 * waves), lds, stream, q, xs, codes, scales, y, (int)n,
                       (int)k, groups, nseg, segs_per_wave, (int)m);
    return hipGetLastError();
}

template <int MC, int R, int DEC>
hipError_t pick_segs(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m, int64_t n,
                     int64_t k, float* y, int per_wave, int waves, int nseg, int chunks,
                     hipStream_t stream) {
    switch (per_wave) {
        case 1: return launch_one<MC, R, 1, DEC>(q, xs, planes, m, n, k, y, waves, nseg, per_wave, chunks, stream);
        case 2: return launch_one<MC, R, 2, DEC>(q, xs, planes, m, n, k, y, waves, nseg, per_wave, chunks, stream);
        case 3: return launch_one<MC, R, 3, DEC>(q, xs, planes, m, n, k, y, waves, nseg, per_wave, chunks, stream);
        default: return launch_one<MC, R, 4, DEC>(q, xs, planes, m, n, k, y, waves, nseg, per_wave, chunks, stream);
    }
}

template <int MC, int DEC>
hipError_t pick_rows(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m, int64_t n,
                     int64_t k, float* y, int rows, int segs, int waves, int nseg, int chunks,
                     hipStream_t stream) {
    switch (rows) {
        case 1: return pick_segs<MC, 1, DEC>(q, xs, planes, m, n, k, y, segs, waves, nseg, chunks, stream);
        case 2: return pick_segs<MC, 2, DEC>(q, xs, planes, m, n, k, y, segs, waves, nseg, chunks, stream);
        case 4: return pick_segs<MC, 4, DEC>(q, xs, planes, m, n, k, y, segs, waves, nseg, chunks, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int DEC>
hipError_t pick_mc(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m, int64_t n,
                   int64_t k, float* y, int mc, int rows, int segs, int waves, int nseg, int chunks,
                   hipStream_t stream) {
#define PQ2_MC_CASE(C) \
    case C: return pick_rows<C, DEC>(q, xs, planes, m, n, k, y, rows, segs, waves, nseg, chunks, stream);
    switch (mc) {
        PQ2_MC_CASE(1) PQ2_MC_CASE(2) PQ2_MC_CASE(3) PQ2_MC_CASE(4)
        PQ2_MC_CASE(5) PQ2_MC_CASE(6) PQ2_MC_CASE(7) PQ2_MC_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef PQ2_MC_CASE
}

}  // namespace

SmallMConfig default_small_m_config(int64_t m, int64_t n, int64_t k) {
    (void)n;
    (void)k;
    SmallMConfig c;
    c.rows_per_lane = 2;
    c.max_waves = 8;
    c.decode = 2;
    return c;
}

hipError_t launch_small_m(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m,
                          int64_t n, int64_t k, float* y, const SmallMConfig& cfg,
                          hipStream_t stream) {
    const int rows = cfg.rows_per_lane;
    if (rows != 1 && rows != 2 && rows != 4) return hipErrorInvalidValue;
    if (cfg.max_waves < 1 || cfg.max_waves > 8) return hipErrorInvalidValue;
    if (cfg.decode != 1 && cfg.decode != 2) return hipErrorInvalidValue;
    const int groups = (int)(k / 128);
    const int nseg = (groups + kGroupLanes - 1) / kGroupLanes;
    // Segments per wave; a wave holds at most 4 segments' loads at a time and
    // loops for longer k.
    const int segs = (nseg + cfg.max_waves - 1) / cfg.max_waves;
    const int waves = (nseg + segs - 1) / segs;
    // Columns per pass: as many as fit the LDS budget (at most 8).
    int mc = (int)(m < 8 ? m : 8);
    while (mc > 1 && lds_bytes(mc, nseg * kGroupLanes, waves, kRowSlots * rows) > kLdsBudget) --mc;
    if (lds_bytes(mc, nseg * kGroupLanes, waves, kRowSlots * rows) > 160 * 1024) return hipErrorInvalidValue;
    const int chunks = (int)((m + mc - 1) / mc);
    mc = (int)((m + chunks - 1) / chunks);  // balance the passes
    if (cfg.decode == 2)
        return pick_mc<2>(q, xs, planes, m, n, k, y, mc, rows, segs, waves, nseg, chunks, stream);
    return pick_mc<1>(q, xs, planes, m, n, k, y, mc, rows, segs, waves, nseg, chunks, stream);
}


}  // namespace pq2
