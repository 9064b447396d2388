// small_m_wg.hip -- workgroup-staged matrix-core engine of the decode /
// small-batch matmul (1..4 activation columns per pass) on gfx950.
//
// What it computes is the definition of pq2_matmul_small_m (page "Baseline
// and the integer breakthrough", "Calculate with small integers"; page
// "Kernel experiments: recorded evidence", section B, Test 6):
//   y[m][n] = sum_g float(dot[m][n][g]) * xs[m][g] * ws[n][g],
//   dot[m][n][g] = sum_{i in group g} q[m][i] * (c[n][i] - 1)   (exact int32).
//
// Why this shape.  A decode call streams 14-24 MB of codes in about two
// microseconds, and the vector memory path of a CU serves its waves' loads
// in the order they were issued.  When every wave loads its own activations
// and then its codes, a wave that starts a little later finds its
// activation loads queued behind the code loads of the waves that started
// first: activations arrive at the pace of the code stream, and the compute
// they gate piles up behind the stream's end.  Here:
//  * one workgroup of 8 waves per CU owns RBW row blocks (8 weight rows each)
//    across all of k, i.e. RBW x nseg units of (8 rows x 1 segment of 8
//    groups);
//  * all waves first issue the loads of the workgroup's activations (every
//    segment, every column), meet at a barrier that waits for nothing, and
//    only then issue the code loads of their units, so in each CU's queue
//    the activations come first and the code stream still starts at once;
//  * the activations are staged into LDS once for the whole workgroup
//    (transposed to plane order with their group sums, or quantised from x
//    on the fused path), while the code loads are in flight;
//  * each wave then runs its units (unit u = wave + 8 i) as their codes
//    arrive: the decode (7 ALU ops per code dword: the four bit planes as
//    bytes 0..3), one v_mfma_i32_16x16x64_i8 per code dword and column pair
//    with the A operand read from LDS, and one FP32 term per (group, row,
//    column).
// Lane roles in a unit are those of small_m_mfma_kernel: for the code loads
// lane l takes row l & 7 and 16-byte chunk l >> 3 of a 128-byte span (whole
// 128-byte lines per instruction); as an MFMA B lane it is k-block l >> 4
// (a group) of column l & 15 = (code half, row); A row 4 ga + 2 mm + hp
// holds the plane-ordered activations of column 2p + mm, half hp, in
// k-block ga only (other k-blocks read a zero area), so the D entries with
// hp equal to the code half are half-group dots and one DPP rotate adds the
// halves into exact group dots.
// Summation order, identical to small_m_kernel and small_m_mfma_kernel with
// one segment per wave: per lane acc = fma(float(dot) * xs, ws, 0) for the
// two group classes kb and 4 + kb of the unit's segment, then (A_kb + A_4+kb)
// and the tree ((A0 + A4) + (A1 + A5)) + ((A2 + A6) + (A3 + A7)) (two lane
// swaps), then the segments in index order.  So every engine gives the same
// bits, for every number of columns.
#include "pq2_internal.h"
#include "small_m_common.h"

namespace pq2 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// Two launch shapes share the kernel:
//  * CU mode: one 8-wave workgroup per CU, up to 12 (row block, segment)
//    items per wave (the activations are staged once per CU);
//  * wave mode: one unit (row block, k slice) per wave, as many waves per
//    workgroup as (row blocks x k slices) of the workgroup, up to 16, so
//    that the grid has thousands of short waves and the staging is still
//    shared by the row blocks of a workgroup.
constexpr int kCuWaves = 8;
constexpr int kCuItems = 12;
constexpr int kMaxWgWaves = 16;

// Zero quads read by A-operand lanes outside their k-block: the largest
// immediate offset an A read adds is (4 * kBlockPitch + 3) quads.
constexpr int kZeroQuads = 4 * kBlockPitch + 4;

// Keeps the scheduler from moving any instruction across this point: the
// kernel relies on the program order of its loads.
__device__ __forceinline__ void keep_order() { __builtin_amdgcn_sched_barrier(0); }

// off if ok, else an offset past every buffer (the load returns zero); no select.
__device__ __forceinline__ uint32_t off_or_oob(bool ok, uint32_t off) {
    return off | (((uint32_t)ok - 1u) & kBufferOOB);
}

// Workgroup barrier after this wave's LDS writes, leaving global loads in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace

// Threads per workgroup and waves per SIMD the registers must leave room
// for: CU mode runs one 8-wave workgroup per CU (2 waves per SIMD); wave mode
// must keep its whole grid resident (up to 8 waves per SIMD for the common
// one-item, few-round shapes); multi-segment units use at most 8 waves per
// workgroup so that their code registers fit.
constexpr int wg_threads(int max_items) { return max_items > 1 ? 64 * kCuWaves : 64 * kMaxWgWaves; }
constexpr int wg_occupancy(int max_items, int rounds, int src) {
    return max_items > 8 ? 2
         : max_items > 1 ? ((src_fused(src) || rounds >= 8) ? 2 : 3)
         : (rounds >= 8 || (src_fused(src) && rounds >= 4)) ? 4
         : src_fused(src) ? 6 : 8;
}

template <int MC, int SRC, int MAX_ITEMS, int ROUNDS>
__global__ __launch_bounds__(wg_threads(MAX_ITEMS)) __attribute__((amdgpu_waves_per_eu(wg_occupancy(MAX_ITEMS, ROUNDS, SRC)))) void small_m_wg_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ xs, const int32_t* __restrict__ qsum,
    const void* __restrict__ x, int64_t x_stride,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, float* __restrict__ y, int n,
    int k, int groups, int nseg, int per_wave, int rbw, int mtotal) {
#pragma clang fp contract(off)
    constexpr bool FUSED = src_fused(SRC);
    constexpr int XL = FUSED ? src_xloads(SRC) : 1;
    constexpr int MP = (MC + 1) / 2;  // column pairs: one matrix instruction each per code dword
    constexpr int BLOCK_QUADS = kSegQuads;  // LDS quads of one (segment, column) block
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    // Matrix roles: code row, 16-byte chunk of the 128-byte span, its group (k-block) and half.
    const int row = lane & 7;
    const int chunk = lane >> 3;
    const int kb = lane >> 4;
    const int h = chunk & 1;
    // A-operand row of this lane: (ga, mm, hp), data only in k-block ga.
    const int ai = lane & 15;
    const int a_mm = (ai >> 1) & 1;
    const int a_hp = ai & 1;
    const bool a_lane = (ai >> 2) == kb;
    const int m0 = blockIdx.y * MC;
    const int mcount = min(MC, mtotal - m0);
    const int row_base = blockIdx.x * rbw * kRowSlots;
    const int rows_here = min(rbw * kRowSlots, n - row_base);
    // A unit is (row block, k slice); a k slice is per_wave consecutive
    // segments, the share of one wave in the other engines' k split.
    const int nslice = (nseg + per_wave - 1) / per_wave;
    const int units = ((rows_here + kRowSlots - 1) / kRowSlots) * nslice;
    const uint32_t k4 = (uint32_t)k >> 2;

    // LDS: the staged activations [segment][column] (kSegQuads quads each:
    // 8 groups x (8 data quads + 1 metadata quad)), a zero area, then one
    // float per (unit, column, row) for the cross-slice sum.
    const int act_quads = nseg * MC * BLOCK_QUADS;
    unsigned char* zero = smem + (size_t)act_quads * 16;
    float* red = reinterpret_cast<float*>(zero + kZeroQuads * 16);
    const uint32_t seg_bytes = MC * BLOCK_QUADS * 16;  // LDS bytes per segment (all columns)

    const auto code_rs = make_rsrc(codes + (size_t)row_base * k4, (uint32_t)rows_here * k4);
    const auto scale_rs = make_rsrc(scales + (size_t)row_base * groups, (uint32_t)(rows_here * groups * 2));
    const auto q_rs = make_rsrc(FUSED ? nullptr : q + (size_t)m0 * k, FUSED ? 0u : (uint32_t)(mcount * k));
    const auto xs_rs = make_rsrc(FUSED ? nullptr : xs + (size_t)m0 * groups, FUSED ? 0u : (uint32_t)(mcount * groups * 4));
    const auto qs_rs = make_rsrc(SRC == kSrcPlanes ? qsum + (size_t)m0 * groups : nullptr,
                                 SRC == kSrcPlanes ? (uint32_t)(mcount * groups * 4) : 0u);
    const auto x_rs = make_rsrc(
        FUSED ? static_cast<const unsigned char*>(x) + (size_t)m0 * x_stride * src_esize(SRC) : nullptr,
        FUSED ? (uint32_t)(((int64_t)(mcount - 1) * x_stride + k) * src_esize(SRC)) : 0u);

    // ---- 1. activation loads of the whole workgroup.  Staging quad Q =
    //      ((s * MC + m) * 8 + slot) * 8 + j is quad j of group slot of segment
    //      s, column m; the 8 quads of a group sit in 8 consecutive lanes.
    const int stage_quads = nseg * MC * 64;
    uint4 qv[ROUNDS];
    uint4 xv[ROUNDS][XL];
    uint32_t xsv[ROUNDS], tv[ROUNDS];
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
        if (nthreads * i >= stage_quads) break;  // uniform
        const int Q = tid + nthreads * i;
        const int j = Q & 7;
        const int slot = (Q >> 3) & 7;
        const int sm = Q >> 6;
        const int s = sm / MC;
        const int m = sm - s * MC;
        const int gq = s * kGroupLanes + slot;
        const bool qok = Q < stage_quads && gq < groups && m < mcount;
        if constexpr (FUSED) {
            const uint32_t off = (uint32_t)((m * x_stride + gq * 128 + j * 16) * src_esize(SRC));
#pragma unroll
            for (int l = 0; l < XL; ++l) xv[i][l] = buf_load16(x_rs, off_or_oob(qok, off + 16u * l));
        } else {
            qv[i] = buf_load16(q_rs, off_or_oob(qok, (uint32_t)(m * k + gq * 128 + j * 16)));
            const uint32_t moff = off_or_oob(qok && j == 0, (uint32_t)((m * groups + gq) * 4));
            xsv[i] = buf_load4(xs_rs, moff);
            if constexpr (SRC == kSrcPlanes) tv[i] = buf_load4(qs_rs, moff);
        }
    }
    keep_order();
    // Every wave's activation loads are in the CU's queue before any code load.
    __builtin_amdgcn_s_barrier();
    keep_order();

    // ---- 2. this wave's items (row block r, segment s) in the order they run:
    //      units u = wave, wave + 8, ..., each the segments of its k slice in
    //      order (uniform scalar bookkeeping), then their code and scale loads
    int it_r[MAX_ITEMS], it_s[MAX_ITEMS], it_u[MAX_ITEMS];
    bool it_first[MAX_ITEMS], it_last[MAX_ITEMS];
    {
        int u = wave;
        int sl = u % nslice;
        int s_cur = sl * per_wave;
#pragma unroll
        for (int i = 0; i < MAX_ITEMS; ++i) {
            const int s_end = min(sl * per_wave + per_wave, nseg);
            it_u[i] = u;
            it_r[i] = u / nslice;
            it_s[i] = s_cur;
            it_first[i] = s_cur == sl * per_wave;
            it_last[i] = s_cur + 1 == s_end;
            if (s_cur + 1 < s_end) {
                ++s_cur;
            } else {
                u += nwaves;
                sl = u % nslice;
                s_cur = sl * per_wave;
            }
        }
    }
    uint4 cw[MAX_ITEMS][2];
    uint32_t wsraw[MAX_ITEMS][2];
#pragma unroll
    for (int i = 0; i < MAX_ITEMS; ++i) {
        if (it_u[i] >= units) break;  // uniform: items run in unit order
        const int g0 = it_s[i] * kGroupLanes;
        const uint32_t rl = (uint32_t)(it_r[i] * kRowSlots + row);
        // rl < 512 and k4, groups < 2^15: the 24-bit multiplier is exact and full rate.
        const uint32_t row_code = __umul24(rl, k4) + (uint32_t)g0 * 32u + 16u * (uint32_t)chunk;
        const uint32_t row_scale = __umul24(rl, (uint32_t)groups) + (uint32_t)(g0 + kb);
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            const bool ok = g0 + 4 * sp + kb < groups;
            cw[i][sp] = buf_load16<kAuxNonTemporal>(code_rs, off_or_oob(ok, row_code + 128u * sp));
            wsraw[i][sp] = buf_load2(scale_rs, off_or_oob(ok, (row_scale + 4u * sp) * 2u));
        }
        keep_order();
    }

    // ---- 3. stage the activations (while the code loads are in flight)
    if (tid < kZeroQuads) reinterpret_cast<uint4*>(zero)[tid] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
        const int Q = tid + nthreads * i;
        if (nthreads * i >= stage_quads) break;  // uniform
        const int j = Q & 7;
        const int slot = (Q >> 3) & 7;
        const int sm = Q >> 6;
        uint4 v = qv[i];
        int sum;
        uint32_t scale_bits;
        if constexpr (FUSED) {
            float xf[16];
            x_to_float16<SRC>(xv[i], xf);
            float scale;
            v = quantize_lane16(xf, sum, scale);
            scale_bits = __float_as_uint(scale);
        } else if constexpr (SRC == kSrcNatural) {
            sum = dot4(v.x, 0x01010101u, 0);
            sum = dot4(v.y, 0x01010101u, sum);
            sum = dot4(v.z, 0x01010101u, sum);
            sum = dot4(v.w, 0x01010101u, sum);
            sum = sum8_i(sum);
            v = to_plane_order(v);
            scale_bits = xsv[i];
        } else {
            sum = (int)tv[i];
            scale_bits = xsv[i];
        }
        if (Q < stage_quads) {
            unsigned char* blk = smem + ((size_t)sm * BLOCK_QUADS + slot * kBlockPitch) * 16;
            *reinterpret_cast<uint4*>(blk + j * 16) = v;
            if (j == 0) *reinterpret_cast<uint2*>(blk + 8 * 16) = make_uint2((uint32_t)sum, scale_bits);
        }
    }
    lds_barrier();

    // ---- 4. the items: decode, matrix cores, exact group dots, FP32 terms
    //      accumulated over a unit's segments; at a unit's last segment the
    //      k-block tree and one float per (unit, column, row) to LDS
    uint32_t a_base[MP], a_seg[MP];
#pragma unroll
    for (int p = 0; p < MP; ++p) {
        const int am = 2 * p + a_mm;
        const bool live = a_lane && am < mcount;
        a_base[p] = live ? (uint32_t)(((am * BLOCK_QUADS) + kb * kBlockPitch + 4 * a_hp) * 16)
                         : (uint32_t)act_quads * 16u;  // the zero area
        a_seg[p] = live ? seg_bytes : 0u;
    }
    const uint32_t meta_base = (uint32_t)((kb * kBlockPitch + 8) * 16);  // sum(q), xs of group kb (+4 sp)
    float acc[MP][2];
#pragma unroll
    for (int i = 0; i < MAX_ITEMS; ++i) {
        if (it_u[i] >= units) break;  // uniform: items run in unit order
        const int s = it_s[i];
        v4i D[MP][2];
#pragma unroll
        for (int p = 0; p < MP; ++p) D[p][0] = D[p][1] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const uint32_t d = word_of(cw[i][sp], st);
                const v4i B = v4i{(int)(d & 0x03030303u), (int)((d >> 2) & 0x03030303u),
                                  (int)((d >> 4) & 0x03030303u), (int)((d >> 6) & 0x03030303u)};
#pragma unroll
                for (int p = 0; p < MP; ++p) {
                    const uint32_t ad = a_base[p] + a_seg[p] * (uint32_t)s + (sp * 4 * kBlockPitch + st) * 16;
                    const v4i A = *reinterpret_cast<const v4i*>(smem + ad);
                    D[p][sp] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, D[p][sp], 0, 0, 0);
                }
            }
        }
        if (it_first[i]) {
#pragma unroll
            for (int p = 0; p < MP; ++p) acc[p][0] = acc[p][1] = 0.0f;
        }
#pragma unroll
        for (int p = 0; p < MP; ++p) {
            const int m = min(2 * p + h, MC - 1);  // a lane past the last column reads a column it never uses
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const uint2 meta = *reinterpret_cast<const uint2*>(
                    smem + seg_bytes * (uint32_t)s + meta_base + (m * BLOCK_QUADS + sp * 4 * kBlockPitch) * 16);
                // Lane (kb, h, row) finishes column 2p + h from its own half D[3h] and
                // the partner lane's (kb, 1 - h, row) half of the same column: D[1]
                // of an h = 1 partner, D[2] of an h = 0 partner (a DPP rotate by 8).
                const v4i& Dv = D[p][sp];
                const int d_h0 = Dv[0] + __builtin_amdgcn_mov_dpp(Dv[1], 0x128, 0xF, 0xF, true);
                const int d_h1 = Dv[3] + __builtin_amdgcn_mov_dpp(Dv[2], 0x128, 0xF, 0xF, true);
                const int dot = (h ? d_h1 : d_h0) - (int)meta.x;
                const float wsf = __half2float(__ushort_as_half((unsigned short)wsraw[i][sp]));
                acc[p][sp] = __builtin_fmaf((float)dot * __uint_as_float(meta.y), wsf, acc[p][sp]);
            }
        }
        if (it_last[i]) {
            const int u = it_u[i];
#pragma unroll
            for (int p = 0; p < MP; ++p) {
                // Classes kb and 4 + kb, then the four k-blocks (lanes 16 apart) as
                // (t0 + t1) + (t2 + t3) through two lane swaps.
                float t = acc[p][0] + acc[p][1];
                const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
                t = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
                const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
                t = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
                if (kb == 0 && 2 * p + h < MC) red[(u * MC + 2 * p + h) * kRowSlots + row] = t;
            }
        }
    }
    lds_barrier();

    // ---- 5. the k slices add in index order; one thread per (column, row)
    const int rows_pad = ((rows_here + kRowSlots - 1) / kRowSlots) * kRowSlots;
    for (int o = tid; o < MC * rows_pad; o += nthreads) {
        const int m = o / rows_pad;
        const int rl = o - m * rows_pad;
        const int r = rl >> 3;
        const float* t = red + ((size_t)(r * nslice) * MC + m) * kRowSlots + (rl & 7);
        float sum = t[0];
        for (int sl = 1; sl < nslice; ++sl) sum += t[(size_t)sl * MC * kRowSlots];
        if (m < mcount && rl < rows_here) y[(size_t)(m0 + m) * n + row_base + rl] = sum;
    }
}

// ------------------------------------------------------------------ host side
namespace {

constexpr size_t kWgLdsLimit = 150 * 1024;
constexpr int kWaveItems = 8;  // wave mode: a unit of up to 8 segments per wave

struct WgPlan {
    int nseg, per_wave, nslice;  // k split: slices of per_wave segments
    int mc, chunks;              // columns per pass, passes
    int waves, items, rounds;    // waves per workgroup, items per wave, staging rounds
    bool wave_mode;
    size_t lds;
};

// Staging rounds the source's registers allow (fp32 input is twice as wide).
int max_rounds(int src) { return src == kSrcF32 ? 4 : 8; }

bool make_plan(int src, int64_t m, int64_t k, int max_waves, int rbw, bool wave_mode, WgPlan* p) {
    if (max_waves < 1 || max_waves > 8 || rbw < 1 || src < 0) return false;
    p->nseg = (int)((k / 128 + kGroupLanes - 1) / kGroupLanes);
    p->per_wave = (p->nseg + max_waves - 1) / max_waves;
    p->nslice = (p->nseg + p->per_wave - 1) / p->per_wave;
    const int units = rbw * p->nslice;
    p->wave_mode = wave_mode;
    if (wave_mode) {
        // Multi-segment units run in the 8-wave (512-thread) instantiation.
        if (units > (p->per_wave > 1 ? kCuWaves : kMaxWgWaves) || p->per_wave > kWaveItems) return false;
        p->waves = units;
        p->items = p->per_wave;
    } else {
        p->waves = kCuWaves;
        p->items = ((units + kCuWaves - 1) / kCuWaves) * p->per_wave;
        if (p->items > kCuItems) return false;
    }
    // Columns per pass: up to four, fewer if the workgroup cannot stage the
    // activations of all of k for more (more passes over the weights then).
    const int64_t stage_cap = (int64_t)max_rounds(src) * p->waves * 64;
    int cap = kWgMaxColumns;
    auto lds_of = [&](int mc) {
        return ((size_t)p->nseg * mc * kSegQuads + kZeroQuads) * 16 + (size_t)units * mc * kRowSlots * 4;
    };
    while (cap > 0 && ((int64_t)p->nseg * cap * 64 > stage_cap || lds_of(cap) > kWgLdsLimit)) --cap;
    if (cap < 1) return false;
    p->chunks = (int)((m + cap - 1) / cap);
    p->mc = (int)((m + p->chunks - 1) / p->chunks);
    const int64_t quads = (int64_t)p->nseg * p->mc * 64;
    const int64_t rounds = (quads + p->waves * 64 - 1) / (p->waves * 64);
    p->rounds = rounds <= 1 ? 1 : rounds <= 2 ? 2 : rounds <= 4 ? 4 : 8;
    p->lds = lds_of(p->mc);
    return true;
}

template <int MC, int SRC, int ITEMS, int ROUNDS>
hipError_t launch_wg_one(const SmallMLaunch& a, const WgPlan& p, int rbw) {
    auto kern = small_m_wg_kernel<MC, SRC, ITEMS, ROUNDS>;
    static bool attr_set = false;  // one instantiation = one static
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(a.planes + a.n * (a.k / 4));
    const int64_t nblk = (a.n + kRowSlots - 1) / kRowSlots;
    const dim3 grid((unsigned)((nblk + rbw - 1) / rbw), (unsigned)p.chunks);
    clear_stale_error();
    hipLaunchKernelGGL(kern, grid, dim3(64 * p.waves), p.lds, a.stream, a.q, a.xs, a.qsum, a.x, a.x_stride, a.planes,
                       scales, a.y, (int)a.n, (int)a.k, (int)(a.k / 128), p.nseg, p.per_wave, rbw, (int)a.m);
    return hipGetLastError();
}

// Instantiations: CU mode (12 items, 8 rounds; 4 for fp32 input) and wave
// mode (1 or 3 items, 2, 4 or 8 rounds).
template <int MC, int SRC>
hipError_t wg_pick_shape(const SmallMLaunch& a, const WgPlan& p, int rbw) {
    constexpr int R8 = SRC == kSrcF32 ? 4 : 8;  // fp32 input stages at most 4 rounds
    if (p.waves == kCuWaves && p.items > 1 && !p.wave_mode) return launch_wg_one<MC, SRC, kCuItems, R8>(a, p, rbw);
    if (p.items == 1) {
        switch (p.rounds) {
            case 1: case 2: return launch_wg_one<MC, SRC, 1, 2>(a, p, rbw);
            case 4: return launch_wg_one<MC, SRC, 1, 4>(a, p, rbw);
            default: return launch_wg_one<MC, SRC, 1, R8>(a, p, rbw);
        }
    }
    switch (p.rounds) {
        case 1: case 2: return launch_wg_one<MC, SRC, kWaveItems, 2>(a, p, rbw);
        case 4: return launch_wg_one<MC, SRC, kWaveItems, 4>(a, p, rbw);
        default: return launch_wg_one<MC, SRC, kWaveItems, R8>(a, p, rbw);
    }
}

template <int SRC>
hipError_t wg_pick_mc(const SmallMLaunch& a, const WgPlan& p, int rbw) {
    switch (p.mc) {
        case 1: return wg_pick_shape<1, SRC>(a, p, rbw);
        case 2: return wg_pick_shape<2, SRC>(a, p, rbw);
        case 3: return wg_pick_shape<3, SRC>(a, p, rbw);
        case 4: return wg_pick_shape<4, SRC>(a, p, rbw);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool wg_supported(int src, int64_t m, int64_t k, int max_waves, int rbw, bool wave_mode) {
    WgPlan p;
    return make_plan(src, m, k, max_waves, rbw, wave_mode, &p);
}

// Row blocks per workgroup.  CU mode: one workgroup per CU when that fits
// the item, staging and LDS budgets, else the most that fits.  Wave mode:
// the most row blocks whose units fit one workgroup (at most 16 waves).
// 0 if no setting fits.
int wg_default_row_blocks(int src, int64_t m, int64_t n, int64_t k, int max_waves, bool wave_mode) {
    const int64_t nblk = (n + kRowSlots - 1) / kRowSlots;
    int rbw = wave_mode ? kMaxWgWaves : (int)((nblk + 255) / 256);
    if (rbw > nblk) rbw = (int)nblk;
    while (rbw > 1 && !wg_supported(src, m, k, max_waves, rbw, wave_mode)) --rbw;
    return wg_supported(src, m, k, max_waves, rbw, wave_mode) ? rbw : 0;
}

hipError_t launch_small_m_wg(int src, const SmallMLaunch& base, int max_waves, int rbw, bool wave_mode) {
    WgPlan p;
    if (!make_plan(src, base.m, base.k, max_waves, rbw, wave_mode, &p)) return hipErrorInvalidValue;
    switch (src) {
        case kSrcPlanes: return wg_pick_mc<kSrcPlanes>(base, p, rbw);
        case kSrcNatural: return wg_pick_mc<kSrcNatural>(base, p, rbw);
        case kSrcBf16: return wg_pick_mc<kSrcBf16>(base, p, rbw);
        case kSrcF16: return wg_pick_mc<kSrcF16>(base, p, rbw);
        case kSrcF32: return wg_pick_mc<kSrcF32>(base, p, rbw);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pq2
