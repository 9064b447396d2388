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
//  * HBM is the bound: every code byte is read once.  A wave is 8 row slots x
//    8 lanes; for one segment (8 groups = 256 contiguous code bytes of a row)
//    lane j of a slot loads bytes 16j.. and 128+16j.. , so each load
//    instruction reads 128 contiguous bytes per row.  A wave issues the loads
//    of all its segments (up to SEGS at a time) before anything else.
//  * With that layout lane j holds half (h = j & 1) of groups j/2 and 4 + j/2.
//    It forms both half-group integer dots, swaps one of them with its
//    partner lane j ^ 1 (one DPP move) and adds: the full, exact dot of group
//    j/2 (h = 0) or 4 + j/2 (h = 1).  Only whole-group dots are scaled, so
//    each output sums exactly k/128 FP32 terms.
//  * Decode: masked code planes (page "Kernel experiments", Test 21 and
//    Diagram 7).  Code dword D gives D & 0x03.., D & 0x0C.., D & 0x30.. and
//    (D >> 2) & 0x30..: plane s holds c << 2s (c << 4 for s = 3), so three
//    INT32 accumulators (scaled by 1, 4, 16) recombine exactly as
//    a0 + (a1 >> 2) + (a23 >> 4), and the code offset -1 becomes one
//    subtraction of sum(q) per group.  5 ALU ops per 16 weights.
//  * The activation operand must pair plane s of a code dword with
//    q[16t + 4j + s]: each 16-byte block of q, 4x4 byte-transposed ("plane
//    order").  Every wave copies the blocks of its own segments into a
//    private LDS region (no workgroup barrier); input that is already in
//    plane order (pq2_quantize_act_i8_planes) is copied as is with its group
//    sums, natural-order input is transposed on the way and its group sums
//    formed with dot4 against 0x01010101.  Rows of 8 blocks are padded to 9
//    so that the 8 distinct blocks one read instruction touches fall in
//    distinct LDS banks and every read address is one register plus an
//    immediate.
//  * k is split over the W waves of a workgroup (consecutive segments); the
//    W partial sums are added through LDS in wave order.  A wave issues the
//    code loads of up to SEGS segments at once and stages one segment's
//    activations at a time, so the LDS footprint does not grow with SEGS.
//  * Two engines compute the same bits: small_m_kernel (packed v_dot4, per
//    column 4 dot instructions per code dword) and small_m_mfma_kernel (INT8
//    matrix cores, whose work per code dword does not grow with the number
//    of columns).  The library picks one per shape.
//  * The fused entry points start from the unquantised activations x: the
//    lanes that stage a group's 16-byte blocks quantise them first (each
//    workgroup quantises the k slice it reads), with results bit-identical to
//    the quantiser kernel, so quantiser + matmul become one launch with the
//    same output bits.
//  * Summation order of an output: each lane accumulates its group terms
//    acc = fma((float)dot * xs, ws, acc) over its segments in order (no other
//    contraction: the pragma below), a fixed DPP tree adds the 8 lanes of a
//    slot, and the wave partials are added in wave order.  That order depends
//    only on the k split, which the library picks from (n, k) alone: outputs
//    are bit-identical whatever the number of columns (batch invariance),
//    the rows per lane, or the input order (natural or plane).
#include "pq2_internal.h"
#include "small_m_common.h"

namespace pq2 {

// Plane-order pairing of activation dwords with code planes, per half group.
// acc0/acc1/acc23 are the three masked-plane accumulators.
template <int R>
__device__ __forceinline__ void half_group_dot(const uint4 (&P)[4], const uint4 (&cw)[R], int (&acc0)[R],
                                               int (&acc1)[R], int (&acc23)[R]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t d = word_of(cw[r], t);
            acc0[r] = dot4(P[t].x, mask_plane<0>(d), acc0[r]);
            acc1[r] = dot4(P[t].y, mask_plane<1>(d), acc1[r]);
            acc23[r] = dot4(P[t].z, mask_plane<2>(d), acc23[r]);
            acc23[r] = dot4(P[t].w, mask_plane<3>(d), acc23[r]);
        }
    }
}

// 16 code bytes of the raw block layout at byte offset off (2-byte aligned:
// blocks are 34 bytes).  An offset of 2 mod 4 reads the dwords from two bytes
// before it plus the ushort at off + 14 and shifts them into place, so no
// read reaches past the block's last byte.
__device__ __forceinline__ uint4 raw_codes16(__amdgpu_buffer_rsrc_t r, bool ok, uint32_t off) {
    const uint32_t sh = (off & 2u) * 8u;  // 0 or 16 bits
    const uint4 a = buf_load16<kAuxNonTemporal>(r, ok ? off & ~3u : kBufferOOB);
    const uint32_t e = buf_load2(r, ok ? off + 14u : kBufferOOB);
    return make_uint4(__builtin_amdgcn_alignbit(a.y, a.x, sh), __builtin_amdgcn_alignbit(a.z, a.y, sh),
                      __builtin_amdgcn_alignbit(a.w, a.z, sh), __builtin_amdgcn_alignbit(e, a.w, sh));
}

// RAW: `codes` is the raw block layout (page "Kernel experiments", section
// A, Tests 4 and 24: each 128-weight block is its fp16 scale then 32 code
// bytes, rows raw_stride bytes apart), read without a preparation pass; each
// lane takes the same 16 code bytes and scale as from the planes.
template <int MC, int R, int SEGS, int SRC, bool RAW = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(SEGS == 1 && R == 1 && MC <= (src_fused(SRC) ? 1 : 4) ? 7 : 1))) void small_m_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ xs, const int32_t* __restrict__ qsum,
    const void* __restrict__ x, int64_t x_stride,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, float* __restrict__ y, int n,
    int k, int groups, int nseg, int segs_per_wave, int mtotal, int raw_stride) {
#pragma clang fp contract(off)
    constexpr bool FUSED = src_fused(SRC);
    constexpr int XL = src_xloads(SRC);
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int RB = kRowSlots * R;
    constexpr int WAVE_QUADS = MC * kSegQuads;  // one segment staged at a time
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop bounds
    const int lane = threadIdx.x & 63;
    const int slot = lane >> 3;
    const int j = lane & 7;
    const int h = j & 1;
    const int gsel = (j >> 1) + 4 * h;  // group (within a segment) whose full dot this lane scales
    const int m0 = blockIdx.y * MC;
    const int mcount = min(MC, mtotal - m0);
    const int row_base = blockIdx.x * RB;
    const int rows_here = min(RB, n - row_base);
    const int seg_begin = wave * segs_per_wave;
    const int seg_end = min(seg_begin + segs_per_wave, nseg);
    const uint32_t k4 = (uint32_t)k >> 2;

    unsigned char* region = smem + (size_t)wave * WAVE_QUADS * 16;
    float* red = reinterpret_cast<float*>(smem + (size_t)nwaves * WAVE_QUADS * 16);
    // One base address per access kind; the (segment, column, quad) parts are immediates.
    unsigned char* wr_ptr = region + (slot * kBlockPitch + j) * 16;          // copies quad j of group `slot`
    const unsigned char* rd_ptr = region + ((j >> 1) * kBlockPitch + 4 * h) * 16;  // half h of group j/2
    const unsigned char* qs_ptr = region + (gsel * kBlockPitch + 8) * 16;     // sum(q) of group gsel

    // Raw rows: the resource starts at the 4-byte boundary at or below this
    // workgroup's first row (rows are 2-byte aligned), and adj re-adds the
    // difference, so an offset's low bits are its address's.
    const uint8_t* raw_rows = codes + (size_t)row_base * raw_stride;
    const uint32_t adj = RAW ? (uint32_t)(reinterpret_cast<uintptr_t>(raw_rows) & 3u) : 0u;
    const auto code_rs = RAW ? make_rsrc(raw_rows - adj, (uint32_t)rows_here * (uint32_t)raw_stride + adj)
                             : make_rsrc(codes + (size_t)row_base * k4, (uint32_t)rows_here * k4);
    const auto scale_rs = make_rsrc(RAW ? nullptr : scales + (size_t)row_base * groups,
                                    RAW ? 0u : (uint32_t)(rows_here * groups * 2));
    const auto q_rs = make_rsrc(FUSED ? nullptr : q + (size_t)m0 * k, FUSED ? 0u : (uint32_t)(mcount * k));
    const auto xs_rs = make_rsrc(FUSED ? nullptr : xs + (size_t)m0 * groups, FUSED ? 0u : (uint32_t)(mcount * groups * 4));
    const auto qs_rs = make_rsrc(SRC == kSrcPlanes ? qsum + (size_t)m0 * groups : nullptr,
                                 SRC == kSrcPlanes ? (uint32_t)(mcount * groups * 4) : 0u);
    const auto x_rs = make_rsrc(
        FUSED ? static_cast<const unsigned char*>(x) + (size_t)m0 * x_stride * src_esize(SRC) : nullptr,
        FUSED ? (uint32_t)(((int64_t)(mcount - 1) * x_stride + k) * src_esize(SRC)) : 0u);

    float acc[MC][R];
#pragma unroll
    for (int m = 0; m < MC; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

    for (int base = seg_begin; base < seg_end; base += SEGS) {
        // 1. Activation blocks, scales and group sums of this step (small, L2-resident) ...
        uint4 qv[SEGS][MC];
        uint4 xv[SEGS][MC][FUSED ? XL : 1];
        uint32_t xsv[SEGS][MC], tv[SEGS][MC];
#pragma unroll
        for (int si = 0; si < SEGS; ++si) {
            const bool sok = base + si < seg_end;
            const int gq = (base + si) * kGroupLanes + slot;  // group whose quad j this lane copies
            const int gs = (base + si) * kGroupLanes + gsel;  // group this lane scales
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const bool qok = sok && gq < groups && m < mcount;
                const bool gok = sok && gs < groups && m < mcount;
                if constexpr (FUSED) {
                    // Elements 16j..16j+15 of group gq (out-of-range groups read zero).
                    const uint32_t off = (uint32_t)((m * x_stride + gq * 128 + j * 16) * src_esize(SRC));
#pragma unroll
                    for (int l = 0; l < XL; ++l) xv[si][m][l] = buf_load16(x_rs, qok ? off + 16u * l : kBufferOOB);
                } else {
                    qv[si][m] = buf_load16(q_rs, qok ? (uint32_t)(m * k + gq * 128 + j * 16) : kBufferOOB);
                    xsv[si][m] = buf_load4(xs_rs, gok ? (uint32_t)((m * groups + gs) * 4) : kBufferOOB);
                }
                if constexpr (SRC == kSrcPlanes)
                    tv[si][m] = buf_load4(qs_rs, gok ? (uint32_t)((m * groups + gs) * 4) : kBufferOOB);
            }
        }
        // 2. ... then every code load of the step (HBM), all in flight together:
        //    lane j reads 16 bytes at 16j (half h of group j/2) and at 128 + 16j
        //    (half h of group 4 + j/2) of the segment's 256 bytes of its row.
        uint4 cw[SEGS][2][R];
        uint32_t wsraw[SEGS][R];
#pragma unroll
        for (int si = 0; si < SEGS; ++si) {
            const int g0 = (base + si) * kGroupLanes;
            const bool sok = base + si < seg_end;
            const bool okA = sok && g0 + (j >> 1) < groups;
            const bool okB = sok && g0 + 4 + (j >> 1) < groups;
            const bool okS = sok && g0 + gsel < groups;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t rl = (uint32_t)(slot + kRowSlots * r);
                if constexpr (RAW) {
                    // Block g of row rl starts at rl * raw_stride + 34 g.
                    const uint32_t row_off = adj + rl * (uint32_t)raw_stride;
                    const uint32_t off = row_off + (uint32_t)(g0 + (j >> 1)) * 34u + 2u + 16u * (uint32_t)h;
                    cw[si][0][r] = raw_codes16(code_rs, okA, off);
                    cw[si][1][r] = raw_codes16(code_rs, okB, off + 4u * 34u);
                    wsraw[si][r] = buf_load2(code_rs, okS ? row_off + (uint32_t)(g0 + gsel) * 34u : kBufferOOB);
                } else {
                    const uint32_t off = rl * k4 + (uint32_t)g0 * 32u + 16u * (uint32_t)j;
                    cw[si][0][r] = buf_load16<kAuxNonTemporal>(code_rs, okA ? off : kBufferOOB);
                    cw[si][1][r] = buf_load16<kAuxNonTemporal>(code_rs, okB ? off + 128u : kBufferOOB);
                    wsraw[si][r] = buf_load2(scale_rs, okS ? (rl * groups + g0 + gsel) * 2u : kBufferOOB);
                }
            }
        }
        // 3./4. Per segment: private LDS copy of its activation blocks (natural
        //    input: transposed here and the group sums formed), then the exact
        //    group dots, partner exchange, FP32 scaling and lane-serial
        //    accumulation.  Only this wave touches its region, and LDS operations
        //    of one wave complete in program order.
#pragma unroll
        for (int si = 0; si < SEGS; ++si) {
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                uint4 v = qv[si][m];
                if constexpr (SRC == kSrcNatural) {
                    int s = dot4(v.x, 0x01010101u, 0);
                    s = dot4(v.y, 0x01010101u, s);
                    s = dot4(v.z, 0x01010101u, s);
                    s = dot4(v.w, 0x01010101u, s);
                    s = sum8_i(s);  // sum(q) of group `slot`, in all 8 lanes of the slot
                    v = to_plane_order(v);
                    if (j == 0) *reinterpret_cast<int*>(wr_ptr + (m * kSegQuads + 8) * 16) = s;
                }
                if constexpr (FUSED) {
                    float xf[16];
                    x_to_float16<SRC>(xv[si][m], xf);
                    int s;
                    float scale;
                    v = quantize_lane16(xf, s, scale);  // group `slot`, all 8 lanes of the slot agree
                    if (j == 0)
                        *reinterpret_cast<uint2*>(wr_ptr + (m * kSegQuads + 8) * 16) =
                            make_uint2((uint32_t)s, __float_as_uint(scale));
                }
                *reinterpret_cast<uint4*>(wr_ptr + m * kSegQuads * 16) = v;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (base + si < seg_end) {
                const unsigned char* blk = rd_ptr;
                int half[2][MC][R];
#pragma unroll
                for (int hg = 0; hg < 2; ++hg) {  // hg 0: group j/2, 1: group 4 + j/2
                    int a0[MC][R], a1[MC][R], a23[MC][R];
#pragma unroll
                    for (int m = 0; m < MC; ++m)
#pragma unroll
                        for (int r = 0; r < R; ++r) a0[m][r] = a1[m][r] = a23[m][r] = 0;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        uint4 P[MC];
#pragma unroll
                        for (int m = 0; m < MC; ++m)
                            P[m] = *reinterpret_cast<const uint4*>(blk + (m * kSegQuads + hg * 4 * kBlockPitch + t) * 16);
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            const uint32_t d = word_of(cw[si][hg][r], t);
                            const uint32_t c0 = mask_plane<0>(d), c1 = mask_plane<1>(d);
                            const uint32_t c2 = mask_plane<2>(d), c3 = mask_plane<3>(d);
#pragma unroll
                            for (int m = 0; m < MC; ++m) {
                                a0[m][r] = dot4(P[m].x, c0, a0[m][r]);
                                a1[m][r] = dot4(P[m].y, c1, a1[m][r]);
                                a23[m][r] = dot4(P[m].z, c2, a23[m][r]);
                                a23[m][r] = dot4(P[m].w, c3, a23[m][r]);
                            }
                        }
                    }
#pragma unroll
                    for (int m = 0; m < MC; ++m)
#pragma unroll
                        for (int r = 0; r < R; ++r) half[hg][m][r] = a0[m][r] + (a1[m][r] >> 2) + (a23[m][r] >> 4);
                }
#pragma unroll
                for (int m = 0; m < MC; ++m) {
                    int sq;
                    float xsf;
                    if constexpr (FUSED) {
                        const uint2 meta = *reinterpret_cast<const uint2*>(qs_ptr + m * kSegQuads * 16);
                        sq = (int)meta.x;
                        xsf = __uint_as_float(meta.y);
                    } else {
                        sq = SRC == kSrcNatural ? *reinterpret_cast<const int*>(qs_ptr + m * kSegQuads * 16)
                                                : (int)tv[si][m];
                        xsf = __uint_as_float(xsv[si][m]);
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        // Lane h = 0 keeps group j/2 and hands its half of group 4 + j/2
                        // to the partner; lane h = 1 the other way round.
                        const int mine = h ? half[1][m][r] : half[0][m][r];
                        const int give = h ? half[0][m][r] : half[1][m][r];
                        const int dot = mine + dpp_i<kDppXor1>(give) - sq;
                        const float wsf = __half2float(__ushort_as_half((unsigned short)wsraw[si][r]));
                        acc[m][r] = __builtin_fmaf((float)dot * xsf, wsf, acc[m][r]);
                    }
                }
            }
        }
    }

    // 5. Reduce over the 8 lanes of a slot (fixed DPP tree), then over waves in index order.
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

// ------------------------------------------------------------------ matrix-core variant
// The same result, bit for bit, from the INT8 matrix cores.  Each wave still
// owns 8 weight rows and the segments of its k split, and reads the codes
// with whole 128-byte lines per row, but lane l takes row l & 7 and 16-byte
// chunk l >> 3 of the 128-byte span (group (l >> 4), half (l >> 3) & 1 of the
// span's four groups).  With that assignment one v_mfma_i32_16x16x64_i8 per
// code dword yields every half-group dot of the span for two columns:
//  * B (64 x 16): lane l supplies k-block l >> 4 (= the group) of column
//    l & 15 = (half h, row); its 16 bytes are the four bit planes of one code
//    dword, code values 0..3 (the -1 offset is again -sum(q) per group);
//  * A (16 x 64): row i = 4 ga + 2 mm + hp holds, in k-block ga only, the
//    plane-ordered activations of column 2 set + mm for half hp -- zero in
//    the other k-blocks, so D[(ga, mm, hp)][(h, row)] is the dot of group ga
//    restricted to (activation half hp, code half h), and the hp == h entries
//    of the lanes (ga, 0, row) and (ga, 1, row) add up (one DPP rotate) to
//    the exact group dot.
// Terms, the lane-serial FP32 accumulation per group class and the final
// tree ((A0 + A4) + (A1 + A5)) + ((A2 + A6) + (A3 + A7)), then waves in
// order, are exactly those of small_m_kernel, so both give identical bits.
template <int MC, int SEGS, int SRC>
__global__ __launch_bounds__(512) void small_m_mfma_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ xs, const int32_t* __restrict__ qsum,
    const void* __restrict__ x, int64_t x_stride,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, float* __restrict__ y, int n,
    int k, int groups, int nseg, int segs_per_wave, int mtotal) {
#pragma clang fp contract(off)
    constexpr bool FUSED = src_fused(SRC);
    constexpr int XL = src_xloads(SRC);
    typedef int v4i __attribute__((ext_vector_type(4)));
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int MP = (MC + 1) / 2;  // matrix-core passes, two columns each
    constexpr int WAVE_QUADS = MC * kSegQuads;  // one segment staged at a time
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // Copy roles (activation blocks): group `slot` of the segment, quad j.
    const int slot = lane >> 3;
    const int j = lane & 7;
    // Matrix roles: code row, k-block (group of the span) and code half.
    const int row = lane & 7;
    const int kb = lane >> 4;
    const int h = (lane >> 3) & 1;
    // A-operand row of this lane: (ga, mm, hp); it carries data only in k-block ga.
    const int ai = lane & 15;
    const int a_mm = (ai >> 1) & 1;
    const int a_hp = ai & 1;
    const bool a_lane = (ai >> 2) == kb;
    const int m0 = blockIdx.y * MC;
    const int mcount = min(MC, mtotal - m0);
    const int row_base = blockIdx.x * kRowSlots;
    const int rows_here = min(kRowSlots, n - row_base);
    const int seg_begin = wave * segs_per_wave;
    const int seg_end = min(seg_begin + segs_per_wave, nseg);
    const uint32_t k4 = (uint32_t)k >> 2;

    // LDS: one all-zero region shared by the workgroup, then one private
    // region per wave, then the reduction area.  A-operand lanes outside
    // their k-block read the zero region at the same offsets, so every A read
    // is unconditional and addressed by one register plus immediates.
    unsigned char* zero_region = smem;
    unsigned char* region = smem + (size_t)(1 + wave) * WAVE_QUADS * 16;
    float* red = reinterpret_cast<float*>(smem + (size_t)(1 + nwaves) * WAVE_QUADS * 16);
    unsigned char* wr_ptr = region + (slot * kBlockPitch + j) * 16;
    const unsigned char* a_base[MP];
#pragma unroll
    for (int p = 0; p < MP; ++p) {
        const int am = 2 * p + a_mm;
        a_base[p] = (a_lane && am < mcount) ? region + ((am * kSegQuads) + kb * kBlockPitch + 4 * a_hp) * 16
                                            : zero_region;
    }
    const unsigned char* meta_ptr = region + (kb * kBlockPitch + 8) * 16;      // sum(q), xs of group kb

    const auto code_rs = make_rsrc(codes + (size_t)row_base * k4, (uint32_t)rows_here * k4);
    const auto scale_rs = make_rsrc(scales + (size_t)row_base * groups, (uint32_t)(rows_here * groups * 2));
    const auto q_rs = make_rsrc(FUSED ? nullptr : q + (size_t)m0 * k, FUSED ? 0u : (uint32_t)(mcount * k));
    const auto xs_rs = make_rsrc(FUSED ? nullptr : xs + (size_t)m0 * groups, FUSED ? 0u : (uint32_t)(mcount * groups * 4));
    const auto qs_rs = make_rsrc(SRC == kSrcPlanes ? qsum + (size_t)m0 * groups : nullptr,
                                 SRC == kSrcPlanes ? (uint32_t)(mcount * groups * 4) : 0u);
    const auto x_rs = make_rsrc(
        FUSED ? static_cast<const unsigned char*>(x) + (size_t)m0 * x_stride * src_esize(SRC) : nullptr,
        FUSED ? (uint32_t)(((int64_t)(mcount - 1) * x_stride + k) * src_esize(SRC)) : 0u);

    float acc[MP][2];
#pragma unroll
    for (int p = 0; p < MP; ++p) acc[p][0] = acc[p][1] = 0.0f;

    for (int base = seg_begin; base < seg_end; base += SEGS) {
        // 1. Activation blocks and per-group metadata (small, L2-resident) ...
        uint4 qv[SEGS][MC];
        uint4 xv[SEGS][MC][FUSED ? XL : 1];
        uint32_t xsv[SEGS][MC], tv[SEGS][MC];
#pragma unroll
        for (int si = 0; si < SEGS; ++si) {
            const bool sok = base + si < seg_end;
            const int gq = (base + si) * kGroupLanes + slot;
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const bool qok = sok && gq < groups && m < mcount;
                if constexpr (FUSED) {
                    const uint32_t off = (uint32_t)((m * x_stride + gq * 128 + j * 16) * src_esize(SRC));
#pragma unroll
                    for (int l = 0; l < XL; ++l) xv[si][m][l] = buf_load16(x_rs, qok ? off + 16u * l : kBufferOOB);
                } else {
                    qv[si][m] = buf_load16(q_rs, qok ? (uint32_t)(m * k + gq * 128 + j * 16) : kBufferOOB);
                    const uint32_t moff = (qok && j == 0) ? (uint32_t)((m * groups + gq) * 4) : kBufferOOB;
                    xsv[si][m] = buf_load4(xs_rs, moff);
                    if constexpr (SRC == kSrcPlanes) tv[si][m] = buf_load4(qs_rs, moff);
                }
            }
        }
        // 2. ... then the code loads of the step: two spans of four groups per segment.
        uint4 cw[SEGS][2];
        uint32_t wsraw[SEGS][2];
#pragma unroll
        for (int si = 0; si < SEGS; ++si) {
            const int g0 = (base + si) * kGroupLanes;
            const bool sok = base + si < seg_end;
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const bool ok = sok && g0 + 4 * sp + kb < groups;
                const uint32_t off = (uint32_t)row * k4 + (uint32_t)g0 * 32u + 128u * sp + 16u * (uint32_t)(lane >> 3);
                cw[si][sp] = buf_load16<kAuxNonTemporal>(code_rs, ok ? off : kBufferOOB);
                wsraw[si][sp] = buf_load2(scale_rs, ok ? ((uint32_t)row * groups + g0 + 4 * sp + kb) * 2u : kBufferOOB);
            }
        }
        // The shared zero region is filled once, while the first loads are in
        // flight; every wave runs this first iteration (each owns >= 1 segment).
        if (base == seg_begin) {
            for (int i = threadIdx.x; i < WAVE_QUADS; i += nthreads)
                reinterpret_cast<uint4*>(zero_region)[i] = make_uint4(0u, 0u, 0u, 0u);
            __syncthreads();
        }
        // 3./4. Per segment: private LDS copy of its activation blocks and
        //    metadata, then the matrix-core group dots, exact recombination and
        //    FP32 terms.
#pragma unroll
        for (int si = 0; si < SEGS; ++si) {
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                uint4 v = qv[si][m];
                int s;
                uint32_t scale_bits;
                if constexpr (FUSED) {
                    float xf[16];
                    x_to_float16<SRC>(xv[si][m], xf);
                    float scale;
                    v = quantize_lane16(xf, s, scale);
                    scale_bits = __float_as_uint(scale);
                } else if constexpr (SRC == kSrcNatural) {
                    s = dot4(v.x, 0x01010101u, 0);
                    s = dot4(v.y, 0x01010101u, s);
                    s = dot4(v.z, 0x01010101u, s);
                    s = dot4(v.w, 0x01010101u, s);
                    s = sum8_i(s);
                    v = to_plane_order(v);
                    scale_bits = xsv[si][m];
                } else {
                    s = (int)tv[si][m];
                    scale_bits = xsv[si][m];
                }
                unsigned char* blk = wr_ptr + m * kSegQuads * 16;
                *reinterpret_cast<uint4*>(blk) = v;
                if (j == 0) *reinterpret_cast<uint2*>(blk + 8 * 16) = make_uint2((uint32_t)s, scale_bits);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (base + si < seg_end) {
#pragma unroll
                for (int p = 0; p < MP; ++p) {
                    // Two independent chains (the two spans), interleaved step by step.
                    v4i D[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
#pragma unroll
                        for (int sp = 0; sp < 2; ++sp) {
                            const uint32_t d = word_of(cw[si][sp], st);
                            const v4i B = v4i{(int)(d & 0x03030303u), (int)((d >> 2) & 0x03030303u),
                                              (int)((d >> 4) & 0x03030303u), (int)((d >> 6) & 0x03030303u)};
                            const uint4 v = *reinterpret_cast<const uint4*>(
                                a_base[p] + (sp * 4 * kBlockPitch + st) * 16);
                            const v4i A = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                            D[sp] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, D[sp], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int sp = 0; sp < 2; ++sp) {
                        // Lane (kb, h, row): column 2p + h; its own half is D[3h], the
                        // partner lane (kb, 1 - h, row) holds the other half.
                        const int give = h ? D[sp][1] : D[sp][2];
                        const int mine = h ? D[sp][3] : D[sp][0];
                        const int dotc = mine + __builtin_amdgcn_update_dpp(0, give, 0x128, 0xF, 0xF, false);
                        const int m = 2 * p + h;
                        if (m < MC) {
                            const uint2 meta = *reinterpret_cast<const uint2*>(
                                meta_ptr + (m * kSegQuads + sp * 4 * kBlockPitch) * 16);
                            const float wsf = __half2float(__ushort_as_half((unsigned short)wsraw[si][sp]));
                            const int dot = dotc - (int)meta.x;
                            acc[p][sp] = __builtin_fmaf((float)dot * __uint_as_float(meta.y), wsf, acc[p][sp]);
                        }
                    }
                }
            }
        }
    }

    // 5. Group classes k-block, 4 + k-block add in the lane; the four k-blocks and
    //    the waves add through LDS in the fixed order of small_m_kernel.
#pragma unroll
    for (int p = 0; p < MP; ++p) {
        const int m = 2 * p + h;
        if (m < MC) red[((wave * 4 + kb) * MC + m) * kRowSlots + row] = acc[p][0] + acc[p][1];
    }
    __syncthreads();
    for (int o = threadIdx.x; o < MC * kRowSlots; o += nthreads) {
        const int m = o / kRowSlots;
        const int r = o - m * kRowSlots;
        float sum = 0.0f;
        for (int w = 0; w < nwaves; ++w) {
            const float* t = red + (size_t)w * 4 * MC * kRowSlots + m * kRowSlots + r;
            const float tw = (t[0] + t[MC * kRowSlots]) + (t[2 * MC * kRowSlots] + t[3 * MC * kRowSlots]);
            sum = w == 0 ? tw : sum + tw;
        }
        if (m < mcount && r < rows_here) y[(size_t)(m0 + m) * n + row_base + r] = sum;
    }
}

// ------------------------------------------------------------------ host side
namespace {

constexpr size_t kLdsLimit = 144 * 1024;

// Private activation regions of all waves, plus one float per (wave, column,
// row) for the cross-wave sum.
size_t lds_bytes(int mc, int segs, int waves, int rows_per_wg) {
    (void)segs;  // one segment is staged at a time
    return (size_t)waves * mc * kSegQuads * 16 + (size_t)waves * mc * rows_per_wg * 4;
}

using Launch = SmallMLaunch;

template <int MC, int R, int SEGS, int SRC, bool RAW = false>
hipError_t launch_one(const Launch& a) {
    auto kern = small_m_kernel<MC, R, SEGS, SRC, RAW>;
    const size_t lds = lds_bytes(MC, SEGS, a.waves, kRowSlots * R);
    static bool attr_set = false;  // one instantiation = one static
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const uint16_t* scales = RAW ? nullptr : reinterpret_cast<const uint16_t*>(a.planes + a.n * (a.k / 4));
    const dim3 grid((unsigned)((a.n + kRowSlots * R - 1) / (kRowSlots * R)), (unsigned)a.chunks);
    clear_stale_error();
    hipLaunchKernelGGL(kern, grid, dim3(64 * a.waves), lds, a.stream, a.q, a.xs, a.qsum, a.x, a.x_stride, a.planes,
                       scales, a.y, (int)a.n, (int)a.k, (int)(a.k / 128), a.nseg, a.per_wave, (int)a.m,
                       (int)a.raw_stride);
    return hipGetLastError();
}

// Segments per load step: 1 or 2 (the register cap in launch_any never asks for more).
template <int MC, int R, int SRC, bool RAW = false>
hipError_t pick_segs(const Launch& a, int segs) {
    return segs == 1 ? launch_one<MC, R, 1, SRC, RAW>(a) : launch_one<MC, R, 2, SRC, RAW>(a);
}

template <int MC, int SRC, bool RAW = false>
hipError_t pick_rows(const Launch& a, int rows, int segs) {
    return rows == 1 ? pick_segs<MC, 1, SRC, RAW>(a, segs) : pick_segs<MC, 2, SRC, RAW>(a, segs);
}

// Fused (quantising) instantiations cover up to 4 columns per pass.
constexpr int max_mc(int src) { return src_fused(src) ? 4 : 8; }

template <int SRC, bool RAW = false>
hipError_t pick_mc(const Launch& a, int mc, int rows, int segs) {
    switch (mc) {
        case 1: return pick_rows<1, SRC, RAW>(a, rows, segs);
        case 2: return pick_rows<2, SRC, RAW>(a, rows, segs);
        case 3: return pick_rows<3, SRC, RAW>(a, rows, segs);
        case 4: return pick_rows<4, SRC, RAW>(a, rows, segs);
        default: break;
    }
    if constexpr (max_mc(SRC) == 8) {
        switch (mc) {
            case 5: return pick_rows<5, SRC, RAW>(a, rows, segs);
            case 6: return pick_rows<6, SRC, RAW>(a, rows, segs);
            case 7: return pick_rows<7, SRC, RAW>(a, rows, segs);
            case 8: return pick_rows<8, SRC, RAW>(a, rows, segs);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

size_t mfma_lds_bytes(int mc, int segs, int waves) {
    (void)segs;  // one segment is staged at a time
    return (size_t)(waves + 1) * mc * kSegQuads * 16 + (size_t)waves * 4 * mc * kRowSlots * 4;
}

template <int MC, int SEGS, int SRC>
hipError_t launch_mfma_one(const Launch& a) {
    auto kern = small_m_mfma_kernel<MC, SEGS, SRC>;
    const size_t lds = mfma_lds_bytes(MC, SEGS, a.waves);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(a.planes + a.n * (a.k / 4));
    const dim3 grid((unsigned)((a.n + kRowSlots - 1) / kRowSlots), (unsigned)a.chunks);
    clear_stale_error();
    hipLaunchKernelGGL(kern, grid, dim3(64 * a.waves), lds, a.stream, a.q, a.xs, a.qsum, a.x, a.x_stride, a.planes,
                       scales, a.y, (int)a.n, (int)a.k, (int)(a.k / 128), a.nseg, a.per_wave, (int)a.m);
    return hipGetLastError();
}

template <int MC, int SRC>
hipError_t mfma_pick_segs(const Launch& a, int segs) {
    return segs == 1 ? launch_mfma_one<MC, 1, SRC>(a) : launch_mfma_one<MC, 2, SRC>(a);
}

template <int SRC>
hipError_t mfma_pick_mc(const Launch& a, int mc, int segs) {
    switch (mc) {
        case 1: return mfma_pick_segs<1, SRC>(a, segs);
        case 2: return mfma_pick_segs<2, SRC>(a, segs);
        case 3: return mfma_pick_segs<3, SRC>(a, segs);
        case 4: return mfma_pick_segs<4, SRC>(a, segs);
        default: break;
    }
    if constexpr (max_mc(SRC) == 8) {
        switch (mc) {
            case 5: return mfma_pick_segs<5, SRC>(a, segs);
            case 6: return mfma_pick_segs<6, SRC>(a, segs);
            case 7: return mfma_pick_segs<7, SRC>(a, segs);
            case 8: return mfma_pick_segs<8, SRC>(a, segs);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

template <int SRC>
hipError_t dispatch(const Launch& a, int engine, int mc, int rows, int segs) {
    return engine == 2 ? mfma_pick_mc<SRC>(a, mc, segs) : pick_mc<SRC>(a, mc, rows, segs);
}

hipError_t launch_any(int src, const Launch& base, const SmallMConfig& cfg) {
    if (cfg.max_waves < 1 || cfg.max_waves > 8) return hipErrorInvalidValue;
    if (cfg.engine == 3 || cfg.engine == 4) return launch_small_m_wg(src, base, cfg.max_waves, cfg.rows, cfg.engine == 4);
    if (cfg.engine != 1 && cfg.engine != 2) return hipErrorInvalidValue;
    const int rows = cfg.engine == 2 ? 1 : cfg.rows;
    if (rows != 1 && rows != 2) return hipErrorInvalidValue;
    const int64_t m = base.m, k = base.k;
    const int groups = (int)(k / 128);
    const int nseg = (groups + kGroupLanes - 1) / kGroupLanes;
    const int per_wave = (nseg + cfg.max_waves - 1) / cfg.max_waves;
    const int waves = (nseg + per_wave - 1) / per_wave;
    auto lds = [&](int mc, int segs) {
        return cfg.engine == 2 ? mfma_lds_bytes(mc, segs, waves) : lds_bytes(mc, segs, waves, kRowSlots * rows);
    };
    int segs = per_wave < 2 ? per_wave : 2;
    const int mc_cap = max_mc(src);
    int mc = (int)(m < mc_cap ? m : mc_cap);
    while (mc > 1 && lds(mc, segs) > kLdsLimit) --mc;
    while (segs > 1 && lds(mc, segs) > kLdsLimit) --segs;
    const int chunks = (int)((m + mc - 1) / mc);
    mc = (int)((m + chunks - 1) / chunks);  // balance the column passes
    // At most two (column x row) units of code loads per lane per step: more
    // segments per step hold more registers than the residency of the whole
    // grid allows (measured at K = 17408), and the loop covers the rest.
    while (mc * rows * segs > 2 && segs > 1) --segs;
    Launch a = base;
    a.waves = waves;
    a.nseg = nseg;
    a.per_wave = per_wave;
    a.chunks = chunks;
    if (a.raw_stride != 0) {  // raw block layout: packed-dot engine, natural-order q
        if (src != kSrcNatural || cfg.engine != 1) return hipErrorInvalidValue;
        return pick_mc<kSrcNatural, true>(a, mc, rows, segs);
    }
    switch (src) {
        case kSrcPlanes: return dispatch<kSrcPlanes>(a, cfg.engine, mc, rows, segs);
        case kSrcNatural: return dispatch<kSrcNatural>(a, cfg.engine, mc, rows, segs);
        case kSrcBf16: return dispatch<kSrcBf16>(a, cfg.engine, mc, rows, segs);
        case kSrcF16: return dispatch<kSrcF16>(a, cfg.engine, mc, rows, segs);
        case kSrcF32: return dispatch<kSrcF32>(a, cfg.engine, mc, rows, segs);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int default_small_m_rows(int engine, int src, int64_t m, int64_t n, int64_t k, int max_waves) {
    switch (engine) {
        case 1: return src_fused(src) ? 2 : (m <= 4 ? 1 : 2);
        case 2: return 1;
        case 3: return wg_default_row_blocks(src, m, n, k, max_waves, false);
        case 4: return wg_default_row_blocks(src, m, n, k, max_waves, true);
        default: return 0;
    }
}

// The k split (max_waves) must depend on (n, k) only: it fixes the summation
// order, and outputs must not change with the number of columns.  Rows per
// lane does not touch the order; two rows per lane halve the LDS reads of
// the activations, which pays from five columns on (measured on the
// K=5120 and K=17408 shapes).
// Every engine gives the same bits, so the engine is free per shape: packed
// dots win at one or two columns, the matrix cores from five columns on and
// from three on when K is long (measured on the K = 5120 and K = 17408
// shapes; the matrix-core work per code dword does not grow with M).
// The fused path quantises the activations inside the matmul.  The
// packed-dot engine repeats that per 16-row workgroup (two rows per lane),
// which is cheapest at one column; from two to eight columns the
// workgroup-staged engine, which quantises once per CU-sized workgroup, is
// faster at every measured shape (K = 5120 and 17408).
SmallMConfig default_small_m_config(int src, int64_t m, int64_t n, int64_t k) {
    SmallMConfig c;
    c.max_waves = 8;
    if (src_fused(src)) {
        c.engine = 1;
        if (m >= 2 && m <= 8 && default_small_m_rows(3, src, m, n, k, c.max_waves) > 0) c.engine = 3;
    } else {
        c.engine = (m >= 5 || (m >= 3 && k >= 8192)) ? 2 : 1;
    }
    c.rows = default_small_m_rows(c.engine, src, m, n, k, c.max_waves);
    return c;
}

hipError_t launch_small_m(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m, int64_t n,
                          int64_t k, float* y, const SmallMConfig& cfg, hipStream_t stream) {
    const Launch a{q, xs, nullptr, nullptr, 0, planes, m, n, k, y, 0, 0, 0, 0, stream};
    return launch_any(kSrcNatural, a, cfg);
}

hipError_t launch_small_m_planes(const int8_t* qp, const float* xs, const int32_t* qsum, const uint8_t* planes,
                                 int64_t m, int64_t n, int64_t k, float* y, const SmallMConfig& cfg,
                                 hipStream_t stream) {
    const Launch a{qp, xs, qsum, nullptr, 0, planes, m, n, k, y, 0, 0, 0, 0, stream};
    return launch_any(kSrcPlanes, a, cfg);
}

hipError_t launch_small_m_raw(const int8_t* q, const float* xs, const uint8_t* raw, int64_t raw_stride, int64_t m,
                              int64_t n, int64_t k, float* y, int max_waves, int rows, hipStream_t stream) {
    Launch a{q, xs, nullptr, nullptr, 0, raw, m, n, k, y, 0, 0, 0, 0, stream};
    a.raw_stride = raw_stride;
    SmallMConfig cfg;
    cfg.engine = 1;
    cfg.max_waves = max_waves;
    cfg.rows = rows;
    return launch_any(kSrcNatural, a, cfg);
}

hipError_t launch_small_m_fused(const void* x, int dtype, int64_t x_stride, const uint8_t* planes, int64_t m,
                                int64_t n, int64_t k, float* y, const SmallMConfig& cfg, hipStream_t stream) {
    const Launch a{nullptr, nullptr, nullptr, x, x_stride, planes, m, n, k, y, 0, 0, 0, 0, stream};
    return launch_any(src_of_dtype(dtype), a, cfg);
}

}  // namespace pq2
