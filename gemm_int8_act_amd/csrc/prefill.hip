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
//  * Workgroup tile BM x BN (128x128, 64x128, 128x64 or 64x64, chosen so
//    the grid fills the chip), WM x 2 waves (WM = 2, or 4 for the 128x128
//    tile on eight waves), each wave (BM/WM) x (BN/2) made of 32 x 32 tiles
//    of v_mfma_i32_32x32x32_i8.  One group (k = 128)
//    = four MFMA k-steps of 32.
//  * Activations come in natural order (transposed while staged) or already
//    in plane order (pq2_quantize_act_i8_planes; copied as they are).
//  * Operand order inside a k-step is free as long as A and B agree: lane l
//    of an MFMA supplies 16 bytes of row (l % 32) of A and of column (l % 32)
//    of B for the same 16 k positions.  Lane half h = l / 32 in k-step kk
//    takes code dword t = 2kk + h, whose four bit planes are the 16 weights
//    16t + 4j + s (plane s, byte j); A is staged byte-transposed to match.
//  * B decode: the 2-bit field of each byte becomes c - 1 through one
//    v_perm_b32 table lookup per plane (table bytes -1, 0, +1, +2), 11 ALU
//    ops per code dword.
//  * LDS is double-buffered: the global loads of later groups are in flight
//    while group g is multiplied, then the next group is written to the
//    other buffer; one barrier per group.  Quads of a row are XOR-swizzled
//    over 16 rows so the 32-row fragment reads and the staging writes hit
//    distinct banks.
//  * Global loads cost by instruction rather than by byte here, so every
//    lane of every load carries data: 16-byte activation loads, one 16-byte
//    code load per group pair (tile layout), and the scales of 8 groups per
//    load (tile layout).
//  * The 128x128 tile on eight waves (tile layout) loads its activations
//    straight into LDS (buffer_load_dwordx4 ... lds), each lane fetching the
//    quad that the swizzle puts in its slot: no registers and no staging
//    writes for A, which keeps the tile at four waves per SIMD, two
//    workgroups per CU.
//  * After the four k-steps of a group each lane rescales its INT32 results:
//    acc += (float(dot) * xs[m]) * ws[n].  That rescale (3 VALU per output
//    and group) makes the VALU the busiest unit: it costs more issue slots
//    than the matrix cores need for the group's 128 multiply-adds.
#include "pq2_device.h"
#include "pq2_internal.h"

#include <hip/hip_fp16.h>

#include <type_traits>

namespace pq2 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr uint32_t kCodeLut = 0x020100FFu;  // code c -> byte c - 1 (as v_perm table)

// 16 bytes per lane straight into LDS, lane l's at lds_addr + 16 l
// (buffer_load_dwordx4 ... lds; offsets past the buffer's range read zero, as
// for buf_load16).  Issued from inline assembly so that the compiler's
// wait-count pass does not see the LDS write: given the builtin, it took the
// write as aliasing every later LDS read and waited for the load before the
// next fragment read.  The caller waits (wait_vm) before other waves read.
// A load the pass does not count only makes its own vmcnt waits longer:
// loads complete in issue order.
__device__ __forceinline__ void buf_load16_lds(i32x4_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N) (GFX9 encoding; expcnt and lgkmcnt left at their
// maxima): all but this wave's N most recent vector-memory instructions have
// completed.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ uint32_t lut_plane(uint32_t fields) {
    return __builtin_amdgcn_perm(0u, kCodeLut, fields);
}

// Quad slot of quad t of row i.  With the row parity, the key (i >> 1) & 7
// makes the 16-byte slots of any 16 consecutive rows distinct modulo 16, so
// 16 lanes of a fragment read (16 rows, one quad each) or of a staging write
// (rows i, i + 1 or (row, half) pairs) touch all 64 banks once.  Of the keys
// measured, this one showed the fewest SQ_LDS_BANK_CONFLICT cycles.
__device__ __forceinline__ int swz(int i, int t) { return i * 8 + (t ^ ((i >> 1) & 7)); }

// TILES: the weights are in the tile layout of the decode GEMV (16-row
// tiles of 4352-byte segment units: four 1 KB code blocks, then 256 bytes of
// scales).  Its 2-bit fields are stored transposed, so the decoded planes of
// a code dword are natural-order weights and natural-order q is staged as it
// is (no byte transpose).  A code block holds the 16 bytes of (row, k-block
// kb) for a pair of groups side by side: the code dwords of k-blocks kb and
// 4 + kb of the even group, then those of the odd group.  Each thread loads
// such 16-byte items once per group pair and stages half of each per group.
// The scale block of a unit holds 16 bytes per row: the fp16 scales of its 8
// groups.
//
// AG: activation group size.  128, or (tile layout only, where k-step kk
// covers natural positions 32kk .. 32kk + 31 of the group) 64 or 32 for the
// smaller activation groups of page "Kernel experiments: recorded evidence",
// section C, Tests 8 and 9: each activation group's k-steps form their own
// INT32 chain; a weight group's terms float(dot) * xs are summed in k order,
// then scaled by its ws into acc.
//
// LDA (the 128 x 128 tile on eight waves, tile layout, 128-element groups):
// A goes straight from memory into LDS, one group ahead, into the buffer the
// previous group used, so it takes no registers and no staging writes, and
// the code and scale loads go two groups ahead; the kernel is held to four
// waves per SIMD (128 registers, a 12-byte spill) so that two workgroups
// share a CU.
template <int BM, int BN, bool PLANE_A, bool TILES, int AG = 128, int WM = 2>
__global__ __launch_bounds__(WM * 128, (WM == 4 && TILES && AG == 128) ? 4 : 1) void prefill_kernel(const int8_t* __restrict__ q,
                                                      const float* __restrict__ xs,
                                                      const uint8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales,
                                                      float* __restrict__ y, int m, int n, int k,
                                                      int groups) {
#pragma clang fp contract(off)
    constexpr int NTH = WM * 128;        // threads: WM x 2 waves
    constexpr int MT = BM / (32 * WM);   // 32-row tiles per wave
    constexpr int NT = BN / 64;          // 32-column tiles per wave
    constexpr int AQ = BM * 8 / NTH;     // A quads staged per thread
    constexpr int BI = BN * 2;           // B items (row, half) per group
    static_assert(MT >= 1 && AQ >= 1 && BI <= NTH && BM + BN <= NTH, "tile / wave split");
    static_assert(!TILES || BN * 4 >= NTH, "tile layout: every thread stages a B item");
    constexpr int S = 128 / AG;          // activation groups per weight group
    constexpr int KS = 4 / S;            // k-steps per activation group
    static_assert(AG == 128 || (TILES && (AG == 64 || AG == 32)), "smaller activation groups: tile layout only");
    // Scale blocks (tile layout, 128-element activation groups): xs and ws of
    // 8 groups are loaded at once, every lane of the load carrying one (row,
    // group) of xs or one (row, group pair) dword of ws, and staged once per
    // 8 groups.  Otherwise each group's scales are loaded and staged with it.
    constexpr bool SBLK = TILES && S == 1;
    // Code items per group pair (tile layout, 128-element activation groups;
    // with smaller groups the second register set would cost a wave per
    // SIMD at 64x128): one 16-byte load per (row, k-block) for both groups.
    // Otherwise one 8-byte load per (row, k-block) and group.
    constexpr bool BPAIR = SBLK;
    constexpr bool LDA = SBLK && WM == 4;
    constexpr int XB = SBLK ? BM * 8 / NTH : 1;   // xs items per thread per block
    constexpr int WB = SBLK ? BN * 4 / NTH : 1;   // ws dwords per thread per block
    static_assert(!SBLK || (XB * NTH == BM * 8 && WB * NTH == BN * 4), "scale block split");
    // The group loop is unrolled so that every register set, LDS buffer and
    // scale slot index is a constant: by 8 with scale blocks, else by 2.
    constexpr int UNR = SBLK ? 8 : 2;

    __shared__ uint4 As[2][BM * 8];
    __shared__ uint4 Bs[2][BN * 8];
    __shared__ float xsS[SBLK ? 1 : 2][S][SBLK ? 1 : BM];
    __shared__ float wsS[SBLK ? 1 : 2][SBLK ? 1 : BN];
    __shared__ float xsB[SBLK ? 8 : 1][SBLK ? BM : 1];       // [group % 8][row]
    __shared__ uint32_t wsB[SBLK ? 4 : 1][SBLK ? BN : 1];    // [(group % 8) / 2][row]: fp16 pair

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int bx = blockIdx.x;
    const int by = blockIdx.y;
    const int nb = bx * BN;
    const int mb = by * BM;
    const int k4 = k >> 2;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // Raw buffer resources over this workgroup's rows: out-of-range rows read
    // zero, and a group's offsets are the first group's plus a uniform step.
    const int mrows = min(BM, m - mb);
    const int nrows = min(BN, n - nb);
    const auto q_rs = make_rsrc(q + (size_t)mb * k, (uint32_t)(mrows * k));
    i32x4_t q_srs{};
    if constexpr (LDA) q_srs = make_srsrc(q + (size_t)mb * k, (uint32_t)(mrows * k));
    // Tile layout: BN is a multiple of 16, so the workgroup's rows are whole
    // tiles; their units are contiguous, (nb / 16) * S8 units from the start.
    const int s8 = (groups + 7) / 8;
    const int tiles_here = (nrows + 15) / 16;
    const auto c_rs = TILES ? make_rsrc(codes + (size_t)(nb / 16) * s8 * 4352, (uint32_t)(tiles_here * s8 * 4352))
                            : make_rsrc(codes + (size_t)nb * k4, (uint32_t)(nrows * k4));
    const auto x_rs = make_rsrc(xs + (size_t)mb * groups * S, (uint32_t)(mrows * groups * S * 4));
    const auto s_rs = make_rsrc(scales + (size_t)nb * groups, (uint32_t)(nrows * groups * 2));
    uint32_t a_off[AQ];
#pragma unroll
    for (int p = 0; p < AQ; ++p) {
        const int it = tid + NTH * p;
        a_off[p] = (uint32_t)((it >> 3) * k + (it & 7) * 16);
    }
    // LDA: slot it = tid + NTH p of an A buffer (row it >> 3, position it & 7)
    // holds quad (it & 7) ^ ((row >> 1) & 7) of the row (the swizzle of the
    // staging writes); wave w's p-th load fills slots (w + NTH/64 p) * 64 ..
    // + 63, lane l the l-th of them.
    uint32_t al_off[LDA ? AQ : 1];
    int wave_u = 0;
    if constexpr (LDA) {
#pragma unroll
        for (int p = 0; p < AQ; ++p) {
            const int it = tid + NTH * p;
            const int row = it >> 3;
            al_off[p] = (uint32_t)(row * k + 16 * ((it & 7) ^ ((row >> 1) & 7)));
        }
        wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    }
    const uint32_t b_off = tid < BI ? (uint32_t)((tid >> 1) * k4 + (tid & 1) * 16) : kBufferOOB;
    // Tile layout: items it = tid + NTH p (p < BN * 4 / NTH) take row it >> 2, k-block it & 3.
    constexpr int TI = TILES ? BN * 4 / NTH : 1;
    uint32_t tb_off[TI];
#pragma unroll
    for (int p = 0; p < TI; ++p) {
        const int it = tid + NTH * p;
        const int row = it >> 2, kbb = it & 3;
        tb_off[p] = (uint32_t)((row >> 4) * s8 * 4352 + 16 * ((row & 15) + 16 * kbb));
    }
    // Per-group scales: thread tid < BM loads xs of row tid, the last BN threads ws.
    const bool s_is_x = tid < BM;
    const bool s_is_w = tid >= NTH - BN;
    const uint32_t s_off = s_is_x ? (uint32_t)(tid * groups * S * 4)
                                  : (s_is_w ? (uint32_t)((tid - (NTH - BN)) * groups * 2) : kBufferOOB);
    // Smaller activation groups (S > 1): a group's xs are BM x S floats, one
    // per thread (item it = tid + NTH p is row it / S, activation group
    // it % S), so the loads carry a value in every lane instead of S loads per
    // thread with most lanes out of range.
    constexpr int XG = !SBLK && S > 1 ? (BM * S + NTH - 1) / NTH : 1;
    uint32_t xg_off[XG];
#pragma unroll
    for (int p = 0; p < XG; ++p) {
        const int it = tid + NTH * p;
        xg_off[p] = it < BM * S ? (uint32_t)(((it / S) * groups * S + it % S) * 4) : kBufferOOB;
    }
    // Scale blocks: xs item it = tid + NTH p is (row it >> 3, group it & 7 of
    // the block), ws item (row it >> 2, dword it & 3 of the row's 16 bytes).
    uint32_t xb_off[XB], wb_off[WB];
    int xb_g[XB];
#pragma unroll
    for (int p = 0; p < XB; ++p) {
        const int it = tid + NTH * p;
        xb_g[p] = it & 7;
        xb_off[p] = (uint32_t)(((it >> 3) * groups + (it & 7)) * 4);
    }
#pragma unroll
    for (int p = 0; p < WB; ++p) {
        const int it = tid + NTH * p;
        const int row = it >> 2;
        wb_off[p] = (uint32_t)((row >> 4) * s8 * 4352 + 4096 + 16 * (row & 15) + 4 * (it & 3));
    }

    // Global loads are issued PD groups ahead of their products: PD = 2 with
    // two register sets (group g's loads land in set g % 2), or PD = 1 with
    // one where two sets would not fit the registers of four waves per SIMD
    // (the 128 x 128 tile on eight waves with A through registers; with A
    // straight into LDS, one group ahead, its other loads go two ahead).
    // Code item pairs are loaded with the even group into set (g / 2) % 2
    // when two pairs can be live at once (PD = 2), else into one set.
    constexpr int PD = WM == 4 && !LDA ? 1 : 2;
    constexpr int TPS = PD == 2 ? 2 : 1;
    uint4 areg[PD][AQ];
    uint4 breg[PD];
    uint4 treg[BPAIR ? TPS : 1][BPAIR ? TI : 1];
    uint2 treg8[TILES && !BPAIR ? PD : 1][TILES && !BPAIR ? TI : 1];
    uint32_t sreg[SBLK ? 1 : PD];
    uint32_t xreg[SBLK ? 1 : PD][S > 1 ? XG : 1];
    uint32_t xbreg[XB], wbreg[WB];

    // Every thread issues the same loads whatever its role and whatever g
    // (threads without a scale role, and groups past the last, read past the
    // buffer's range, which returns zero): no branch around a load, so the
    // compiler's wait for one register set counts only that set's loads.
    // JC: g modulo the unroll (a constant); loads of group g land in set
    // g % PD.
    auto load_stage = [&](int g, auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int st = j % PD;
        if constexpr (!LDA) {
#pragma unroll
            for (int p = 0; p < AQ; ++p) areg[st][p] = buf_load16s(q_rs, a_off[p], (uint32_t)g * 128u);
        }
        if constexpr (BPAIR) {
            if constexpr (j % 2 == 0) {
                // Unit (tile, g / 8), block (g % 8) / 2: both groups of the pair.
                const uint32_t goff = (uint32_t)((g >> 3) * 4352 + ((g & 7) >> 1) * 1024);
#pragma unroll
                for (int p = 0; p < TI; ++p) treg[(j / 2) % TPS][p] = buf_load16s(c_rs, tb_off[p], goff);
            }
        } else if constexpr (TILES) {
            // Unit (tile, g / 8), block (g % 8) / 2, this group's half of the item.
            const uint32_t goff = (uint32_t)((g >> 3) * 4352 + ((g & 7) >> 1) * 1024 + (g & 1) * 8);
#pragma unroll
            for (int p = 0; p < TI; ++p) treg8[st][p] = buf_load8s(c_rs, tb_off[p], goff);
        } else {
            breg[st] = buf_load16s(c_rs, b_off, (uint32_t)g * 32u);
        }
        if constexpr (SBLK) {
            if constexpr (j % 8 == 0) {
                // Groups g .. g + 7: xs of the workgroup's rows and the unit's scale block.
#pragma unroll
                for (int p = 0; p < XB; ++p)
                    xbreg[p] = buf_load4(x_rs, g + xb_g[p] < groups ? xb_off[p] + (uint32_t)g * 4u : kBufferOOB);
#pragma unroll
                for (int p = 0; p < WB; ++p) wbreg[p] = buf_load4(c_rs, wb_off[p] + (uint32_t)(g >> 3) * 4352u);
            }
        } else {
            if constexpr (S > 1) {
#pragma unroll
                for (int p = 0; p < XG; ++p)
                    xreg[st][p] = buf_load4(x_rs, g < groups ? xg_off[p] + (uint32_t)(g * S) * 4u : kBufferOOB);
            } else {
                xreg[st][0] = buf_load4(x_rs, s_is_x && g < groups ? s_off + (uint32_t)g * 4u : kBufferOOB);
            }
            if constexpr (TILES)
                // The dword holding the scales of groups g & ~1 and g | 1 (a
                // 16-bit load would be zero-extended right after it is issued,
                // which waits for it); store_stage takes half g % 2.
                sreg[st] = buf_load4(c_rs, s_is_w && g < groups
                                               ? (uint32_t)((((tid - (NTH - BN)) >> 4) * s8 + (g >> 3)) * 4352 + 4096 +
                                                            16 * ((tid - (NTH - BN)) & 15) + 4 * ((g & 7) >> 1))
                                               : kBufferOOB);
            else
                sreg[st] = buf_load2(s_rs, s_is_w && g < groups ? s_off + (uint32_t)g * 2u : kBufferOOB);
        }
    };
    // LDA: group g's A into LDS buffer JC % 2 (all waves are past their
    // reads of it: the previous group's barrier).
    auto load_a = [&](int g, auto jc) {
        constexpr int buf = decltype(jc)::value % 2;
#pragma unroll
        for (int p = 0; p < AQ; ++p)
            buf_load16_lds(q_srs, al_off[p], __builtin_amdgcn_readfirstlane((uint32_t)g * 128u),
                           __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
                               (__attribute__((address_space(3))) uint4*)(&As[buf][(wave_u + (NTH / 64) * p) * 64]))));
    };
    // Vector-memory instructions load_stage issues under LDA for group JC
    // (modulo the unroll): code items on even groups, the scale block every 8.
    auto rest_loads = [](auto jc) constexpr {
        constexpr int j = decltype(jc)::value;
        return (j % 2 == 0 ? TI : 0) + (j % 8 == 0 ? XB + WB : 0);
    };
    // LDS slots this thread writes (fixed for the whole kernel).
    int a_slot[AQ];
#pragma unroll
    for (int p = 0; p < AQ; ++p) {
        const int it = tid + NTH * p;
        a_slot[p] = swz(it >> 3, it & 7);
    }
    int b_slot[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) b_slot[c] = swz(tid >> 1, 4 * (tid & 1) + c);
    // Stage group h (JC = h modulo the unroll) into LDS buffer h % 2.
    auto store_stage = [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int buf = j % 2;   // LDS buffer = parity of the group
        constexpr int st = j % PD;   // register set
        if constexpr (!LDA) {
#pragma unroll
            for (int p = 0; p < AQ; ++p)
                As[buf][a_slot[p]] = (PLANE_A || TILES) ? areg[st][p] : to_plane_order(areg[st][p]);
        }
        if constexpr (TILES) {
#pragma unroll
            for (int p = 0; p < TI; ++p) {
                const int it = tid + NTH * p;
                const int row = it >> 2, kbb = it & 3;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // Weights 16 (4h + kb) .. +15 of this group, natural planes.
                    uint32_t d;
                    if constexpr (BPAIR) {
                        const uint4 v = treg[(j / 2) % TPS][p];
                        d = buf ? (h ? v.w : v.z) : (h ? v.y : v.x);
                    } else {
                        d = h ? treg8[st][p].y : treg8[st][p].x;
                    }
                    Bs[buf][swz(row, 4 * h + kbb)] =
                        make_uint4(lut_plane(d & 0x03030303u), lut_plane((d >> 2) & 0x03030303u),
                                   lut_plane((d >> 4) & 0x03030303u), lut_plane((d >> 6) & 0x03030303u));
                }
            }
        } else if (tid < BI) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t d = word_of(breg[st], c);
                Bs[buf][b_slot[c]] =
                    make_uint4(lut_plane(d & 0x03030303u), lut_plane((d >> 2) & 0x03030303u),
                               lut_plane((d >> 4) & 0x03030303u), lut_plane((d >> 6) & 0x03030303u));
            }
        }
        if constexpr (SBLK) {
            if constexpr (j % 8 == 0) {
#pragma unroll
                for (int p = 0; p < XB; ++p) {
                    const int it = tid + NTH * p;
                    xsB[it & 7][it >> 3] = __uint_as_float(xbreg[p]);
                }
#pragma unroll
                for (int p = 0; p < WB; ++p) {
                    const int it = tid + NTH * p;
                    wsB[it & 3][it >> 2] = wbreg[p];
                }
            }
        } else {
            if constexpr (S > 1) {
#pragma unroll
                for (int p = 0; p < XG; ++p) {
                    const int it = tid + NTH * p;
                    if (it < BM * S) xsS[buf][it % S][it / S] = __uint_as_float(xreg[st][p]);
                }
            } else if (s_is_x) {
                xsS[buf][0][tid] = __uint_as_float(xreg[st][0]);
            }
            if (s_is_w) {
                const uint32_t h = TILES ? (buf ? sreg[st] >> 16 : sreg[st] & 0xFFFFu) : sreg[st];
                wsS[buf][tid - (NTH - BN)] = __half2float(__ushort_as_half((unsigned short)h));
            }
        }
    };
    // Fragment read slots per k-step (fixed for the whole kernel).
    int af_slot[4][MT], bf_slot[4][NT];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) af_slot[kk][mt] = swz(wm * (BM / WM) + mt * 32 + l32, 2 * kk + hi);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) bf_slot[kk][nt] = swz(wn * (BN / 2) + nt * 32 + l32, 2 * kk + hi);
    }

    float acc[MT][NT][16];
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    if constexpr (LDA) load_a(0, C0{});
    load_stage(0, C0{});
    if constexpr (PD == 2) load_stage(1, C1{});
    store_stage(C0{});
    if constexpr (LDA) wait_vm<rest_loads(C0{}) + (PD == 2 ? rest_loads(C1{}) : 0)>();
    __syncthreads();

    // One group g (JC = g modulo the unroll): its products and rescale from
    // LDS buffer g % 2 (a constant, so every LDS address is a register plus an
    // immediate), while group g + PD is loaded and group g + 1 (loaded PD - 1
    // groups earlier) is staged into the other buffer.
    auto group_step = [&](int g, auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int buf = j % 2;
        if constexpr (LDA) {
            // Unconditional: past the last group the offsets are out of range
            // and the buffer is not read again.  (Under a branch the compiler
            // waited on the previous group's loads before the first fragment
            // read.)
            load_a(g + 1, std::integral_constant<int, (j + 1) % UNR>{});
            __builtin_amdgcn_sched_barrier(0);
        }
        load_stage(g + PD, std::integral_constant<int, (j + PD) % UNR>{});

        // Activation group t of this weight group: k-steps KS*t .. KS*t + KS - 1.
        // With S > 1 the group's terms float(dot_t) * xs_t are summed first
        // (gs), then scaled by ws once: 2S + 1 VALU per output, not 3S.
        float gs[S > 1 ? MT : 1][S > 1 ? NT : 1][16];
#pragma unroll
        for (int t = 0; t < S; ++t) {
        v16i D[MT][NT];
#pragma unroll
        for (int u = 0; u < KS; ++u) {
            const int kk = KS * t + u;
            v4i af[MT], bf[NT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint4 v = As[buf][af_slot[kk][mt]];
                af[mt] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const uint4 v = Bs[buf][bf_slot[kk][nt]];
                bf[nt] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if (u == 0)
                        D[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mt], bf[nt], v16i{}, 0, 0, 0);
                    else
                        D[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mt], bf[nt], D[mt][nt], 0, 0, 0);
                }
        }

        // Rescale: lane holds column l32 of each 32x32 tile and rows
        // 8*(r/4) + 4*hi + (r%4), r = 0..15.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int col = wn * (BN / 2) + nt * 32 + l32;
            float wsv = 0.0f;
            if constexpr (SBLK) {
                const uint32_t wp = wsB[(j % 8) >> 1][col];
                wsv = __half2float(__ushort_as_half((unsigned short)(j % 2 ? wp >> 16 : wp & 0xFFFFu)));
            } else if constexpr (S == 1) {
                wsv = wsS[buf][col];
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int row = wm * (BM / WM) + mt * 32 + rb * 8 + hi * 4;
                    float4 xv;
                    if constexpr (SBLK)
                        xv = *reinterpret_cast<const float4*>(&xsB[j % 8][row]);
                    else
                        xv = *reinterpret_cast<const float4*>(&xsS[buf][t][row]);
                    const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = rb * 4 + e;
                        if constexpr (S == 1) {
                            acc[mt][nt][r] = __builtin_fmaf((float)D[mt][nt][r] * xa[e], wsv, acc[mt][nt][r]);
                        } else if (t == 0) {
                            gs[mt][nt][r] = (float)D[mt][nt][r] * xa[e];
                        } else {
                            gs[mt][nt][r] = __builtin_fmaf((float)D[mt][nt][r], xa[e], gs[mt][nt][r]);
                        }
                    }
                }
            }
        }
        // One activation group's chain at a time: the empty statement takes
        // the partial sums as operands and orders memory, so this group's
        // terms are added before the next group's fragments are read.  Without
        // it the compiler starts every group's products first and holds S sets
        // of D.
        if constexpr (S > 1) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(gs[mt][nt][r]) : : "memory");
        }
        }
        if constexpr (S > 1) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float wsv = wsS[buf][wn * (BN / 2) + nt * 32 + l32];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mt][nt][r] = __builtin_fmaf(gs[mt][nt][r], wsv, acc[mt][nt][r]);
            }
        }
        if (g + 1 < groups) {
            // The scale block has one LDS copy: before group g + 1 opens a new
            // block, every wave must be done with this group's rescale.
            if constexpr (SBLK && (j + 1) % 8 == 0) __syncthreads();
            store_stage(std::integral_constant<int, (j + 1) % UNR>{});
        }
        // LDA: group g + 1's A is in LDS once every vector-memory instruction
        // but the ones issued after it (group g + PD's loads) has completed.
        if constexpr (LDA) wait_vm<rest_loads(std::integral_constant<int, (j + PD) % UNR>{})>();
        __syncthreads();
    };
    for (int g = 0; g < groups; g += UNR) {
        group_step(g, C0{});
        if (g + 1 < groups) group_step(g + 1, C1{});
        if constexpr (UNR >= 4) {
            if (g + 2 < groups) group_step(g + 2, std::integral_constant<int, 2>{});
            if (g + 3 < groups) group_step(g + 3, std::integral_constant<int, 3>{});
        }
        if constexpr (UNR >= 8) {
            if (g + 4 < groups) group_step(g + 4, std::integral_constant<int, 4>{});
            if (g + 5 < groups) group_step(g + 5, std::integral_constant<int, 5>{});
            if (g + 6 < groups) group_step(g + 6, std::integral_constant<int, 6>{});
            if (g + 7 < groups) group_step(g + 7, std::integral_constant<int, 7>{});
        }
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int col = nb + wn * (BN / 2) + nt * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = mb + wm * (BM / WM) + mt * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
                if (row < m && col < n) y[(size_t)row * n + col] = acc[mt][nt][r];
            }
        }
}

namespace {

template <int BM, int BN, bool PLANE_A, bool TILES, int AG = 128, int WM = 2>
hipError_t launch_tile(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m, int64_t n,
                       int64_t k, float* y, hipStream_t stream) {
    const uint16_t* scales = TILES ? nullptr : reinterpret_cast<const uint16_t*>(planes + n * (k / 4));
    const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
    clear_stale_error();
    hipLaunchKernelGGL((prefill_kernel<BM, BN, PLANE_A, TILES, AG, WM>), grid, dim3(WM * 128), 0, stream, q, xs, planes,
                       scales, y, (int)m, (int)n, (int)k, (int)(k / 128));
    return hipGetLastError();
}

template <bool PLANE_A, bool TILES, int AG = 128>
hipError_t launch_any_tile(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m, int64_t n,
                           int64_t k, float* y, int tile, hipStream_t stream) {
    switch (tile) {
        case 1: return launch_tile<128, 128, PLANE_A, TILES, AG>(q, xs, planes, m, n, k, y, stream);
        case 2: return launch_tile<64, 128, PLANE_A, TILES, AG>(q, xs, planes, m, n, k, y, stream);
        case 3: return launch_tile<64, 64, PLANE_A, TILES, AG>(q, xs, planes, m, n, k, y, stream);
        case 4: return launch_tile<128, 64, PLANE_A, TILES, AG>(q, xs, planes, m, n, k, y, stream);
        case 5: return launch_tile<128, 128, PLANE_A, TILES, AG, 4>(q, xs, planes, m, n, k, y, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Tile choice.  A tile's workgroups run in rounds of as many as the chip
// holds at once (256 CUs; per CU four 64x64, three 64x128 or two 128x128
// workgroups on eight waves), each workgroup one chain over all k groups.
// Below 512 workgroups of 64x128 the 64x64 tile, whose grid fills more of
// the chip.  From there, for the tile layout with 128-element groups, the
// 64x128 tile or the 128x128 tile on eight waves (A straight into LDS), by a
// cost counted in rounds (round_cost): a full round of 128x128 workgroups
// takes about 1.1 times one of 64x128 at k = 5120, and a partial round
// costs more the fewer full rounds run before it, since the workgroups of
// the first rounds start together and finish together.  Measured on one
// box (µs, 64x128 against 128x128): FFN up m = 256 / 512 / 1024 / 2048,
// 52.3 / 88.1 / 156.4 / 303.2 against 54.6 / 89.4 / 145.1 / 266.8; gate
// (n = 6144) m = 1024 / 2048, 57.8 / 110.7 against 56.1 / 97.4; n = 16384,
// m = 512 / 1024, 78.0 / 144.9 against 64.7 / 124.1; n = 8192, m = 1024,
// 77.3 against 65.5.  The rule picks the faster tile at each of these but
// FFN up m = 512 (1.5% apart).  The other weight layouts keep
// 128x128 from 2048 workgroups of 64x128 on.  Activation groups of 64 or 32
// stay on 64x128: there the 128x128 tile on eight waves needs 146-148
// registers, one workgroup per CU.  The 128x128 tile on four waves needs
// more than 256 registers per lane (one wave per SIMD); it stays available
// through the tuning entry points.
constexpr int64_t kPrefillCUs = 256;

// Time of `rounds` rounds of workgroups in units of one full round.
static double round_cost(double rounds) {
    const double full = (double)(int64_t)rounds;
    const double part = rounds - full;
    if (part == 0.0) return full;
    if (full == 0.0) return 0.6 + 0.4 * part;
    if (full == 1.0) return full + 0.35 + 0.45 * part;
    return full + 0.05 + 0.65 * part;
}

static int default_prefill_tile(int64_t m, int64_t n, bool tile_layout, int agroup = 128) {
    const int64_t wgs2 = ((n + 127) / 128) * ((m + 63) / 64);
    if (wgs2 < 512) return 3;
    if (agroup != 128) return 2;
    if (!tile_layout) return wgs2 >= 2048 ? 5 : 2;
    const int64_t wgs5 = ((n + 127) / 128) * ((m + 127) / 128);
    const double t2 = round_cost((double)wgs2 / (3 * kPrefillCUs));
    const double t5 = 1.1 * round_cost((double)wgs5 / (2 * kPrefillCUs));
    return t5 < t2 ? 5 : 2;
}

hipError_t launch_prefill(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m,
                          int64_t n, int64_t k, float* y, int tile, bool plane_a, hipStream_t stream) {
    if (tile == 0) tile = default_prefill_tile(m, n, false);
    return plane_a ? launch_any_tile<true, false>(q, xs, planes, m, n, k, y, tile, stream)
                   : launch_any_tile<false, false>(q, xs, planes, m, n, k, y, tile, stream);
}

hipError_t launch_prefill_tiles(const int8_t* q, const float* xs, const uint8_t* tiles, int64_t m, int64_t n,
                                int64_t k, float* y, int tile, hipStream_t stream) {
    if (tile == 0) tile = default_prefill_tile(m, n, true);
    return launch_any_tile<false, true>(q, xs, tiles, m, n, k, y, tile, stream);
}

hipError_t launch_prefill_tiles_g(const int8_t* q, const float* xs, const uint8_t* tiles, int64_t m, int64_t n,
                                  int64_t k, float* y, int tile, int agroup, hipStream_t stream) {
    if (tile == 0) tile = default_prefill_tile(m, n, true, agroup);
    switch (agroup) {
        case 128: return launch_any_tile<false, true>(q, xs, tiles, m, n, k, y, tile, stream);
        case 64: return launch_any_tile<false, true, 64>(q, xs, tiles, m, n, k, y, tile, stream);
        case 32: return launch_any_tile<false, true, 32>(q, xs, tiles, m, n, k, y, tile, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pq2
