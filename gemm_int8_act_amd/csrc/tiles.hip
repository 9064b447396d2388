// tiles.hip -- tile-major weight layout for the decode GEMV, and the
// matrix-core small-m engine that reads it.
//
// Why a second layout (page "Kernel experiments: recorded evidence",
// section H, Tests 24 and 25: storing the pieces a warp loads next to each
// other lifted copy-only code reads to the streaming limit, and the
// tile-major integer projection kept the output bits): the INT8 matrix
// core's operand layout on gfx950 gives each lane 16 bytes of one weight row
// and one 16-weight k block, so with row-major codes one load instruction
// can cover at most 64 bytes of a row.  Here every load instruction of a
// wave reads one contiguous kilobyte.
//
// Layout (sizes in bytes; T = ceil(n/16) tiles of 16 rows, G = k/128
// groups, S8 = ceil(G/8) segments of 8 groups): T x S8 segment units of
// 4352 bytes, unit (t, sb) at (t*S8 + sb)*4352, each
//   four code blocks b = 0..3 of 1024 (groups 8sb + 2b and 8sb + 2b + 1):
//               lane l = j + 16*kb (j = row within the tile, kb = 0..3) owns
//               bytes 1024*b + 16*l .. +15; its dword u = 0..3 holds the 16
//               weights k0 .. k0+15 of row 16t+j, k0 = 128*(8sb + 2b + u/2)
//               + 64*(u%2) + 16*kb, and bits 2s..2s+1 of its byte v hold the
//               code of weight k0 + 4s + v.  (The prepared planes keep weight
//               4v + s there: inside each dword the 2-bit fields are
//               4x4-transposed, so bit plane s of a dword is the
//               natural-order activation dword s.)
//   then 256 bytes of scales: row j at 4096 + 16*j, the eight fp16 scales of
//               groups 8sb .. 8sb+7, next to the codes they scale (the wave
//               reads them from the same DRAM pages).
//   Rows >= n and groups >= G are padding: code 1 (weight 0), scale 0.
// When G % 8 == 0 (every shape measured here) and n % 16 == 0 the size
// equals the prepared planes', n*k/128*34.
//
// Engine (the summation order of small_m.hip):
//  * A workgroup owns one 16-row tile; its waves split k into consecutive
//    segments of 8 groups over at most 16 waves (by default), which is the
//    other small-m engines' split wherever k <= 8192, so the bits are theirs
//    there.
//  * Per group one wave issues v_mfma_i32_16x16x64_i8 twice with B = the two
//    code dwords' bit planes (codes 0..3, natural order) and A = the
//    activations of up to four columns; D starts from -sum(q) of each group
//    and column, so the accumulated D is the exact dot of the codes minus 1
//    with no decode of the -1 offset.
//  * The wave stages its segment's activation blocks in a private LDS region
//    (one load per column for the whole segment, no workgroup barrier) and
//    reads the A operand from there; the fp32 terms
//    fma((float)dot * xs, ws, acc) are accumulated per group class over the
//    wave's segments, the classes added as ((A0+A4)+(A1+A5))+((A2+A6)+(A3+A7)),
//    then the waves in index order.
#include "pq2_internal.h"
#include "small_m_common.h"

#include <hip/hip_fp16.h>

namespace pq2 {

namespace {

constexpr int kTileRows = 16;
constexpr int kCodeBlock = 1024;   // one (tile, group pair) code block
constexpr int kSegUnit = 4 * kCodeBlock + 256;  // one (tile, 8 groups) unit: codes then scales
constexpr int kTilesMaxColumns = 8;

struct TileGeometry {
    int64_t tiles, s8, total;
};

TileGeometry geometry(int64_t n, int64_t k) {
    TileGeometry t;
    t.tiles = (n + kTileRows - 1) / kTileRows;
    t.s8 = (k / 128 + 7) / 8;
    t.total = t.tiles * t.s8 * kSegUnit;
    return t;
}

// out byte v, field s = in byte s, field v (4x4 transpose of 2-bit fields).
__device__ uint32_t transpose_fields(uint32_t d) {
    uint32_t out = 0;
    for (int v = 0; v < 4; ++v)
        for (int s = 0; s < 4; ++s) out |= ((d >> (8 * s + 2 * v)) & 3u) << (8 * v + 2 * s);
    return out;
}

// One thread per 16-byte lane chunk of a code block: chunk c = (unit, b, lane).
__global__ void prepare_tile_codes_kernel(const uint8_t* __restrict__ raw, int64_t stride, int64_t n, int groups,
                                          int s8, int64_t chunks, uint8_t* __restrict__ out) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= chunks) return;
    const int lane = (int)(c & 63);
    const int b = (int)((c >> 6) & 3);
    const int64_t unit = c >> 8;  // t * S8 + sb
    const int sb = (int)(unit % s8);
    const int64_t row = (unit / s8) * kTileRows + (lane & 15);
    const int kb = lane >> 4;
    uint32_t w[4];
    for (int u = 0; u < 4; ++u) {
        const int g = 8 * sb + 2 * b + (u >> 1);
        if (row < n && g < groups) {
            const uint8_t* src = raw + row * stride + (int64_t)g * 34 + 2 + 16 * (u & 1) + 4 * kb;
            const uint32_t d = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16) |
                               ((uint32_t)src[3] << 24);
            w[u] = transpose_fields(d);
        } else {
            w[u] = 0x55555555u;
        }
    }
    *reinterpret_cast<uint4*>(out + unit * kSegUnit + b * kCodeBlock + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
}

// One thread per (unit, row): the eight fp16 scales after the unit's codes.
__global__ void prepare_tile_scales_kernel(const uint8_t* __restrict__ raw, int64_t stride, int64_t n, int groups,
                                           int s8, int64_t chunks, uint8_t* __restrict__ out) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= chunks) return;
    const int j = (int)(c & 15);
    const int64_t unit = c >> 4;
    const int sb = (int)(unit % s8);
    const int64_t row = (unit / s8) * kTileRows + j;
    uint32_t h[8];
    for (int e = 0; e < 8; ++e) {
        const int g = 8 * sb + e;
        h[e] = 0;
        if (row < n && g < groups) {
            const uint8_t* src = raw + row * stride + (int64_t)g * 34;
            h[e] = (uint32_t)src[0] | ((uint32_t)src[1] << 8);
        }
    }
    *reinterpret_cast<uint4*>(out + unit * kSegUnit + 4 * kCodeBlock + 16 * j) =
        make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

__device__ __forceinline__ void keep_order() { __builtin_amdgcn_sched_barrier(0); }

// s_waitcnt vmcnt(0) (GFX9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15): this
// wave's vector memory operations, stores included, have completed.  The
// signal fences keep the compiler from moving memory operations across it.
__device__ __forceinline__ void wait_stores_complete() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// j mod mcount for j < 16 and mcount = 1..8 (mcount is uniform), without
// the generic integer division.
__device__ __forceinline__ int small_mod(int j, int mcount) {
    if (mcount == 4 || mcount == 8) return j & (mcount - 1);
    if (mcount == 3) return j - 3 * ((j * 11) >> 5);  // (j * 11) >> 5 == j / 3 for j < 16
    if (mcount == 2) return j & 1;
    if (mcount > 4) return j >= 2 * mcount ? j - 2 * mcount : (j >= mcount ? j - mcount : j);
    return 0;
}

// Per-wave LDS: the staged columns of CPW groups (each padded by 64 bytes:
// the columns of one A read fall in distinct banks), then 8 x 8 floats of xs
// and 8 x 8 ints of -sum(q) (group class x column, up to eight columns).
// With activation groups of ag < 128 elements the xs and -sum(q) tables hold
// 128/ag entries per class, and ag = 32 adds a zero block that the lanes
// outside a 32-element group read as their A operand.
__host__ __device__ constexpr int tiles_col_pitch(int cpw) { return 128 * cpw + 64; }
// Staged columns: MC, plus a spare column that takes the stores of lanes
// past the last column when a staging load spans more columns than remain
// (8 / CPW columns per load).
__host__ __device__ constexpr int tiles_cols_staged(int mc, int cpw) {
    return mc + (((mc + 8 / cpw - 1) / (8 / cpw)) * (8 / cpw) > mc ? 1 : 0);
}
// With 128-element activation groups the -sum(q) table holds 8 classes x 4
// columns x 4 copies (512 bytes: a lane's C operand is four copies of one
// column's value) instead of 8 x 8 ints.
__host__ __device__ constexpr int tiles_region_bytes(int mc, int cpw, int ag = 128) {
    return tiles_cols_staged(mc, cpw) * tiles_col_pitch(cpw) + 512 * (128 / ag) + (ag == 128 ? 256 : 0) +
           (ag == 32 ? 128 * cpw : 0);
}

__device__ __forceinline__ float half_of(const uint4& v, int c) {
    const uint32_t w = word_of(v, c >> 1);
    return __half2float(__ushort_as_half((unsigned short)((c & 1) ? (w >> 16) : (w & 0xFFFFu))));
}

// SRC: kSrcNatural reads q and xs; kSrcBf16 / kSrcF16 / kSrcF32 read x and
// quantise each staged group in the wave (the exact in-kernel quantiser, so
// the codes and scales are those of pq2_quantize_act_i8).
//
// MC: columns per pass, 1..4 or 8.  A row i holds column i mod mcount, so D
// row 4*kb + r is column 4*kb + r: with MC = 8 the lanes kb = 0 and 1 both
// hold outputs (columns 0..3 and 4..7), one decode of each code word feeding
// eight columns.
//
// AG: activation group size (128; 64 or 32 for the smaller activation groups
// of page "Kernel experiments: recorded evidence", section C, Tests 8 and 9).  Each activation group has its own D chain seeded
// with its own -sum(q); the weight group's terms (float)dot * xs_a are summed
// in k order, then scaled by ws into the class accumulator, fma(sum, ws, acc).
//
// SPLIT: the k slices of a tile are spread over `ks` workgroups (grid.x =
// tiles * ks, workgroup p taking slices p * nwaves .. p * nwaves + nwaves - 1,
// one segment each).  Each wave stores its slice's class sum to
// partials[slice][column][row] (write-through device-scope stores, waited
// for before the workgroup's barrier); the workgroup that draws the last
// ticket from the tile's counter (a device-scope vector atomic) adds the
// slices in index order, writes y and puts the counter back to zero.  No
// workgroup waits for another.  The sum is the one the single-workgroup
// kernel forms for the same slices (slice sums added in index order).
template <int MC, int CPW, int SRC, int AG = 128, bool SPLIT = false>
__global__ __launch_bounds__(1024) void small_m_tiles_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ xs, const void* __restrict__ x, int64_t x_stride,
    const uint8_t* __restrict__ tiles, float* __restrict__ y, int n, int k, int groups, int s8, int nseg,
    int per_wave, int mtotal, float* __restrict__ partials, uint32_t* __restrict__ counters, int ks) {
#pragma clang fp contract(off)
    constexpr bool FUSED = src_fused(SRC);
    constexpr int XL = src_xloads(SRC);
    typedef int v4i __attribute__((ext_vector_type(4)));
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int WPS = 8 / CPW;            // waves per k slice (each takes CPW group classes)
    constexpr int CHUNKS = 8 * CPW;         // 16-byte chunks of one column's activations per segment
    constexpr int COLS_PER_LOAD = 64 / CHUNKS;
    constexpr int QLOADS = (MC + COLS_PER_LOAD - 1) / COLS_PER_LOAD;
    constexpr int PITCH = tiles_col_pitch(CPW);
    constexpr int S = 128 / AG;             // activation groups per weight group
    constexpr int LPS = AG / 16;            // staging lanes per activation group
    constexpr int XSV = CPW * S * MC;       // xs values of one segment (AG < 128)
    constexpr int XSL = (XSV + 63) / 64;    // their loads per lane
    static_assert(AG == 128 || AG == 64 || AG == 32, "activation group");
    static_assert(MC <= 4 || (MC == 8 && AG == 128), "eight-column passes take 128-element activation groups");
    // COLK (2..4 columns, natural-order q or quantised in the kernel): A rows
    // 4c..4c+3 all carry column c, so the lanes of k block kb hold column kb
    // in every D row and one output each: the epilogue takes 3 VALU per group
    // whatever the column count, against 3 per group and column with rows =
    // columns.  A lane takes its column's xs from memory, or from the LDS
    // copy the in-kernel quantiser writes.
    constexpr bool COLK = AG == 128 && MC >= 2 && MC <= 4;
    constexpr int R = COLK ? 1 : (MC < 4 ? MC : 4);  // outputs per lane and class (D rows 4*kb + r)
    constexpr int KBU = COLK ? MC : (MC > 4 ? 2 : 1);  // lane groups kb holding outputs
    constexpr bool XS_VEC = !src_fused(SRC) && (AG < 128 || MC > 4);  // xs through LDS from vector loads
    static_assert(!SPLIT || (CPW == 8 && !src_fused(SRC) && AG == 128), "split k: natural q, one wave per slice");
    const int nwaves = blockDim.x >> 6;
    const int nslices = SPLIT ? (nseg + per_wave - 1) / per_wave : nwaves / WPS;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tile = SPLIT ? (int)blockIdx.x / ks : (int)blockIdx.x;
    const int slice = SPLIT ? ((int)blockIdx.x - tile * ks) * nwaves + wave : wave / WPS;
    const int c_lo = (wave % WPS) * CPW;  // first group class of this wave
    const int lane = threadIdx.x & 63;
    const int j = lane & 15;   // B column (row of the tile) and A row (activation column)
    const int kb = lane >> 4;  // k block of the 64-wide MFMA step
    const int m0 = blockIdx.y * MC;
    const int mcount = min(MC, mtotal - m0);
    const int seg_begin = slice * per_wave;
    const int seg_end = min(seg_begin + per_wave, nseg);

    const auto tile_rs = make_rsrc(tiles + (size_t)tile * s8 * kSegUnit, (uint32_t)(s8 * kSegUnit));
    const auto q_rs = make_rsrc(FUSED ? nullptr : q + (size_t)m0 * k, FUSED ? 0u : (uint32_t)(mcount * k));
    const i32x4_t xs_srs = make_srsrc(FUSED ? nullptr : xs + (size_t)m0 * groups, FUSED ? 0u : (uint32_t)(mcount * groups * 4));
    const auto xsc_rs = make_rsrc(COLK && !FUSED ? xs + (size_t)m0 * groups : nullptr,
                                  COLK && !FUSED ? (uint32_t)(mcount * groups * 4) : 0u);
    const auto xsa_rs = make_rsrc(XS_VEC ? xs + (size_t)m0 * groups * S : nullptr,
                                  XS_VEC ? (uint32_t)(mcount * groups * S * 4) : 0u);
    const auto x_rs = make_rsrc(
        FUSED ? static_cast<const unsigned char*>(x) + (size_t)m0 * x_stride * src_esize(SRC) : nullptr,
        FUSED ? (uint32_t)(((int64_t)(mcount - 1) * x_stride + k) * src_esize(SRC)) : 0u);
    // Staging roles: chunk ch of column (load t) * COLS_PER_LOAD + sub.
    const int ch = lane % CHUNKS;
    const int sub = lane / CHUNKS;

    // 1. One segment's loads: the activation chunks of the wave's classes,
    //    then the weight scales, then the code blocks in use order (loads
    //    complete in order, so the first group pair can start while the later
    //    blocks are in flight), then xs.  Groups past the end read zeros.
    // One segment's registers.  (Issuing the next segment's loads before a
    // segment's arithmetic, with two sets of these, measured slower at
    // K = 17408: the waves' tails grow.)
    struct Seg {
        uint4 qv[QLOADS];
        uint4 xraw[QLOADS][FUSED ? XL : 1];
        float xss[FUSED || XS_VEC || COLK ? 1 : MC][CPW];  // xs of the wave's groups, scalar loads (uniform)
        uint4 xlv[COLK && !FUSED ? 2 : 1];           // COLK: xs of this lane's column, vector loads
        uint32_t xsa[XS_VEC ? XSL : 1];              // xs through LDS (AG < 128 or MC > 4), vector loads
        uint4 wsv;
        uint4 cw[CPW / 2];
    };
    auto issue = [&](int s, Seg& g) {
        const uint32_t qoff = (uint32_t)(s * 1024 + 128 * c_lo + 16 * ch);  // element offset in the row
#pragma unroll
        for (int t = 0; t < QLOADS; ++t) {
            const int m = t * COLS_PER_LOAD + sub;
            const bool ok = m < mcount && (int)qoff < k;
            if constexpr (FUSED) {
                const uint32_t off = (uint32_t)((m * x_stride + qoff) * src_esize(SRC));
#pragma unroll
                for (int l = 0; l < XL; ++l) g.xraw[t][l] = buf_load16(x_rs, ok ? off + 16u * l : kBufferOOB);
            } else {
                g.qv[t] = buf_load16(q_rs, ok ? (uint32_t)(m * k) + qoff : kBufferOOB);
            }
        }
        const uint32_t unit_off = (uint32_t)(s * kSegUnit);
        g.wsv = buf_load16<kAuxNonTemporal>(tile_rs, unit_off + 4 * kCodeBlock + 16 * j);
        keep_order();
#pragma unroll
        for (int b = 0; b < CPW / 2; ++b)
            g.cw[b] = buf_load16<kAuxNonTemporal>(tile_rs, unit_off + (c_lo / 2 + b) * kCodeBlock + 16 * lane);
        keep_order();
        if constexpr (XS_VEC) {
            // Value i of the segment: column i / (CPW*S), activation group
            // (8s + c_lo)*S + i % (CPW*S).
#pragma unroll
            for (int t = 0; t < XSL; ++t) {
                const int i = t * 64 + lane;
                const int col = i / (CPW * S);
                const int a = (8 * s + c_lo) * S + i % (CPW * S);
                const bool ok = i < XSV && col < mcount && a < groups * S;
                g.xsa[t] = buf_load4(xsa_rs, ok ? (uint32_t)((col * groups * S + a) * 4) : kBufferOOB);
            }
        } else if constexpr (COLK && !FUSED) {
            // The eight xs of this lane's column (lanes past the last column
            // read the last one; past the last group the values are never
            // used: those groups' dots are zero).
            const uint32_t xoff = (uint32_t)((min(kb, mcount - 1) * groups + 8 * s + c_lo) * 4);
            g.xlv[0] = buf_load16(xsc_rs, xoff);
            g.xlv[1] = buf_load16(xsc_rs, xoff + 16u);
        } else if constexpr (!FUSED) {
            // xs of the wave's groups: uniform offsets, so the scalar unit
            // fetches them, outside the vector memory queue.  Columns past
            // the last re-read it (their D rows are never used).  A segment
            // that runs past the last group reads dword by dword, so the
            // missing groups read zero and the others their values.
            const int g0 = 8 * s + c_lo;
#pragma unroll
            for (int r = 0; r < MC; ++r) {
                const int off = (min(r, mcount - 1) * groups + g0) * 4;
                if (g0 + CPW <= groups) {
                    sbuf_load_f32<CPW>(xs_srs, off, g.xss[r]);
                } else {
#pragma unroll
                    for (int c = 0; c < CPW; ++c) sbuf_load_f32<1>(xs_srs, off + 4 * c, &g.xss[r][c]);
                }
            }
        }
    };
    // Private region: the staged columns (CPW groups each), then per class c
    // of the wave 8 floats xs[c][m] (COLK: xs[m][c]) and 8 ints -sum(q)[c][m]
    // (COLK: four copies of each).
    unsigned char* region = smem + (size_t)wave * tiles_region_bytes(MC, CPW, AG);
    float* red = reinterpret_cast<float*>(smem + (size_t)nwaves * tiles_region_bytes(MC, CPW, AG));
    constexpr int NCOLS = tiles_cols_staged(MC, CPW);
    float* xs_lds = reinterpret_cast<float*>(region + NCOLS * PITCH);
    int* nsq_lds = reinterpret_cast<int*>(region + NCOLS * PITCH + 256 * S);
    const unsigned char* zero_lds = region + NCOLS * PITCH + 512 * S;  // AG == 32 only
    // A row i reads column i mod mcount: rows >= mcount repeat real columns,
    // so one read touches at most 4 x 16 distinct banks, and the D rows they
    // produce are never used.
    const unsigned char* a_base = region + small_mod(COLK ? j >> 2 : j, mcount) * PITCH + 16 * kb;
    // COLK: this lane's column and its -sum(q) copies (4 per class and column).
    const int* nsq_colk = nsq_lds + 4 * small_mod(kb, mcount);
#pragma unroll
    for (int i = 0; i < (AG == 128 ? 2 : S); ++i) nsq_lds[lane + 64 * i] = 0;
    if constexpr (AG == 32) {
        if (lane < 8 * CPW) *reinterpret_cast<uint4*>(const_cast<unsigned char*>(zero_lds) + 16 * lane) = make_uint4(0, 0, 0, 0);
    }
    // With 32-element activation groups lanes kb = 2s, 2s + 1 hold group s of
    // each 64-wide half; the others read zeros for that group's product.
    const unsigned char* a_grp[2] = {AG == 32 && (kb >> 1) != 0 ? zero_lds : a_base,
                                     AG == 32 && (kb >> 1) != 1 ? zero_lds : a_base};

    float acc[CPW][R];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[c][r] = 0.0f;
    const int col4 = COLK ? kb : (MC > 4 ? 4 * (kb & 1) : 0);  // first column of this lane's D rows

    // Every wave has at least one segment (slice * per_wave < nseg), so the
    // loop has no zero-trip test and the kernel arguments load in one go.
    // (With SPLIT the last workgroup of a tile may hold waves past the last
    // slice; they skip the loop and store nothing.)
    auto body = [&](int s, Seg& g) {

        // 2. Stage the activations, xs and each group's -sum(q) (dot4 against
        //    ones over the lane's 16 bytes, then the 8 lanes of the group).
        //    Lanes past the last column write their (zero) chunk to the spare column.
#pragma unroll
        for (int t = 0; t < QLOADS; ++t) {
            const int m = t * COLS_PER_LOAD + sub;
            uint4 v;
            int sq;
            if constexpr (FUSED) {
                float xf[16];
                x_to_float16<SRC>(g.xraw[t], xf);
                float scale;
                v = quantize_lane16<false, LPS>(xf, sq, scale);  // the LPS lanes of the group agree
                if ((lane & (LPS - 1)) == 0 && m < MC) {
                    if constexpr (COLK) xs_lds[m * 8 + c_lo + (ch >> 3)] = scale;
                    else xs_lds[((c_lo + (ch >> 3)) * S + (ch & 7) / LPS) * 8 + m] = scale;
                }
            } else {
                v = g.qv[t];
                sq = dot4(v.x, 0x01010101u, 0);
                sq = dot4(v.y, 0x01010101u, sq);
                sq = dot4(v.z, 0x01010101u, sq);
                sq = dot4(v.w, 0x01010101u, sq);
                if constexpr (AG == 128) {
                    sq = sum8_i(sq);
                } else {
                    sq += dpp_i<kDppXor1>(sq);
                    if constexpr (AG == 64) sq += dpp_i<kDppXor2>(sq);
                }
            }
            *reinterpret_cast<uint4*>(region + (m < MC ? m : MC) * PITCH + 16 * ch) = v;
            if constexpr (COLK) {
                if ((lane & 7) == 0 && m < MC)
                    *reinterpret_cast<int4*>(nsq_lds + ((c_lo + (ch >> 3)) * 4 + m) * 4) = make_int4(-sq, -sq, -sq, -sq);
            } else if ((lane & (LPS - 1)) == 0 && m < MC) {
                nsq_lds[((c_lo + (ch >> 3)) * S + (ch & 7) / LPS) * 8 + m] = -sq;
            }
        }
        if constexpr (XS_VEC) {
#pragma unroll
            for (int t = 0; t < XSL; ++t) {
                const int i = t * 64 + lane;
                if (i < XSV) xs_lds[(c_lo * S + i % (CPW * S)) * 8 + i / (CPW * S)] = __uint_as_float(g.xsa[t]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // COLK: the activation scales of this lane's column (loaded for
        // column min(kb, mcount - 1), or read from the quantiser's LDS copy;
        // lanes past the last column are never stored).
        float xl[COLK ? CPW : 1];
        if constexpr (COLK) {
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                if constexpr (FUSED) xl[c] = xs_lds[small_mod(kb, mcount) * 8 + c_lo + c];
                else xl[c] = __uint_as_float(word_of(g.xlv[c >> 2], c & 3));
            }
        }

        // 3. Group dots on the matrix cores, two groups at a time: D starts
        //    at -sum(q) of its column (the code offset), then adds the two
        //    64-wide halves of codes 0..3 times q.
#pragma unroll
        for (int c0 = 0; c0 < CPW; c0 += 2) {
          if constexpr (AG < 128) {
            // One chain per activation group, seeded with its -sum(q); its
            // term uses its own xs.  The groups' terms are added in k order.
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int c = c0 + p;
                v4i Bh[2], Dt[S];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t d = word_of(g.cw[c >> 1], 2 * (c & 1) + h);
                    Bh[h] = v4i{(int)(d & 0x03030303u), (int)((d >> 2) & 0x03030303u),
                                (int)((d >> 4) & 0x03030303u), (int)((d >> 6) & 0x03030303u)};
                }
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    const int4 nsq = *reinterpret_cast<const int4*>(nsq_lds + ((c_lo + c) * S + t) * 8);
                    Dt[t] = v4i{nsq.x, nsq.y, nsq.z, nsq.w};
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int u = 0; u < S / 2; ++u) {  // activation group t = h * S/2 + u of this weight group
                        const uint4 a = *reinterpret_cast<const uint4*>((S == 2 ? a_base : a_grp[u]) + 128 * c + 64 * h);
                        const int t = h * (S / 2) + u;
                        Dt[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w},
                                                                      Bh[h], Dt[t], 0, 0, 0);
                    }
                }
                // The weight group's terms float(dot_t) * xs_t in k order, then
                // one scale by ws into the class accumulator.
                const float wsf = half_of(g.wsv, c_lo + c);
                float gsum[R];
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    const float4 xg = *reinterpret_cast<const float4*>(xs_lds + ((c_lo + c) * S + t) * 8);
                    const float xv[4] = {xg.x, xg.y, xg.z, xg.w};
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        gsum[r] = t == 0 ? (float)Dt[t][r] * xv[r] : __builtin_fmaf((float)Dt[t][r], xv[r], gsum[r]);
                }
#pragma unroll
                for (int r = 0; r < R; ++r) acc[c][r] = __builtin_fmaf(gsum[r], wsf, acc[c][r]);
            }
          } else {
            v4i D[2];
            v4i A[2][2];
            v4i B[2][2];
            float4 xsg[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int c = c0 + p;  // class c_lo + c
                const uint4 a0 = *reinterpret_cast<const uint4*>(a_base + 128 * c);
                const uint4 a1 = *reinterpret_cast<const uint4*>(a_base + 128 * c + 64);
                A[p][0] = v4i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w};
                A[p][1] = v4i{(int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                const int4 nsq = COLK ? *reinterpret_cast<const int4*>(nsq_colk + (c_lo + c) * 16)
                                      : *reinterpret_cast<const int4*>(nsq_lds + (c_lo + c) * 8 + col4);
                D[p] = v4i{nsq.x, nsq.y, nsq.z, nsq.w};
                if constexpr ((FUSED || XS_VEC) && !COLK) xsg[p] = *reinterpret_cast<const float4*>(xs_lds + (c_lo + c) * 8 + col4);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t d = word_of(g.cw[c >> 1], 2 * (c & 1) + h);
                    B[p][h] = v4i{(int)(d & 0x03030303u), (int)((d >> 2) & 0x03030303u),
                                  (int)((d >> 4) & 0x03030303u), (int)((d >> 6) & 0x03030303u)};
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int p = 0; p < 2; ++p) D[p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[p][h], B[p][h], D[p], 0, 0, 0);
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int c = c0 + p;
                const float wsf = half_of(g.wsv, c_lo + c);
                float xv[4];
                if constexpr (COLK) {
                    xv[0] = xl[c];
                } else if constexpr (FUSED || XS_VEC) {
                    xv[0] = xsg[p].x; xv[1] = xsg[p].y; xv[2] = xsg[p].z; xv[3] = xsg[p].w;
                } else {
#pragma unroll
                    for (int r = 0; r < R; ++r) xv[r] = g.xss[r][c];
                }
#pragma unroll
                for (int r = 0; r < R; ++r) acc[c][r] = __builtin_fmaf((float)D[p][r] * xv[r], wsf, acc[c][r]);
            }
          }
        }
        // The next segment rewrites the region: every lane's reads of this one
        // are done (LDS operations of one wave complete in order).
        __builtin_amdgcn_wave_barrier();
    };
    Seg g;
    int s = seg_begin;
    if (!SPLIT || seg_begin < seg_end) do {
        issue(s, g);
        body(s, g);
    } while (++s < seg_end);

    // 4. Class sums ((A0+A4)+(A1+A5))+((A2+A6)+(A3+A7)) per slice, then the
    //    slices in index order.  D row 4*kb + r is column 4*kb + r, so the
    //    columns live in the lanes with kb = 0.  A wave that holds all eight
    //    classes adds them in registers.
    if constexpr (CPW == 8) {
        float part[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            part[r] = ((acc[0][r] + acc[4][r]) + (acc[1][r] + acc[5][r])) +
                      ((acc[2][r] + acc[6][r]) + (acc[3][r] + acc[7][r]));
        const int row = tile * kTileRows + j;
        if constexpr (SPLIT) {
            const size_t plane = (size_t)mtotal * n;  // one slice's [column][row] sums
            // Partial sums, tickets and their reads are device-scope atomics
            // (relaxed: write-through stores and loads that bypass the
            // per-XCD caches), so no cache write-back or invalidation is
            // needed.  Order: every wave waits for its stores to complete
            // before the barrier, thread 0 takes the ticket after it, and the
            // last workgroup reads the sums after its ticket returns.
            if (seg_begin < seg_end && kb < KBU && row < n) {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (col4 + r < mcount)
                        __hip_atomic_store(partials + (size_t)slice * plane + (size_t)(m0 + col4 + r) * n + row, part[r],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            wait_stores_complete();
            __syncthreads();
            int* last = reinterpret_cast<int*>(red);
            if (threadIdx.x == 0) {
                const int ntiles = (int)gridDim.x / ks;
                uint32_t* ctr = counters + (size_t)blockIdx.y * ntiles + tile;
                const uint32_t before = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int is_last = before == (uint32_t)(ks - 1);
                if (is_last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                *last = is_last;
            }
            __syncthreads();
            if (*last == 0) return;
            // The slices in index order (loads in batches of eight, slots past
            // the last slice re-read it and are not added).
#pragma unroll
            for (int o0 = 0; o0 < MC * kTileRows; o0 += 64) {
                const int o = o0 + lane;
                const int col = o >> 4;
                if (wave == 0 && o < MC * kTileRows && col < mcount && row < n) {
                    const float* p = partials + (size_t)(m0 + col) * n + row;
                    float sum = 0.0f;
                    for (int b = 0; b < nslices; b += 8) {
                        float v[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            v[i] = __hip_atomic_load(p + (size_t)min(b + i, nslices - 1) * plane, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            if (b + i < nslices) sum = b + i == 0 ? v[i] : sum + v[i];
                    }
                    y[(size_t)(m0 + col) * n + row] = sum;
                }
            }
            return;
        }
        if (nwaves == 1) {
            if (kb < KBU && row < n) {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (col4 + r < mcount) y[(size_t)(m0 + col4 + r) * n + row] = part[r];
            }
            return;
        }
        if (kb < KBU) {
#pragma unroll
            for (int r = 0; r < R; ++r) red[(wave * MC + col4 + r) * kTileRows + j] = part[r];
        }
        __syncthreads();
        // Wave 0 adds the slices (up to 16) in index order.  Each batch of
        // eight reads goes out before its adds; slots past the last slice
        // re-read the last one and are not added.
#pragma unroll
        for (int o0 = 0; o0 < MC * kTileRows; o0 += 64) {
            const int o = o0 + lane;
            if (wave == 0 && o < MC * kTileRows) {
                const int col = o >> 4;
                float sum = 0.0f;
                for (int b = 0; b < nwaves; b += 8) {
                    float v[8];
#pragma unroll
                    for (int w = 0; w < 8; ++w) v[w] = red[(min(b + w, nwaves - 1) * MC + col) * kTileRows + j];
#pragma unroll
                    for (int w = 0; w < 8; ++w)
                        if (b + w < nwaves) sum = b + w == 0 ? v[w] : sum + v[w];
                }
                if (col < mcount && row < n) y[(size_t)(m0 + col) * n + row] = sum;
            }
        }
        return;
    }
    if (kb < KBU) {
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int r = 0; r < R; ++r) red[((slice * 8 + c_lo + c) * MC + col4 + r) * kTileRows + j] = acc[c][r];
    }
    __syncthreads();
#pragma unroll
    for (int o0 = 0; o0 < MC * kTileRows; o0 += 64) {
        const int o = o0 + lane;
        if (wave == 0 && o < MC * kTileRows) {
            const int col = o >> 4;
            constexpr int C = MC * kTileRows;  // stride between classes
            float t[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const float* a = red + ((size_t)min(w, nslices - 1) * 8 * MC + col) * kTileRows + j;
                t[w] = ((a[0] + a[4 * C]) + (a[1 * C] + a[5 * C])) + ((a[2 * C] + a[6 * C]) + (a[3 * C] + a[7 * C]));
            }
            float sum = t[0];
#pragma unroll
            for (int w = 1; w < 8; ++w)
                if (w < nslices) sum += t[w];
            const int row = tile * kTileRows + j;
            if (col < mcount && row < n) y[(size_t)(m0 + col) * n + row] = sum;
        }
    }
}

struct TilesArgs {
    const int8_t* q;
    const float* xs;
    const void* x;
    int64_t x_stride;
    const uint8_t* tiles;
    int64_t m, n, k;
    float* y;
    hipStream_t stream;
};

template <int MC, int CPW, int SRC, int AG>
hipError_t launch_tiles_one(const TilesArgs& a, int slices, int nseg, int per_wave, int chunks) {
    const int64_t m = a.m, n = a.n, k = a.k;
    const TileGeometry t = geometry(n, k);
    const int waves = slices * (8 / CPW);
    const size_t lds = (size_t)waves * tiles_region_bytes(MC, CPW, AG) +
                       (size_t)(CPW == 8 ? waves : slices * 8) * MC * kTileRows * 4;
    const dim3 grid((unsigned)t.tiles, (unsigned)chunks);
    clear_stale_error();
    hipLaunchKernelGGL((small_m_tiles_kernel<MC, CPW, SRC, AG>), grid, dim3(64 * waves), lds, a.stream, a.q, a.xs, a.x,
                       a.x_stride, a.tiles, a.y, (int)n, (int)k, (int)(k / 128), (int)t.s8, nseg, per_wave, (int)m,
                       nullptr, nullptr, 1);
    return hipGetLastError();
}

// Split k: `ks` workgroups of `waves` waves per tile, one segment per wave.
template <int MC>
hipError_t launch_tiles_splitk_one(const TilesArgs& a, float* partials, uint32_t* counters, int ks, int waves,
                                   int nseg, int chunks) {
    const TileGeometry t = geometry(a.n, a.k);
    const size_t lds = (size_t)waves * tiles_region_bytes(MC, 8) + (size_t)waves * MC * kTileRows * 4;
    const dim3 grid((unsigned)(t.tiles * ks), (unsigned)chunks);
    clear_stale_error();
    hipLaunchKernelGGL((small_m_tiles_kernel<MC, 8, kSrcNatural, 128, true>), grid, dim3(64 * waves), lds, a.stream,
                       a.q, a.xs, nullptr, (int64_t)0, a.tiles, a.y, (int)a.n, (int)a.k, (int)(a.k / 128), (int)t.s8,
                       nseg, 1, (int)a.m, partials, counters, ks);
    return hipGetLastError();
}

template <int CPW, int SRC, int AG>
hipError_t launch_tiles_mc(int mc, const TilesArgs& a, int slices, int nseg, int per_wave, int chunks) {
    switch (mc) {
        case 1: return launch_tiles_one<1, CPW, SRC, AG>(a, slices, nseg, per_wave, chunks);
        case 2: return launch_tiles_one<2, CPW, SRC, AG>(a, slices, nseg, per_wave, chunks);
        case 3: return launch_tiles_one<3, CPW, SRC, AG>(a, slices, nseg, per_wave, chunks);
        case 4: return launch_tiles_one<4, CPW, SRC, AG>(a, slices, nseg, per_wave, chunks);
        case 8:
            if constexpr (AG == 128) return launch_tiles_one<8, CPW, SRC, AG>(a, slices, nseg, per_wave, chunks);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <int SRC, int AG = 128>
hipError_t launch_tiles_split(int split, int mc, const TilesArgs& a, int slices, int nseg, int per_wave, int chunks) {
    switch (split) {
        case 1: return launch_tiles_mc<8, SRC, AG>(mc, a, slices, nseg, per_wave, chunks);
        case 2: return launch_tiles_mc<4, SRC, AG>(mc, a, slices, nseg, per_wave, chunks);
        default: return launch_tiles_mc<2, SRC, AG>(mc, a, slices, nseg, per_wave, chunks);
    }
}

}  // namespace

int64_t tiles_bytes(int64_t n, int64_t k) { return geometry(n, k).total; }

hipError_t launch_prepare_tiles(const uint8_t* raw, int64_t stride, int64_t n, int64_t k, uint8_t* tiles,
                                hipStream_t stream) {
    const TileGeometry t = geometry(n, k);
    const int groups = (int)(k / 128);
    const int64_t code_chunks = t.tiles * t.s8 * 4 * 64;
    const int64_t scale_chunks = t.tiles * t.s8 * kTileRows;
    clear_stale_error();
    hipLaunchKernelGGL(prepare_tile_codes_kernel, dim3((unsigned)((code_chunks + 255) / 256)), dim3(256), 0, stream,
                       raw, stride, n, groups, (int)t.s8, code_chunks, tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prepare_tile_scales_kernel, dim3((unsigned)((scale_chunks + 255) / 256)), dim3(256), 0, stream,
                       raw, stride, n, groups, (int)t.s8, scale_chunks, tiles);
    return hipGetLastError();
}

// The k split is the one every small-m engine uses for (n, k) and max_waves,
// so the outputs are bit-identical to pq2_matmul_small_m's.  split = waves
// per k slice (1, 2 or 4; each takes 8/split of the segment's group
// classes), at most 16 waves per workgroup.
static int tiles_slices(int64_t k, int max_waves, int* nseg, int* per_wave) {
    const int groups = (int)(k / 128);
    *nseg = (groups + 7) / 8;
    *per_wave = (*nseg + max_waves - 1) / max_waves;
    return (*nseg + *per_wave - 1) / *per_wave;
}

// One wave per slice: with the activation scales through the scalar unit
// and eight-column passes, splitting a slice over two waves no longer pays
// at any measured shape (K = 17408: 9.71 against 9.87 us at four columns,
// 16.6 against 21.0 us at sixteen); the split never changes the bits.
int tiles_default_split(int64_t m, int64_t k, int max_waves) {
    (void)m, (void)k, (void)max_waves;
    return 1;
}

bool tiles_supported(int64_t k, int max_waves, int split) {
    if (max_waves < 1 || max_waves > 16 || (split != 1 && split != 2 && split != 4)) return false;
    int nseg, per_wave;
    return tiles_slices(k, max_waves, &nseg, &per_wave) * split <= 16;
}

// Activation groups of 64 or 32: any split from natural-order q; from x (the
// fused sources) one wave per k slice.
template <int SRC>
hipError_t launch_tiles_g(int agroup, int split, int mc, const TilesArgs& a, int slices, int nseg, int per_wave,
                          int chunks) {
    if constexpr (SRC == kSrcNatural) {
        return agroup == 64 ? launch_tiles_split<SRC, 64>(split, mc, a, slices, nseg, per_wave, chunks)
                            : launch_tiles_split<SRC, 32>(split, mc, a, slices, nseg, per_wave, chunks);
    } else {
        if (split != 1) return hipErrorInvalidValue;
        return agroup == 64 ? launch_tiles_mc<8, SRC, 64>(mc, a, slices, nseg, per_wave, chunks)
                            : launch_tiles_mc<8, SRC, 32>(mc, a, slices, nseg, per_wave, chunks);
    }
}

static hipError_t launch_tiles_any(int src, const TilesArgs& a, int max_waves, int split, int agroup = 128) {
    if (!tiles_supported(a.k, max_waves, split)) return hipErrorInvalidValue;
    int nseg, per_wave;
    const int slices = tiles_slices(a.k, max_waves, &nseg, &per_wave);
    // Up to four columns: one pass of exactly M.  More: passes of at most
    // four, or, when every wave holds several segments (long k) and the
    // activation groups are 128, passes of eight, the last one partial.
    // (Eight-column passes halve the weight reads; at short k with many
    // tiles they measured no faster: up, M = 8: 12.3 against 12.1 us.)
    int mc = (int)(a.m < 4 ? a.m : 4);
    int chunks = (int)((a.m + mc - 1) / mc);
    mc = (int)((a.m + chunks - 1) / chunks);
    if (a.m > 4 && agroup == 128 && per_wave >= 2) {
        mc = kTilesMaxColumns;
        chunks = (int)((a.m + kTilesMaxColumns - 1) / kTilesMaxColumns);
    }
    if (agroup != 128) {
        switch (src) {
            case kSrcNatural: return launch_tiles_g<kSrcNatural>(agroup, split, mc, a, slices, nseg, per_wave, chunks);
            case kSrcBf16: return launch_tiles_g<kSrcBf16>(agroup, split, mc, a, slices, nseg, per_wave, chunks);
            case kSrcF16: return launch_tiles_g<kSrcF16>(agroup, split, mc, a, slices, nseg, per_wave, chunks);
            case kSrcF32: return launch_tiles_g<kSrcF32>(agroup, split, mc, a, slices, nseg, per_wave, chunks);
            default: return hipErrorInvalidValue;
        }
    }
    switch (src) {
        case kSrcNatural: return launch_tiles_split<kSrcNatural>(split, mc, a, slices, nseg, per_wave, chunks);
        case kSrcBf16: return launch_tiles_split<kSrcBf16>(split, mc, a, slices, nseg, per_wave, chunks);
        case kSrcF16: return launch_tiles_split<kSrcF16>(split, mc, a, slices, nseg, per_wave, chunks);
        case kSrcF32: return launch_tiles_split<kSrcF32>(split, mc, a, slices, nseg, per_wave, chunks);
        default: return hipErrorInvalidValue;
    }
}

// Split-k geometry: one segment per wave, `waves` (1..16) waves per
// workgroup, ks = ceil(nseg / waves) workgroups per tile, then the waves
// evened out over the ks workgroups.  Column passes: one of m at m <= 4,
// else passes of eight (the last one partial).
SplitKPlan splitk_plan(int64_t m, int64_t n, int64_t k, int waves) {
    SplitKPlan p;
    const TileGeometry t = geometry(n, k);
    p.nseg = (int)t.s8;
    p.ks = (p.nseg + waves - 1) / waves;
    p.waves = (p.nseg + p.ks - 1) / p.ks;
    p.mc = m <= 4 ? (int)m : kTilesMaxColumns;
    p.chunks = (int)((m + p.mc - 1) / p.mc);
    p.tiles = t.tiles;
    p.partial_floats = (int64_t)p.nseg * m * n;
    p.counters = (int64_t)kSplitKMaxChunks * t.tiles;
    return p;
}

hipError_t launch_small_m_tiles_splitk(const int8_t* q, const float* xs, const uint8_t* tiles, int64_t m, int64_t n,
                                       int64_t k, float* y, float* partials, uint32_t* counters, int waves,
                                       hipStream_t stream) {
    const SplitKPlan p = splitk_plan(m, n, k, waves);
    const TilesArgs a{q, xs, nullptr, 0, tiles, m, n, k, y, stream};
    switch (p.mc) {
        case 1: return launch_tiles_splitk_one<1>(a, partials, counters, p.ks, p.waves, p.nseg, p.chunks);
        case 2: return launch_tiles_splitk_one<2>(a, partials, counters, p.ks, p.waves, p.nseg, p.chunks);
        case 3: return launch_tiles_splitk_one<3>(a, partials, counters, p.ks, p.waves, p.nseg, p.chunks);
        case 4: return launch_tiles_splitk_one<4>(a, partials, counters, p.ks, p.waves, p.nseg, p.chunks);
        case 8: return launch_tiles_splitk_one<8>(a, partials, counters, p.ks, p.waves, p.nseg, p.chunks);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_small_m_tiles(const int8_t* q, const float* xs, const uint8_t* tiles, int64_t m, int64_t n,
                                int64_t k, float* y, int max_waves, int split, hipStream_t stream) {
    const TilesArgs a{q, xs, nullptr, 0, tiles, m, n, k, y, stream};
    return launch_tiles_any(kSrcNatural, a, max_waves, split);
}

hipError_t launch_small_m_tiles_fused(const void* x, int dtype, int64_t x_stride, const uint8_t* tiles, int64_t m,
                                      int64_t n, int64_t k, float* y, int max_waves, int split, hipStream_t stream) {
    const TilesArgs a{nullptr, nullptr, x, x_stride, tiles, m, n, k, y, stream};
    return launch_tiles_any(src_of_dtype(dtype), a, max_waves, split);
}

hipError_t launch_small_m_tiles_fused_g(const void* x, int dtype, int64_t x_stride, const uint8_t* tiles, int64_t m,
                                        int64_t n, int64_t k, int agroup, float* y, int max_waves, int split,
                                        hipStream_t stream) {
    if (agroup != 128 && agroup != 64 && agroup != 32) return hipErrorInvalidValue;
    const TilesArgs a{nullptr, nullptr, x, x_stride, tiles, m, n, k, y, stream};
    return launch_tiles_any(src_of_dtype(dtype), a, max_waves, split, agroup);
}

hipError_t launch_small_m_tiles_g(const int8_t* q, const float* xs, const uint8_t* tiles, int64_t m, int64_t n,
                                  int64_t k, int agroup, float* y, int max_waves, int split, hipStream_t stream) {
    if (agroup != 128 && agroup != 64 && agroup != 32) return hipErrorInvalidValue;
    const TilesArgs a{q, xs, nullptr, 0, tiles, m, n, k, y, stream};
    return launch_tiles_any(kSrcNatural, a, max_waves, split, agroup);
}

}  // namespace pq2
