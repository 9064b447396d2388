// probe.hip -- read-only probes of the weight layouts: the decode engines'
// weight loads with no arithmetic, the ceiling their matmuls are measured
// against.
//
// Page "Kernel experiments: recorded evidence", section H, Test 24 timed
// copy-free read patterns of the weight layouts (row-major segments against
// tile-major) to separate what the access pattern allows from what the
// kernel's work costs.  These probes issue exactly the weight loads of the
// gfx950 decode engines: the same grid, waves, k split (segments of 8
// groups over at most 16 waves for the tile layout, 8 for the planes),
// instruction widths and cache policy, one segment at a time.  Each wave folds what it reads with XOR (so no load is dead)
// and writes one word.  Every byte of the layout is read once, so the XOR of
// all output words is the XOR of the layout's dwords (code dwords and tile
// units; the planes' fp16 scales each zero-extended), which the tests check.
#include "pq2_device.h"
#include "pq2_internal.h"

namespace pq2 {

namespace {

// Tile layout (pq2_prepare_tiles): per 16-row tile and 8-group segment one
// 4352-byte unit, four 1 KB code blocks (one 16-byte MFMA operand per lane)
// then the 16 rows' 8 fp16 scales.
constexpr int kProbeTileRows = 16;
constexpr int kProbeCodeBlock = 1024;
constexpr int kProbeUnit = 4 * kProbeCodeBlock + 256;
// Planes: a wave is 8 row slots of 8 lanes, as in the packed-dot engine.
constexpr int kProbeRowSlots = 8;
constexpr int kProbeMaxWaves = 8;       // planes: the packed-dot engine's k split
constexpr int kProbeTileMaxWaves = 16;  // tiles: the tile engine's

__device__ __forceinline__ uint32_t fold4(const uint4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

__device__ __forceinline__ uint32_t wave_xor(uint32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v ^= (uint32_t)__shfl_xor((int)v, d);
    return v;
}

// Grid: one workgroup per 16-row tile, one wave per k slice.  Per segment a
// wave reads the unit's 256 scale bytes (16 bytes per lane; lanes 16..63
// repeat lanes 0..15 as in the matmul and are not folded) and its four code
// blocks (16 bytes per lane each, streamed).
__global__ __launch_bounds__(1024) void read_probe_tiles_kernel(const uint8_t* __restrict__ tiles, int s8,
                                                               int per_wave, uint32_t* __restrict__ out) {
    const int nwaves = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int tile = blockIdx.x;
    const auto rs = make_rsrc(tiles + (size_t)tile * s8 * kProbeUnit, (uint32_t)(s8 * kProbeUnit));
    const int seg_end = min((wave + 1) * per_wave, s8);
    uint32_t f = 0;
    for (int s = wave * per_wave; s < seg_end; ++s) {
        const uint32_t unit = (uint32_t)(s * kProbeUnit);
        const uint4 ws = buf_load16<kAuxNonTemporal>(rs, unit + 4 * kProbeCodeBlock + 16 * (lane & 15));
        uint4 cw[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) cw[b] = buf_load16<kAuxNonTemporal>(rs, unit + b * kProbeCodeBlock + 16 * lane);
        f ^= fold4(cw[0]) ^ fold4(cw[1]) ^ fold4(cw[2]) ^ fold4(cw[3]) ^ (lane < 16 ? fold4(ws) : 0u);
    }
    f = wave_xor(f);
    if (lane == 0) out[(size_t)tile * nwaves + wave] = f;
}

// Grid: one workgroup per 8 rows, one wave per k slice.  Per segment lane j
// of row slot r reads code bytes 16j and 128 + 16j of the row's 256 (the
// halves of groups j/2 and 4 + j/2; groups past the end are not read) and
// the fp16 scale of one of the segment's 8 groups.
__global__ __launch_bounds__(512) void read_probe_planes_kernel(const uint8_t* __restrict__ codes,
                                                                const uint16_t* __restrict__ scales, int n, int k,
                                                                int groups, int per_wave, int nseg,
                                                                uint32_t* __restrict__ out) {
    const int nwaves = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int slot = lane >> 3;
    const int j = lane & 7;
    const int gsel = (j >> 1) + 4 * (j & 1);
    const int row_base = blockIdx.x * kProbeRowSlots;
    const int rows_here = min(kProbeRowSlots, n - row_base);
    const uint32_t k4 = (uint32_t)k >> 2;
    const auto code_rs = make_rsrc(codes + (size_t)row_base * k4, (uint32_t)rows_here * k4);
    const auto scale_rs = make_rsrc(scales + (size_t)row_base * groups, (uint32_t)(rows_here * groups * 2));
    const int seg_end = min((wave + 1) * per_wave, nseg);
    uint32_t f = 0;
    for (int s = wave * per_wave; s < seg_end; ++s) {
        const int g0 = s * 8;
        const bool okA = g0 + (j >> 1) < groups;
        const bool okB = g0 + 4 + (j >> 1) < groups;
        const bool okS = g0 + gsel < groups;
        const uint32_t off = (uint32_t)slot * k4 + (uint32_t)g0 * 32u + 16u * (uint32_t)j;
        const uint4 a = buf_load16<kAuxNonTemporal>(code_rs, okA ? off : kBufferOOB);
        const uint4 b = buf_load16<kAuxNonTemporal>(code_rs, okB ? off + 128u : kBufferOOB);
        const uint32_t w = buf_load2(scale_rs, okS ? ((uint32_t)slot * groups + g0 + gsel) * 2u : kBufferOOB);
        f ^= fold4(a) ^ fold4(b) ^ w;
    }
    f = wave_xor(f);
    if (lane == 0) out[(size_t)blockIdx.x * nwaves + wave] = f;
}

// Linear stream read of `bytes` bytes, shaped like no decode engine:
// grid-stride over wave chunks of U KB.  Iteration i, workgroup w, wave v
// reads the U consecutive 1 KB blocks starting at block ((i * G + w) * W + v)
// * U, one 16-byte load per lane per block, all U loads issued before any is
// used, so a lane has U loads in flight.  POLICY picks the load:
//   0, 1  buffer_load_dwordx4 into registers (1: non-temporal); bytes past
//         the end read zero (buffer range check);
//   2, 3  global_load_lds_dwordx4 into a per-wave LDS slot of U KB (3:
//         non-temporal), then, once the loads have landed, each lane reads
//         16 bytes back (bytes is a multiple of 1 KB, so a block is wholly
//         in or out of range: a wave-uniform branch).
// Each wave folds what it read with XOR.  store_all = 1 writes every wave's
// fold (the XOR of all words is the XOR of the buffer's dwords); store_all =
// 0 writes only from a lane whose own fold equals `sentinel` (practically
// never), so a timed run is a pure read (any output store adds the latency of
// one store to the end of a launch).
template <int U, int POLICY>
__global__ __launch_bounds__(1024) void stream_probe_kernel(const uint8_t* __restrict__ buf, uint32_t bytes, int iters,
                                                            int store_all, uint32_t sentinel,
                                                            uint32_t* __restrict__ out) {
    constexpr int kAux = (POLICY & 1) ? kAuxNonTemporal : 0;
    const int nwaves = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint32_t wave_id = (uint32_t)blockIdx.x * nwaves + wave;
    const uint32_t stride = gridDim.x * (uint32_t)nwaves * (uint32_t)(U * 1024);
    uint32_t base = wave_id * (uint32_t)(U * 1024);  // wave-uniform start of this iteration's chunk
    uint32_t f = 0;
    if constexpr (POLICY < 2) {
        const auto rs = make_rsrc(buf, bytes);
        for (int i = 0; i < iters; ++i, base += stride) {
            uint4 r[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t off = base + u * 1024u + 16u * lane;
                r[u] = buf_load16<kAux>(rs, off < bytes ? off : kBufferOOB);
            }
            // Keep the scheduler from starting the fold (and its waits)
            // before the last load has issued: U loads in flight.
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) f ^= fold4(r[u]);
        }
    } else {
        extern __shared__ uint4 stream_slots[];  // U KB per wave
        uint4* slot = stream_slots + (size_t)wave * U * 64;
#pragma nounroll
        for (int i = 0; i < iters; ++i, base += stride) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (base + u * 1024u < bytes)
                    __builtin_amdgcn_global_load_lds(
                        (const void __attribute__((address_space(1)))*)(buf + base + u * 1024u + 16u * lane),
                        (void __attribute__((address_space(3)))*)(slot + u * 64), 16, 0, kAux);
            // The compiler does not order these LDS reads after the loads
            // that fill the slot: wait for every vector-memory load of the
            // wave (vmcnt 0; expcnt and lgkmcnt left at their maxima).
            __builtin_amdgcn_s_waitcnt(0x0F70);
            // Every slot is read (LDS, always in range); a block past the
            // end holds stale bytes and is dropped from the fold.
            uint4 r[U];
#pragma unroll
            for (int u = 0; u < U; ++u) r[u] = slot[u * 64 + lane];
#pragma unroll
            for (int u = 0; u < U; ++u) f ^= base + u * 1024u < bytes ? fold4(r[u]) : 0u;
        }
    }
    if (store_all) {
        f = wave_xor(f);
        if (lane == 0) out[wave_id] = f;
    } else if (f == sentinel) {
        out[wave_id] = f;  // the timed mode: a lane's own fold, practically never equal
    }
}

// An empty kernel: the launch floor of a graph of back-to-back launches.
__global__ void empty_probe_kernel(uint32_t* out, int never) {
    if (never == 1 && threadIdx.x == 0) out[blockIdx.x] = 0;
}

struct ProbeGrid {
    int64_t blocks;
    int waves, per_wave, nseg;
};

// The engines' k split: segments of 8 groups over at most 8 waves (planes)
// or 16 (tiles).
ProbeGrid probe_grid(int layout, int64_t n, int64_t k) {
    ProbeGrid g;
    const int max_waves = layout == 1 ? kProbeTileMaxWaves : kProbeMaxWaves;
    g.nseg = (int)((k / 128 + 7) / 8);
    g.per_wave = (g.nseg + max_waves - 1) / max_waves;
    g.waves = (g.nseg + g.per_wave - 1) / g.per_wave;
    g.blocks = layout == 1 ? (n + kProbeTileRows - 1) / kProbeTileRows : (n + kProbeRowSlots - 1) / kProbeRowSlots;
    return g;
}

}  // namespace

hipError_t launch_stream_probe(const uint8_t* buf, int64_t bytes, int64_t workgroups, int waves, int loads,
                               int policy, int store_all, uint32_t sentinel, uint32_t* out, hipStream_t stream) {
    const int64_t per_iter = workgroups * waves * loads * 1024;
    const int iters = (int)((bytes + per_iter - 1) / per_iter);
    const size_t lds = policy >= 2 ? (size_t)waves * loads * 1024 : 0;
    decltype(&stream_probe_kernel<1, 0>) fn = nullptr;
#define PQ2_STREAM_CASE(u)                                                                                 \
    if (loads == u)                                                                                        \
        fn = policy == 0   ? stream_probe_kernel<u, 0>                                                     \
             : policy == 1 ? stream_probe_kernel<u, 1>                                                     \
             : policy == 2 ? stream_probe_kernel<u, 2>                                                     \
                           : stream_probe_kernel<u, 3>;
    PQ2_STREAM_CASE(1)
    PQ2_STREAM_CASE(2)
    PQ2_STREAM_CASE(4)
    PQ2_STREAM_CASE(8)
    PQ2_STREAM_CASE(16)
#undef PQ2_STREAM_CASE
    if (!fn) return hipErrorInvalidValue;
    clear_stale_error();
    hipLaunchKernelGGL(fn, dim3((unsigned)workgroups), dim3(64 * waves), lds, stream, buf, (uint32_t)bytes, iters,
                       store_all, sentinel, out);
    return hipGetLastError();
}

hipError_t launch_empty_probe(int64_t workgroups, int waves, hipStream_t stream) {
    clear_stale_error();
    hipLaunchKernelGGL(empty_probe_kernel, dim3((unsigned)workgroups), dim3(64 * waves), 0, stream, nullptr, 0);
    return hipGetLastError();
}

int64_t read_probe_words(int layout, int64_t n, int64_t k) {
    const ProbeGrid g = probe_grid(layout, n, k);
    return g.blocks * g.waves;
}

hipError_t launch_read_probe(const uint8_t* weights, int layout, int64_t n, int64_t k, uint32_t* out,
                             hipStream_t stream) {
    const ProbeGrid g = probe_grid(layout, n, k);
    clear_stale_error();
    if (layout == 1) {
        hipLaunchKernelGGL(read_probe_tiles_kernel, dim3((unsigned)g.blocks), dim3(64 * g.waves), 0, stream, weights,
                           g.nseg, g.per_wave, out);
    } else {
        const uint16_t* scales = reinterpret_cast<const uint16_t*>(weights + n * (k / 4));
        hipLaunchKernelGGL(read_probe_planes_kernel, dim3((unsigned)g.blocks), dim3(64 * g.waves), 0, stream, weights,
                           scales, (int)n, (int)k, (int)(k / 128), g.per_wave, g.nseg, out);
    }
    return hipGetLastError();
}

}  // namespace pq2
