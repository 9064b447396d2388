// pq2_internal.h -- host-side launchers shared between the libpq2 sources.
// Arguments reaching these functions are already validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pq2 {

// Where a small-m kernel's activations come from.
enum : int {
    kSrcPlanes = 0,   // plane-order q and group sums (pq2_quantize_act_i8_planes)
    kSrcNatural = 1,  // natural-order q (pq2_quantize_act_i8): transposed and summed while staged
    kSrcBf16 = 2,     // unquantised x of this element type, quantised while staged
    kSrcF16 = 3,
    kSrcF32 = 4,
};
constexpr bool src_fused(int src) { return src >= kSrcBf16; }
constexpr int src_esize(int src) { return src == kSrcF32 ? 4 : 2; }
constexpr int src_xloads(int src) { return src == kSrcF32 ? 4 : 2; }  // 16-byte loads per lane and group
inline int src_of_dtype(int dtype) { return dtype == 0 ? kSrcBf16 : dtype == 1 ? kSrcF16 : dtype == 2 ? kSrcF32 : -1; }

// Discard an error another library left in this thread's HIP error slot, so
// the hipGetLastError() that follows our launch reports our launch only.
inline void clear_stale_error() { (void)hipGetLastError(); }

// Returns a hipError_t from launching (hipSuccess on success).
hipError_t launch_prepare(const uint8_t* raw, int64_t stride, int64_t n, int64_t k, uint8_t* planes,
                          hipStream_t stream);

hipError_t launch_quantize(const void* x, int dtype, int64_t row_stride, int64_t m, int64_t k,
                           int8_t* q, float* xs, hipStream_t stream);

// Activation groups of agroup = 128, 64 or 32 elements (q [m][k], xs [m][k/agroup]).
hipError_t launch_quantize_g(const void* x, int dtype, int64_t row_stride, int64_t m, int64_t k, int agroup,
                             int8_t* q, float* xs, hipStream_t stream);
hipError_t launch_quantize_planes(const void* x, int dtype, int64_t row_stride, int64_t m, int64_t k,
                                  int8_t* qp, float* xs, int32_t* qsum, hipStream_t stream);

struct SmallMConfig {
    int rows;       // engine 1: weight rows per lane (1, 2); engines 3, 4: 8-row blocks per workgroup
    int max_waves;  // 1..8: waves that split k inside one workgroup
    int engine;     // 1 = packed dot products (v_dot4), 2 = INT8 matrix cores, one row block per
                    // workgroup, 3 = INT8 matrix cores, one 8-wave workgroup staging the
                    // activations for `rows` row blocks, 4 = the same kernel with one
                    // unit per wave; same bits
};

// Arguments of one small-m launch, any engine.  waves, nseg, per_wave and
// chunks (k split and column passes) are filled in by the dispatcher.
struct SmallMLaunch {
    const int8_t* q;
    const float* xs;
    const int32_t* qsum;
    const void* x;
    int64_t x_stride;
    const uint8_t* planes;
    int64_t m, n, k;
    float* y;
    int waves, nseg, per_wave, chunks;
    hipStream_t stream;
    int64_t raw_stride = 0;  // nonzero: `planes` is the raw block layout with this row stride in bytes
};

// Columns one pass of the workgroup-staged engine covers; more columns take
// several passes over the weights.
constexpr int kWgMaxColumns = 4;

// Workgroup-staged matrix-core engine (small_m_wg.hip); src is a kSrc* value
// and rows the row blocks (8 weight rows) per workgroup.  wave_mode false:
// one 8-wave workgroup per CU (engine 3); true: one unit per wave (engine 4).
bool wg_supported(int src, int64_t m, int64_t k, int max_waves, int rows, bool wave_mode);
int wg_default_row_blocks(int src, int64_t m, int64_t n, int64_t k, int max_waves, bool wave_mode);  // 0: none
hipError_t launch_small_m_wg(int src, const SmallMLaunch& a, int max_waves, int rows, bool wave_mode);

// Tile-major weight layout and its matrix-core decode engine (tiles.hip).
int64_t tiles_bytes(int64_t n, int64_t k);
hipError_t launch_prepare_tiles(const uint8_t* raw, int64_t stride, int64_t n, int64_t k, uint8_t* tiles,
                                hipStream_t stream);
int tiles_default_split(int64_t m, int64_t k, int max_waves);
// The tile engine splits k over up to 16 waves of one workgroup (the other
// small-m engines over up to 8): at K = 17408 that is 9 slices of two
// segments instead of 6 of three, 0.3-1.0 us faster at 2-4 columns.  The
// split depends on k only, so every column count sums in one order.
constexpr int kTilesDefaultWaves = 16;
bool tiles_supported(int64_t k, int max_waves, int split);
hipError_t launch_small_m_tiles(const int8_t* q, const float* xs, const uint8_t* tiles, int64_t m, int64_t n,
                                int64_t k, float* y, int max_waves, int split, hipStream_t stream);
// Split-k tile engine: one segment per wave, the k slices of a tile spread
// over several workgroups; partial sums [nseg][m][n] fp32 and one counter per
// (column pass, tile) (kSplitKMaxChunks x tiles words, zero before the call
// and left zero by it).  `waves` (1..16) bounds the waves per workgroup.
constexpr int kSplitKMaxChunks = 4;    // column passes for m <= 16 (passes of m <= 4, or of eight)
constexpr int kSplitKDefaultWaves = 6;
struct SplitKPlan {
    int nseg, ks, waves, mc, chunks;
    int64_t tiles, partial_floats, counters;
};
SplitKPlan splitk_plan(int64_t m, int64_t n, int64_t k, int waves);
hipError_t launch_small_m_tiles_splitk(const int8_t* q, const float* xs, const uint8_t* tiles, int64_t m, int64_t n,
                                       int64_t k, float* y, float* partials, uint32_t* counters, int waves,
                                       hipStream_t stream);
hipError_t launch_prefill_tiles(const int8_t* q, const float* xs, const uint8_t* tiles, int64_t m, int64_t n,
                                int64_t k, float* y, int tile, hipStream_t stream);
// Read-only probes of the weight layouts (layout 0 = planes, 1 = tiles): the
// decode engines' weight loads without arithmetic; out gets
// read_probe_words(layout, n, k) XOR folds.
int64_t read_probe_words(int layout, int64_t n, int64_t k);
hipError_t launch_read_probe(const uint8_t* weights, int layout, int64_t n, int64_t k, uint32_t* out,
                             hipStream_t stream);
// Linear stream read of a buffer (workgroups x waves, grid-stride over
// chunks of `loads` KB per wave, `loads` 16-byte loads per lane in flight;
// policy 0..3 as in pq2_measure.h).  Writes workgroups x waves words.
hipError_t launch_stream_probe(const uint8_t* buf, int64_t bytes, int64_t workgroups, int waves, int loads,
                               int policy, int store_all, uint32_t sentinel, uint32_t* out, hipStream_t stream);
// An empty kernel of workgroups x waves: the launch floor.
hipError_t launch_empty_probe(int64_t workgroups, int waves, hipStream_t stream);
// Packed-dot small-m matmul straight from the raw block layout (34 bytes per
// 128 weights: fp16 scale, then 32 code bytes; rows raw_stride bytes apart),
// natural-order q; max_waves fixes the k split as for launch_small_m.
hipError_t launch_small_m_raw(const int8_t* q, const float* xs, const uint8_t* raw, int64_t raw_stride, int64_t m,
                              int64_t n, int64_t k, float* y, int max_waves, int rows, hipStream_t stream);
// Tile-layout prefill with activation groups of agroup = 128, 64 or 32
// (natural-order q, xs [m][k/agroup]); tile 0 picks the default.
hipError_t launch_prefill_tiles_g(const int8_t* q, const float* xs, const uint8_t* tiles, int64_t m, int64_t n,
                                  int64_t k, float* y, int tile, int agroup, hipStream_t stream);
hipError_t launch_small_m_tiles_fused(const void* x, int dtype, int64_t x_stride, const uint8_t* tiles, int64_t m,
                                      int64_t n, int64_t k, float* y, int max_waves, int split, hipStream_t stream);
// The fused tile matmul (x quantised while staged) with activation groups of
// agroup = 128, 64 or 32; split must be 1 below 128.
hipError_t launch_small_m_tiles_fused_g(const void* x, int dtype, int64_t x_stride, const uint8_t* tiles, int64_t m,
                                        int64_t n, int64_t k, int agroup, float* y, int max_waves, int split,
                                        hipStream_t stream);
// Tile engine with activation groups of agroup = 128, 64 or 32 (natural-order
// q from launch_quantize_g, xs [m][k/agroup]).
hipError_t launch_small_m_tiles_g(const int8_t* q, const float* xs, const uint8_t* tiles, int64_t m, int64_t n,
                                  int64_t k, int agroup, float* y, int max_waves, int split, hipStream_t stream);

// The library's choice for activations of kind src; the k split (max_waves)
// depends on (n, k) only, so every source and column count sums in one order.
SmallMConfig default_small_m_config(int src, int64_t m, int64_t n, int64_t k);
// The `rows` setting an engine uses by default at this shape (0: the engine
// cannot run it).
int default_small_m_rows(int engine, int src, int64_t m, int64_t n, int64_t k, int max_waves);

// Natural-order q (the kernel transposes blocks and forms the group sums).
// Returns hipErrorInvalidValue for a configuration the library has no kernel for.
hipError_t launch_small_m(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m,
                          int64_t n, int64_t k, float* y, const SmallMConfig& cfg,
                          hipStream_t stream);

// Plane-order q with its group sums (from launch_quantize_planes).
hipError_t launch_small_m_planes(const int8_t* qp, const float* xs, const int32_t* qsum, const uint8_t* planes,
                                 int64_t m, int64_t n, int64_t k, float* y, const SmallMConfig& cfg,
                                 hipStream_t stream);

// Unquantised activations x (dtype 0 bf16, 1 f16, 2 f32; rows x_stride
// elements apart), quantised inside the matmul kernel with the quantiser's
// exact results: same output bits as launch_quantize + launch_small_m.
hipError_t launch_small_m_fused(const void* x, int dtype, int64_t x_stride, const uint8_t* planes, int64_t m,
                                int64_t n, int64_t k, float* y, const SmallMConfig& cfg, hipStream_t stream);

// tile: 0 = default, 1 = 128x128, 2 = 64x128, 3 = 64x64, 4 = 128x64 outputs
// per workgroup.  plane_a: q is in plane order (pq2_quantize_act_i8_planes).
hipError_t launch_prefill(const int8_t* q, const float* xs, const uint8_t* planes, int64_t m,
                          int64_t n, int64_t k, float* y, int tile, bool plane_a, hipStream_t stream);

}  // namespace pq2
