// pq2_internal.h -- host-side launchers shared between the libpq2 sources.
// Arguments reaching these functions are already validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pq2 {

// Discard an error another library left in this thread's HIP error slot, so
// the hipGetLastError() that follows our launch reports our launch only.
inline void clear_stale_error() { (void)hipGetLastError(); }

// Returns a hipError_t from launching (hipSuccess on success).
hipError_t launch_prepare(const uint8_t* raw, int64_t stride, int64_t n, int64_t k, uint8_t* planes,
                          hipStream_t stream);

hipError_t launch_quantize(const void* x, int dtype, int64_t row_stride, int64_t m, int64_t k,
                           int8_t* q, float* xs, hipStream_t stream);

hipError_t launch_quantize_planes(const void* x, int dtype, int64_t row_stride, int64_t m, int64_t k,
                                  int8_t* qp, float* xs, int32_t* qsum, hipStream_t stream);

struct SmallMConfig {
    int rows_per_lane;  // 1 or 2 (dot-product engine only)
    int max_waves;      // 1..8: waves that split k inside one workgroup
    int engine;         // 1 = packed dot products (v_dot4), 2 = INT8 matrix cores; same bits
};

SmallMConfig default_small_m_config(int64_t m, int64_t n, int64_t k);
SmallMConfig default_small_m_fused_config(int64_t m, int64_t n, int64_t k);  // same k split

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
