// api.hip -- the C ABI of libpq2 (declared in include/pq2.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, returns a status instead of aborting, and enqueues its kernel
// on the caller's stream.  Buffers are owned by the caller.
#include "../../include/pq2.h"
#include "../../include/pq2_measure.h"
#include "../../include/pq2_tuning.h"
#include "pq2_internal.h"

#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>

namespace {

constexpr int64_t kGroup = 128;
constexpr int64_t kMaxPrefillM = (int64_t)65535 * 64;  // grid.y limit x smallest tile rows
constexpr int64_t kMaxN = (int64_t)1 << 30;
// Raw rows read in place: a workgroup's 16 rows stay below 2^31 bytes, the
// range of the kernels' 32-bit buffer offsets.
constexpr int64_t kMaxRawStride = (int64_t)1 << 26;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Is the current device a gfx950?  Cached per device ordinal.
int check_device() {
    static int known[64];  // 0 unknown, 1 yes, 2 no
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PQ2_EDEVICE;
    if (dev >= 0 && dev < 64 && known[dev]) return known[dev] == 1 ? PQ2_OK : PQ2_EDEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return PQ2_EDEVICE;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev >= 0 && dev < 64) known[dev] = ok ? 1 : 2;
    return ok ? PQ2_OK : PQ2_EDEVICE;
}

thread_local hipError_t last_hip_error = hipSuccess;

int launch_status(hipError_t e) {
    last_hip_error = e;
    return e == hipSuccess ? PQ2_OK : PQ2_ELAUNCH;
}

int check_k(int64_t k) {
    if (k < kGroup || k % kGroup || k > PQ2_MAX_K) return PQ2_ESHAPE;
    return PQ2_OK;
}

int check_matmul_args(const int8_t* q, const float* xs, const void* planes, int64_t m, int64_t n,
                      int64_t k, float* y, int64_t m_max, bool tiles = false) {
    if (!q || !xs || !planes || !y) return PQ2_EINVAL;
    if (m < 1 || m > m_max || n < 1 || n > kMaxN) return PQ2_ESHAPE;
    if (int rc = check_k(k)) return rc;
    if (!aligned(q, 16) || !aligned(planes, 16) || !aligned(xs, 4) || !aligned(y, 4)) return PQ2_EALIGN;
    const size_t ybytes = (size_t)m * n * 4;
    if (overlap(y, ybytes, q, (size_t)m * k) || overlap(y, ybytes, xs, (size_t)m * (k / kGroup) * 4) ||
        overlap(y, ybytes, planes, tiles ? (size_t)pq2::tiles_bytes(n, k) : (size_t)n * (k / kGroup) * 34))
        return PQ2_EINVAL;
    return PQ2_OK;
}

// Default small-m configuration with the caller's overrides (0 = default).
// An explicit engine without explicit rows takes that engine's default rows.
int small_m_config(int src, int64_t m, int64_t n, int64_t k, int rows, int max_waves, int engine,
                   pq2::SmallMConfig* cfg) {
    *cfg = pq2::default_small_m_config(src, m, n, k);
    if (max_waves) cfg->max_waves = max_waves;
    if (cfg->max_waves < 1 || cfg->max_waves > 8) return PQ2_EINVAL;
    if (engine && engine != cfg->engine) {
        cfg->engine = engine;
        cfg->rows = pq2::default_small_m_rows(engine, src, m, n, k, cfg->max_waves);
    } else if (max_waves && cfg->engine >= 3) {
        cfg->rows = pq2::default_small_m_rows(cfg->engine, src, m, n, k, cfg->max_waves);
    }
    if (rows) cfg->rows = rows;
    switch (cfg->engine) {
        case 1: return (cfg->rows == 1 || cfg->rows == 2) ? PQ2_OK : PQ2_EINVAL;
        case 2: return cfg->rows == 1 ? PQ2_OK : PQ2_EINVAL;
        case 3: return pq2::wg_supported(src, m, k, cfg->max_waves, cfg->rows, false) ? PQ2_OK : PQ2_EINVAL;
        case 4: return pq2::wg_supported(src, m, k, cfg->max_waves, cfg->rows, true) ? PQ2_OK : PQ2_EINVAL;
        default: return PQ2_EINVAL;
    }
}

// Scratch of pq2_gemv_tiles_static: the quantised activations q
// [PQ2_MAX_SMALL_M][PQ2_MAX_K] int8, then their scales xs
// [PQ2_MAX_SMALL_M][PQ2_MAX_K / 128] float, the largest shape any small-m
// entry point accepts (1 MiB + 32 KiB per GPU, held until the process ends).
constexpr size_t kStaticQBytes = (size_t)PQ2_MAX_SMALL_M * PQ2_MAX_K;
constexpr size_t kStaticXsBytes = (size_t)PQ2_MAX_SMALL_M * (PQ2_MAX_K / 128) * 4;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticQBytes + kStaticXsBytes];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (each GPU holds its own copy of the array).  In host code the
// array's name is not a device address; only this pointer is passed on.
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PQ2_EDEVICE;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return launch_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return PQ2_OK;
}

}  // namespace

extern "C" {

int pq2_layout_version(void) { return 1; }

const char* pq2_last_hip_error(void) { return hipGetErrorName(last_hip_error); }

const char* pq2_status_str(int status) {
    switch (status) {
        case PQ2_OK: return "ok";
        case PQ2_EINVAL: return "invalid argument (null pointer, dtype, or overlapping buffers)";
        case PQ2_ESHAPE: return "unsupported shape (k % 128, m/n/k range, or row stride)";
        case PQ2_EALIGN: return "misaligned pointer or stride";
        case PQ2_ELAUNCH: return "kernel launch failed";
        case PQ2_EDEVICE: return "current device is not gfx950";
        default: return "unknown status";
    }
}

int pq2_prepare_planes(const void* raw, int64_t raw_row_stride_bytes, int64_t n, int64_t k,
                       void* planes, void* stream) {
    if (!raw || !planes) return PQ2_EINVAL;
    if (n < 1 || n > kMaxN) return PQ2_ESHAPE;
    if (int rc = check_k(k)) return rc;
    if (raw_row_stride_bytes < (k / kGroup) * 34) return PQ2_ESHAPE;
    if (!aligned(planes, 16)) return PQ2_EALIGN;
    const size_t raw_bytes = (size_t)(n - 1) * raw_row_stride_bytes + (size_t)(k / kGroup) * 34;
    if (overlap(raw, raw_bytes, planes, (size_t)n * (k / kGroup) * 34)) return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_prepare(static_cast<const uint8_t*>(raw), raw_row_stride_bytes, n, k,
                                             static_cast<uint8_t*>(planes), (hipStream_t)stream));
}

int64_t pq2_tiles_bytes(int64_t n, int64_t k) {
    if (n < 1 || n > kMaxN || check_k(k)) return -1;
    return pq2::tiles_bytes(n, k);
}

int pq2_prepare_tiles(const void* raw, int64_t raw_row_stride_bytes, int64_t n, int64_t k, void* tiles,
                      void* stream) {
    if (!raw || !tiles) return PQ2_EINVAL;
    if (n < 1 || n > kMaxN) return PQ2_ESHAPE;
    if (int rc = check_k(k)) return rc;
    if (raw_row_stride_bytes < (k / kGroup) * 34) return PQ2_ESHAPE;
    if (!aligned(tiles, 16)) return PQ2_EALIGN;
    const size_t raw_bytes = (size_t)(n - 1) * raw_row_stride_bytes + (size_t)(k / kGroup) * 34;
    if (overlap(raw, raw_bytes, tiles, (size_t)pq2::tiles_bytes(n, k))) return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_prepare_tiles(static_cast<const uint8_t*>(raw), raw_row_stride_bytes, n, k,
                                                   static_cast<uint8_t*>(tiles), (hipStream_t)stream));
}

int pq2_matmul_small_m_tiles_tuned(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                                   int64_t k, float* y, int max_waves, int split, void* stream) {
    if (int rc = check_matmul_args(q, xs, tiles, m, n, k, y, PQ2_MAX_SMALL_M, true)) return rc;
    if (max_waves < 0 || max_waves > 16) return PQ2_EINVAL;
    const int waves = max_waves ? max_waves : pq2::kTilesDefaultWaves;
    if (!split) split = pq2::tiles_default_split(m, k, waves);
    if (!pq2::tiles_supported(k, waves, split)) return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_small_m_tiles(q, xs, static_cast<const uint8_t*>(tiles), m, n, k, y, waves,
                                                   split, (hipStream_t)stream));
}

int pq2_matmul_small_m_tiles(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                             int64_t k, float* y, void* stream) {
    return pq2_matmul_small_m_tiles_tuned(q, xs, tiles, m, n, k, y, 0, 0, stream);
}

// Arguments of the fused tile matmul: x is read in place with 16-byte loads.
static int check_tiles_fused_args(const void* x, int dtype, int64_t x_row_stride_elems, const void* tiles, int64_t m,
                                  int64_t n, int64_t k, const float* y) {
    if (!x || !tiles || !y) return PQ2_EINVAL;
    if (dtype != PQ2_BF16 && dtype != PQ2_F16 && dtype != PQ2_F32) return PQ2_EINVAL;
    if (m < 1 || m > PQ2_MAX_SMALL_M || n < 1 || n > kMaxN) return PQ2_ESHAPE;
    if (int rc = check_k(k)) return rc;
    if (x_row_stride_elems < k) return PQ2_ESHAPE;
    const int esize = dtype == PQ2_F32 ? 4 : 2;
    const size_t xbytes = ((size_t)(m - 1) * x_row_stride_elems + k) * esize;
    if (xbytes >= ((size_t)1 << 31)) return PQ2_ESHAPE;  // the kernel addresses x with 32-bit offsets
    if (!aligned(x, 16) || (x_row_stride_elems * esize) % 16 || !aligned(tiles, 16) || !aligned(y, 4))
        return PQ2_EALIGN;
    const size_t ybytes = (size_t)m * n * 4;
    if (overlap(y, ybytes, x, xbytes) || overlap(y, ybytes, tiles, (size_t)pq2::tiles_bytes(n, k))) return PQ2_EINVAL;
    return PQ2_OK;
}

int pq2_matmul_small_m_tiles_fused_tuned(const void* x, int dtype, int64_t x_row_stride_elems, const void* tiles,
                                         int64_t m, int64_t n, int64_t k, float* y, int max_waves, int split,
                                         void* stream) {
    if (int rc = check_tiles_fused_args(x, dtype, x_row_stride_elems, tiles, m, n, k, y)) return rc;
    if (max_waves < 0 || max_waves > 16) return PQ2_EINVAL;
    const int waves = max_waves ? max_waves : pq2::kTilesDefaultWaves;
    if (!split) split = pq2::tiles_default_split(m, k, waves);
    if (!pq2::tiles_supported(k, waves, split)) return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_small_m_tiles_fused(x, dtype, x_row_stride_elems,
                                                         static_cast<const uint8_t*>(tiles), m, n, k, y, waves, split,
                                                         (hipStream_t)stream));
}

int pq2_matmul_small_m_tiles_fused(const void* x, int dtype, int64_t x_row_stride_elems, const void* tiles,
                                   int64_t m, int64_t n, int64_t k, float* y, void* stream) {
    return pq2_matmul_small_m_tiles_fused_tuned(x, dtype, x_row_stride_elems, tiles, m, n, k, y, 0, 0, stream);
}

int pq2_quantize_act_i8(const void* x, int dtype, int64_t x_row_stride_elems, int64_t m, int64_t k,
                        int8_t* q, float* xs, void* stream) {
    if (!x || !q || !xs) return PQ2_EINVAL;
    if (dtype != PQ2_BF16 && dtype != PQ2_F16 && dtype != PQ2_F32) return PQ2_EINVAL;
    if (m < 1 || m > ((int64_t)1 << 31)) return PQ2_ESHAPE;
    if (int rc = check_k(k)) return rc;
    if (x_row_stride_elems < k) return PQ2_ESHAPE;
    const int esize = dtype == PQ2_F32 ? 4 : 2;
    if (!aligned(x, esize) || !aligned(q, 8) || !aligned(xs, 4)) return PQ2_EALIGN;
    const size_t xbytes = ((size_t)(m - 1) * x_row_stride_elems + k) * esize;
    if (overlap(q, (size_t)m * k, x, xbytes) || overlap(xs, (size_t)m * (k / kGroup) * 4, x, xbytes) ||
        overlap(q, (size_t)m * k, xs, (size_t)m * (k / kGroup) * 4))
        return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_quantize(x, dtype, x_row_stride_elems, m, k, q, xs, (hipStream_t)stream));
}

int pq2_gemv_tiles(const void* x, int dtype, int64_t x_row_stride_elems, const void* tiles, int64_t m, int64_t n,
                   int64_t k, float* y, int8_t* q_work, float* xs_work, void* stream) {
    // The single launch repeats the quantisation in every 16-row tile; the
    // two-launch path pays a second launch (about 2 us in a graph).  The
    // fused launch wins while m * tiles is small and every wave holds one
    // segment (K = 5120: qkv 5.2 against 6.8 us at one column and 6.3
    // against 6.8 at two; up 6.9 against 8.3 at one column, but 9.2 against
    // 8.5 at two, m * tiles = 2176).  Both give the same bits.  x that the
    // fused kernel cannot read (not 16-byte aligned rows, or a span of 2^31
    // bytes or more) takes the two-launch path when scratch is given.
    if (m <= 2 && k <= 8192 && m * ((n + 15) / 16) <= 1600) {
        const int esize = dtype == PQ2_F32 ? 4 : 2;
        const bool fused_ok = x && aligned(x, 16) && (x_row_stride_elems * esize) % 16 == 0 && m >= 1 &&
                              x_row_stride_elems >= k &&
                              ((size_t)(m - 1) * x_row_stride_elems + k) * esize < ((size_t)1 << 31);
        if (fused_ok || !q_work || !xs_work)
            return pq2_matmul_small_m_tiles_fused(x, dtype, x_row_stride_elems, tiles, m, n, k, y, stream);
    }
    if (!x || !q_work || !xs_work) return PQ2_EINVAL;
    if (dtype != PQ2_BF16 && dtype != PQ2_F16 && dtype != PQ2_F32) return PQ2_EINVAL;
    if (int rc = check_matmul_args(q_work, xs_work, tiles, m, n, k, y, PQ2_MAX_SMALL_M, true)) return rc;
    if (x_row_stride_elems < k) return PQ2_ESHAPE;
    const int esize = dtype == PQ2_F32 ? 4 : 2;
    if (!aligned(x, esize)) return PQ2_EALIGN;
    const size_t xbytes = ((size_t)(m - 1) * x_row_stride_elems + k) * esize;
    const size_t qbytes = (size_t)m * k, sbytes = (size_t)m * (k / kGroup) * 4, ybytes = (size_t)m * n * 4;
    if (overlap(q_work, qbytes, x, xbytes) || overlap(xs_work, sbytes, x, xbytes) ||
        overlap(q_work, qbytes, xs_work, sbytes) || overlap(y, ybytes, x, xbytes) ||
        overlap(q_work, qbytes, tiles, (size_t)pq2::tiles_bytes(n, k)) ||
        overlap(xs_work, sbytes, tiles, (size_t)pq2::tiles_bytes(n, k)))
        return PQ2_EINVAL;
    if (int rc = pq2_quantize_act_i8(x, dtype, x_row_stride_elems, m, k, q_work, xs_work, stream)) return rc;
    return pq2_matmul_small_m_tiles(q_work, xs_work, tiles, m, n, k, y, stream);
}

int64_t pq2_tiles_splitk_partial_floats(int64_t m, int64_t n, int64_t k) {
    if (m < 1 || m > PQ2_MAX_SMALL_M || n < 1 || n > kMaxN || check_k(k)) return -1;
    return pq2::splitk_plan(m, n, k, pq2::kSplitKDefaultWaves).partial_floats;
}

int64_t pq2_tiles_splitk_counter_words(int64_t n) {
    if (n < 1 || n > kMaxN) return -1;
    return (int64_t)pq2::kSplitKMaxChunks * ((n + 15) / 16);
}

int pq2_matmul_small_m_tiles_splitk_tuned(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                                          int64_t k, float* y, float* partials, uint32_t* counters, int waves,
                                          void* stream) {
    if (int rc = check_matmul_args(q, xs, tiles, m, n, k, y, PQ2_MAX_SMALL_M, true)) return rc;
    if (!partials || !counters) return PQ2_EINVAL;
    if (waves < 0 || waves > 16) return PQ2_EINVAL;
    if (!aligned(partials, 4) || !aligned(counters, 4)) return PQ2_EALIGN;
    const size_t pbytes = (size_t)pq2_tiles_splitk_partial_floats(m, n, k) * 4;
    const size_t cbytes = (size_t)pq2_tiles_splitk_counter_words(n) * 4;
    const size_t tbytes = (size_t)pq2::tiles_bytes(n, k);
    const void* bufs[5] = {partials, counters, y, q, xs};
    const size_t lens[5] = {pbytes, cbytes, (size_t)m * n * 4, (size_t)m * k, (size_t)m * (k / kGroup) * 4};
    for (int i = 0; i < 2; ++i) {
        if (overlap(bufs[i], lens[i], tiles, tbytes)) return PQ2_EINVAL;
        for (int j = i + 1; j < 5; ++j)
            if (overlap(bufs[i], lens[i], bufs[j], lens[j])) return PQ2_EINVAL;
    }
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_small_m_tiles_splitk(q, xs, static_cast<const uint8_t*>(tiles), m, n, k, y,
                                                          partials, counters,
                                                          waves ? waves : pq2::kSplitKDefaultWaves,
                                                          (hipStream_t)stream));
}

int pq2_matmul_small_m_tiles_splitk(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                                    int64_t k, float* y, float* partials, uint32_t* counters, void* stream) {
    return pq2_matmul_small_m_tiles_splitk_tuned(q, xs, tiles, m, n, k, y, partials, counters, 0, stream);
}

int64_t pq2_stream_probe_words(int64_t workgroups) {
    if (workgroups < 1 || workgroups > 65536) return 0;
    return workgroups * 4;
}

int pq2_stream_probe(const void* buf, int64_t bytes, int64_t workgroups, int store_all, uint32_t sentinel,
                     uint32_t* out, void* stream) {
    return pq2_stream_probe_cfg(buf, bytes, workgroups, 4, 1, PQ2_STREAM_BUFFER_NT, store_all, sentinel, out,
                                stream);
}

int pq2_stream_probe_cfg(const void* buf, int64_t bytes, int64_t workgroups, int waves, int loads_per_lane,
                         int policy, int store_all, uint32_t sentinel, uint32_t* out, void* stream) {
    if (!buf || !out || policy < PQ2_STREAM_BUFFER || policy > PQ2_STREAM_LDS_NT) return PQ2_EINVAL;
    const int u = loads_per_lane;
    if (bytes < 16 || bytes % 16 || bytes >= ((int64_t)1 << 31) || workgroups < 1 || workgroups > 65536 ||
        waves < 1 || waves > 16 || (u != 1 && u != 2 && u != 4 && u != 8 && u != 16) || waves * u > 64 ||
        workgroups * waves * u * 1024 > ((int64_t)1 << 30) || (policy >= PQ2_STREAM_LDS && bytes % 1024))
        return PQ2_ESHAPE;
    if (!aligned(buf, 16) || !aligned(out, 4)) return PQ2_EALIGN;
    if (overlap(out, (size_t)(workgroups * waves) * 4, buf, (size_t)bytes)) return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_stream_probe(static_cast<const uint8_t*>(buf), bytes, workgroups, waves, u,
                                                  policy, store_all ? 1 : 0, sentinel, out, (hipStream_t)stream));
}

int pq2_empty_probe(int64_t workgroups, int waves, void* stream) {
    if (workgroups < 1 || workgroups > ((int64_t)1 << 20) || waves < 1 || waves > 16) return PQ2_ESHAPE;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_empty_probe(workgroups, waves, (hipStream_t)stream));
}

int pq2_gemv_tiles_static(const void* x, int dtype, int64_t x_row_stride_elems, const void* tiles, int64_t m,
                          int64_t n, int64_t k, float* y, void* stream) {
    if (m < 1 || m > PQ2_MAX_SMALL_M || n < 1 || n > kMaxN) return PQ2_ESHAPE;
    if (int rc = check_k(k)) return rc;
    if ((size_t)m * k > kStaticQBytes || (size_t)m * (k / kGroup) * 4 > kStaticXsBytes) return PQ2_ESHAPE;
    if (int rc = check_device()) return rc;
    void* base = nullptr;
    if (int rc = scratch_address(&base)) return rc;
    int8_t* q_work = static_cast<int8_t*>(base);
    float* xs_work = reinterpret_cast<float*>(static_cast<unsigned char*>(base) + kStaticQBytes);
    return pq2_gemv_tiles(x, dtype, x_row_stride_elems, tiles, m, n, k, y, q_work, xs_work, stream);
}

int pq2_quantize_act_i8_g(const void* x, int dtype, int64_t x_row_stride_elems, int64_t m, int64_t k,
                          int64_t agroup, int8_t* q, float* xs, void* stream) {
    if (!x || !q || !xs) return PQ2_EINVAL;
    if (dtype != PQ2_BF16 && dtype != PQ2_F16 && dtype != PQ2_F32) return PQ2_EINVAL;
    if (agroup != 128 && agroup != 64 && agroup != 32) return PQ2_EINVAL;
    if (m < 1 || m > ((int64_t)1 << 31)) return PQ2_ESHAPE;
    if (int rc = check_k(k)) return rc;
    if (x_row_stride_elems < k) return PQ2_ESHAPE;
    const int esize = dtype == PQ2_F32 ? 4 : 2;
    if (!aligned(x, esize) || !aligned(q, 8) || !aligned(xs, 4)) return PQ2_EALIGN;
    const size_t xbytes = ((size_t)(m - 1) * x_row_stride_elems + k) * esize;
    const size_t sbytes = (size_t)m * (k / agroup) * 4;
    if (overlap(q, (size_t)m * k, x, xbytes) || overlap(xs, sbytes, x, xbytes) || overlap(q, (size_t)m * k, xs, sbytes))
        return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(
        pq2::launch_quantize_g(x, dtype, x_row_stride_elems, m, k, (int)agroup, q, xs, (hipStream_t)stream));
}

int pq2_matmul_small_m_tiles_g(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n, int64_t k,
                               int64_t agroup, float* y, void* stream) {
    if (agroup != 128 && agroup != 64 && agroup != 32) return PQ2_EINVAL;
    if (int rc = check_matmul_args(q, xs, tiles, m, n, k, y, PQ2_MAX_SMALL_M, true)) return rc;
    if (overlap(y, (size_t)m * n * 4, xs, (size_t)m * (k / agroup) * 4)) return PQ2_EINVAL;
    const int waves = pq2::kTilesDefaultWaves;
    const int split = pq2::tiles_default_split(m, k, waves);
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_small_m_tiles_g(q, xs, static_cast<const uint8_t*>(tiles), m, n, k, (int)agroup,
                                                     y, waves, split, (hipStream_t)stream));
}

int pq2_matmul_small_m_tiles_fused_g(const void* x, int dtype, int64_t x_row_stride_elems, const void* tiles,
                                     int64_t m, int64_t n, int64_t k, int64_t agroup, float* y, void* stream) {
    if (agroup != 128 && agroup != 64 && agroup != 32) return PQ2_EINVAL;
    if (int rc = check_tiles_fused_args(x, dtype, x_row_stride_elems, tiles, m, n, k, y)) return rc;
    const int waves = pq2::kTilesDefaultWaves;
    const int split = pq2::tiles_default_split(m, k, waves);
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_small_m_tiles_fused_g(x, dtype, x_row_stride_elems,
                                                           static_cast<const uint8_t*>(tiles), m, n, k, (int)agroup,
                                                           y, waves, split, (hipStream_t)stream));
}

int pq2_quantize_act_i8_planes(const void* x, int dtype, int64_t x_row_stride_elems, int64_t m, int64_t k,
                               int8_t* qp, float* xs, int32_t* qsum, void* stream) {
    if (!x || !qp || !xs || !qsum) return PQ2_EINVAL;
    if (dtype != PQ2_BF16 && dtype != PQ2_F16 && dtype != PQ2_F32) return PQ2_EINVAL;
    if (m < 1 || m > ((int64_t)1 << 31)) return PQ2_ESHAPE;
    if (int rc = check_k(k)) return rc;
    if (x_row_stride_elems < k) return PQ2_ESHAPE;
    const int esize = dtype == PQ2_F32 ? 4 : 2;
    if (!aligned(x, esize) || !aligned(qp, 16) || !aligned(xs, 4) || !aligned(qsum, 4)) return PQ2_EALIGN;
    const size_t xbytes = ((size_t)(m - 1) * x_row_stride_elems + k) * esize;
    const size_t qbytes = (size_t)m * k, gbytes = (size_t)m * (k / kGroup) * 4;
    if (overlap(qp, qbytes, x, xbytes) || overlap(xs, gbytes, x, xbytes) || overlap(qsum, gbytes, x, xbytes) ||
        overlap(qp, qbytes, xs, gbytes) || overlap(qp, qbytes, qsum, gbytes) || overlap(xs, gbytes, qsum, gbytes))
        return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(
        pq2::launch_quantize_planes(x, dtype, x_row_stride_elems, m, k, qp, xs, qsum, (hipStream_t)stream));
}

int pq2_matmul_small_m_planes_tuned(const int8_t* qp, const float* xs, const int32_t* qsum, const void* planes,
                                    int64_t m, int64_t n, int64_t k, float* y, int rows,
                                    int max_waves, int engine, void* stream) {
    if (!qsum) return PQ2_EINVAL;
    if (int rc = check_matmul_args(qp, xs, planes, m, n, k, y, PQ2_MAX_SMALL_M)) return rc;
    if (!aligned(qsum, 4)) return PQ2_EALIGN;
    if (overlap(y, (size_t)m * n * 4, qsum, (size_t)m * (k / kGroup) * 4)) return PQ2_EINVAL;
    pq2::SmallMConfig cfg;
    if (int rc = small_m_config(pq2::kSrcPlanes, m, n, k, rows, max_waves, engine, &cfg)) return rc;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_small_m_planes(qp, xs, qsum, static_cast<const uint8_t*>(planes), m, n, k, y,
                                                    cfg, (hipStream_t)stream));
}

int pq2_matmul_small_m_planes(const int8_t* qp, const float* xs, const int32_t* qsum, const void* planes,
                              int64_t m, int64_t n, int64_t k, float* y, void* stream) {
    return pq2_matmul_small_m_planes_tuned(qp, xs, qsum, planes, m, n, k, y, 0, 0, 0, stream);
}

int pq2_matmul_small_m_tuned(const int8_t* q, const float* xs, const void* planes, int64_t m,
                             int64_t n, int64_t k, float* y, int rows, int max_waves, int engine,
                             void* stream) {
    if (int rc = check_matmul_args(q, xs, planes, m, n, k, y, PQ2_MAX_SMALL_M)) return rc;
    pq2::SmallMConfig cfg;
    if (int rc = small_m_config(pq2::kSrcNatural, m, n, k, rows, max_waves, engine, &cfg)) return rc;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_small_m(q, xs, static_cast<const uint8_t*>(planes), m, n, k, y, cfg,
                                             (hipStream_t)stream));
}

int pq2_matmul_small_m(const int8_t* q, const float* xs, const void* planes, int64_t m, int64_t n,
                       int64_t k, float* y, void* stream) {
    return pq2_matmul_small_m_tuned(q, xs, planes, m, n, k, y, 0, 0, 0, stream);
}

int64_t pq2_read_probe_words(int layout, int64_t n, int64_t k) {
    if ((layout != PQ2_LAYOUT_PLANES && layout != PQ2_LAYOUT_TILES) || n < 1 || n > kMaxN || check_k(k)) return 0;
    return pq2::read_probe_words(layout, n, k);
}

int pq2_read_probe(const void* weights, int layout, int64_t n, int64_t k, uint32_t* out, void* stream) {
    if (!weights || !out) return PQ2_EINVAL;
    if (layout != PQ2_LAYOUT_PLANES && layout != PQ2_LAYOUT_TILES) return PQ2_EINVAL;
    if (n < 1 || n > kMaxN) return PQ2_ESHAPE;
    if (int rc = check_k(k)) return rc;
    if (!aligned(weights, 16) || !aligned(out, 4)) return PQ2_EALIGN;
    const size_t wbytes = layout == PQ2_LAYOUT_TILES ? (size_t)pq2::tiles_bytes(n, k) : (size_t)n * (k / kGroup) * 34;
    if (overlap(out, (size_t)pq2::read_probe_words(layout, n, k) * 4, weights, wbytes)) return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(
        pq2::launch_read_probe(static_cast<const uint8_t*>(weights), layout, n, k, out, (hipStream_t)stream));
}

int pq2_matmul_small_m_raw(const int8_t* q, const float* xs, const void* raw, int64_t raw_row_stride_bytes, int64_t m,
                           int64_t n, int64_t k, float* y, void* stream) {
    if (!q || !xs || !raw || !y) return PQ2_EINVAL;
    if (m < 1 || m > PQ2_MAX_SMALL_M || n < 1 || n > kMaxN) return PQ2_ESHAPE;
    if (int rc = check_k(k)) return rc;
    const int64_t row_bytes = k / kGroup * 34;
    if (raw_row_stride_bytes < row_bytes || (raw_row_stride_bytes & 1) || raw_row_stride_bytes > kMaxRawStride)
        return PQ2_ESHAPE;
    if (!aligned(q, 16) || !aligned(xs, 4) || !aligned(raw, 2) || !aligned(y, 4)) return PQ2_EALIGN;
    const size_t ybytes = (size_t)m * n * 4;
    if (overlap(y, ybytes, q, (size_t)m * k) || overlap(y, ybytes, xs, (size_t)m * (k / kGroup) * 4) ||
        overlap(y, ybytes, raw, (size_t)(n - 1) * raw_row_stride_bytes + row_bytes))
        return PQ2_EINVAL;
    const pq2::SmallMConfig cfg = pq2::default_small_m_config(pq2::kSrcNatural, m, n, k);
    const int rows = pq2::default_small_m_rows(1, pq2::kSrcNatural, m, n, k, cfg.max_waves);
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_small_m_raw(q, xs, static_cast<const uint8_t*>(raw), raw_row_stride_bytes, m, n,
                                                 k, y, cfg.max_waves, rows, (hipStream_t)stream));
}

int pq2_matmul_small_m_fused_tuned(const void* x, int dtype, int64_t x_row_stride_elems, const void* planes,
                                   int64_t m, int64_t n, int64_t k, float* y, int rows, int max_waves,
                                   int engine, void* stream) {
    if (!x || !planes || !y) return PQ2_EINVAL;
    if (dtype != PQ2_BF16 && dtype != PQ2_F16 && dtype != PQ2_F32) return PQ2_EINVAL;
    if (m < 1 || m > PQ2_MAX_SMALL_M || n < 1 || n > kMaxN) return PQ2_ESHAPE;
    if (int rc = check_k(k)) return rc;
    if (x_row_stride_elems < k) return PQ2_ESHAPE;
    const int esize = dtype == PQ2_F32 ? 4 : 2;
    const size_t xbytes = ((size_t)(m - 1) * x_row_stride_elems + k) * esize;
    if (xbytes >= ((size_t)1 << 31)) return PQ2_ESHAPE;  // the kernel addresses x with 32-bit offsets
    if (!aligned(x, 16) || (x_row_stride_elems * esize) % 16 || !aligned(planes, 16) || !aligned(y, 4))
        return PQ2_EALIGN;
    const size_t ybytes = (size_t)m * n * 4;
    if (overlap(y, ybytes, x, xbytes) || overlap(y, ybytes, planes, (size_t)n * (k / kGroup) * 34))
        return PQ2_EINVAL;
    pq2::SmallMConfig cfg;
    if (int rc = small_m_config(pq2::src_of_dtype(dtype), m, n, k, rows, max_waves, engine, &cfg)) return rc;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_small_m_fused(x, dtype, x_row_stride_elems, static_cast<const uint8_t*>(planes),
                                                   m, n, k, y, cfg, (hipStream_t)stream));
}

int pq2_matmul_small_m_fused(const void* x, int dtype, int64_t x_row_stride_elems, const void* planes, int64_t m,
                             int64_t n, int64_t k, float* y, void* stream) {
    return pq2_matmul_small_m_fused_tuned(x, dtype, x_row_stride_elems, planes, m, n, k, y, 0, 0, 0, stream);
}

int pq2_matmul_prefill_tuned(const int8_t* q, const float* xs, const void* planes, int64_t m, int64_t n,
                             int64_t k, float* y, int tile, void* stream) {
    if (int rc = check_matmul_args(q, xs, planes, m, n, k, y, kMaxPrefillM)) return rc;
    if (tile < 0 || tile > 5) return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_prefill(q, xs, static_cast<const uint8_t*>(planes), m, n, k, y, tile, false,
                                             (hipStream_t)stream));
}

int pq2_matmul_prefill_tiles_tuned(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                                   int64_t k, float* y, int tile, void* stream) {
    if (int rc = check_matmul_args(q, xs, tiles, m, n, k, y, kMaxPrefillM, true)) return rc;
    if (tile < 0 || tile > 5) return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_prefill_tiles(q, xs, static_cast<const uint8_t*>(tiles), m, n, k, y, tile,
                                                   (hipStream_t)stream));
}

int pq2_matmul_prefill_tiles(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                             int64_t k, float* y, void* stream) {
    return pq2_matmul_prefill_tiles_tuned(q, xs, tiles, m, n, k, y, 0, stream);
}

int pq2_matmul_prefill_tiles_g(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n, int64_t k,
                               int64_t agroup, float* y, void* stream) {
    if (agroup != 128 && agroup != 64 && agroup != 32) return PQ2_EINVAL;
    if (int rc = check_matmul_args(q, xs, tiles, m, n, k, y, kMaxPrefillM, true)) return rc;
    if (overlap(y, (size_t)m * n * 4, xs, (size_t)m * (k / agroup) * 4)) return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_prefill_tiles_g(q, xs, static_cast<const uint8_t*>(tiles), m, n, k, y, 0,
                                                     (int)agroup, (hipStream_t)stream));
}

int pq2_matmul_prefill(const int8_t* q, const float* xs, const void* planes, int64_t m, int64_t n,
                       int64_t k, float* y, void* stream) {
    return pq2_matmul_prefill_tuned(q, xs, planes, m, n, k, y, 0, stream);
}

int pq2_matmul_prefill_planes_tuned(const int8_t* qp, const float* xs, const void* planes, int64_t m, int64_t n,
                                    int64_t k, float* y, int tile, void* stream) {
    if (int rc = check_matmul_args(qp, xs, planes, m, n, k, y, kMaxPrefillM)) return rc;
    if (tile < 0 || tile > 5) return PQ2_EINVAL;
    if (int rc = check_device()) return rc;
    return launch_status(pq2::launch_prefill(qp, xs, static_cast<const uint8_t*>(planes), m, n, k, y, tile, true,
                                             (hipStream_t)stream));
}

int pq2_matmul_prefill_planes(const int8_t* qp, const float* xs, const void* planes, int64_t m, int64_t n,
                              int64_t k, float* y, void* stream) {
    return pq2_matmul_prefill_planes_tuned(qp, xs, planes, m, n, k, y, 0, stream);
}

}  // extern "C"
