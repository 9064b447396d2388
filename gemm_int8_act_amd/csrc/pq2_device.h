// pq2_device.h -- device-side helpers shared by the gfx950 kernels of libpq2.
//
// Wave64 cross-lane primitives (DPP), the byte transpose that puts INT8
// activations into code-plane order, and the two exact 2-bit decodes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pq2 {

// ---------------------------------------------------------------- DPP
// dpp_ctrl encodings (GFX9 DPP): quad_perm [1,0,3,2] swaps neighbours,
// [2,3,0,1] swaps pairs, row_half_mirror reverses each 8-lane half-row,
// row_mirror reverses each 16-lane row.
enum : int {
    kDppXor1 = 0xB1,
    kDppXor2 = 0x4E,
    kDppHalfMirror = 0x141,
    kDppMirror = 0x140,
};

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 8 lanes; every lane of the group gets the
// same value (each step pairs a with b and b with a, and FP addition is
// commutative, so partner lanes agree bit for bit).
__device__ __forceinline__ float sum8_f(float v) {
#pragma clang fp contract(off)
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    return v;
}

__device__ __forceinline__ int sum8_i(int v) {
    v += dpp_i<kDppXor1>(v);
    v += dpp_i<kDppXor2>(v);
    v += dpp_i<kDppHalfMirror>(v);
    return v;
}

// Max over each aligned group of 8 lanes; all lanes of the group agree.
__device__ __forceinline__ float max8_f(float v) {
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    return v;
}

// Max over each aligned group of 16 lanes (one DPP row); all lanes agree.
__device__ __forceinline__ float max16_f(float v) {
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    return v;
}

// ---------------------------------------------------------------- dot4
// Signed 4 x int8 dot product accumulated into a signed int32 (v_dot4_i32_i8).
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int acc) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, acc, false);
}

// ---------------------------------------------------------------- plane order
// A code dword (4 code bytes = 16 consecutive weights 16t..16t+15 of a block)
// splits into four planes: plane s holds weights 16t+4j+s, j = 0..3, one per
// byte.  The matching activation dword holds q[16t+4j+s] in byte j, i.e. byte
// s of each of the four natural-order activation dwords Q0..Q3 = a 4x4 byte
// transpose.  __builtin_amdgcn_perm(hi, lo, sel): result byte i is byte
// sel.i of the 8-byte value {hi:lo} (selector 0..3 = lo, 4..7 = hi).
__device__ __forceinline__ uint4 to_plane_order(uint4 Q) {
    const uint32_t l01 = __builtin_amdgcn_perm(Q.y, Q.x, 0x05010400u);  // Q0b0 Q1b0 Q0b1 Q1b1
    const uint32_t h01 = __builtin_amdgcn_perm(Q.y, Q.x, 0x07030602u);  // Q0b2 Q1b2 Q0b3 Q1b3
    const uint32_t l23 = __builtin_amdgcn_perm(Q.w, Q.z, 0x05010400u);
    const uint32_t h23 = __builtin_amdgcn_perm(Q.w, Q.z, 0x07030602u);
    uint4 P;
    P.x = __builtin_amdgcn_perm(l23, l01, 0x05040100u);  // byte 0 of Q0..Q3
    P.y = __builtin_amdgcn_perm(l23, l01, 0x07060302u);  // byte 1
    P.z = __builtin_amdgcn_perm(h23, h01, 0x05040100u);  // byte 2
    P.w = __builtin_amdgcn_perm(h23, h01, 0x07060302u);  // byte 3
    return P;
}

// ---------------------------------------------------------------- decodes
// Masked planes: byte values c * 4^S for S = 0,1,2 and, for S = 3, the field
// shifted down by two (c * 16) so every byte stays below 128.
template <int S>
__device__ __forceinline__ uint32_t mask_plane(uint32_t d) {
    if constexpr (S == 0) return d & 0x03030303u;
    if constexpr (S == 1) return d & 0x0C0C0C0Cu;
    if constexpr (S == 2) return d & 0x30303030u;
    return (d >> 2) & 0x30303030u;
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer resources (gfx9 descriptor, stride 0): a load whose byte offset
// lies at or beyond num_records returns zero instead of touching memory, so
// padded rows, groups and columns need no branch around their loads.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kBufferOOB = 0x80000000u;  // an offset past any record count used here
constexpr int kBufferFlags = 0x00020000;
constexpr int kAuxNonTemporal = 2;          // cache-policy bit: streamed, not reused

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

template <int AUX = 0>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The same with a uniform byte offset in the instruction's scalar operand
// (no per-lane add for an offset shared by the wave).
template <int AUX = 0>
__device__ __forceinline__ uint4 buf_load16s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, AUX);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return make_uint2(v.x, v.y);
}

__device__ __forceinline__ uint2 buf_load8s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, 0);
    return make_uint2(v.x, v.y);
}

__device__ __forceinline__ uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

// Scalar buffer loads (uniform offset, results in SGPRs): the same range
// check, dword by dword, without a slot in the vector memory queue.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
extern "C" __device__ float pq2_sbuf_load_f32(i32x4_t rsrc, int off, int aux) __asm("llvm.amdgcn.s.buffer.load.f32");
extern "C" __device__ f32x2_t pq2_sbuf_load_f32x2(i32x4_t rsrc, int off, int aux) __asm("llvm.amdgcn.s.buffer.load.v2f32");
extern "C" __device__ f32x4_t pq2_sbuf_load_f32x4(i32x4_t rsrc, int off, int aux) __asm("llvm.amdgcn.s.buffer.load.v4f32");
extern "C" __device__ f32x8_t pq2_sbuf_load_f32x8(i32x4_t rsrc, int off, int aux) __asm("llvm.amdgcn.s.buffer.load.v8f32");

__device__ __forceinline__ i32x4_t make_srsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4_t{(int)(uint32_t)a, (int)((a >> 32) & 0xFFFFu), (int)bytes, kBufferFlags};
}

// N = 1, 2, 4 or 8 consecutive floats at byte offset off (a multiple of 4).
template <int N>
__device__ __forceinline__ void sbuf_load_f32(i32x4_t r, int off, float* out) {
    if constexpr (N == 8) {
        const f32x8_t v = pq2_sbuf_load_f32x8(r, off, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = v[i];
    } else if constexpr (N == 4) {
        const f32x4_t v = pq2_sbuf_load_f32x4(r, off, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = v[i];
    } else if constexpr (N == 2) {
        const f32x2_t v = pq2_sbuf_load_f32x2(r, off, 0);
        out[0] = v[0];
        out[1] = v[1];
    } else {
        out[0] = pq2_sbuf_load_f32(r, off, 0);
    }
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

}  // namespace pq2
