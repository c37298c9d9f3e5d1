// Device helpers shared by the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq8 {

typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer resources: one 128-bit scalar descriptor per array, so a load is
// a lane offset (VGPR) plus a wave-uniform offset (SGPR) and no per-lane
// 64-bit address has to be kept live. The plan keeps every array below 2^31
// bytes, so 32-bit offsets cover them; an offset past the end reads zero.
constexpr int kBufferFlags = 0x00020000;  // gfx9 dword 3: 32-bit raw buffer
constexpr int kOob = 0x7ffffff0;           // an offset beyond every such array
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, kBufferFlags);
}

// The dispatcher hands workgroup b to XCD b % 8, and each XCD has its own L2.
// Renumbering so that XCD x runs one contiguous range of logical blocks puts
// neighbouring work items (which share input rows or operand panels) behind
// the same L2. The map is a bijection on [0, nb) for any nb.
__device__ __forceinline__ int xcd_block(int b, int nb) {
    constexpr int kXcd = 8;
    const int q = nb / kXcd, r = nb % kXcd, x = b % kXcd;
    return x * q + min(x, r) + b / kXcd;
}

// x + 1.5 * 2^23 rounds x (|x| < 2^22) to an integer with ties to even, which
// is rint(x); the low byte of the sum's bits is that integer in two's
// complement. Codes here satisfy |x| <= 127 (1 + 2^-24)^2 < 127.5, so the
// clamp to +-127 never binds.
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

// Four codes (low byte of each float's bits) -> one dword, byte k = x[k].
__device__ __forceinline__ uint32_t pack4(float x0, float x1, float x2, float x3) {
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(x3), __float_as_uint(x2), 0x04000c0cu);
    return lo | hi;
}

__device__ __forceinline__ float load_act(const float *p) { return *p; }
__device__ __forceinline__ float load_act(const uint16_t *p) {
    return __uint_as_float((uint32_t)(*p) << 16);  // bf16 -> f32, exact
}
__device__ __forceinline__ void store_act(float *p, float v) { *p = v; }
__device__ __forceinline__ uint16_t to_bf16(float v) {
    const uint32_t u = __float_as_uint(v);  // f32 -> bf16, nearest even (finite input)
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ void store_act(uint16_t *p, float v) { *p = to_bf16(v); }
// Two adjacent outputs; p must be aligned to the pair's size.
__device__ __forceinline__ void store_act2(float *p, float a, float b) { *(float2 *)p = float2{a, b}; }
__device__ __forceinline__ void store_act2(uint16_t *p, float a, float b) {
    *(uint32_t *)p = (uint32_t)to_bf16(a) | (uint32_t)to_bf16(b) << 16;
}

}  // namespace wq8
