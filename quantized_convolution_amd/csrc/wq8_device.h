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


// Max over aligned segments of SEG lanes (SEG a power of two <= 64).
template <int SEG>
__device__ __forceinline__ float seg_max(float a) {
#pragma unroll
    for (int s = 1; s < SEG; s <<= 1) a = fmaxf(a, __shfl_xor(a, s));
    return a;
}

// --------------------------------------------------- per-channel transforms
// Each lane owns one channel; a group of G channels spans SEG lanes of one
// wave, or GW whole waves when G > 64. The block (256 threads) holds TPB
// "rows" (tiles for stage 1, output channels for the weights).
template <int G>
struct GroupShape {
    static constexpr int GW = G > 64 ? G / 64 : 1;   // waves per group
    static constexpr int TPB = 4 / GW;               // rows per block
    static constexpr int SEG = G < 64 ? G : 64;      // lanes reduced in-wave
    static constexpr int CPB = 64 * GW;              // channels per block
};

// The group maxima are taken on bit patterns of |v|: non-negative floats
// order like their unsigned bit patterns, so an integer max gives the float
// max. (A float max of values that arrive through the integer cross-lane
// moves would first have to quiet possible signalling NaNs, one more
// instruction per operand.)

// Reduce-scatter steps: pair value i with value i + K/2 (values come from
// src(i)); each lane keeps one half, a[i] for i < K/2 (the max over itself and
// its partner), and returns 1 if it kept the upper half.
template <int K, typename F>
__device__ __forceinline__ int rs_swap32(uint32_t (&a)[64], F src) {
#pragma unroll
    for (int i = 0; i < K / 2; ++i) {
        auto r = __builtin_amdgcn_permlane32_swap(src(i), src(i + K / 2), false, false);
        a[i] = max(r[0], r[1]);
    }
    auto lab = __builtin_amdgcn_permlane32_swap(0u, 1u, false, false);
    return (int)lab[0];
}

template <int K, typename F>
__device__ __forceinline__ int rs_swap16(uint32_t (&a)[64], F src) {
#pragma unroll
    for (int i = 0; i < K / 2; ++i) {
        auto r = __builtin_amdgcn_permlane16_swap(src(i), src(i + K / 2), false, false);
        a[i] = max(r[0], r[1]);
    }
    auto lab = __builtin_amdgcn_permlane16_swap(0u, 1u, false, false);
    return (int)lab[0];
}

// DPP exchange with the lane given by CTRL; BIT is a lane-id bit that differs
// between partners and decides which half a lane keeps.
template <int K, int CTRL, int BIT, typename F>
__device__ __forceinline__ int rs_dpp(uint32_t (&a)[64], int lane, F src) {
    const bool up = (lane >> BIT) & 1;
#pragma unroll
    for (int i = 0; i < K / 2; ++i) {
        const uint32_t lo = src(i), hi = src(i + K / 2);
        const uint32_t send = up ? lo : hi, keep = up ? hi : lo;
        // old value 0 (the identity of the max) lets the move fold into the max
        const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, CTRL, 0xf, 0xf, false);
        a[i] = max(keep, recv);
    }
    return up;
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppXor7 = 0x141;       // row_half_mirror: lane ^ 7 inside 8 lanes
constexpr int kDppXor8 = 0x128;       // row_ror:8: lane ^ 8 inside 16 lanes

// Max over SEG aligned lanes, for 64 values per lane (bit patterns of
// non-negative floats, value i = src(i)); the first step reads src, so the
// caller need not hold a copy of all 64. On return a[j], j < 64/SEG, holds
// the max for value index base + j (base is returned).
template <int SEG, typename F>
__device__ __forceinline__ int reduce_scatter_max(uint32_t (&a)[64], int lane, F src) {
    const auto in = [&](int i) { return a[i]; };
    int base = 0;
    if constexpr (SEG == 64) {
        base += rs_swap32<64>(a, src) * 32;
        base += rs_swap16<32>(a, in) * 16;
        base += rs_dpp<16, kDppXor8, 3>(a, lane, in) * 8;
        base += rs_dpp<8, kDppXor7, 2>(a, lane, in) * 4;
        base += rs_dpp<4, kDppXor2, 1>(a, lane, in) * 2;
        base += rs_dpp<2, kDppXor1, 0>(a, lane, in);
    } else if constexpr (SEG == 32) {
        base += rs_swap16<64>(a, src) * 32;
        base += rs_dpp<32, kDppXor8, 3>(a, lane, in) * 16;
        base += rs_dpp<16, kDppXor7, 2>(a, lane, in) * 8;
        base += rs_dpp<8, kDppXor2, 1>(a, lane, in) * 4;
        base += rs_dpp<4, kDppXor1, 0>(a, lane, in) * 2;
    } else {
        static_assert(SEG == 16, "group lanes must be 16, 32 or 64");
        base += rs_dpp<64, kDppXor8, 3>(a, lane, src) * 32;
        base += rs_dpp<32, kDppXor7, 2>(a, lane, in) * 16;
        base += rs_dpp<16, kDppXor2, 1>(a, lane, in) * 8;
        base += rs_dpp<8, kDppXor1, 0>(a, lane, in) * 4;
    }
    return base;
}

// Stage-1 quantizer for one lane's NT transformed values (one channel of one
// tile): the absmax of each (tap, group) over the group's lanes (a
// reduce-scatter leaves each lane the max of 64/SEG taps; for groups over
// several waves the per-wave maxima meet in `red`), then per (tap, group) the
// IEEE divisions 127/a and a/127 once, the scale stored by the group's first
// wave, the reciprocals passed to the group's lanes through `inv_lds`, and
// each value rounded with x + 1.5*2^23 (its low byte is rint(x)) and stored as
// a code. Codes go to Vq[tap][t][c] (tap stride `plane` bytes), scales to
// sV[tap][t][c / G] (tap stride `splane` floats). A lane with `skip` only
// meets the barriers (the waves of one group skip together); `ok` = the lane's
// channel exists. Holds one block barrier (two for groups over several waves),
// so every wave of the block calls it.
template <int NT, int G, int NW>
__device__ __forceinline__ void s1_quantize_store(const float (&v)[NT], bool skip, bool ok, int wave, int lane,
                                                  int c, int t, int Cin, int ng, int plane, int splane,
                                                  __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rs,
                                                  float (*red)[64],
                                                  float (*inv_lds)[64 / GroupShape<G>::SEG][64]) {
    using S = GroupShape<G>;
    constexpr int KF = 64 / S::SEG;  // taps per lane after the reduce-scatter
    const int seg = lane / S::SEG;
    // the maxima run on bit patterns of |v| (v itself is kept)
    uint32_t a[64];
    int base = 0;
    if (!skip)
        base = reduce_scatter_max<S::SEG>(
            a, lane, [&](int i) { return i < NT ? __float_as_uint(v[i]) & 0x7fffffffu : 0u; });
    if constexpr (S::GW > 1) {
        if (!skip)
#pragma unroll
            for (int j = 0; j < KF; ++j) red[wave][base + j] = __uint_as_float(a[j]);
        __syncthreads();
        const int w0 = (wave / S::GW) * S::GW;
        if (!skip)
#pragma unroll
            for (int j = 0; j < KF; ++j) {
                float m = red[w0][base + j];
#pragma unroll
                for (int k = 1; k < S::GW; ++k) m = fmaxf(m, red[w0 + k][base + j]);
                a[j] = __float_as_uint(m);
            }
    }
    if (!skip)
#pragma unroll
        for (int j = 0; j < KF; ++j) {
            const int tap = base + j;
            const float am = __uint_as_float(a[j]);
            float inv = 0.0f, sc = 0.0f;
            if (am != 0.0f) {
                inv = 127.0f / am;
                sc = am / 127.0f;
            }
            inv_lds[wave][seg][tap] = inv;
            if (ok && tap < NT && (S::GW == 1 || wave % S::GW == 0))
                // tap differs between lanes, so it goes in the vector offset
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rs, (tap * splane + t * ng + c / G) * 4,
                                                      0, 0);
        }
    __syncthreads();
    if (ok) {
        const int voff = t * Cin + c;
#pragma unroll
        for (int q4 = 0; q4 < (NT + 3) / 4; ++q4) {
            const float4 iv = *(const float4 *)&inv_lds[wave][seg][4 * q4];
            const float ivs[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tap = 4 * q4 + e;
                if (tap < NT) {
                    const float y = v[tap] * ivs[e] + kRoundMagic;
                    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)__float_as_uint(y), rq, voff, tap * plane, 0);
                }
            }
        }
    }
}

}  // namespace wq8
