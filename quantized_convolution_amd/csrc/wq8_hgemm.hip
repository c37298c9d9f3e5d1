// Stage 2 (staged schedule): the n*n Hadamard GEMMs over input channels on
// int8 MFMA with group dequantization into fp32 M.
//
//   P_g[tap][t][co] = sum_{c in group g} Vq[tap][t][c] Uq[tap][co][c]   (int32, exact)
//   M[tap][t][co]   = fp32 fma chain over g ascending of fl(sV sU) * P_g
//
// Block: one tap, BT = 16 RT tiles x BC = 16 CT NWV output channels. RT is
// chosen per layer so that the tiles need as little padding as possible (72
// tiles take 80 rows, 288 take 3 x 96). Each of the NWV waves owns 16 CT
// output channels and all BT tiles: RT x CT MFMA 16x16 blocks with U as the A
// operand (rows = output channels) and V as B (columns = tiles). A lane then
// holds 4 consecutive output channels of one tile, so its 4 weight scales are
// one 16-byte LDS read, its tile scale one 4-byte read, and its M values
// leave as one 16-byte store.
//
// Input channels run in chunks of KC = max(128, G) bytes per row (GPC whole
// groups; a chunk row is one cache line). The two operands travel differently:
//   - V (the tile rows, shared by every wave of the block and by every block
//     of the tap, mostly served by L2) is staged in LDS, double-buffered:
//     while the block computes chunk c, each thread holds chunk c+1 in
//     registers and writes it to the other buffer, then loads chunk c+2. The
//     chunk's group scales of V and U go the same way.
//   - U (the weights, 16 CT rows private to each wave and read once from
//     HBM) goes straight from global memory into registers, DU chunks ahead
//     (a ring of registers), so each wave keeps its next chunk's HBM round
//     trip in flight. A lane loads 16 contiguous bytes of its row per 64
//     bytes; for groups of 32 one permlane32 swap per 8 bytes then gives every
//     lane 8 bytes of each of the two groups in those 64 bytes.
//
// MFMA operand layout (16x16xK, int8): lane l holds row l % 16 of A / column
// l % 16 of B and 8 (K = 32) or 16 (K = 64) bytes of the group in K-slot
// l / 16. Which channels a K-slot carries is free as long as A and B agree
// (the int32 dot product is exact); for groups of 32 slot q carries bytes
// 16 (q & 1) + 8 (q >> 1) of the group, the layout the swap leaves. Result:
// lane l holds rows 4 (l / 16) + i, column l % 16. Groups of 16 use the
// K = 32 form with the upper K slots zero. The dequantization is the fma
// chain above in group order, so M is bit-identical to the definition.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq8_device.h"
#include "wq8_internal.h"

namespace wq8 {

template <int G_, int RT_, int CT_, int NWV_>
struct H2 {
    static constexpr int G = G_, RT = RT_, CT = CT_, NWV = NWV_;
    static constexpr int NT = 64 * NWV;                  // threads per block
    static constexpr int BT = 16 * RT;                   // tile rows (V)
    static constexpr int BC = 16 * CT * NWV;             // output-channel rows (U)
    static constexpr int KC = G > 128 ? G : 128;         // chunk bytes per row (one cache line or more)
    static constexpr int GPC = KC / G;                   // groups per chunk
    // LDS row stride of V: B fragments are read as 8-byte (K = 32) or 16-byte
    // (K = 64) pieces of 16 consecutive rows; a stride of 18 (or 20, 36)
    // dwords puts the 16 rows of an 8-byte read (8 rows of a 16-byte read) on
    // distinct banks
    static constexpr int LDR = G <= 32 ? KC + 8 : KC + 16;
    static constexpr int PPR = KC / 16;                  // 16-byte pieces per V row
    static constexpr int LPV = (BT * PPR + NT - 1) / NT; // V pieces per thread per chunk
    static constexpr int SPV = (BT * GPC + NT - 1) / NT; // V scales per thread per chunk
    static constexpr int SPU = (BC * GPC + NT - 1) / NT; // U scales per thread per chunk
    // LDS rows the threads' pieces cover (at least BT, BC): the rows past the
    // block's take the zeros loaded for them, so the commit needs no bounds
    static constexpr int VR = LPV * NT / PPR;            // V rows
    static constexpr int SVR = SPV * NT / GPC;           // V scale rows per group
    static constexpr int SUR = SPU * NT / GPC;           // U scale rows per group
    static constexpr bool K64 = G >= 64;
    static constexpr int NK = K64 ? G / 64 : 1;          // MFMA steps per group
    // U registers per lane per chunk and channel tile, in 16-byte pieces
    // (G = 16: each piece holds two 8-byte group slices)
    static constexpr int UP = G == 16 ? KC / 32 : KC / 64;
    // U chunks in flight per wave: 4 for the shapes that still fit in 128
    // registers with them (four waves per SIMD; the deeper ring hides more of
    // HBM's latency when the weights are not cached), else 2 (more registers
    // would cost a wave per SIMD, which costs more than the ring gains).
    // Groups of 32 keep 2: their software-pipelined chunk needs the
    // registers, and gains more than the deeper ring
    static constexpr int DU = RT <= 5 && CT == 1 && NWV == 4 && G >= 64 && G <= 128 ? 4 : 2;
};

struct H2Pos {
    int tap, t0, c0;
};

// Per-thread byte offsets of the chunk loads without the chunk's position
// along the input channels; kOob where the thread has nothing to load. The
// chunk's position is added to the lane offset (not the scalar one) so the
// buffer's range check sees the whole offset: kOob plus any chunk position
// stays out of range, and a last chunk that runs past the end of the last
// row reads zero.
template <class C>
struct H2Base {
    uint32_t v[C::LPV], sv[C::SPV], su[C::SPU];
    uint32_t u[C::CT];
};

// Registers of one chunk of V and of its group scales between global load
// and LDS.
template <class C>
struct H2Stage {
    v4i v[C::LPV];
    float sv[C::SPV], su[C::SPU];
};

template <class C, bool I32>
__device__ __forceinline__ void h2_bases(H2Base<C> &bs, const H2Pos &ps, const Geo &g) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int j = 0; j < C::LPV; ++j) {
        const int pce = tid + C::NT * j;
        const int row = pce / C::PPR, qq = pce % C::PPR;
        const int t = ps.t0 + row;
        bs.v[j] = row < C::BT && t < g.T ? (uint32_t)((ps.tap * (int)g.T + t) * g.Cin + 16 * qq) : (uint32_t)kOob;
    }
#pragma unroll
    for (int j = 0; j < C::SPV; ++j) {
        const int e = tid + C::NT * j;
        const int row = e / C::GPC, k = e % C::GPC;
        const int t = ps.t0 + row;
        bs.sv[j] = !I32 && row < C::BT && t < g.T ? (uint32_t)(((ps.tap * (int)g.T + t) * g.ng + k) * 4)
                                                  : (uint32_t)kOob;
    }
#pragma unroll
    for (int j = 0; j < C::SPU; ++j) {
        const int e = tid + C::NT * j;
        const int row = e / C::GPC, k = e % C::GPC;
        const int co = ps.c0 + row;
        bs.su[j] = !I32 && row < C::BC && co < g.Cout ? (uint32_t)(((ps.tap * g.Cout + co) * g.ng + k) * 4)
                                                      : (uint32_t)kOob;
    }
    // U: lane (r, q) of the wave loads row 16 ct + r of its channel tile;
    // groups of 16: the 8 bytes of K-slot q < 2 of each group, else 16 bytes
    // at 16 q
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
        const int co = ps.c0 + 16 * C::CT * wave + 16 * ct + r;
        const bool ok = co < g.Cout && (C::G != 16 || q < 2);
        bs.u[ct] = ok ? (uint32_t)((ps.tap * g.Cout + co) * g.Cin + (C::G == 16 ? 8 * q : 16 * q)) : (uint32_t)kOob;
    }
}

// Issue the loads of chunk c of V and of the chunk's group scales. A chunk
// that ends past a row's last group reads the next row's bytes (or zero past
// the buffer) into group slots that are never computed. For a chunk past the
// last one (c >= nch) the offsets are out of range: the loads return zero
// and fetch nothing.
template <class C, bool I32>
__device__ __forceinline__ void h2_issue_v(H2Stage<C> &st, int c, int nch, const H2Base<C> &bs,
                                           const H2Pos &ps, const Geo &g, __amdgpu_buffer_rsrc_t rV,
                                           __amdgpu_buffer_rsrc_t rsV, __amdgpu_buffer_rsrc_t rsU) {
    const uint32_t cb = c < nch ? (uint32_t)(c * C::KC) : (uint32_t)kOob;
#pragma unroll
    for (int j = 0; j < C::LPV; ++j) st.v[j] = __builtin_amdgcn_raw_buffer_load_b128(rV, (int)(bs.v[j] + cb), 0, 0);
    if constexpr (!I32) {
        const uint32_t sb = c < nch ? (uint32_t)(c * C::GPC * 4) : (uint32_t)kOob;
        // groups of 32 (M only, h2_chunk_pipe32) run every group slot of a
        // chunk: the slots past the row's last group load zero scales, so
        // fma(0, P, M) leaves M as it is (M is never -0: its chain starts at
        // +0 and no scale is negative)
        const int gend = g.ng - c * C::GPC;
#pragma unroll
        for (int j = 0; j < C::SPV; ++j) {
            const int k = (threadIdx.x + C::NT * j) % C::GPC;
            const uint32_t o = C::G != 32 || k < gend ? bs.sv[j] + sb : (uint32_t)kOob;
            st.sv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsV, (int)o, 0, 0));
        }
#pragma unroll
        for (int j = 0; j < C::SPU; ++j) {
            const int k = (threadIdx.x + C::NT * j) % C::GPC;
            const uint32_t o = C::G != 32 || k < gend ? bs.su[j] + sb : (uint32_t)kOob;
            st.su[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsU, (int)o, 0, 0));
        }
    }
}

// Write a chunk of V (rows 0..VR-1; rows from BT on hold zeros) and its
// scales, transposed to [group][row], to LDS. No bounds: every thread's
// pieces have rows in the padded buffers.
template <class C, bool I32>
__device__ __forceinline__ void h2_commit_v(const H2Stage<C> &st, int8_t *op, float *ssv, float *ssu) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < C::LPV; ++j) {
        const int pce = tid + C::NT * j;
        const int row = pce / C::PPR, qq = pce % C::PPR;
        int8_t *p = &op[row * C::LDR + 16 * qq];
        if constexpr (C::LDR % 16 == 0) {
            *(v4i *)p = st.v[j];
        } else {  // rows are 8-byte aligned
            typedef int v2i __attribute__((ext_vector_type(2)));
            ((v2i *)p)[0] = v2i{st.v[j].x, st.v[j].y};
            ((v2i *)p)[1] = v2i{st.v[j].z, st.v[j].w};
        }
    }
    if constexpr (!I32) {
#pragma unroll
        for (int j = 0; j < C::SPV; ++j) {
            const int e = tid + C::NT * j;
            const int row = e / C::GPC, k = e % C::GPC;
            ssv[k * C::SVR + row] = st.sv[j];
        }
#pragma unroll
        for (int j = 0; j < C::SPU; ++j) {
            const int e = tid + C::NT * j;
            const int row = e / C::GPC, k = e % C::GPC;
            ssu[k * C::SUR + row] = st.su[j];
        }
    }
}

// Issue the U loads of chunk c into one ring slot (out of range, so zero and
// no fetch, for a chunk past the last one).
template <class C>
__device__ __forceinline__ void h2_issue_u(v4i (&u)[C::CT][C::UP], int c, int nch, const H2Base<C> &bs,
                                           __amdgpu_buffer_rsrc_t rU) {
    const uint32_t cb = c < nch ? (uint32_t)(c * C::KC) : (uint32_t)kOob;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
        if constexpr (C::G == 16) {
            // groups of 16: 8 bytes of each at 16 k (+ 8 q), two per piece
            typedef int v2i __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int h = 0; h < C::UP; ++h) {
                const v2i a = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(rU, (int)(bs.u[ct] + cb + 32 * h), 0, 0));
                const v2i b = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(rU, (int)(bs.u[ct] + cb + 32 * h + 16), 0, 0));
                u[ct][h] = v4i{a.x, a.y, b.x, b.y};
            }
        } else {
#pragma unroll
            for (int p = 0; p < C::UP; ++p) u[ct][p] = __builtin_amdgcn_raw_buffer_load_b128(rU, (int)(bs.u[ct] + cb + 64 * p), 0, 0);
        }
    }
}

__device__ __forceinline__ long pack64(int lo, int hi) {
    return (long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Groups of 32, M only: B fragment (8 bytes of tile row 16 rt + r; K-slot q
// carries bytes 16 (q & 1) + 8 (q >> 1) of group k) and A fragment (8 bytes
// of channel tile ct's group k; each 16-byte piece of U holds 8 bytes of two
// groups after the swap).
template <class C>
__device__ __forceinline__ long h2_bfrag32(const int8_t *sb, int k, int rt, int r, int q) {
    return *(const long *)&sb[(16 * rt + r) * C::LDR + 32 * k + 16 * (q & 1) + 8 * (q >> 1)];
}

template <class C>
__device__ __forceinline__ long h2_afrag32(const v4i (&u)[C::CT][C::UP], int k, int ct) {
    const v4i w = u[ct][k >> 1];
    return (k & 1) ? pack64(w.z, w.w) : pack64(w.x, w.y);
}

// A chunk for groups of 32 (M only), software-pipelined over its GPC group
// slots: right after the dequantization of group k has read a 16x16 block's
// products, the block's MFMA of group k + 1 writes the same registers, so a
// wave's matrix core works on the next group while its vector ALU
// dequantizes the current one; the next group's B fragments are read from
// LDS before that dequantization starts. Every output's fma chain still runs
// over the groups in ascending order (M is bit-identical to one group at a
// time). Slots past a row's last group have zero scales (h2_issue_v), so
// fma(0, P, M) leaves M as it is. The scheduling fences keep the compiler
// from hoisting later groups' reads, which would cost registers and a wave
// per SIMD.
template <class C>
__device__ __forceinline__ void h2_chunk_pipe32(float (&acc)[C::CT][C::RT][4], const v4i (&u)[C::CT][C::UP],
                                                const int8_t *sb, const float *ssv, const float *ssu) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int wc0 = 16 * C::CT * wave;
    const v4i zero = v4i{0, 0, 0, 0};
    v4i P[C::CT][C::RT];
    long bb[C::RT];
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) bb[rt] = h2_bfrag32<C>(sb, 0, rt, r, q);
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
            P[ct][rt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(h2_afrag32<C>(u, 0, ct), bb[rt], zero, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < C::GPC; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        if (k + 1 < C::GPC) {
#pragma unroll
            for (int rt = 0; rt < C::RT; ++rt) bb[rt] = h2_bfrag32<C>(sb, k + 1, rt, r, q);
        }
        float4 su[C::CT];
        float sv[C::RT];
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) su[ct] = *(const float4 *)&ssu[k * C::SUR + wc0 + 16 * ct + 4 * q];
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) sv[rt] = ssv[k * C::SVR + 16 * rt + r];
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) {
            const float sus[4] = {su[ct].x, su[ct].y, su[ct].z, su[ct].w};
            const long a = k + 1 < C::GPC ? h2_afrag32<C>(u, k + 1, ct) : 0;
#pragma unroll
            for (int rt = 0; rt < C::RT; ++rt) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[ct][rt][i] = __builtin_fmaf(sv[rt] * sus[i], (float)P[ct][rt][i], acc[ct][rt][i]);
                if (k + 1 < C::GPC) P[ct][rt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bb[rt], zero, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// One chunk: GPC groups (gin of them present), A from the U ring slot, B
// from the V buffer in LDS.
template <class C, bool I32>
__device__ __forceinline__ void h2_chunk(float (&acc)[C::CT][C::RT][4], v4i (&u)[C::CT][C::UP], int c,
                                         int gin, const int8_t *sb, const float *ssv, const float *ssu,
                                         const H2Pos &ps, const Geo &g, int32_t *Po) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int wc0 = 16 * C::CT * wave;
    if constexpr (C::G == 32) {
        // lane q < 2 holds bytes [16 q, 16 q + 16) of group 0, lane q + 2 the
        // same of group 1; swap the upper 8 bytes of the lower lanes with the
        // lower 8 bytes of the upper lanes: each lane then has 8 bytes of both
        // groups (dwords 0, 1: group 0; 2, 3: group 1; K-slot q carries bytes
        // 16 (q & 1) + 8 (q >> 1))
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
            for (int p = 0; p < C::UP; ++p) {
                const auto s0 = __builtin_amdgcn_permlane32_swap((uint32_t)u[ct][p].x, (uint32_t)u[ct][p].z, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap((uint32_t)u[ct][p].y, (uint32_t)u[ct][p].w, false, false);
                u[ct][p] = v4i{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
            }
    }
    if constexpr (!I32 && C::G == 32) {
        h2_chunk_pipe32<C>(acc, u, sb, ssv, ssu);
        return;
    }
#pragma unroll
    for (int k = 0; k < C::GPC; ++k) {
        if (k >= gin) break;
        v4i P[C::CT][C::RT];
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
            for (int rt = 0; rt < C::RT; ++rt) P[ct][rt] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < C::NK; ++s) {
            if constexpr (C::K64) {
                const int kb = k * C::G + 64 * s + 16 * q;
                v4i bb[C::RT];
#pragma unroll
                for (int rt = 0; rt < C::RT; ++rt) bb[rt] = *(const v4i *)&sb[(16 * rt + r) * C::LDR + kb];
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
                    for (int rt = 0; rt < C::RT; ++rt)
                        P[ct][rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(u[ct][k * C::NK + s], bb[rt], P[ct][rt], 0, 0, 0);
            } else {
                // groups of 32: K-slot q carries bytes 16 (q & 1) + 8 (q >> 1);
                // groups of 16: K-slots 2, 3 are zero
                long bb[C::RT];
#pragma unroll
                for (int rt = 0; rt < C::RT; ++rt) {
                    if constexpr (C::G == 32)
                        bb[rt] = *(const long *)&sb[(16 * rt + r) * C::LDR + 32 * k + 16 * (q & 1) + 8 * (q >> 1)];
                    else
                        bb[rt] = q < 2 ? *(const long *)&sb[(16 * rt + r) * C::LDR + 16 * k + 8 * q] : 0;
                }
                // each 16-byte piece of U holds 8 bytes of two groups (after
                // the swap for G = 32; as loaded for G = 16)
                long a[C::CT];
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) {
                    const v4i w = u[ct][k >> 1];
                    a[ct] = (k & 1) ? pack64(w.z, w.w) : pack64(w.x, w.y);
                }
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
                    for (int rt = 0; rt < C::RT; ++rt)
                        P[ct][rt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[ct], bb[rt], P[ct][rt], 0, 0, 0);
            }
        }
        if constexpr (I32) {
            const int gi = c * C::GPC + k;
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
                for (int rt = 0; rt < C::RT; ++rt) {
                    const int t = ps.t0 + 16 * rt + r;
                    const int co = ps.c0 + wc0 + 16 * ct + 4 * q;
                    if (t >= g.T) continue;
                    int32_t *pp = Po + (((size_t)ps.tap * g.ng + gi) * g.T + t) * g.Cout + co;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (co + i < g.Cout) pp[i] = P[ct][rt][i];
                }
        } else {
            float4 su[C::CT];
            float sv[C::RT];
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) su[ct] = *(const float4 *)&ssu[k * C::SUR + wc0 + 16 * ct + 4 * q];
#pragma unroll
            for (int rt = 0; rt < C::RT; ++rt) sv[rt] = ssv[k * C::SVR + 16 * rt + r];
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) {
                const float sus[4] = {su[ct].x, su[ct].y, su[ct].z, su[ct].w};
#pragma unroll
                for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[ct][rt][i] = __builtin_fmaf(sv[rt] * sus[i], (float)P[ct][rt][i], acc[ct][rt][i]);
            }
        }
    }
}

template <int G, int RT, int CT, int NWV, bool I32>
__global__ __launch_bounds__(64 * NWV) void k_hgemm(const int8_t *__restrict__ Vq,
                                                    const float *__restrict__ sV,
                                                    const int8_t *__restrict__ Uq,
                                                    const float *__restrict__ sU,
                                                    float *__restrict__ Mo, int32_t *__restrict__ Po,
                                                    Geo g) {
    using C = H2<G, RT, CT, NWV>;
    __shared__ __attribute__((aligned(16))) int8_t s_v[2][C::VR * C::LDR];
    __shared__ __attribute__((aligned(16))) float s_sv[2][C::GPC * C::SVR];
    __shared__ __attribute__((aligned(16))) float s_su[2][C::GPC * C::SUR];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    // Block order: channel blocks fastest, then tile blocks, then taps, laid
    // out so that each XCD runs a contiguous range: the blocks of a tap (which
    // all read its V) and the tile blocks reading one slice of U share an L2.
    const int ntb = (int)((g.T + C::BT - 1) / C::BT), ncb = (g.Cout + C::BC - 1) / C::BC;
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    H2Pos ps;
    ps.tap = lb / (ntb * ncb);
    ps.t0 = ((lb / ncb) % ntb) * C::BT;
    ps.c0 = (lb % ncb) * C::BC;
    const int n2 = g.n * g.n;
    const auto rV = make_rsrc(Vq, (size_t)n2 * g.T * g.Cin);
    const auto rU = make_rsrc(Uq, (size_t)n2 * g.Cout * g.Cin);
    const auto rsV = make_rsrc(sV, I32 ? 0 : (size_t)n2 * g.T * g.ng * 4);
    const auto rsU = make_rsrc(sU, I32 ? 0 : (size_t)n2 * g.Cout * g.ng * 4);
    const int nch = (g.ng + C::GPC - 1) / C::GPC;

    H2Base<C> bs;
    h2_bases<C, I32>(bs, ps, g);

    float acc[C::CT][C::RT][4];
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[ct][rt][i] = 0.0f;

    // U ring: chunk c lives in slot c % DU from its load until its compute.
    // Loads are issued without conditions, also for chunks past the last one
    // (with out-of-range offsets, chosen by a select, so they fetch nothing):
    // with no branch between a load and its use the compiler waits for
    // exactly the loads a step needs, not for every outstanding one.
    v4i ur[C::DU][C::CT][C::UP];
#pragma unroll
    for (int d = 0; d < C::DU; ++d) h2_issue_u<C>(ur[d], d, nch, bs, rU);
    H2Stage<C> st;
    h2_issue_v<C, I32>(st, 0, nch, bs, ps, g, rV, rsV, rsU);
    h2_commit_v<C, I32>(st, s_v[0], s_sv[0], s_su[0]);
    h2_issue_v<C, I32>(st, 1, nch, bs, ps, g, rV, rsV, rsU);
    for (int c0 = 0; c0 < nch; c0 += C::DU) {
#pragma unroll
        for (int d = 0; d < C::DU; ++d) {
            const int c = c0 + d;
            if (c >= nch) break;
            const int b = d & 1;  // c & 1, as DU is even and c0 a multiple of DU
            __syncthreads();      // chunk c is in buffer b; buffer b ^ 1 is free
            h2_commit_v<C, I32>(st, s_v[b ^ 1], s_sv[b ^ 1], s_su[b ^ 1]);
            h2_issue_v<C, I32>(st, c + 2, nch, bs, ps, g, rV, rsV, rsU);
            const int gin = min(C::GPC, g.ng - c * C::GPC);
            h2_chunk<C, I32>(acc, ur[d], c, gin, s_v[b], s_sv[b], s_su[b], ps, g, Po);
            h2_issue_u<C>(ur[d], c + C::DU, nch, bs, rU);
        }
    }
    if constexpr (!I32) {
        float *Mp = Mo + (size_t)ps.tap * g.T * g.Cout;
        const bool vec = g.Cout % 4 == 0;
        typedef float f4v __attribute__((ext_vector_type(4)));
        if constexpr (C::CT == 1 && C::BT * (C::BC + 4) * 4 <= (int)sizeof(s_v)) {
            if (vec) {
                // M goes through LDS (the V buffers, free after the last
                // chunk) so that each store instruction writes whole 128-byte
                // lines of M's rows: a wave's own results cover 64 bytes of a
                // tile row, and with the non-temporal hint two half-line
                // stores reach HBM as two writes (31.6 instead of 23.6 MB per
                // launch on the 1280-channel layer).
                constexpr int SR = C::BC + 4;  // LDS row stride, floats
                constexpr int P4 = C::BC / 4;  // 16-byte pieces per row
                float *sm = reinterpret_cast<float *>(&s_v[0][0]);
                __syncthreads();  // every wave is done with the V buffers
#pragma unroll
                for (int rt = 0; rt < C::RT; ++rt)
                    *(float4 *)&sm[(16 * rt + r) * SR + 16 * wave + 4 * q] =
                        float4{acc[0][rt][0], acc[0][rt][1], acc[0][rt][2], acc[0][rt][3]};
                __syncthreads();
#pragma unroll
                for (int j = 0; j < (C::BT * P4 + C::NT - 1) / C::NT; ++j) {
                    const int pce = threadIdx.x + C::NT * j;
                    const int row = pce / P4, c4 = pce % P4;
                    const int t = ps.t0 + row, co = ps.c0 + 4 * c4;
                    if (row < C::BT && t < g.T && co < g.Cout) {
                        const float4 v = *(const float4 *)&sm[row * SR + 4 * c4];
                        __builtin_nontemporal_store(f4v{v.x, v.y, v.z, v.w}, (f4v *)(Mp + (size_t)t * g.Cout + co));
                    }
                }
                return;
            }
        }
        const int wc0 = 16 * C::CT * wave;
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
            for (int rt = 0; rt < C::RT; ++rt) {
                const int t = ps.t0 + 16 * rt + r;
                const int co = ps.c0 + wc0 + 16 * ct + 4 * q;
                if (t >= g.T || co >= g.Cout) continue;
                float *mp = Mp + (size_t)t * g.Cout + co;
                if (vec) {
                    // non-temporal: M leaves in one burst as the blocks finish
                    // (stage 2 of the 1280-channel layer 47.8 -> 44.2 us; the
                    // same hint on stage 3's 8-byte output stores made that
                    // kernel 1.5-2x slower)
                    __builtin_nontemporal_store(f4v{acc[ct][rt][0], acc[ct][rt][1], acc[ct][rt][2], acc[ct][rt][3]},
                                                (f4v *)mp);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (co + i < g.Cout) mp[i] = acc[ct][rt][i];
                }
            }
    }
}

// ------------------------------------------------------------- launches
template <int G, int RT, int CT, int NWV>
static void hgemm_launch(const Geo &g, const int8_t *Vq, const float *sV, const int8_t *Uq,
                         const float *sU, float *M, int32_t *P, hipStream_t s) {
    using C = H2<G, RT, CT, NWV>;
    const unsigned nb = (unsigned)(((g.T + C::BT - 1) / C::BT) * ((g.Cout + C::BC - 1) / C::BC) * (g.n * g.n));
    if (P)
        hipLaunchKernelGGL((k_hgemm<G, RT, CT, NWV, true>), dim3(nb), dim3(C::NT), 0, s, Vq, sV, Uq, sU, M, P, g);
    else
        hipLaunchKernelGGL((k_hgemm<G, RT, CT, NWV, false>), dim3(nb), dim3(C::NT), 0, s, Vq, sV, Uq, sU, M, P, g);
}

// Tile rows per block: the RT (16-tile MFMA columns) that pads the layer's
// tiles least; ties to the larger RT (fewer re-reads of U).
static int hgemm_rows(int64_t T) {
    int best = 4;
    int64_t best_pad = -1;
    for (int rt = 4; rt <= 8; ++rt) {
        if (rt == 7) continue;
        const int64_t rows = ((T + 16 * rt - 1) / (16 * rt)) * 16 * rt;
        if (best_pad < 0 || rows - T <= best_pad) {
            best = rt;
            best_pad = rows - T;
        }
    }
    return best;
}

// Block shape: tiles per block 16 RT (the layer's padding is smallest),
// then wave tiles of 16 CT channels and NWV waves per block such that the
// busiest SIMD, given the waves spread evenly over the device's SIMDs, does
// the least MFMA-block work (ceil(waves / SIMDs) x RT x CT; ties to more
// channels per wave, then 4 waves).
static void hgemm_shape(const Geo &g, int cus, int &rt, int &ct, int &nwv) {
    rt = g.s2_rows ? g.s2_rows : hgemm_rows(g.T);
    const int64_t ntb = (g.T + 16 * rt - 1) / (16 * rt), n2 = g.n * g.n;
    int64_t best = -1;
    for (int c = (rt <= 5 ? 2 : 1); c >= 1; --c) {
        if (g.s2_cols && c != g.s2_cols) continue;
        for (int w = 4; w >= 2; w -= 2) {
            if (g.s2_waves && w != g.s2_waves) continue;
            const int64_t nb = ntb * ((g.Cout + 16 * c * w - 1) / (16 * c * w)) * n2;
            const int64_t simds = 4 * (int64_t)cus;
            const int64_t load = ((nb * w + simds - 1) / simds) * rt * c;
            if (best < 0 || load < best) {
                best = load;
                ct = c;
                nwv = w;
            }
        }
    }
}

template <int G>
static void hgemm_g(const Geo &g, const int8_t *Vq, const float *sV, const int8_t *Uq,
                    const float *sU, float *M, int32_t *P, hipStream_t s) {
    int rt = 4, ct = 1, nwv = 4;
    hgemm_shape(g, device_cus(), rt, ct, nwv);
#define WQ8_H2(RT_, CT_)                                                      \
    do {                                                                      \
        if (nwv == 2) hgemm_launch<G, RT_, CT_, 2>(g, Vq, sV, Uq, sU, M, P, s); \
        else hgemm_launch<G, RT_, CT_, 4>(g, Vq, sV, Uq, sU, M, P, s);          \
    } while (0)
    if (rt == 4 && ct == 2) WQ8_H2(4, 2);
    else if (rt == 4) WQ8_H2(4, 1);
    else if (rt == 5 && ct == 2) WQ8_H2(5, 2);
    else if (rt == 5) WQ8_H2(5, 1);
    else if (rt == 6) WQ8_H2(6, 1);
    else WQ8_H2(8, 1);
#undef WQ8_H2
}

wq8_status launch_hgemm(const Geo &g, const int8_t *Vq, const float *sV, const int8_t *Uq,
                        const float *sU, float *M, int32_t *P, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    switch (g.G) {
        case 16: hgemm_g<16>(g, Vq, sV, Uq, sU, M, P, s); break;
        case 32: hgemm_g<32>(g, Vq, sV, Uq, sU, M, P, s); break;
        case 64: hgemm_g<64>(g, Vq, sV, Uq, sU, M, P, s); break;
        case 128: hgemm_g<128>(g, Vq, sV, Uq, sU, M, P, s); break;
        default: hgemm_g<256>(g, Vq, sV, Uq, sU, M, P, s); break;
    }
    return check_launch("Hadamard GEMM");
}

}  // namespace wq8
