// HIP kernels for group-wise fully quantized Winograd F(m,3) on gfx950.
//
//   k_weights  U = G g G^T, per-group int8 (offline weight preparation)
//   k_stage1   V = B^T d B, per-group int8 (input transform)
//   k_stage2   n*n int8 GEMMs over input channels on MFMA, group dequant
//   k_stage3   Y requant over the n*n taps of a (tile, co), A^T Yq A, crop
//   k_fused23  stages 2 and 3 in one kernel, M kept on chip (16 x 16 blocks)
//   k_fused23w the same with 32 x 32 blocks, for F(6,3) layers with many tiles
//
// Numerics follow the library contract bit for bit: every transform sum is an
// fp32 fma chain in index order starting from +0, the quantizer divides with
// IEEE fp32 division and rounds with rint (ties to even). Build with
// -ffp-contract=off so nothing else is fused. The one exception is the fused
// kernel's output transform (fp16 matrix cores on split factors, ~1e-6 of the
// output RMS from the fp32 chain); its codes and scales are still exact.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "wq8_device.h"
#include "wq8_internal.h"

namespace wq8 {

// Symmetric absmax quantizer pieces (a = group absmax > 0).
__device__ __forceinline__ int quant_code(float v, float inv) {
    float r = __builtin_rintf(v * inv);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// Quantize NT values per lane with per-tap group absmax and store codes and
// scales. plane_codes/plane_scales are the per-tap strides.
template <int NT, int G>
__device__ __forceinline__ void quantize_store(const float (&v)[NT], bool ok, int c, int wave,
                                               int8_t *codes, size_t plane_codes, float *scales,
                                               size_t plane_scales, float (*red)[NT]) {
    using S = GroupShape<G>;
    float amax[NT];
#pragma unroll
    for (int tap = 0; tap < NT; ++tap) amax[tap] = seg_max<S::SEG>(fabsf(v[tap]));
    if constexpr (S::GW > 1) {
        const int lane = threadIdx.x & 63;
        if (lane == 0)
#pragma unroll
            for (int tap = 0; tap < NT; ++tap) red[wave][tap] = amax[tap];
        __syncthreads();
        const int w0 = (wave / S::GW) * S::GW;
#pragma unroll
        for (int tap = 0; tap < NT; ++tap) {
            float a = red[w0][tap];
#pragma unroll
            for (int k = 1; k < S::GW; ++k) a = fmaxf(a, red[w0 + k][tap]);
            amax[tap] = a;
        }
    }
    if (!ok) return;
#pragma unroll
    for (int tap = 0; tap < NT; ++tap) {
        const float a = amax[tap];
        int q = 0;
        float s = 0.0f;
        if (a != 0.0f) {
            const float inv = 127.0f / a;
            q = quant_code(v[tap], inv);
            s = a / 127.0f;
        }
        codes[tap * plane_codes] = (int8_t)q;
        if (c % G == 0) scales[tap * plane_scales] = s;
    }
}

// ------------------------------------------------------------- stage 1
// One lane per input channel, one wave per (tile, 64-channel chunk); a block
// takes one strip of adjacent tiles of a tile row (the work item below). Per
// tile:
//   1. the strip's input window is staged in LDS (zero outside the image) and
//      each lane reads its channel's n x n patch from there;
//   2. V = B^T d B as fp32 fma chains in index order (terms whose B^T entry is
//      structurally zero are skipped when the host has verified the pattern;
//      fma(0, d, acc) == acc, so the chains stay bit-identical);
//   3. group absmax per tap by a reduce-scatter butterfly over the group's
//      lanes (permlane32/16 swaps, then DPP exchanges), leaving each lane the
//      max of 64/SEG taps, so the IEEE divisions 127/a and a/127 run once per
//      (tap, group) instead of once per value;
//   4. reciprocals go through LDS to every lane of the group; each value is
//      rounded with x + 1.5*2^23, whose low byte is rint(x) in two's
//      complement (|x| <= 127 (1 + 2^-24)^2 < 127.5, so the clamp to +-127
//      never binds and is omitted).

// Stage 1 work item: a strip of TPB horizontally adjacent tiles of one tile
// row, for CPB input channels. The strip's input window (CPB channels x n rows
// x WC columns, zero outside the image) is copied to LDS, then each wave reads
// its tile's n x n patch per channel from LDS (one channel per lane; the
// channel stride in LDS is odd, so these reads are free of bank conflicts).
//
// The window starts at the 4-aligned column at or before the strip's first
// input column, so every lane loads an aligned quad of 4 columns. When W is a
// multiple of 4 such a quad lies wholly inside or wholly outside the image
// and is one 16-byte (bf16: 8-byte) load; otherwise each column is loaded on
// its own. One load instruction covers CPI channels x QPR quads of one window
// row; which row and channels is the same for all lanes, so that part of the
// address, and the zero fill of rows outside the image, go in the scalar
// offset (a raw buffer load returns zero past the buffer's end).
template <int M, int G, int TPB_, bool RH = false>
struct S1Shape {
    static constexpr int N = M + 2;
    static constexpr int NR = RH ? N / 2 : N;                // window rows held in LDS at once
    static constexpr int GW = GroupShape<G>::GW;             // waves per tile
    static constexpr int TPB = TPB_;
    static constexpr int NW = TPB * GW;                      // waves per block
    static constexpr int CPB = 64 * GW;
    static constexpr int NEED = 3 + TPB * M + 2;             // window columns used, at most
    static constexpr int QPR = NEED <= 8 ? 2 : NEED <= 16 ? 4 : 8;  // quads per window row
    static constexpr int WC = 4 * QPR;
    static constexpr int CPI = 64 / QPR;                     // channels per load instruction
    static constexpr int CS = NR * WC + 1;                   // LDS floats per channel (odd)
    static constexpr int ITERS = CPB / CPI * NR / NW;        // load instructions per wave
    static_assert(NEED <= WC && ITERS * NW * CPI == CPB * NR, "stage-1 window shape");
    static_assert(16 % CPI == 0, "a load instruction must not straddle a channel group");
};

// One thread's share of a strip window in flight between load and LDS.
template <int M, int G, int TPB, bool RH = false>
struct S1Loads {
    float f[S1Shape<M, G, TPB, RH>::ITERS][4];
};

// A work item's position: image, tile row, first tile column, first channel.
struct S1Item {
    int img, ty, tx0, c0;
};

template <int M, int G, int TPB>
__device__ __forceinline__ S1Item s1_item(int item, const Geo &g) {
    const int nstrip = (g.tW + TPB - 1) / TPB;
    const int strip = item % nstrip;
    const int rem = item / nstrip;
    const int rows = g.N * g.tH;
    const int rowid = rem % rows;
    S1Item it;
    it.c0 = (rem / rows) * GroupShape<G>::CPB;
    it.ty = rowid % g.tH;
    it.img = rowid / g.tH;
    it.tx0 = strip * TPB;
    return it;
}

// First window column (4-aligned, may be negative) of a work item.
template <int M>
__device__ __forceinline__ int s1_w0(const S1Item &it, const Geo &g) {
    return ((it.tx0 * M - g.pad) >> 2) << 2;  // arithmetic shift: floor
}

// Issue all of this thread's window loads for one strip: window rows
// r0 .. r0 + NR - 1 of the strip's n input rows.
template <int M, int G, int TPB, bool VEC, typename XT, bool RH = false>
__device__ __forceinline__ void s1_issue(S1Loads<M, G, TPB, RH> &ld, __amdgpu_buffer_rsrc_t rx,
                                         const S1Item &it, const Geo &g, int wave, int r0 = 0) {
    using SS = S1Shape<M, G, TPB, RH>;
    auto &f = ld.f;
    constexpr int ES = sizeof(XT);
    constexpr int OOB = 0x7ffffff0;  // beyond every buffer the plan accepts; two sum below 2^32
    const int lane = threadIdx.x & 63;
    const int chs = lane / SS::QPR, part = lane % SS::QPR;
    const int col = s1_w0<M>(it, g) + 4 * part;
    const int hw = g.H * g.W;
    const int h0 = it.ty * M - g.pad;
    const int lrow = (it.img * g.Cin + it.c0 + chs) * hw;  // this lane's channel plane
    int vb[VEC ? 1 : 4];
    if constexpr (VEC) {
        vb[0] = col >= 0 && col < g.W ? (lrow + col) * ES : OOB;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) vb[e] = col + e >= 0 && col + e < g.W ? (lrow + col + e) * ES : OOB;
    }
#pragma unroll
    for (int i = 0; i < SS::ITERS; ++i) {
        const int j = i * SS::NW + wave;  // uniform: window row and channel slice
        const int row = j % SS::NR, cho = (j / SS::NR) * SS::CPI;
        const int h = h0 + r0 + row;
        const int so = h >= 0 && h < g.H && it.c0 + cho < g.Cin ? (cho * hw + h * g.W) * ES : OOB;
        if constexpr (VEC) {
            if constexpr (ES == 4) {
                const v4i q = __builtin_amdgcn_raw_buffer_load_b128(rx, vb[0], so, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) f[i][e] = __int_as_float(q[e]);
            } else {
                const auto q = __builtin_amdgcn_raw_buffer_load_b64(rx, vb[0], so, 0);
                f[i][0] = __uint_as_float(q[0] << 16);
                f[i][1] = __uint_as_float(q[0] & 0xffff0000u);
                f[i][2] = __uint_as_float(q[1] << 16);
                f[i][3] = __uint_as_float(q[1] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (ES == 4)
                    f[i][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx, vb[e], so, 0));
                else
                    f[i][e] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rx, vb[e], so, 0)
                                              << 16);
            }
        }
    }
}

// Write the loaded quads to the LDS window.
template <int M, int G, int TPB, bool RH = false>
__device__ __forceinline__ void s1_commit(float *win, const S1Loads<M, G, TPB, RH> &ld, int wave) {
    using SS = S1Shape<M, G, TPB, RH>;
    const int lane = threadIdx.x & 63;
    float *lp = win + (lane / SS::QPR) * SS::CS + 4 * (lane % SS::QPR);
#pragma unroll
    for (int i = 0; i < SS::ITERS; ++i) {
        const int j = i * SS::NW + wave;
        const int row = j % SS::NR, cho = (j / SS::NR) * SS::CPI;
        float *p = lp + cho * SS::CS + row * SS::WC;
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = ld.f[i][e];
    }
}

// IQ selects the integer input stage: the patches of a (tile, group) share one
// absmax scale sx, the transform runs on their codes and the codes of B^T
// (mt.Bq) in exact int32 arithmetic (24-bit multiplies: |codes| <= 127 and
// the first pass stays below n * 127^2 < 2^23), and
// V = float(Wi) * ((sq_i * sq_j) * sx) goes on to the same V quantization.
// RH (fp32 input stage only): the LDS window holds half of the n input rows
// at a time. Both halves' loads are issued at once; the first pass of the
// transform (B^T d, an fma chain over rows in index order) runs over the
// first half, the second half then replaces it in LDS and the chains
// continue, so the sums are unchanged. Half the LDS lets twice as many
// blocks be resident.
template <int M, int G, int TPB, uint64_t BMASK, bool VEC, typename XT, bool IQ, bool RH>
__global__ __launch_bounds__((64 * S1Shape<M, G, TPB>::NW), RH ? 4 : 1) void k_stage1(
    const XT *__restrict__ x, int8_t *__restrict__ Vq, float *__restrict__ sV, Mats mt, Geo g) {
    static_assert(!(RH && IQ), "the integer input stage needs the whole patch at once");
    constexpr int N = M + 2, NT = N * N;
    using S = GroupShape<G>;
    using SS = S1Shape<M, G, TPB, RH>;
    __shared__ float win[SS::CPB * SS::CS];
    __shared__ float red[S::GW > 1 ? SS::NW : 1][64];
    __shared__ __attribute__((aligned(16))) float inv_lds[SS::NW][64 / S::SEG][64];
    __shared__ float redx[IQ && S::GW > 1 ? SS::NW : 1];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int tl = wave / S::GW;                // this wave's tile in the strip
    const int cl = (wave % S::GW) * 64 + lane;  // this lane's channel in the block
    const int n2 = N * N;
    const int plane = (int)g.T * g.Cin, splane = (int)g.T * g.ng;
    const auto rx = make_rsrc(x, (size_t)g.N * g.Cin * g.H * g.W * sizeof(XT));
    const auto rq = make_rsrc(Vq, (size_t)n2 * plane);
    const auto rs = make_rsrc(sV, (size_t)n2 * splane * 4);

    const S1Item cur = s1_item<M, G, TPB>(xcd_block(blockIdx.x, gridDim.x), g);
    S1Loads<M, G, TPB, RH> f;
    s1_issue<M, G, TPB, VEC, XT, RH>(f, rx, cur, g, wave);
    [[maybe_unused]] S1Loads<M, G, TPB, RH> f2;  // RH: the second half of the rows
    if constexpr (RH) s1_issue<M, G, TPB, VEC, XT, RH>(f2, rx, cur, g, wave, SS::NR);
    s1_commit<M, G, TPB, RH>(win, f, wave);
    __syncthreads();
    {
        const int c = cur.c0 + cl, tx = cur.tx0 + tl;
        // A wave whose tile lies past the end of the tile row (the strip's
        // last slots) only helps load the window and meets the barriers.
        // (With the integer input stage and groups over several waves the
        // transform holds a barrier, so there every wave runs it.)
        const bool act = tx < g.tW;
        const bool skip = !act && !(IQ && S::GW > 1);
        const bool ok = c < g.Cin && act;
        const int t = (cur.img * g.tH + cur.ty) * g.tW + tx;
        const float *src = win + cl * SS::CS + (cur.tx0 * M - g.pad - s1_w0<M>(cur, g)) + tl * M;
        float v[NT];
        if constexpr (RH) {
            float t1[N][N];
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int l = 0; l < N; ++l)
                    t1[i][l] = (BMASK >> (i * N)) & ((1ull << SS::NR) - 1) ? __builtin_nondeterministic_value(0.0f) : 0.0f;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                if (hh == 1) {
                    __syncthreads();  // every wave has read the first half
                    s1_commit<M, G, TPB, RH>(win, f2, wave);
                    __syncthreads();
                }
                if (skip) continue;
                float d[SS::NR][N];
#pragma unroll
                for (int k = 0; k < SS::NR; ++k)
#pragma unroll
                    for (int l = 0; l < N; ++l) d[k][l] = src[k * SS::WC + l];
#pragma unroll
                for (int i = 0; i < N; ++i)
#pragma unroll
                    for (int l = 0; l < N; ++l)
#pragma unroll
                        for (int kk = 0; kk < SS::NR; ++kk) {
                            const int k = hh * SS::NR + kk;
                            const bool first = hh == 0 && !((BMASK >> (i * N)) & ((1ull << k) - 1));
                            if ((BMASK >> (i * N + k)) & 1)
                                t1[i][l] = __builtin_fmaf(mt.Bt[i * N + k], d[kk][l], first ? 0.0f : t1[i][l]);
                        }
            }
            if (!skip)
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int j = 0; j < N; ++j) {
                    float acc = 0.0f;
#pragma unroll
                    for (int l = 0; l < N; ++l)
                        if ((BMASK >> (j * N + l)) & 1) acc = __builtin_fmaf(t1[i][l], mt.Bt[j * N + l], acc);
                    v[i * N + j] = acc;
                }
        } else if (!skip) {
        float d[N][N];
#pragma unroll
        for (int k = 0; k < N; ++k)
#pragma unroll
            for (int l = 0; l < N; ++l) d[k][l] = src[k * SS::WC + l];

        if constexpr (IQ) {
            float ax = 0.0f;
#pragma unroll
            for (int k = 0; k < N; ++k)
#pragma unroll
                for (int l = 0; l < N; ++l) ax = fmaxf(ax, fabsf(d[k][l]));
            ax = seg_max<S::SEG>(ax);
            if constexpr (S::GW > 1) {
                if (lane == 0) redx[wave] = ax;
                __syncthreads();
                const int w0 = (wave / S::GW) * S::GW;
                ax = redx[w0];
#pragma unroll
                for (int k = 1; k < S::GW; ++k) ax = fmaxf(ax, redx[w0 + k]);
            }
            float invx = 0.0f, sx = 0.0f;
            if (ax != 0.0f) {
                invx = 127.0f / ax;
                sx = ax / 127.0f;
            }
            int dq[N][N];
#pragma unroll
            for (int k = 0; k < N; ++k)
#pragma unroll
                for (int l = 0; l < N; ++l) dq[k][l] = (int)__builtin_rintf(d[k][l] * invx);
            int t1[N][N];
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int l = 0; l < N; ++l) {
                    int acc = 0;
#pragma unroll
                    for (int k = 0; k < N; ++k)
                        if ((BMASK >> (i * N + k)) & 1) acc += __mul24(mt.Bq[i * N + k], dq[k][l]);
                    t1[i][l] = acc;
                }
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int j = 0; j < N; ++j) {
                    int acc = 0;
#pragma unroll
                    for (int l = 0; l < N; ++l)
                        if ((BMASK >> (j * N + l)) & 1) acc += __mul24(t1[i][l], mt.Bq[j * N + l]);
                    v[i * N + j] = (float)acc * ((mt.sqb[i] * mt.sqb[j]) * sx);
                }
        } else {
            float t1[N][N];
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int l = 0; l < N; ++l) {
                    float acc = 0.0f;
#pragma unroll
                    for (int k = 0; k < N; ++k)
                        if ((BMASK >> (i * N + k)) & 1) acc = __builtin_fmaf(mt.Bt[i * N + k], d[k][l], acc);
                    t1[i][l] = acc;
                }
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int j = 0; j < N; ++j) {
                    float acc = 0.0f;
#pragma unroll
                    for (int l = 0; l < N; ++l)
                        if ((BMASK >> (j * N + l)) & 1) acc = __builtin_fmaf(t1[i][l], mt.Bt[j * N + l], acc);
                    v[i * N + j] = acc;
                }
        }
        }
        s1_quantize_store<NT, G, SS::NW>(v, skip, ok, wave, lane, c, t, g.Cin, g.ng, plane, splane, rq, rs,
                                         red, inv_lds);
    }
}

template <int M, int G>
__global__ __launch_bounds__(256) void k_weights(const float *__restrict__ w, int8_t *__restrict__ Uq,
                                                 float *__restrict__ sU, Mats mt, Geo g) {
    constexpr int N = M + 2, NT = N * N;
    using S = GroupShape<G>;
    __shared__ float red[S::GW > 1 ? 4 : 1][NT];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int co = blockIdx.x * S::TPB + wave / S::GW;
    const int ci = blockIdx.y * S::CPB + (wave % S::GW) * 64 + lane;
    const bool ok = co < g.Cout && ci < g.Cin;

    float u[NT];
    {
        float gw[3][3];
        const float *wp = w + ((size_t)(ok ? co : 0) * g.Cin + (ok ? ci : 0)) * 9;
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = 0; b < 3; ++b) gw[a][b] = ok ? wp[a * 3 + b] : 0.0f;
        float t2[N][3];
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int b = 0; b < 3; ++b) {
                float acc = 0.0f;
#pragma unroll
                for (int a = 0; a < 3; ++a) acc = __builtin_fmaf(mt.G[i * 3 + a], gw[a][b], acc);
                t2[i][b] = acc;
            }
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int j = 0; j < N; ++j) {
                float acc = 0.0f;
#pragma unroll
                for (int b = 0; b < 3; ++b) acc = __builtin_fmaf(t2[i][b], mt.G[j * 3 + b], acc);
                u[i * N + j] = acc;
            }
    }
    const size_t plane = (size_t)g.Cout * g.Cin, splane = (size_t)g.Cout * g.ng;
    quantize_store<NT, G>(u, ok, ci, wave, Uq + (size_t)co * g.Cin + ci, plane,
                          sU + (size_t)co * g.ng + ci / G, splane, red);
}

// ------------------------------------------------------- Hadamard GEMMs
// Grid (ceil(T/64), ceil(Cout/BC), n*n). A block computes M for 64 tiles x BC
// output channels of one tap; its 4 waves form 2 x 2, wave (wt, wc) owning
// tiles 32wt.. and channels (BC/2)wc.. as 2 x BC/32 MFMA 16x16 blocks.
//
// K (input channels) runs in chunks of KC bytes (the largest power of two up
// to 128 dividing Cin). Each chunk's operand rows (64 tile rows of V, BC
// channel rows of U) and the scales of the groups that end inside it are
// staged in LDS, double-buffered: while the block computes chunk c, every
// thread holds chunk c+1 in registers (loaded during chunk c-1) and writes it
// to the other buffer, then issues the loads of chunk c+2. All global loads
// are 16-byte pieces of whole rows, so each cache line is fetched once.
//
// Per group: the int32 dot products on MFMA (16x16x32 for G <= 32, with zero
// K slots for G = 16; else G/64 steps of 16x16x64), then
// M = fma(fl(sV sU), P, M) in group order, so M is bit-identical to the
// definition. MFMA operand layout (16x16xK, int8): lane l holds row (l % 16)
// of A / column (l % 16) of B, K-slice (l / 16). A and B use the same K
// mapping, so the exact int32 dot product does not depend on the order the
// hardware sums the K slots in. Result: lane l holds rows 4 (l / 16) + i,
// column l % 16. I32: store each group's int32 products (P) instead of M.
template <int G, int BC>
struct S2 {
    static constexpr int BT = 64, KCM = 128;
    static constexpr int ROWS = BT + BC;                    // operand rows of a chunk
    static constexpr int LDR = KCM + 16;                    // LDS row stride in bytes
    static constexpr int NGM = G < KCM ? KCM / G : 1;       // groups ending in one chunk, at most
    static constexpr int LPT = 2 * (BT * KCM / 16 / 256);   // 16-byte loads per thread per chunk, at most
    static constexpr int SPT = 2 * ((BT * NGM + 255) / 256); // scale loads per thread per chunk, at most
    static constexpr int NJ = BC / 32;                      // MFMA blocks per wave along the channels
    static constexpr bool K64 = G >= 64;
    static_assert(BC == BT && BT * KCM / 16 % 256 == 0, "whole loads per thread and operand");
};

// Where a thread's pieces of chunk c come from and go. Rows 0..BT-1 of a
// chunk are tile rows of V, rows BT.. output-channel rows of U; each row is
// split into 16-byte pieces (ppr = KC / 16 = 1 << lppr of them).
struct S2Pos {
    int tap, t0, c0, KC, lppr;
};

// Groups whose scales chunk c stages: [first, first + count).
template <int G>
__device__ __forceinline__ void s2_chunk_groups(int c, int KC, int &first, int &count) {
    if (G <= KC) {
        first = c * (KC / G);
        count = KC / G;
    } else {
        first = ((c + 1) * KC) / G - 1;
        count = ((c + 1) * KC) % G == 0 ? 1 : 0;
    }
}

// Loads of one chunk into registers: LPH 16-byte pieces per thread for each
// of the two operands (a separate loop each, so the buffer resource stays
// uniform), and the chunk's group scales.
template <int G, int BC, bool I32, int LN, int SN>
__device__ __forceinline__ void s2_issue(v4i (&ld)[LN], float (&ls)[SN], int c, const S2Pos &ps,
                                         const Geo &g, __amdgpu_buffer_rsrc_t rV,
                                         __amdgpu_buffer_rsrc_t rU, __amdgpu_buffer_rsrc_t rsV,
                                         __amdgpu_buffer_rsrc_t rsU) {
    using C = S2<G, BC>;
    constexpr int LPH = LN / 2;
    const int tid = threadIdx.x;
    const int npo = C::BT << ps.lppr;  // pieces per operand (BC == BT)
#pragma unroll
    for (int j = 0; j < LPH; ++j) {
        const int pce = tid + 256 * j;
        const int row = pce >> ps.lppr, q = pce & ((1 << ps.lppr) - 1);
        const int t = ps.t0 + row < g.T ? ps.t0 + row : 0;  // unused rows read row 0
        const int off = pce < npo ? (ps.tap * (int)g.T + t) * g.Cin + c * ps.KC + 16 * q : kOob;
        ld[j] = __builtin_amdgcn_raw_buffer_load_b128(rV, off, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < LPH; ++j) {
        const int pce = tid + 256 * j;
        const int row = pce >> ps.lppr, q = pce & ((1 << ps.lppr) - 1);
        const int co = ps.c0 + row < g.Cout ? ps.c0 + row : 0;
        const int off = pce < npo ? (ps.tap * g.Cout + co) * g.Cin + c * ps.KC + 16 * q : kOob;
        ld[LPH + j] = __builtin_amdgcn_raw_buffer_load_b128(rU, off, 0, 0);
    }
    if constexpr (!I32) {
        int first, count;
        s2_chunk_groups<G>(c, ps.KC, first, count);
        // thread e < count * BT: row e / count, group first + e % count
        const int lc = count == 8 ? 3 : count == 4 ? 2 : count == 2 ? 1 : 0;
        constexpr int SPH = SN / 2;
#pragma unroll
        for (int j = 0; j < SPH; ++j) {
            const int e = tid + 256 * j;
            const int row = e >> lc, k = e & (count - 1);
            const bool in = count && row < C::BT;
            const int offv = in && ps.t0 + row < g.T ? ((ps.tap * (int)g.T + ps.t0 + row) * g.ng + first + k) * 4 : kOob;
            const int offu = in && ps.c0 + row < g.Cout ? ((ps.tap * g.Cout + ps.c0 + row) * g.ng + first + k) * 4 : kOob;
            ls[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsV, offv, 0, 0));
            ls[SPH + j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsU, offu, 0, 0));
        }
    }
}

template <int G, int BC, bool I32, int LN, int SN, int NR>
__device__ __forceinline__ void s2_commit(const v4i (&ld)[LN], const float (&ls)[SN], int c, const S2Pos &ps,
                                          int8_t *op, float (*sc)[NR]) {
    using C = S2<G, BC>;
    constexpr int LPH = LN / 2;
    const int tid = threadIdx.x;
    const int npo = C::BT << ps.lppr;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < LPH; ++j) {
            const int pce = tid + 256 * j;
            const int row = pce >> ps.lppr, q = pce & ((1 << ps.lppr) - 1);
            if (pce < npo) *(v4i *)&op[(h * C::BT + row) * C::LDR + 16 * q] = ld[h * LPH + j];
        }
    if constexpr (!I32) {
        int first, count;
        s2_chunk_groups<G>(c, ps.KC, first, count);
        const int lc = count == 8 ? 3 : count == 4 ? 2 : count == 2 ? 1 : 0;
        constexpr int SPH = SN / 2;
#pragma unroll
        for (int j = 0; j < SPH; ++j) {
            const int e = tid + 256 * j;
            const int row = e >> lc, k = e & (count - 1);
            if (count && row < C::BT) {
                sc[k][row] = ls[j];
                sc[k][C::BT + row] = ls[SPH + j];
            }
        }
    }
}

// One group's products are complete: dequantize them into M (or store them)
// and clear them. k: the group's slot among the chunk's staged scales.
template <int G, int BC, bool I32, int NJ, int NR>
__device__ __forceinline__ void s2_finish(v4i (&P)[2][NJ], float (&acc)[2][NJ][4], int gi,
                                          const float (*sc)[NR], int k, const S2Pos &ps, const Geo &g,
                                          int32_t *Po) {
    using C = S2<G, BC>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, kq = lane >> 4, wt = wave & 1, wc = wave >> 1;
    if constexpr (I32) {
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < C::NJ; ++bj) {
                const int col = ps.c0 + (BC / 2) * wc + 16 * bj + r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = ps.t0 + 32 * wt + 16 * bi + 4 * kq + i;
                    if (row < g.T && col < g.Cout)
                        Po[(((size_t)ps.tap * g.ng + gi) * g.T + row) * g.Cout + col] = P[bi][bj][i];
                }
            }
    } else {
        float su[C::NJ];
#pragma unroll
        for (int bj = 0; bj < C::NJ; ++bj) su[bj] = sc[k][C::BT + (BC / 2) * wc + 16 * bj + r];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
            const float4 sv = *(const float4 *)&sc[k][32 * wt + 16 * bi + 4 * kq];
            const float svs[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
            for (int bj = 0; bj < C::NJ; ++bj)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[bi][bj][i] = __builtin_fmaf(svs[i] * su[bj], (float)P[bi][bj][i], acc[bi][bj][i]);
        }
    }
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < C::NJ; ++bj) P[bi][bj] = v4i{0, 0, 0, 0};
}

template <int G, int BC, bool I32>
__global__ __launch_bounds__(256) void k_stage2(const int8_t *__restrict__ Vq,
                                                const float *__restrict__ sV,
                                                const int8_t *__restrict__ Uq,
                                                const float *__restrict__ sU, float *__restrict__ Mo,
                                                int32_t *__restrict__ Po, Geo g, int KC) {
    using C = S2<G, BC>;
    __shared__ __attribute__((aligned(16))) int8_t s_op[2][C::ROWS * C::LDR];
    __shared__ __attribute__((aligned(16))) float s_sc[2][C::NGM][C::ROWS];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, kq = lane >> 4;
    const int wt = wave & 1, wc = wave >> 1;
    // Block order: tile blocks fastest, then channel blocks, then taps, laid
    // out so that each XCD runs a contiguous range of it: the tile blocks that
    // share a slice of U, and all blocks of a tap (which share its V), then
    // meet in one L2 instead of fetching the same bytes into several.
    const int ntb = (int)((g.T + C::BT - 1) / C::BT), ncb = (g.Cout + BC - 1) / BC;
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    S2Pos ps;
    ps.tap = lb / (ntb * ncb);
    ps.t0 = (lb % ntb) * C::BT;
    ps.c0 = ((lb / ntb) % ncb) * BC;
    ps.KC = KC;
    ps.lppr = KC == 128 ? 3 : KC == 64 ? 2 : KC == 32 ? 1 : 0;
    const int n2 = g.n * g.n;
    const auto rV = make_rsrc(Vq, (size_t)n2 * g.T * g.Cin);
    const auto rU = make_rsrc(Uq, (size_t)n2 * g.Cout * g.Cin);
    const auto rsV = make_rsrc(sV, (size_t)n2 * g.T * g.ng * 4);
    const auto rsU = make_rsrc(sU, (size_t)n2 * g.Cout * g.ng * 4);
    const int nch = g.Cin / KC;

    float acc[2][C::NJ][4];
    v4i P[2][C::NJ];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < C::NJ; ++bj) {
            P[bi][bj] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[bi][bj][i] = 0.0f;
        }
    const int arow = (32 * wt + r) * C::LDR, brow = (C::BT + (BC / 2) * wc + r) * C::LDR;
    const bool kin = C::K64 || 8 * kq < G;

    v4i ld[C::LPT];
    float ls[C::SPT];
    s2_issue<G, BC, I32>(ld, ls, 0, ps, g, rV, rU, rsV, rsU);
    s2_commit<G, BC, I32>(ld, ls, 0, ps, s_op[0], s_sc[0]);
    if (nch > 1) s2_issue<G, BC, I32>(ld, ls, 1, ps, g, rV, rU, rsV, rsU);
    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        __syncthreads();  // chunk c is in buffer b; buffer b^1 is free
        if (c + 1 < nch) {
            s2_commit<G, BC, I32>(ld, ls, c + 1, ps, s_op[b ^ 1], s_sc[b ^ 1]);
            if (c + 2 < nch) s2_issue<G, BC, I32>(ld, ls, c + 2, ps, g, rV, rU, rsV, rsU);
        }
        const int8_t *sa = &s_op[b][arow];
        const int8_t *sb = &s_op[b][brow];
        if constexpr (!C::K64) {
            // groups of 16 or 32 channels, one 16x16x32 step each
            const int ngc = KC / G;
            for (int k = 0; k < ngc; ++k) {
                const int kb = k * G + (kin ? 8 * kq : 0);
                long a8[2], b8[C::NJ];
#pragma unroll
                for (int bi = 0; bi < 2; ++bi) a8[bi] = kin ? *(const long *)&sa[16 * bi * C::LDR + kb] : 0;
#pragma unroll
                for (int bj = 0; bj < C::NJ; ++bj) b8[bj] = kin ? *(const long *)&sb[16 * bj * C::LDR + kb] : 0;
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                    for (int bj = 0; bj < C::NJ; ++bj)
                        P[bi][bj] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a8[bi], b8[bj], P[bi][bj], 0, 0, 0);
                s2_finish<G, BC, I32>(P, acc, c * ngc + k, s_sc[b], k, ps, g, Po);
            }
        } else {
            // 64-channel steps; a group ends every G / 64 steps
            const int nst = KC / 64;
            for (int st = 0; st < nst; ++st) {
                const int kb = 64 * st + 16 * kq;
                v4i a[2], bb[C::NJ];
#pragma unroll
                for (int bi = 0; bi < 2; ++bi) a[bi] = *(const v4i *)&sa[16 * bi * C::LDR + kb];
#pragma unroll
                for (int bj = 0; bj < C::NJ; ++bj) bb[bj] = *(const v4i *)&sb[16 * bj * C::LDR + kb];
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                    for (int bj = 0; bj < C::NJ; ++bj)
                        P[bi][bj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[bi], bb[bj], P[bi][bj], 0, 0, 0);
                const int kend = c * KC + 64 * (st + 1);  // channels done
                if (kend % G == 0)
                    s2_finish<G, BC, I32>(P, acc, kend / G - 1, s_sc[b], G <= KC ? (64 * (st + 1)) / G - 1 : 0,
                                          ps, g, Po);
            }
        }
    }
    if constexpr (!I32) {
        float *Mp = Mo + (size_t)ps.tap * g.T * g.Cout;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < C::NJ; ++bj) {
                const int col = ps.c0 + (BC / 2) * wc + 16 * bj + r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = ps.t0 + 32 * wt + 16 * bi + 4 * kq + i;
                    if (row < g.T && col < g.Cout) Mp[(size_t)row * g.Cout + col] = acc[bi][bj][i];
                }
            }
    }
}

// ------------------------------------------ Y requant + output transform
// A block takes 8 tiles x 32 output channels; thread (ti, ci) = (tid / 32,
// tid % 32) owns one (tile, co) pair, so M is read 32 channels (one 128-byte
// line) at a time. ROWS: one Y scale per row of taps, applied to the codes before the
// transform; otherwise one scale over all taps, applied to the result. The
// m x m outputs go through LDS and leave as output rows: consecutive threads
// write consecutive tiles of one row of one channel.
// Codes are rounded with x + 1.5 * 2^23 (exactly rint of the fp32 product,
// which stays within +-127.5; the code is that sum minus 1.5 * 2^23, and its
// low byte in two's complement). AMASK: the nonzero pattern of A^T when the
// host has verified it (the standard points'); the chains skip the zero
// terms, which is bit-identical (fma(0, y, acc) == acc: a chain starting at
// +0 never holds -0).
// Stage-3 outputs of a block of NTH threads (TI tiles x CI output channels,
// m x m pixels each, in LDS as s_out[ci][ti][pixel]) to y, one output row of
// one tile per thread step, consecutive threads on consecutive tiles. (Left
// rolled: unrolling this loop made stage 3 5-8 % slower.)
template <int M, int CI, int TI, int NTH, typename YT>
__device__ __forceinline__ void s3_store(const float (*s_out)[TI][M * M + 1], int t0, int c0, YT *y,
                                         const Geo &g) {
    for (int e = threadIdx.x; e < CI * TI * M; e += NTH) {
        const int eti = e % TI, rest = e / TI;
        const int aa = rest % M, eci = rest / M;
        const int et = t0 + eti, eco = c0 + eci;
        if (et >= g.T || eco >= g.Cout) continue;
        const int tx = et % g.tW, rr = et / g.tW, ty = rr % g.tH, img = rr / g.tH;
        const int h = ty * M + aa;
        if (h >= g.Ho) continue;
        YT *yp = y + (((size_t)img * g.Cout + eco) * g.Ho + h) * g.Wo + (size_t)tx * M;
        const int nb = min(M, g.Wo - tx * M);
        if constexpr (M % 2 == 0) {
            // with m and Wo even a tile's row starts at an even element, so
            // pairs of pixels go out as one store (8 bytes fp32, 4 bytes bf16)
            if (g.Wo % 2 == 0) {
#pragma unroll
                for (int b = 0; b < M; b += 2) {
                    const float v0 = s_out[eci][eti][aa * M + b], v1 = s_out[eci][eti][aa * M + b + 1];
                    if (b + 1 < nb) store_act2(yp + b, v0, v1);
                    else if (b < nb) store_act(yp + b, v0);
                }
                continue;
            }
        }
#pragma unroll
        for (int b = 0; b < M; ++b)
            if (b < nb) store_act(yp + b, s_out[eci][eti][aa * M + b]);
    }
}

template <int M, bool ROWS, typename YT, uint64_t AMASK>
__global__ __launch_bounds__(256) void k_stage3(const float *__restrict__ Mi, YT *__restrict__ y,
                                                int8_t *__restrict__ Yq, float *__restrict__ sY,
                                                Mats mt, Geo g) {
    constexpr int N = M + 2, NT = N * N, MM = M * M;
    constexpr int TI = 8, CI = 32;
    __shared__ float s_out[CI][TI][MM + 1];  // [ci][ti][pixel]
    const int tid = threadIdx.x;
    const int ti = tid / CI, ci = tid % CI;
    const int t0 = blockIdx.x * TI, c0 = blockIdx.y * CI;
    const int t = t0 + ti, co = c0 + ci;
    const bool ok = t < g.T && co < g.Cout;
    const size_t plane = (size_t)g.T * g.Cout;
    const size_t idx = (size_t)t * g.Cout + co;
    // raw buffer loads: no branch per load; pairs outside the layer read zero
    // (kOob plus a tap plane offset, below 2^31, stays below 2^32)
    const auto rM = make_rsrc(Mi, (size_t)NT * plane * 4);
    const int moff = ok ? (int)idx * 4 : kOob;
    float mv[NT];
#pragma unroll
    for (int tap = 0; tap < NT; ++tap)
        mv[tap] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rM, moff, tap * (int)plane * 4, 0));
    float r[NT];  // x + 1.5 * 2^23 per tap (the code is r - 1.5 * 2^23)
    float yd[NT];
    float s = 1.0f;
#pragma unroll
    for (int blk = 0; blk < (ROWS ? N : 1); ++blk) {
        // one scale over taps [k0, k0 + len)
        constexpr int len = ROWS ? N : NT;
        const int k0 = blk * len;
        float a = 0.0f;
#pragma unroll
        for (int k = 0; k < len; ++k) a = fmaxf(a, fabsf(mv[k0 + k]));
        float sc = 0.0f, inv = 0.0f;  // a == 0: every code rounds to 0
        if (a != 0.0f) {
            inv = 127.0f / a;
            sc = a / 127.0f;
        }
#pragma unroll
        for (int k = 0; k < len; ++k) r[k0 + k] = mv[k0 + k] * inv + kRoundMagic;
        if (ok && sY) sY[ROWS ? idx * N + blk : idx] = sc;
        if constexpr (ROWS) {
#pragma unroll
            for (int k = 0; k < len; ++k) yd[k0 + k] = sc * (r[k0 + k] - kRoundMagic);
        } else {
            s = sc;
#pragma unroll
            for (int k = 0; k < len; ++k) yd[k] = r[k] - kRoundMagic;
        }
    }
    if (ok && Yq) {
        uint32_t *yq = (uint32_t *)(Yq + idx * NT);  // NT is a multiple of 4
#pragma unroll
        for (int k = 0; k < NT; k += 4) yq[k / 4] = pack4(r[k], r[k + 1], r[k + 2], r[k + 3]);
    }

    float z[M][N];
#pragma unroll
    for (int aa = 0; aa < M; ++aa)
#pragma unroll
        for (int j = 0; j < N; ++j) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < N; ++i)
                if ((AMASK >> (aa * N + i)) & 1) acc = __builtin_fmaf(mt.At[aa * N + i], yd[i * N + j], acc);
            z[aa][j] = acc;
        }
#pragma unroll
    for (int aa = 0; aa < M; ++aa)
#pragma unroll
        for (int b = 0; b < M; ++b) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < N; ++j)
                if ((AMASK >> (b * N + j)) & 1) acc = __builtin_fmaf(z[aa][j], mt.At[b * N + j], acc);
            s_out[ci][ti][aa * M + b] = ROWS ? acc : acc * s;
        }
    __syncthreads();
    s3_store<M, CI, TI, 256>(s_out, t0, c0, y, g);
}

// Stage 3 with two lanes per (tile, co) pair, for layers with few pairs
// (one lane per pair would leave the SIMDs one or two waves each). Lane l
// (half h = l / 32) and lane l + 32 share a pair; lane h holds the taps of
// columns [h n/2, (h+1) n/2) of all n rows. The Y absmax (of the pair, or of
// each row of taps) meets across the halves through one permlane32 swap; the
// first pass z = A^T Yq runs over rows in index order inside each lane (its
// columns); then a permlane32 swap per (row of z, column) gives lane h rows
// [h m/2, (h+1) m/2) of z with all n columns, in column order, and the second
// pass O = z A over columns in index order produces those output rows. Every
// chain is the one-lane kernel's chain, so codes, scales and outputs are
// bit-identical to it.
template <int M, bool ROWS, typename YT, uint64_t AMASK>
__global__ __launch_bounds__(256) void k_stage3h(const float *__restrict__ Mi, YT *__restrict__ y,
                                                 int8_t *__restrict__ Yq, float *__restrict__ sY,
                                                 Mats mt, Geo g) {
    constexpr int N = M + 2, NT = N * N, MM = M * M;
    constexpr int NH = N / 2, MH = M / 2;  // columns and output rows per lane
    constexpr int TI = 4, CI = 32;         // one tile per wave, 32 channels per half
    __shared__ float s_out[CI][TI][MM + 1];
    const int lane = threadIdx.x & 63, h = lane >> 5, ci = lane & 31;
    const int ti = threadIdx.x >> 6;
    const int t0 = blockIdx.x * TI, c0 = blockIdx.y * CI;
    const int t = t0 + ti, co = c0 + ci;
    const bool ok = t < g.T && co < g.Cout;
    const int plane = (int)g.T * g.Cout;  // n^2 * plane * 4 (M's bytes) is below 2^31
    const int idx = t * g.Cout + co;
    const auto rM = make_rsrc(Mi, (size_t)NT * plane * 4);
    // tap (i, h NH + jj) at byte idx * 4 + tap * plane * 4; the lane's column
    // offset goes in the vector offset, the tap's row and column in the
    // scalar one (out of range for pairs outside the layer)
    const int moff = ok ? (idx + h * NH * plane) * 4 : kOob;
    float mv[N][NH];
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int jj = 0; jj < NH; ++jj)
            mv[i][jj] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rM, moff, (i * N + jj) * plane * 4, 0));
    // max of the two halves' non-negative maxima, on bit patterns
    auto pair_max = [](float a) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
        return __uint_as_float(max(r[0], r[1]));
    };
    float r[N][NH];   // x + 1.5 * 2^23 per tap (the code is r - 1.5 * 2^23)
    float yd[N][NH];
    float s = 1.0f;
#pragma unroll
    for (int blk = 0; blk < (ROWS ? N : 1); ++blk) {
        constexpr int rows = ROWS ? 1 : N;  // rows of taps under one scale
        const int i0 = blk * rows;
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < rows; ++i)
#pragma unroll
            for (int jj = 0; jj < NH; ++jj) a = fmaxf(a, fabsf(mv[i0 + i][jj]));
        a = pair_max(a);
        float sc = 0.0f, inv = 0.0f;  // a == 0: every code rounds to 0
        if (a != 0.0f) {
            inv = 127.0f / a;
            sc = a / 127.0f;
        }
#pragma unroll
        for (int i = 0; i < rows; ++i)
#pragma unroll
            for (int jj = 0; jj < NH; ++jj) r[i0 + i][jj] = mv[i0 + i][jj] * inv + kRoundMagic;
        if (ok && sY && h == 0) sY[ROWS ? (size_t)idx * N + blk : (size_t)idx] = sc;
        if constexpr (ROWS) {
#pragma unroll
            for (int jj = 0; jj < NH; ++jj) yd[blk][jj] = sc * (r[blk][jj] - kRoundMagic);
        } else {
            s = sc;
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int jj = 0; jj < NH; ++jj) yd[i][jj] = r[i][jj] - kRoundMagic;
        }
    }
    if (ok && Yq) {
        int8_t *yq = Yq + (size_t)idx * NT + h * NH;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if constexpr (NH == 4)
                *(uint32_t *)(yq + i * N) = pack4(r[i][0], r[i][1], r[i][2], r[i][3]);
            else
#pragma unroll
                for (int jj = 0; jj < NH; ++jj) yq[i * N + jj] = (int8_t)__float_as_uint(r[i][jj]);
        }
    }
    // first pass on this lane's columns: z[aa][jj] = sum_i A^T[aa][i] yd[i][jj]
    float z[M][NH];
#pragma unroll
    for (int aa = 0; aa < M; ++aa)
#pragma unroll
        for (int jj = 0; jj < NH; ++jj) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < N; ++i)
                if ((AMASK >> (aa * N + i)) & 1) acc = __builtin_fmaf(mt.At[aa * N + i], yd[i][jj], acc);
            z[aa][jj] = acc;
        }
    // swap(x = z[rr], y = z[MH + rr]): the lower half gets row rr (its own
    // columns in r0, the upper half's in r1), the upper half row MH + rr (the
    // lower half's columns in r0, its own in r1)
    float zr[MH][N];
#pragma unroll
    for (int rr = 0; rr < MH; ++rr)
#pragma unroll
        for (int jj = 0; jj < NH; ++jj) {
            const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(z[rr][jj]), __float_as_uint(z[MH + rr][jj]),
                                                            false, false);
            zr[rr][jj] = __uint_as_float(w[0]);
            zr[rr][NH + jj] = __uint_as_float(w[1]);
        }
#pragma unroll
    for (int rr = 0; rr < MH; ++rr)
#pragma unroll
        for (int b = 0; b < M; ++b) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < N; ++j)
                if ((AMASK >> (b * N + j)) & 1) acc = __builtin_fmaf(zr[rr][j], mt.At[b * N + j], acc);
            s_out[ci][ti][(h * MH + rr) * M + b] = ROWS ? acc : acc * s;
        }
    __syncthreads();
    s3_store<M, CI, TI, 256>(s_out, t0, c0, y, g);
}

// ------------------------------------------------- fused stages 2 + 3
// The Winograd-domain output M never leaves the chip. A block owns 16 tiles x
// 16 output channels (256 (tile, co) pairs) and all n*n taps.
//
// Hadamard part: wave w computes taps [w*NT/4, (w+1)*NT/4) of the 16 x 16
// block on int8 MFMA with U as the A operand (rows = output channels) and V as
// the B operand (columns = tiles), so lane (r, kq) ends with the four
// (co = 4kq + i, t = r) pairs for its taps. The per-group dequantization is
// the same fma chain over groups as stage 2, so M is bit-identical to it. The
// group scales of a wave's taps are staged in LDS, one group at a time, the
// next group's loaded while the current one is computed.
//
// Y: the absmax of a pair over all taps combines the four waves' partial
// maxima through LDS; one thread per pair computes 127/a and a/127 (the same
// IEEE divisions as stage 3) and the codes are rounded by the wave that holds
// the values, then stored in LDS as bytes biased by +128.
//
// Output transform: for each pair, vec(O) = (A^T (x) A^T) vec(Yq), one dense
// product for all 256 pairs of the block on fp16 MFMA (16x16x32, fp32
// accumulation). Codes are exact in fp16. The Kronecker matrix K (built per
// block in LDS from A^T) is scaled by a power of two and split into fp16 high
// and low parts, K = Kh + Kl, so Kh*Yq + Kl*Yq carries about 22 significant
// bits of K: the result differs from an fp32 evaluation of A^T Yq A by ~1e-6
// of its RMS, well inside the tolerance of the output (which, unlike the
// codes, is not required to be bit-exact). Product rows are (a, b) with b
// padded to BS, so a lane's four rows are adjacent pixels of one output row.
//
// LDS stays below 40 KB and registers below 128 so that four blocks share a
// CU: with 800 blocks (16 x 16 blocks on the ResNet-18 layer) they then run
// in a single wave of residency instead of 768 plus a tail of 32.
constexpr float kBiasedMagic = 12583040.0f;  // 1.5 * 2^23 + 128 (even)

// Code rows: 64 bytes per pair; 8-byte chunk c of pair p at c ^ ((p >> 2) & 7).
__device__ __forceinline__ int cswz(int p, int c) { return (p << 6) + ((c ^ ((p >> 2) & 7)) << 3); }
// K rows: 64 fp16 per row; 16-byte chunk c of row q at c ^ ((q >> 1) & 7).
__device__ __forceinline__ int kswz(int q, int c) { return (q << 6) + ((c ^ ((q >> 1) & 7)) << 3); }

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

// Eight biased code bytes -> eight fp16 codes: bytes u become fp16 bit
// patterns 0x6400 | u = 1024 + u, and 1024 + u - 1152 = u - 128 exactly.
__device__ __forceinline__ h8 unbias8(v2i w) {
    h8 r;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t x = (uint32_t)w[k];
        const uint32_t p0 = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
        const uint32_t p1 = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
        const h2 q0 = __builtin_bit_cast(h2, p0) - h2{(_Float16)1152.0f, (_Float16)1152.0f};
        const h2 q1 = __builtin_bit_cast(h2, p1) - h2{(_Float16)1152.0f, (_Float16)1152.0f};
        r[4 * k + 0] = q0[0];
        r[4 * k + 1] = q0[1];
        r[4 * k + 2] = q1[0];
        r[4 * k + 3] = q1[1];
    }
    return r;
}

// K = A^T (x) A^T (rows a * m + b, taps i * n + j), scaled by the plan's
// power of two and split into fp16 hi + lo parts, written to LDS by the NTH
// threads of a block. at_lds holds A^T (m x n) and is visible to them all.
template <int M, int NTH>
__device__ __forceinline__ void fused_build_ktab(const float *at_lds, _Float16 (*ktab)[M * M * 64],
                                                 float kscale) {
    constexpr int N = M + 2, NT = N * N, MM = M * M;
    const int tid = threadIdx.x;
    for (int task = tid; task < MM * 8; task += NTH) {
        const int q = task >> 3, c = task & 7;
        const int a = q / M, b = q % M;
        h8 hi, lo;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int tap = 8 * c + u;
            float kv = 0.0f;
            if (tap < NT) {
                const int i = tap / N, j = tap - (tap / N) * N;
                kv = (at_lds[a * N + i] * kscale) * at_lds[b * N + j];
            }
            const _Float16 h = (_Float16)kv;
            hi[u] = h;
            lo[u] = (_Float16)(kv - (float)h);
        }
        *(h8 *)&ktab[0][kswz(q, c)] = hi;
        *(h8 *)&ktab[1][kswz(q, c)] = lo;
    }
}

// Output transform and stores of a fused block: D[row][pair] = sum_tap
// K[row][tap] * Yq[tap][pair] on fp16 MFMA, for this wave's CBW column blocks
// cb = wave + WPB c (pairs 16 cb .. 16 cb + 15, code rows in LDS). All of a
// wave's column blocks cover the same 16 tiles, t0w .. t0w + 15 (lane
// nl = lane % 16 takes tile t0w + nl; tiles from t_end on belong to no pair
// of the block and are not stored); column block c is output channel
// co_base + co_step c. Taps NT..63 of a code row hold stale bytes: finite
// codes, multiplied by K = 0 there.
template <int M, int WPB, int CBW, typename YT>
__device__ __forceinline__ void fused_output(const uint8_t *codes, const _Float16 (*ktab)[M * M * 64],
                                             const float *s_out, int wave, int t0w, int t_end, int co_base,
                                             int co_step, YT *y, const Geo &g) {
    constexpr int BS = M == 6 ? 8 : 4;  // output row a, column b -> product row a * BS + b
    constexpr int RB = M * BS / 16;     // 16-row blocks of the output product
    constexpr int ES = sizeof(YT);
    const int lane = threadIdx.x & 63;
    const int kg = lane >> 4, nl = lane & 15;
    h8 bq[CBW][2];
#pragma unroll
    for (int c = 0; c < CBW; ++c)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            bq[c][ks] = unbias8(*(const v2i *)&codes[cswz(16 * (wave + WPB * c) + nl, 4 * ks + kg)]);
    float so[CBW];
#pragma unroll
    for (int c = 0; c < CBW; ++c) so[c] = s_out[16 * (wave + WPB * c) + nl];

    // This lane's tile; per row block, the output pixel (a, b0) of its first
    // row 16rb + 4kg and how many of its 4 adjacent pixels b0..b0+3 are inside
    // the image (rows a * BS + b with b >= m are padding).
    const int t = t0w + nl;
    int ooff[RB], nv[RB];
    {
        const int tx = t % g.tW, rr = t / g.tW, ty = rr % g.tH, img = rr / g.tH;
        const int hv = g.Ho - ty * M, wv = g.Wo - tx * M;
        const int base = (img * g.Cout * g.Ho + ty * M) * g.Wo + tx * M;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int row0 = 16 * rb + 4 * kg;
            const int a = row0 / BS, b0 = row0 % BS;
            const int n = min(4, min(M, wv) - b0);
            nv[rb] = t < t_end && a < hv && n > 0 ? n : 0;
            ooff[rb] = (base + a * g.Wo + b0) * ES;
        }
    }
    const auto ry = make_rsrc(y, (size_t)g.N * g.Cout * g.Ho * g.Wo * ES);
    const int hw = g.Ho * g.Wo;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        // A fragment: product row 16rb + nl = (a, b); padding rows are zero
        h8 ka[2][2];
        const int prow = 16 * rb + nl, pa = prow / BS, pb = prow % BS;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                if (pb < M) ka[ks][part] = *(const h8 *)&ktab[part][kswz(pa * M + pb, 4 * ks + kg)];
                else ka[ks][part] = h8{0, 0, 0, 0, 0, 0, 0, 0};
            }
#pragma unroll
        for (int cb = 0; cb < CBW; ++cb) {
            f4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int part = 0; part < 2; ++part)
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[ks][part], bq[cb][ks], d, 0, 0, 0);
            const int co = co_base + co_step * cb;
            if (co < g.Cout) {
                const int soff = co * hw * ES;
                const int o = ooff[rb], n = nv[rb];
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = d[i] * so[cb];
                if constexpr (ES == 4) {
                    if (n == 4) {
                        const v4i q = {(int)__float_as_uint(v[0]), (int)__float_as_uint(v[1]),
                                       (int)__float_as_uint(v[2]), (int)__float_as_uint(v[3])};
                        __builtin_amdgcn_raw_buffer_store_b128(q, ry, o, soff, 0);
                    } else {
                        if (n >= 2) {
                            const v2i q = {(int)__float_as_uint(v[0]), (int)__float_as_uint(v[1])};
                            __builtin_amdgcn_raw_buffer_store_b64(q, ry, o, soff, 0);
                        }
                        if (n & 1) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[n - 1]), ry, o + 4 * (n - 1), soff, 0);
                    }
                } else {
                    uint32_t hb[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t u = __float_as_uint(v[i]);
                        hb[i] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
                    }
                    if (n == 4) {
                        const v2i q = {(int)(hb[0] | hb[1] << 16), (int)(hb[2] | hb[3] << 16)};
                        __builtin_amdgcn_raw_buffer_store_b64(q, ry, o, soff, 0);
                    } else {
                        if (n >= 2) __builtin_amdgcn_raw_buffer_store_b32(hb[0] | hb[1] << 16, ry, o, soff, 0);
                        if (n & 1) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hb[n - 1], ry, o + 2 * (n - 1), soff, 0);
                    }
                }
            }
        }
    }
}

// WPB: waves per block (the block's taps are split evenly between them).
// MULTI: more than one quantization group along Cin (the group loop runs and
// prefetches across groups).
template <int M, int G, int WPB, bool MULTI, typename YT>
__global__ __launch_bounds__(64 * WPB, WPB == 4 && MULTI ? 3 : 4) void k_fused23(const int8_t *__restrict__ Vq,
                                                 const float *__restrict__ sV,
                                                 const int8_t *__restrict__ Uq,
                                                 const float *__restrict__ sU, YT *__restrict__ y,
                                                 Mats mt, Geo g) {
    constexpr int N = M + 2, NT = N * N, TPW = NT / WPB, MM = M * M, NTH = 64 * WPB;
    constexpr int CBW = 16 / WPB;       // output column blocks (16 pairs) per wave
    constexpr bool K64 = G % 64 == 0;
    constexpr int KSTEPS = K64 ? G / 64 : 1;
    static_assert(NT <= 64 && TPW * WPB == NT && TPW <= 16 && CBW * WPB == 16, "taps per wave");
    // codes: 256 pairs x 64 bytes; during the Hadamard part each wave uses its
    // share (16 KB / WPB) for one group's scales [2][TPW taps][16 rows], then
    // for its partial maxima (256 floats)
    constexpr int WLDS = 4096 / WPB;  // floats per wave
    static_assert(WLDS >= 256 && WLDS >= 2 * TPW * 16, "per-wave LDS share");
    __shared__ __attribute__((aligned(16))) uint8_t codes[256 * 64];
    __shared__ __attribute__((aligned(16))) _Float16 ktab[2][MM * 64];  // K rows a * m + b
    __shared__ float s_inv[256], s_out[256];
    __shared__ float at_lds[M * N];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int nco = (g.Cout + 15) / 16;
    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int ntb = (int)((g.T + 15) / 16);
    const int cob = g.co_major ? blk / ntb : blk % nco;
    const int tb = g.co_major ? blk % ntb : blk / nco;
    const int t0 = tb * 16, co0 = cob * 16;
    const int tap0 = wave * TPW;
    const size_t vplane = (size_t)g.T * g.Cin, uplane = (size_t)g.Cout * g.Cin;
    float *wlds = reinterpret_cast<float *>(codes) + wave * WLDS;

    // ---- K = A^T (x) A^T (rows a * m + b, taps i * n + j), scaled, fp16 hi/lo
    if (tid < M * N) at_lds[tid] = mt.At[tid];
    __syncthreads();
    fused_build_ktab<M, NTH>(at_lds, ktab, mt.kscale);

    // ---- Hadamard GEMMs for this wave's taps
    // Rows past T or Cout read row 0 instead: they only feed (tile, co) pairs
    // that are never stored, and unconditional loads let the compiler keep
    // many taps' operands in flight.
    const int tB = t0 + r;          // B column: tile
    const int coA = co0 + r;        // A row: output channel
    const int tBc = tB < g.T ? tB : 0, coAc = coA < g.Cout ? coA : 0;
    const int n2 = g.n * g.n;
    const auto rV = make_rsrc(Vq, (size_t)n2 * vplane);
    const auto rU = make_rsrc(Uq, (size_t)n2 * uplane);
    const auto rsV = make_rsrc(sV, (size_t)n2 * g.T * g.ng * 4);
    const auto rsU = make_rsrc(sU, (size_t)n2 * g.Cout * g.ng * 4);
    // lane offsets (bytes) that do not change with the tap or group
    const bool kin = K64 || 8 * kq < G;          // K slots inside the group
    const int koff = K64 ? 16 * kq : (kin ? 8 * kq : 0);
    const int voff = tBc * g.Cin + koff;
    const int uoff = coAc * g.Cin + koff;
    float acc[TPW][4];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = 0.0f;

    // Operands of one tap for one group (G < 64: one 8-byte K slice each).
    struct TapOps {
        v4i a[K64 ? KSTEPS : 0], b[K64 ? KSTEPS : 0];
        long a8, b8;
    };
    auto load_tap = [&](int j, int gi, TapOps &o) {
        const int tap = tap0 + j;
        const int vs = tap * (int)vplane + gi * G, us = tap * (int)uplane + gi * G;
        if constexpr (K64) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                o.a[ks] = __builtin_amdgcn_raw_buffer_load_b128(rU, uoff, us + ks * 64, 0);
                o.b[ks] = __builtin_amdgcn_raw_buffer_load_b128(rV, voff, vs + ks * 64, 0);
            }
        } else {
            const auto a2 = __builtin_amdgcn_raw_buffer_load_b64(rU, uoff, us, 0);
            const auto b2 = __builtin_amdgcn_raw_buffer_load_b64(rV, voff, vs, 0);
            o.a8 = ((long)(uint32_t)a2[1] << 32) | (uint32_t)a2[0];
            o.b8 = ((long)(uint32_t)b2[1] << 32) | (uint32_t)b2[0];
        }
    };
    // Group scales of this wave's taps for one group, staged in its LDS
    // quarter: wlds[(s * 16 + j) * 16 + row], s = 0 for sV (row = tile), 1 for
    // sU (row = output channel). The next group's are loaded into registers
    // while the current group is computed.
    // slot e = 64k + lane: s = e / (16 TPW) (0: sV, row = tile; 1: sU, row =
    // output channel), tap j = (e / 16) % TPW, row = e % 16
    constexpr int SL = (2 * TPW * 16 + 63) / 64;  // scale loads per lane
    auto load_scales = [&](int gi, float (&sreg)[SL]) {
        const int row = lane & 15;
        const int tr = t0 + row < g.T ? t0 + row : 0, cr = co0 + row < g.Cout ? co0 + row : 0;
#pragma unroll
        for (int k = 0; k < SL; ++k) {
            const int e = 64 * k + lane;
            const int sw = e / (16 * TPW), j = (e / 16) % TPW;
            const int tap = tap0 + j;
            const int off = sw == 0 ? ((tap * (int)g.T + tr) * g.ng + gi) * 4 : ((tap * g.Cout + cr) * g.ng + gi) * 4;
            // slots past 2 * TPW * 16 (sw == 2) read past the end: zero, never stored
            sreg[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sw == 0 ? rsV : rsU,
                                                                           sw < 2 ? off : 0x7ffffff0, 0, 0));
        }
    };
    auto put_scales = [&](const float (&sreg)[SL]) {
#pragma unroll
        for (int k = 0; k < SL; ++k) {
            const int e = 64 * k + lane;
            if (e < 2 * TPW * 16) wlds[e] = sreg[k];
        }
    };
    auto use_tap = [&](int j, const TapOps &o) {
        v4i P = v4i{0, 0, 0, 0};
        if constexpr (K64) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                P = __builtin_amdgcn_mfma_i32_16x16x64_i8(o.a[ks], o.b[ks], P, 0, 0, 0);
        } else {
            // K = 32; for G = 16 the upper 16 K slots are zero
            P = __builtin_amdgcn_mfma_i32_16x16x32_i8(kin ? o.a8 : 0, kin ? o.b8 : 0, P, 0, 0, 0);
        }
        const float sv = wlds[j * 16 + r];
        const float4 su = *(const float4 *)&wlds[(TPW + j) * 16 + 4 * kq];
        const float sus[4] = {su.x, su.y, su.z, su.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float sc = sv * sus[i];
            acc[j][i] = __builtin_fmaf(sc, (float)P[i], acc[j][i]);
        }
    };
    // Two batches of taps in flight: the next batch's loads (of this group or,
    // when a group has an even number of batches, of the next group) are
    // issued before the current batch's MFMAs and dequantization. With 8
    // waves per block a wave's 8 taps of a group are loaded at once.
    constexpr int BATCH = KSTEPS >= 2 ? 1
                          : WPB == 8 ? TPW
                          : TPW % 4 == 0 && TPW / 4 % 2 == 0 && !K64 ? 4
                          : TPW % 2 == 0 ? 2 : TPW % 3 == 0 ? 3 : 1;
    constexpr int NB = TPW / BATCH;
    constexpr bool XG = NB % 2 == 0;  // prefetch across group boundaries
    static_assert(NB * BATCH == TPW, "batches per group");
    TapOps buf[2][BATCH];
    float snext[SL];
    load_scales(0, snext);
    if constexpr (XG) {
#pragma unroll
        for (int b = 0; b < BATCH; ++b) load_tap(b, 0, buf[0][b]);
    }
    const int ng = MULTI ? g.ng : 1;
    for (int gi = 0; gi < ng; ++gi) {
        put_scales(snext);
        const int gnext = gi + 1 < ng ? gi + 1 : gi;  // the last group reloads itself (unused)
        load_scales(gnext, snext);
        if constexpr (!XG) {
#pragma unroll
            for (int b = 0; b < BATCH; ++b) load_tap(b, gi, buf[0][b]);
        }
#pragma unroll
        for (int jb = 0; jb < TPW; jb += BATCH) {
            const int cur = (jb / BATCH) & 1;
            if (jb + BATCH < TPW) {
#pragma unroll
                for (int b = 0; b < BATCH; ++b) load_tap(jb + BATCH + b, gi, buf[cur ^ 1][b]);
            } else if (XG) {
#pragma unroll
                for (int b = 0; b < BATCH; ++b) load_tap(b, gnext, buf[cur ^ 1][b]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < BATCH; ++b) use_tap(jb + b, buf[cur][b]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- Y absmax per pair: partial maxima of this wave's taps (its own LDS
    // quarter is free once its Hadamard part is done)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < TPW; ++j) m = fmaxf(m, fabsf(acc[j][i]));
        wlds[(4 * kq + i) * 16 + r] = m;
    }
    __syncthreads();
    if (tid < 256) {
        const float *pm = reinterpret_cast<const float *>(codes);
        float am = pm[tid];
#pragma unroll
        for (int w = 1; w < WPB; ++w) am = fmaxf(am, pm[w * WLDS + tid]);
        float inv = 0.0f, sy = 0.0f;
        if (am != 0.0f) {
            inv = 127.0f / am;
            sy = am / 127.0f;
        }
        s_inv[tid] = inv;
        s_out[tid] = sy * mt.oscale;
    }
    __syncthreads();
    // ---- codes of this wave's taps, biased bytes, into the pair rows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = (4 * kq + i) * 16 + r;
        const float inv = s_inv[p];
        float yb[TPW];
#pragma unroll
        for (int j = 0; j < TPW; ++j) yb[j] = acc[j][i] * inv + kBiasedMagic;  // low byte: code + 128
        if constexpr (TPW % 8 == 0) {
#pragma unroll
            for (int c = 0; c < TPW / 8; ++c) {
                const v2i w = {(int)pack4(yb[8 * c], yb[8 * c + 1], yb[8 * c + 2], yb[8 * c + 3]),
                               (int)pack4(yb[8 * c + 4], yb[8 * c + 5], yb[8 * c + 6], yb[8 * c + 7])};
                *(v2i *)&codes[cswz(p, tap0 / 8 + c)] = w;
            }
        } else if constexpr (TPW == 4) {
            *(uint32_t *)&codes[cswz(p, tap0 >> 3) + (tap0 & 7)] = pack4(yb[0], yb[1], yb[2], yb[3]);
        } else {
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int tap = tap0 + j;
                codes[cswz(p, tap >> 3) + (tap & 7)] = (uint8_t)__float_as_uint(yb[j]);
            }
        }
    }
    __syncthreads();

    // ---- output transform: column block cb = wave + WPB c holds tiles
    // t0 .. t0 + 15 of output channel co0 + cb
    fused_output<M, WPB, CBW, YT>(codes, ktab, s_out, wave, t0, (int)g.T, co0 + wave, WPB, y, g);
}

// Wide fused blocks, F(6,3): HT x 16 tiles by HC x 16 output channels, with
// (HT, HC) = (2, 2), (2, 1) or (1, 2), and 4 HT HC waves of NT / (4 HT HC)
// taps each. Per tap a wave computes the HC x HT 16 x 16 products of the
// block's channel and tile halves, so each operand byte it loads feeds HT or
// HC MFMAs (a 16 x 16 block loads 2 KB per tap for 256 pairs; a 32 x 32 one
// 4 KB for 1024). Pair p = 16 HT (co - co0) + (t - t0); 16 consecutive pairs
// (one channel, 16 tiles) form an output column block as in k_fused23, and
// the Y quantization and output transform are those of k_fused23 over the
// block's column blocks, so the output is bit for bit that of k_fused23.
template <int M, int G, int HT, int HC, bool MULTI, typename YT>
__global__ __launch_bounds__(256 * HT * HC, 1) void k_fused23w(const int8_t *__restrict__ Vq,
                                                               const float *__restrict__ sV,
                                                               const int8_t *__restrict__ Uq,
                                                               const float *__restrict__ sU,
                                                               YT *__restrict__ y, Mats mt, Geo g) {
    constexpr int N = M + 2, NT = N * N, MM = M * M, WPB = 4 * HT * HC, NTH = 64 * WPB;
    constexpr int TPW = NT / WPB;            // taps per wave: 4 or 8
    constexpr int NP = 256 * HT * HC;        // pairs per block
    constexpr int CBW = NP / 16 / WPB;       // output column blocks per wave (4)
    constexpr int RT = 16 * HT, RC = 16 * HC;  // tile rows of V, channel rows of U
    constexpr bool K64 = G % 64 == 0;
    constexpr int KSTEPS = K64 ? G / 64 : 1;
    constexpr int WLDS = NP * 64 / 4 / WPB;  // floats of the code rows per wave (1024)
    constexpr int NSV = TPW * RT, NSC = TPW * (RT + RC);  // staged scales per wave
    static_assert(M == 6 && TPW * WPB == NT && (TPW == 4 || TPW == 8), "F(6,3): 4 or 8 taps per wave");
    static_assert(HT * HC >= 2 && HT <= 2 && HC <= 2, "2 x 2, 2 x 1 or 1 x 2 halves");
    static_assert(WLDS >= NP && WLDS >= NSC && NSC % 64 == 0, "per-wave LDS share");
    __shared__ __attribute__((aligned(16))) uint8_t codes[NP * 64];
    __shared__ __attribute__((aligned(16))) _Float16 ktab[2][MM * 64];
    __shared__ float s_inv[NP], s_out[NP];
    __shared__ float at_lds[M * N];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int nco = (g.Cout + RC - 1) / RC;
    const int ntb = g.fused_ntb;  // at least ceil(T / RT), so a block has at most RT tiles
    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int cob = g.co_major ? blk / ntb : blk % nco;
    const int tb = g.co_major ? blk % ntb : blk / nco;
    const int t0 = (int)((int64_t)tb * g.T / ntb), t1 = (int)((int64_t)(tb + 1) * g.T / ntb);
    const int co0 = cob * RC;
    const int tap0 = wave * TPW;
    const size_t vplane = (size_t)g.T * g.Cin, uplane = (size_t)g.Cout * g.Cin;
    float *wlds = reinterpret_cast<float *>(codes) + wave * WLDS;

    // ---- K = A^T (x) A^T, scaled, fp16 hi/lo
    if (tid < M * N) at_lds[tid] = mt.At[tid];
    __syncthreads();
    fused_build_ktab<M, NTH>(at_lds, ktab, mt.kscale);

    // ---- Hadamard GEMMs: A = U rows co0 + 16 hc + r, B = V rows t0 + 16 ht + r
    // (channel rows past Cout read row 0 and tile rows past the block's last
    // tile read zero: they feed pairs that are never stored)
    const int n2 = g.n * g.n;
    const auto rV = make_rsrc(Vq, (size_t)n2 * vplane);
    const auto rU = make_rsrc(Uq, (size_t)n2 * uplane);
    const auto rsV = make_rsrc(sV, (size_t)n2 * g.T * g.ng * 4);
    const auto rsU = make_rsrc(sU, (size_t)n2 * g.Cout * g.ng * 4);
    const bool kin = K64 || 8 * kq < G;
    const int koff = K64 ? 16 * kq : (kin ? 8 * kq : 0);
    int voff[HT], uoff[HC];
#pragma unroll
    for (int h = 0; h < HT; ++h) {
        const int tB = t0 + 16 * h + r;
        voff[h] = tB < t1 ? tB * g.Cin + koff : kOob;
    }
#pragma unroll
    for (int h = 0; h < HC; ++h) {
        const int coA = co0 + 16 * h + r;
        uoff[h] = (coA < g.Cout ? coA : 0) * g.Cin + koff;
    }
    float acc[TPW][HC][HT][4];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int hc = 0; hc < HC; ++hc)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[j][hc][ht][i] = 0.0f;

    struct TapOps {
        v4i a[HC][K64 ? KSTEPS : 0], b[HT][K64 ? KSTEPS : 0];
        long a8[HC], b8[HT];
    };
    auto load_tap = [&](int j, int gi, TapOps &o) {
        const int tap = tap0 + j;
        const int vs = tap * (int)vplane + gi * G, us = tap * (int)uplane + gi * G;
#pragma unroll
        for (int h = 0; h < HC; ++h) {
            if constexpr (K64) {
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    o.a[h][ks] = __builtin_amdgcn_raw_buffer_load_b128(rU, uoff[h], us + ks * 64, 0);
            } else {
                const auto a2 = __builtin_amdgcn_raw_buffer_load_b64(rU, uoff[h], us, 0);
                o.a8[h] = ((long)(uint32_t)a2[1] << 32) | (uint32_t)a2[0];
            }
        }
#pragma unroll
        for (int h = 0; h < HT; ++h) {
            if constexpr (K64) {
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    o.b[h][ks] = __builtin_amdgcn_raw_buffer_load_b128(rV, voff[h], vs + ks * 64, 0);
            } else {
                const auto b2 = __builtin_amdgcn_raw_buffer_load_b64(rV, voff[h], vs, 0);
                o.b8[h] = ((long)(uint32_t)b2[1] << 32) | (uint32_t)b2[0];
            }
        }
    };
    // group scales of this wave's taps, staged in its LDS share: sV of tap j
    // at wlds[j * RT + row] (row = tile), then sU at wlds[NSV + j * RC + row]
    constexpr int SL = NSC / 64;
    auto load_scales = [&](int gi, float (&sreg)[SL]) {
#pragma unroll
        for (int k = 0; k < SL; ++k) {
            const int e = 64 * k + lane;
            const bool isv = e < NSV;
            const int ev = isv ? e : e - NSV;
            const int rows = isv ? RT : RC;
            const int j = ev / rows, row = ev % rows;
            const int tap = tap0 + j;
            int off;
            if (isv) {
                const int tr = t0 + row < t1 ? t0 + row : 0;
                off = ((tap * (int)g.T + tr) * g.ng + gi) * 4;
            } else {
                const int cr = co0 + row < g.Cout ? co0 + row : 0;
                off = ((tap * g.Cout + cr) * g.ng + gi) * 4;
            }
            // which descriptor is uniform per load: NSV is a multiple of 64
            sreg[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(64 * k < NSV ? rsV : rsU, off, 0, 0));
        }
    };
    auto put_scales = [&](const float (&sreg)[SL]) {
#pragma unroll
        for (int k = 0; k < SL; ++k) wlds[64 * k + lane] = sreg[k];
    };
    auto use_tap = [&](int j, const TapOps &o) {
#pragma unroll
        for (int hc = 0; hc < HC; ++hc)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                v4i P = v4i{0, 0, 0, 0};
                if constexpr (K64) {
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ++ks)
                        P = __builtin_amdgcn_mfma_i32_16x16x64_i8(o.a[hc][ks], o.b[ht][ks], P, 0, 0, 0);
                } else {
                    P = __builtin_amdgcn_mfma_i32_16x16x32_i8(kin ? o.a8[hc] : 0, kin ? o.b8[ht] : 0, P, 0, 0, 0);
                }
                const float sv = wlds[j * RT + 16 * ht + r];
                const float4 su = *(const float4 *)&wlds[NSV + j * RC + 16 * hc + 4 * kq];
                const float sus[4] = {su.x, su.y, su.z, su.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[j][hc][ht][i] = __builtin_fmaf(sv * sus[i], (float)P[i], acc[j][hc][ht][i]);
            }
    };
    // one tap per batch, the next tap's (or the next group's first tap's)
    // operands in flight while the current one is computed
    TapOps buf[2];
    float snext[SL];
    load_scales(0, snext);
    load_tap(0, 0, buf[0]);
    const int ng = MULTI ? g.ng : 1;
    for (int gi = 0; gi < ng; ++gi) {
        put_scales(snext);
        const int gnext = gi + 1 < ng ? gi + 1 : gi;  // the last group reloads itself (unused)
        load_scales(gnext, snext);
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int cur = j & 1;
            if (j + 1 < TPW) load_tap(j + 1, gi, buf[cur ^ 1]);
            else load_tap(0, gnext, buf[cur ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
            use_tap(j, buf[cur]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- Y absmax per pair: this wave's partial maxima in its LDS share
#pragma unroll
    for (int hc = 0; hc < HC; ++hc)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float m = 0.0f;
#pragma unroll
                for (int j = 0; j < TPW; ++j) m = fmaxf(m, fabsf(acc[j][hc][ht][i]));
                wlds[(16 * hc + 4 * kq + i) * RT + 16 * ht + r] = m;
            }
    __syncthreads();
    for (int p = tid; p < NP; p += NTH) {
        const float *pm = reinterpret_cast<const float *>(codes);
        float am = pm[p];
#pragma unroll
        for (int w = 1; w < WPB; ++w) am = fmaxf(am, pm[w * WLDS + p]);
        float inv = 0.0f, sy = 0.0f;
        if (am != 0.0f) {
            inv = 127.0f / am;
            sy = am / 127.0f;
        }
        s_inv[p] = inv;
        s_out[p] = sy * mt.oscale;
    }
    __syncthreads();
    // ---- codes of this wave's taps, biased bytes, into the pair rows
#pragma unroll
    for (int hc = 0; hc < HC; ++hc)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = (16 * hc + 4 * kq + i) * RT + 16 * ht + r;
                const float inv = s_inv[p];
                float yb[TPW];
#pragma unroll
                for (int j = 0; j < TPW; ++j) yb[j] = acc[j][hc][ht][i] * inv + kBiasedMagic;
                if constexpr (TPW == 8) {
                    const v2i w = {(int)pack4(yb[0], yb[1], yb[2], yb[3]), (int)pack4(yb[4], yb[5], yb[6], yb[7])};
                    *(v2i *)&codes[cswz(p, tap0 >> 3)] = w;
                } else {
                    *(uint32_t *)&codes[cswz(p, tap0 >> 3) + (tap0 & 7)] = pack4(yb[0], yb[1], yb[2], yb[3]);
                }
            }
    __syncthreads();

    // ---- output transform: column block cb = wave + WPB c holds pairs
    // 16 cb .. 16 cb + 15, i.e. channel co0 + cb / HT and tiles
    // t0 + 16 (cb % HT) + 0..15; cb % HT == wave % HT for all of a wave's blocks
    fused_output<M, WPB, CBW, YT>(codes, ktab, s_out, wave, t0 + 16 * (wave % HT), t1, co0 + wave / HT, WPB / HT,
                                  y, g);
}

// ------------------------------------------------------------- launchers
wq8_status check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(WQ8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return WQ8_OK;
}

template <int M, int G>
static void weights_m_g(const Geo &g, const Mats &mt, const float *w, int8_t *Uq, float *sU,
                        hipStream_t s) {
    using S = GroupShape<G>;
    dim3 grid((g.Cout + S::TPB - 1) / S::TPB, (g.Cin + S::CPB - 1) / S::CPB);
    hipLaunchKernelGGL((k_weights<M, G>), grid, dim3(256), 0, s, w, Uq, sU, mt, g);
}

template <int M>
static void weights_m(const Geo &g, const Mats &mt, const float *w, int8_t *Uq, float *sU,
                      hipStream_t s) {
    switch (g.G) {
        case 16: weights_m_g<M, 16>(g, mt, w, Uq, sU, s); break;
        case 32: weights_m_g<M, 32>(g, mt, w, Uq, sU, s); break;
        case 64: weights_m_g<M, 64>(g, mt, w, Uq, sU, s); break;
        case 128: weights_m_g<M, 128>(g, mt, w, Uq, sU, s); break;
        default: weights_m_g<M, 256>(g, mt, w, Uq, sU, s); break;
    }
}

wq8_status launch_weights(const Geo &g, const Mats &mt, const float *w, int8_t *Uq, float *sU,
                          void *stream) {
    hipStream_t s = (hipStream_t)stream;
    if (g.m == 4) weights_m<4>(g, mt, w, Uq, sU, s);
    else weights_m<6>(g, mt, w, Uq, sU, s);
    return check_launch("weight transform");
}

// Compute units of the current device (queried once per device).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int M, int G, int TPB, uint64_t BMASK, typename XT, bool IQ, bool RH>
static void stage1_launch_q(const Geo &g, const Mats &mt, const XT *x, int8_t *Vq, float *sV,
                            hipStream_t s) {
    using SS = S1Shape<M, G, TPB, RH>;
    const int nstrip = (g.tW + TPB - 1) / TPB;
    const int chunks = (g.Cin + SS::CPB - 1) / SS::CPB;
    const unsigned blocks = (unsigned)(nstrip * g.N * g.tH * chunks);
    if (g.W % 4 == 0)
        hipLaunchKernelGGL((k_stage1<M, G, TPB, BMASK, true, XT, IQ, RH>), dim3(blocks), dim3(64 * SS::NW), 0,
                           s, x, Vq, sV, mt, g);
    else
        hipLaunchKernelGGL((k_stage1<M, G, TPB, BMASK, false, XT, IQ, RH>), dim3(blocks), dim3(64 * SS::NW),
                           0, s, x, Vq, sV, mt, g);
}

template <int M, int G, int TPB, uint64_t BMASK, typename XT>
static void stage1_launch(const Geo &g, const Mats &mt, const XT *x, int8_t *Vq, float *sV,
                          hipStream_t s) {
    if (g.in_quant) {
        stage1_launch_q<M, G, TPB, BMASK, XT, true, false>(g, mt, x, Vq, sV, s);
        return;
    }
    // half-row windows when the strips outnumber the blocks that full
    // windows let the GPU hold at once (one generation instead of two)
    bool rh = g.s1_rows == 2;
    if (g.s1_rows == 0) {
        // resident full-window blocks per CU for this instantiation (both load
        // forms use the same LDS and nearly the same registers)
        static std::atomic<int> per_cu_cache{-1};
        int per_cu = per_cu_cache.load(std::memory_order_relaxed);
        if (per_cu < 0) {
            int n = 0;
            using SS = S1Shape<M, G, TPB>;
            const auto k = k_stage1<M, G, TPB, BMASK, true, XT, false, false>;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, 64 * SS::NW, 0) != hipSuccess) {
                n = 0;                 // full windows; the failed query must not
                (void)hipGetLastError();  // surface as a launch error
            }
            per_cu = n;
            per_cu_cache.store(n, std::memory_order_relaxed);
        }
        using SS = S1Shape<M, G, TPB>;
        const int64_t nblk = (int64_t)((g.tW + TPB - 1) / TPB) * g.N * g.tH * ((g.Cin + SS::CPB - 1) / SS::CPB);
        rh = per_cu > 0 && nblk > (int64_t)per_cu * device_cus();
    }
    if (rh) stage1_launch_q<M, G, TPB, BMASK, XT, false, true>(g, mt, x, Vq, sV, s);
    else stage1_launch_q<M, G, TPB, BMASK, XT, false, false>(g, mt, x, Vq, sV, s);
}

template <int M, int G, typename XT>
static void stage1_m_g(const Geo &g, const Mats &mt, const XT *x, int8_t *Vq, float *sV,
                       hipStream_t s) {
    constexpr uint64_t pat = M == 4 ? kBtPattern4 : kBtPattern6;
    // tiles per block: 4 (one wave each) up to 128-channel groups; 1 for 256
    constexpr int tpb = GroupShape<G>::GW <= 2 ? 4 : 1;
    if (g.bt_std) stage1_launch<M, G, tpb, pat, XT>(g, mt, x, Vq, sV, s);
    else stage1_launch<M, G, tpb, ~0ull, XT>(g, mt, x, Vq, sV, s);
}

template <int M, typename XT>
static void stage1_m(const Geo &g, const Mats &mt, const XT *x, int8_t *Vq, float *sV,
                     hipStream_t s) {
    switch (g.G) {
        case 16: stage1_m_g<M, 16>(g, mt, x, Vq, sV, s); break;
        case 32: stage1_m_g<M, 32>(g, mt, x, Vq, sV, s); break;
        case 64: stage1_m_g<M, 64>(g, mt, x, Vq, sV, s); break;
        case 128: stage1_m_g<M, 128>(g, mt, x, Vq, sV, s); break;
        default: stage1_m_g<M, 256>(g, mt, x, Vq, sV, s); break;
    }
}

wq8_status launch_stage1(const Geo &g, const Mats &mt, wq8_dtype xdt, const void *x, int8_t *Vq,
                         float *sV, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    if (xdt == WQ8_F32) {
        if (g.m == 4) stage1_m<4>(g, mt, (const float *)x, Vq, sV, s);
        else stage1_m<6>(g, mt, (const float *)x, Vq, sV, s);
    } else {
        if (g.m == 4) stage1_m<4>(g, mt, (const uint16_t *)x, Vq, sV, s);
        else stage1_m<6>(g, mt, (const uint16_t *)x, Vq, sV, s);
    }
    return check_launch("input transform");
}

template <int G>
static void stage2_g(const Geo &g, const int8_t *Vq, const float *sV, const int8_t *Uq,
                     const float *sU, float *M, int32_t *P, hipStream_t s) {
    constexpr int BC = 64;  // 128-channel blocks measured 7-22 % slower on every layer
    int kc = S2<G, BC>::KCM;
    while (g.Cin % kc) kc >>= 1;  // Cin is a multiple of G >= 16
    // one dimension: the kernel derives (tile block, channel block, tap)
    const unsigned nb = (unsigned)((g.T + S2<G, BC>::BT - 1) / S2<G, BC>::BT) * ((g.Cout + BC - 1) / BC) * (g.n * g.n);
    dim3 grid(nb);
    if (P) hipLaunchKernelGGL((k_stage2<G, BC, true>), grid, dim3(256), 0, s, Vq, sV, Uq, sU, M, P, g, kc);
    else hipLaunchKernelGGL((k_stage2<G, BC, false>), grid, dim3(256), 0, s, Vq, sV, Uq, sU, M, P, g, kc);
}

wq8_status launch_stage2(const Geo &g, const int8_t *Vq, const float *sV, const int8_t *Uq,
                         const float *sU, float *M, int32_t *P, void *stream) {
    // Up to 128 input channels (one or two chunks) the LDS-pipelined kernel
    // below is faster (ResNet-18 56 x 56 layer, staged: 14.6 against 20 us);
    // from 256 channels on the register-streamed kernel (c5 layers: 70 -> 45
    // us for 1280 channels, G = 32). stage2_rows forces one: 1 this kernel,
    // 4, 5, 6 or 8 the other.
    if (g.s2_rows > 1 || (g.s2_rows == 0 && g.Cin > 128)) return launch_hgemm(g, Vq, sV, Uq, sU, M, P, stream);
    hipStream_t s = (hipStream_t)stream;
    switch (g.G) {
        case 16: stage2_g<16>(g, Vq, sV, Uq, sU, M, P, s); break;
        case 32: stage2_g<32>(g, Vq, sV, Uq, sU, M, P, s); break;
        case 64: stage2_g<64>(g, Vq, sV, Uq, sU, M, P, s); break;
        case 128: stage2_g<128>(g, Vq, sV, Uq, sU, M, P, s); break;
        default: stage2_g<256>(g, Vq, sV, Uq, sU, M, P, s); break;
    }
    return check_launch("Hadamard GEMM");
}

// Two lanes per (tile, co) pair when one lane per pair gives the device
// fewer than 1.25 waves per SIMD (the plan's stage3_lanes may force 1 or 2).
// Measured stage 3 (one lane -> two): 7 x 7, C = 512 (1.0 waves per SIMD)
// 6.8 -> 5.6 us; 14 x 14, C = 256 (1.1) 8.7 -> 7.9 us; 16 x 16, C = 1280
// (1.4) 10.0 either way; 64 x 64, C = 320, F(4,3) (2.5) 6.9 -> 7.3 us;
// 32 x 32, C = 640 (2.8) 15.3 -> 17.6 us.
static bool stage3_split(const Geo &g, int cus) {
    if (g.s3_lanes) return g.s3_lanes == 2;
    const int64_t waves = (g.T * (int64_t)g.Cout + 63) / 64;
    return 4 * waves < 5 * 4 * (int64_t)cus;
}

template <int M, typename YT>
static void stage3_m(const Geo &g, const Mats &mt, const float *Mi, YT *y, int8_t *Yq, float *sY,
                     hipStream_t s) {
    constexpr uint64_t pat = M == 4 ? kAtPattern4 : kAtPattern6;
    if (stage3_split(g, device_cus())) {
        dim3 grid((unsigned)((g.T + 3) / 4), (g.Cout + 31) / 32);
#define WQ8_S3(ROWS_, MASK_) hipLaunchKernelGGL((k_stage3h<M, ROWS_, YT, MASK_>), grid, dim3(256), 0, s, Mi, y, Yq, sY, mt, g)
        if (g.y_rows) {
            if (g.at_std) WQ8_S3(true, pat);
            else WQ8_S3(true, ~0ull);
        } else {
            if (g.at_std) WQ8_S3(false, pat);
            else WQ8_S3(false, ~0ull);
        }
#undef WQ8_S3
        return;
    }
    dim3 grid((unsigned)((g.T + 7) / 8), (g.Cout + 31) / 32);
#define WQ8_S3(ROWS_, MASK_) hipLaunchKernelGGL((k_stage3<M, ROWS_, YT, MASK_>), grid, dim3(256), 0, s, Mi, y, Yq, sY, mt, g)
    if (g.y_rows) {
        if (g.at_std) WQ8_S3(true, pat);
        else WQ8_S3(true, ~0ull);
    } else {
        if (g.at_std) WQ8_S3(false, pat);
        else WQ8_S3(false, ~0ull);
    }
#undef WQ8_S3
}

// Fused block shape for a layer: waves per 16 x 16 block and the wide form
// (0 16 x 16; 1 32 x 32, 2 32 tiles x 16 channels, 3 16 tiles x 32 channels).
// The plan's values win where it forced one.
//   Waves: with at least three 16 x 16 blocks per CU, 4-wave blocks keep every
//   block resident at once (up to five fit a CU); with fewer blocks, 8-wave
//   blocks (F(6,3): 8 taps per wave, all loaded at once) put more loads in
//   flight per block: 4-10 % faster on the deeper layers, 2 % slower on the
//   56 x 56 ResNet-18 layer. 16 waves were never faster.
//   Wide blocks (F(6,3), G <= 64) let each tap's operands feed two MFMAs
//   (48 operand rows per block instead of 2 x 32 for two 16 x 16 blocks).
//   The busiest CU loads (its blocks) x (tile rows + channel rows) operand
//   rows per tap and K byte; the shape with the fewest wins, ties to 16 x 32,
//   then 32 x 16. A wide block holds T / ntb tiles (fused_tile_blocks), a
//   16 x 16 block 16. Measured fused stage (16 x 16 -> 16 x 32, 16-tile
//   wide blocks): 56 x 56 ResNet-18 layer 18.5 -> 15.4 us, 28 x 28 22.8 ->
//   20.2 us, 14 x 14 39.1 -> 31.6 us; where 16 x 16 blocks already give each
//   CU one block (7 x 7, C = 512) the model keeps them (42 vs 61 us). With
//   the tile blocks evened out over the CUs the model picks 32 x 16 on the
//   56 x 56 and 28 x 28 layers (15.4 -> 15.1 us, 20.4 -> 18.6 us). 32 x 32
//   blocks of 16 waves run slower than the model says on those layers and
//   are only taken when forced.
// Tile blocks of the wide fused kernel. At least ceil(T / rt), so that no
// block holds more than rt tiles; raised so that the blocks come out to the
// same count on every compute unit. With b blocks on the busiest unit either
// way, each block then holds T / ntb tiles instead of rt, so that unit loads
// fewer tile rows (its weight rows are the same).
static int64_t fused_tile_blocks(int64_t T, int rt, int64_t nco, int cus) {
    const int64_t ntb0 = (T + rt - 1) / rt;
    const int64_t per = (ntb0 * nco + cus - 1) / cus;  // blocks of the busiest unit
    return std::max(ntb0, std::min(T, per * cus / nco));
}

static void fused_shape(const Geo &g, int cus, int &waves, int &wide) {
    const int64_t nblk = ((g.T + 15) / 16) * (int64_t)((g.Cout + 15) / 16);
    waves = g.fused_waves ? g.fused_waves : g.m == 6 && nblk < 3 * (int64_t)cus ? 8 : 4;
    if (g.fused_wide >= 0) {
        wide = g.fused_wide;
        return;
    }
    wide = 0;
    if (g.m == 6 && g.G <= 64) {
        // operand rows of the busiest CU per tap and K byte, in units of 1 / ntb
        // rows (wide blocks hold T / ntb tiles, 16 x 16 blocks 16)
        auto busiest = [&](int64_t rt, int64_t rc, bool even) {
            const int64_t nco = (g.Cout + rc - 1) / rc;
            const int64_t per = (((g.T + rt - 1) / rt) * nco + cus - 1) / cus;
            const int64_t ntb = even ? fused_tile_blocks(g.T, (int)rt, nco, cus) : (g.T + rt - 1) / rt;
            return std::make_pair(per * (even ? g.T : rt * ntb) + per * rc * ntb, ntb);
        };
        auto less = [](std::pair<int64_t, int64_t> a, std::pair<int64_t, int64_t> b) {
            return (__int128)a.first * b.second < (__int128)b.first * a.second;
        };
        const auto c0 = busiest(16, 16, false), c2 = busiest(32, 16, true), c3 = busiest(16, 32, true);
        if (!less(c2, c3) && less(c3, c0)) wide = 3;
        else if (less(c2, c0)) wide = 2;
    }
}

template <int M, int G, typename YT>
static void fused_m_g(const Geo &g, const Mats &mt, const int8_t *Vq, const float *sV,
                      const int8_t *Uq, const float *sU, YT *y, hipStream_t s) {
    const unsigned blocks = (unsigned)(((g.T + 15) / 16) * ((g.Cout + 15) / 16));
    const int cus = device_cus();
    int waves, wide;
    fused_shape(g, cus, waves, wide);
    if constexpr (M == 6 && G <= 64) {
        if (wide) {
            // 1: 32 x 32 blocks, 2: 32 tiles x 16 channels, 3: 16 tiles x 32 channels
            const int ht = wide == 3 ? 1 : 2, hc = wide == 2 ? 1 : 2;
            const int64_t nco = (g.Cout + 16 * hc - 1) / (16 * hc);
            Geo gw = g;
            gw.fused_ntb = (int)fused_tile_blocks(g.T, 16 * ht, nco, cus);
            const unsigned wblocks = (unsigned)(gw.fused_ntb * nco);
            const dim3 th(256 * ht * hc);
#define WQ8_WIDE(HT_, HC_)                                                                                   \
    do {                                                                                                     \
        if (g.ng == 1)                                                                                       \
            hipLaunchKernelGGL((k_fused23w<M, G, HT_, HC_, false, YT>), dim3(wblocks), th, 0, s, Vq, sV, Uq, sU, y, mt, gw); \
        else                                                                                                 \
            hipLaunchKernelGGL((k_fused23w<M, G, HT_, HC_, true, YT>), dim3(wblocks), th, 0, s, Vq, sV, Uq, sU, y, mt, gw);  \
    } while (0)
            if (ht == 2 && hc == 2) WQ8_WIDE(2, 2);
            else if (ht == 2) WQ8_WIDE(2, 1);
            else WQ8_WIDE(1, 2);
#undef WQ8_WIDE
            return;
        }
    }
    // waves per block as the plan chose (8 or 16 split the taps further; F(4,3)
    // has 36 taps and always uses 4)
    if constexpr (M == 6) {
        if (waves == 8) {
            if (g.ng == 1)
                hipLaunchKernelGGL((k_fused23<M, G, 8, false, YT>), dim3(blocks), dim3(512), 0, s, Vq, sV, Uq, sU, y, mt, g);
            else
                hipLaunchKernelGGL((k_fused23<M, G, 8, true, YT>), dim3(blocks), dim3(512), 0, s, Vq, sV, Uq, sU, y, mt, g);
            return;
        }
        if (waves == 16) {
            if (g.ng == 1)
                hipLaunchKernelGGL((k_fused23<M, G, 16, false, YT>), dim3(blocks), dim3(1024), 0, s, Vq, sV, Uq, sU, y, mt, g);
            else
                hipLaunchKernelGGL((k_fused23<M, G, 16, true, YT>), dim3(blocks), dim3(1024), 0, s, Vq, sV, Uq, sU, y, mt, g);
            return;
        }
    }
    {
        if (g.ng == 1)
            hipLaunchKernelGGL((k_fused23<M, G, 4, false, YT>), dim3(blocks), dim3(256), 0, s, Vq, sV, Uq, sU, y, mt, g);
        else
            hipLaunchKernelGGL((k_fused23<M, G, 4, true, YT>), dim3(blocks), dim3(256), 0, s, Vq, sV, Uq, sU, y, mt, g);
    }
}

template <int M, typename YT>
static void fused_m(const Geo &g, const Mats &mt, const int8_t *Vq, const float *sV,
                    const int8_t *Uq, const float *sU, YT *y, hipStream_t s) {
    switch (g.G) {
        case 16: fused_m_g<M, 16>(g, mt, Vq, sV, Uq, sU, y, s); break;
        case 32: fused_m_g<M, 32>(g, mt, Vq, sV, Uq, sU, y, s); break;
        case 64: fused_m_g<M, 64>(g, mt, Vq, sV, Uq, sU, y, s); break;
        case 128: fused_m_g<M, 128>(g, mt, Vq, sV, Uq, sU, y, s); break;
        default: fused_m_g<M, 256>(g, mt, Vq, sV, Uq, sU, y, s); break;
    }
}

wq8_status launch_fused23(const Geo &g, const Mats &mt, wq8_dtype ydt, const int8_t *Vq,
                          const float *sV, const int8_t *Uq, const float *sU, void *y,
                          void *stream) {
    hipStream_t s = (hipStream_t)stream;
    if (ydt == WQ8_F32) {
        if (g.m == 4) fused_m<4>(g, mt, Vq, sV, Uq, sU, (float *)y, s);
        else fused_m<6>(g, mt, Vq, sV, Uq, sU, (float *)y, s);
    } else {
        if (g.m == 4) fused_m<4>(g, mt, Vq, sV, Uq, sU, (uint16_t *)y, s);
        else fused_m<6>(g, mt, Vq, sV, Uq, sU, (uint16_t *)y, s);
    }
    return check_launch("fused Hadamard + output transform");
}

wq8_status launch_stage3(const Geo &g, const Mats &mt, wq8_dtype ydt, const float *Mi, void *y,
                         int8_t *Yq, float *sY, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    if (ydt == WQ8_F32) {
        if (g.m == 4) stage3_m<4>(g, mt, Mi, (float *)y, Yq, sY, s);
        else stage3_m<6>(g, mt, Mi, (float *)y, Yq, sY, s);
    } else {
        if (g.m == 4) stage3_m<4>(g, mt, Mi, (uint16_t *)y, Yq, sY, s);
        else stage3_m<6>(g, mt, Mi, (uint16_t *)y, Yq, sY, s);
    }
    return check_launch("output transform");
}

}  // namespace wq8
