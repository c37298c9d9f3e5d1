// HIP kernels for the group-wise W8A8 direct 3x3 convolution on gfx950: the
// non-Winograd baseline of the method's speed comparison (group-quantized
// direct kernels).
//
//   k_dq_w   per-(kernel tap, output channel, group) int8 weights (offline)
//   k_dq_x   per-(pixel, group) int8 activations, NCHW values -> NHWC codes
//   k_dconv_row, k_dconv_flat
//            implicit GEMM over (group, tap) on int8 MFMA with the group
//            dequantization as one fp32 fma chain per output; blocks of one
//            output row's pixels (wide rows) or of consecutive pixels across
//            rows and images (rows of at most 32 pixels)
//
// Same quantizer as the Winograd path (absmax, IEEE 127/a, rint ties to even,
// codes in +-127, zero group -> codes 0 and scale 0). The chain runs over
// groups ascending and, inside a group, taps kh*3+kw ascending; taps outside
// the image contribute nothing (their codes and scales are zero, and
// fma(0, 0, acc) == acc).
#include <type_traits>

#include "wq8_device.h"
#include "wq8_internal.h"

namespace wq8 {

// ------------------------------------------------------------------ weights
// Thread per (tap, co, group): G weights w[co][g*G + c][kh][kw].
template <int G>
__global__ __launch_bounds__(256) void k_dq_w(const float *__restrict__ w, int8_t *__restrict__ wq,
                                              float *__restrict__ sw, Geo g) {
    const int ng = g.Cin / G;
    const long id = (long)blockIdx.x * 256 + threadIdx.x;
    if (id >= 9L * g.Cout * ng) return;
    const int gi = (int)(id % ng);
    const int co = (int)((id / ng) % g.Cout);
    const int tap = (int)(id / ((long)ng * g.Cout));
    const float *wp = w + ((size_t)co * g.Cin + (size_t)gi * G) * 9 + tap;
    float a = 0.0f;
    for (int c = 0; c < G; ++c) a = fmaxf(a, fabsf(wp[c * 9]));
    float inv = 0.0f, sc = 0.0f;
    if (a != 0.0f) {
        inv = 127.0f / a;
        sc = a / 127.0f;
    }
    int8_t *q = wq + ((size_t)tap * g.Cout + co) * g.Cin + (size_t)gi * G;
    for (int c = 0; c < G; ++c) q[c] = (int8_t)__float_as_uint(wp[c * 9] * inv + kRoundMagic);
    sw[((size_t)tap * g.Cout + co) * ng + gi] = sc;
}

// -------------------------------------------------------------- activations
// Thread per (pixel, group): G channel values (coalesced across the block's
// consecutive pixels), absmax, codes packed 16 to a store. Block row y holds
// one group for 256 consecutive pixels.
template <int G, typename XT>
__global__ __launch_bounds__(256) void k_dq_x(const XT *__restrict__ x, int8_t *__restrict__ xq,
                                              float *__restrict__ sx, Geo g) {
    constexpr int CH = G < 64 ? G : 64;  // channels held in registers at once
    const int hw = g.H * g.W;
    const long px = (long)blockIdx.x * 256 + threadIdx.x;
    if (px >= (long)g.N * hw) return;
    const int img = (int)(px / hw), rem = (int)(px % hw);
    const XT *xp = x + (size_t)img * g.Cin * hw + rem;
    const int ng = g.Cin / G;
    const int gi = blockIdx.y;
    const XT *gp = xp + (size_t)gi * G * hw;
    float v[CH];
    float a = 0.0f;
    for (int c0 = 0; c0 < G; c0 += CH) {  // one pass for G <= 64
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            v[c] = load_act(gp + (size_t)(c0 + c) * hw);
            a = fmaxf(a, fabsf(v[c]));
        }
    }
    float inv = 0.0f, sc = 0.0f;
    if (a != 0.0f) {
        inv = 127.0f / a;
        sc = a / 127.0f;
    }
    for (int c0 = 0; c0 < G; c0 += CH) {
        if (G > CH) {  // second pass: reload this chunk
#pragma unroll
            for (int c = 0; c < CH; ++c) v[c] = load_act(gp + (size_t)(c0 + c) * hw);
        }
        int8_t *q = xq + (size_t)px * g.Cin + (size_t)gi * G + c0;
#pragma unroll
        for (int c = 0; c < CH; c += 16) {
            float y[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) y[e] = v[c + e] * inv + kRoundMagic;
            const v4i pk = {(int)pack4(y[0], y[1], y[2], y[3]), (int)pack4(y[4], y[5], y[6], y[7]),
                            (int)pack4(y[8], y[9], y[10], y[11]), (int)pack4(y[12], y[13], y[14], y[15])};
            *(v4i *)(q + c) = pk;
        }
    }
    sx[(size_t)px * ng + gi] = sc;
}

// ----------------------------------------- convolution, flattened pixels
// For rows of at most 32 pixels. Block: 64 consecutive output pixels in (image, row, column) order, so rows
// narrower than 64 pixels share a block, x 64 output channels (channel block
// slowest, so each XCD's contiguous range of blocks reads one slice of the
// weights); wave (wp, wc)
// computes 32 pixels x 32 channels as 2 x 2 MFMA tiles with the weights as A
// (rows = output channels) and the shifted input codes as B (columns =
// pixels), so lane (r, kq) ends with channels 16ic + 4kq + i of pixel
// 32wp + 16ip + r of the block.
//
// The reduction runs over the steps (group, tap) in chain order. Operands
// travel through a ring of D register sets, D - 1 steps ahead of the step
// being computed and across group boundaries; steps past the last one load
// with out-of-range offsets (zero, no fetch). Each group's weight and
// activation scales for the block's pixels and taps are staged in LDS, double
// buffered, one group ahead: one barrier per group.
template <int G>
struct DC {
    static constexpr bool K64 = G % 64 == 0;
    static constexpr int KSTEPS = K64 ? G / 64 : 1;
    // ring depth (register sets of one step's operands): 3 where the
    // registers allow, 2 keeps G = 64 at 4 blocks per CU
    static constexpr int D = G <= 32 ? 3 : (G <= 128 ? 2 : 1);
};

template <int G, typename YT>
__global__ __launch_bounds__(256) void k_dconv_flat(const int8_t *__restrict__ xq, const float *__restrict__ sx,
                                               const int8_t *__restrict__ wq, const float *__restrict__ sw,
                                               YT *__restrict__ y, Geo g) {
    using C = DC<G>;
    constexpr bool K64 = C::K64;
    constexpr int KSTEPS = C::KSTEPS, D = C::D;
    __shared__ float sw_l[2][9][64];   // [buffer][tap][output channel in block]
    __shared__ float sx_l[2][9][64];   // [buffer][tap][pixel in block]
    __shared__ int s_img[64], s_ho[64], s_wo[64];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int wp = wave & 1, wc = wave >> 1;
    const int ncb = (g.Cout + 63) / 64;
    // N Ho Wo < 2^31: the plan keeps every array below 2^31 bytes
    const int npx = g.N * g.Ho * g.Wo;
    const int npb = (npx + 63) / 64;
    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int cb = blk / npb;
    const int p0 = (blk % npb) * 64;
    const int co0 = cb * 64;
    const int ng = g.Cin / G;
    const int nsteps = 9 * ng;

    if (tid < 64) {
        const int p = p0 + tid;
        const bool ok = p < npx;
        const int wo = ok ? (int)(p % g.Wo) : 0;
        const int rr = ok ? p / g.Wo : 0;
        s_wo[tid] = wo;
        s_ho[tid] = ok ? rr % g.Ho : -(1 << 20);  // a row no tap reaches
        s_img[tid] = ok ? rr / g.Ho : 0;
    }
    __syncthreads();

    const auto rX = make_rsrc(xq, (size_t)g.N * g.H * g.W * g.Cin);
    const auto rW = make_rsrc(wq, (size_t)9 * g.Cout * g.Cin);
    const bool kin = K64 || 8 * kq < G;  // K slots inside the group (G = 16: half)
    const int koff = K64 ? 16 * kq : (kin ? 8 * kq : 0);
    // A rows (output channels), clamped to a valid row: rows past Cout only
    // feed outputs that are never stored
    int coA[2];
#pragma unroll
    for (int ic = 0; ic < 2; ++ic) {
        const int co = co0 + 32 * wc + 16 * ic + r;
        coA[ic] = co < g.Cout ? co : 0;
    }
    int pimg[2], pho[2], pwo[2];  // B columns: output pixel
#pragma unroll
    for (int ip = 0; ip < 2; ++ip) {
        const int pl = 32 * wp + 16 * ip + r;
        pimg[ip] = s_img[pl];
        pho[ip] = s_ho[pl];
        pwo[ip] = s_wo[pl];
    }

    // Scales of group gi: element e = tid + 256 j of [tap][channel or pixel]
    // (576 of them). They are loaded into registers one group before they
    // are written to LDS, so the write never waits on a load in flight (a
    // wait for the newest loads would drain the operand ring as well).
    constexpr int SE = (9 * 64 + 255) / 256;
    uint32_t swo[SE], sxo[SE];  // byte offsets without the group; kOob where none
#pragma unroll
    for (int j = 0; j < SE; ++j) {
        const int e = tid + 256 * j;
        const int tap = e / 64, c = e % 64, co = co0 + c;
        const int kh = tap / 3, kw = tap % 3;
        const int h = s_ho[c] + kh - g.pad, w = s_wo[c] + kw - g.pad;
        swo[j] = e < 9 * 64 && co < g.Cout ? (uint32_t)(((tap * g.Cout + co) * ng) * 4) : (uint32_t)kOob;
        sxo[j] = e < 9 * 64 && h >= 0 && h < g.H && w >= 0 && w < g.W
                     ? (uint32_t)((((s_img[c] * g.H + h) * g.W + w) * ng) * 4) : (uint32_t)kOob;
    }
    const auto rsW = make_rsrc(sw, (size_t)9 * g.Cout * ng * 4);
    const auto rsX = make_rsrc(sx, (size_t)g.N * g.H * g.W * ng * 4);
    float swr[SE], sxr[SE];
    auto fetch = [&](int gi) {  // past the last group: zero, no fetch
        const uint32_t go = gi < ng ? (uint32_t)(gi * 4) : (uint32_t)kOob;
#pragma unroll
        for (int j = 0; j < SE; ++j) {
            swr[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsW, (int)(swo[j] + go), 0, 0));
            sxr[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsX, (int)(sxo[j] + go), 0, 0));
        }
    };
    auto commit = [&](int b) {
#pragma unroll
        for (int j = 0; j < SE; ++j) {
            const int e = tid + 256 * j;
            if (e < 9 * 64) {
                (&sw_l[b][0][0])[e] = swr[j];
                (&sx_l[b][0][0])[e] = sxr[j];
            }
        }
    };

    float acc[2][2][4];
#pragma unroll
    for (int ic = 0; ic < 2; ++ic)
#pragma unroll
        for (int ip = 0; ip < 2; ++ip)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[ic][ip][i] = 0.0f;

    struct Ops {
        v4i a[2][K64 ? KSTEPS : 0], b[2][K64 ? KSTEPS : 0];
        long a8[2], b8[2];
    };
    // per-lane parts of the operand offsets: the B pixel's own input
    // position (a tap adds a uniform delta) and the A row
    int xb[2], wb[2];
#pragma unroll
    for (int ip = 0; ip < 2; ++ip) {
        // pixels past the layer carry a sentinel row; their offsets are never
        // used (every tap selects kOob), so row 0 keeps the product in range
        const int h = pho[ip] < 0 ? 0 : pho[ip];
        xb[ip] = ((pimg[ip] * g.H + h) * g.W + pwo[ip]) * g.Cin + koff;
    }
#pragma unroll
    for (int ic = 0; ic < 2; ++ic) wb[ic] = coA[ic] * g.Cin + koff;
    // operands of step st = (group st / 9, tap st % 9); zero past the last
    // step. Branch-free: every offset is a select, so the compiler keeps its
    // waits for the ring partial.
    auto load = [&](int st, Ops &o) {
        const bool in = st < nsteps;
        const int gi = in ? st / 9 : 0, tap = in ? st % 9 : 0;
        const int kh = tap / 3, kw = tap % 3;
        const int dx = ((kh - g.pad) * g.W + (kw - g.pad)) * g.Cin + gi * G;  // uniform
#pragma unroll
        for (int ip = 0; ip < 2; ++ip) {
            const bool ok = in && (unsigned)(pho[ip] + kh - g.pad) < (unsigned)g.H &&
                            (unsigned)(pwo[ip] + kw - g.pad) < (unsigned)g.W;
            const int off = ok ? xb[ip] + dx : kOob;
            if constexpr (K64) {
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    o.b[ip][ks] = __builtin_amdgcn_raw_buffer_load_b128(rX, off, 64 * ks, 0);
            } else {
                const auto qv = __builtin_amdgcn_raw_buffer_load_b64(rX, off, 0, 0);
                o.b8[ip] = ((long)(uint32_t)qv[1] << 32) | (uint32_t)qv[0];
            }
        }
#pragma unroll
        for (int ic = 0; ic < 2; ++ic) {
            const int off = in ? wb[ic] + tap * g.Cout * g.Cin + gi * G : kOob;
            if constexpr (K64) {
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    o.a[ic][ks] = __builtin_amdgcn_raw_buffer_load_b128(rW, off, 64 * ks, 0);
            } else {
                const auto qv = __builtin_amdgcn_raw_buffer_load_b64(rW, off, 0, 0);
                o.a8[ic] = ((long)(uint32_t)qv[1] << 32) | (uint32_t)qv[0];
            }
        }
    };
    auto use = [&](int tap, int b, const Ops &o) {
#pragma unroll
        for (int ic = 0; ic < 2; ++ic) {
            const float4 s4 = *(const float4 *)&sw_l[b][tap][32 * wc + 16 * ic + 4 * kq];
            const float swv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int ip = 0; ip < 2; ++ip) {
                v4i P = {0, 0, 0, 0};
                if constexpr (K64) {
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ++ks)
                        P = __builtin_amdgcn_mfma_i32_16x16x64_i8(o.a[ic][ks], o.b[ip][ks], P, 0, 0, 0);
                } else {
                    P = __builtin_amdgcn_mfma_i32_16x16x32_i8(kin ? o.a8[ic] : 0, kin ? o.b8[ip] : 0, P, 0, 0, 0);
                }
                const float sxv = sx_l[b][tap][32 * wp + 16 * ip + r];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[ic][ip][i] = __builtin_fmaf(sxv * swv[i], (float)P[i], acc[ic][ip][i]);
            }
        }
    };

    fetch(0);
    commit(0);
    fetch(1);
    // step st = (group st / 9, tap st % 9) lives in ring slot st % D
    Ops ring[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) load(d, ring[d]);
    // the steps run in whole rings; steps past the last one (fewer than D)
    // load zero codes and read zero scales (the buffer of the group past the
    // last holds the zeros fetched for it), and fma(0, 0, acc) == acc
    for (int s0 = 0; s0 < nsteps; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int st = s0 + d;
            const int gi = st / 9, tap = st - 9 * gi;
            if (tap == 0) {
                // group gi's scales are in buffer gi & 1; buffer (gi + 1) & 1
                // was last read by group gi - 1, which every wave has left.
                // Group gi + 1's scales (in registers since the last group
                // boundary) go there; group gi + 2's are fetched.
                __syncthreads();
                commit((gi + 1) & 1);
                fetch(gi + 2);
            }
            load(st + D - 1, ring[(d + D - 1) % D]);
            __builtin_amdgcn_sched_barrier(0);
            use(tap, gi & 1, ring[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // outputs: 16 lanes of one channel are 16 consecutive pixels
#pragma unroll
    for (int ic = 0; ic < 2; ++ic)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int co = co0 + 32 * wc + 16 * ic + 4 * kq + i;
            if (co >= g.Cout) continue;
#pragma unroll
            for (int ip = 0; ip < 2; ++ip)
                if (pho[ip] >= 0)
                    store_act(y + (((size_t)pimg[ip] * g.Cout + co) * g.Ho + pho[ip]) * g.Wo + pwo[ip],
                              acc[ic][ip][i]);
        }
}

// ------------------------------------------------ convolution, row blocks
// Block: 64 output pixels of one output row x 64 output channels; wave
// (wp, wc) computes 32 pixels x 32 channels as 2 x 2 MFMA tiles with the
// weights as A (rows = output channels) and the shifted input codes as B
// (columns = pixels), so lane (r, kq) ends with channels 16ic + 4kq + i of
// pixel 16ip + r. One group's scales are staged in LDS at a time; each tap's
// operands are loaded while the previous tap is computed.
template <int G, typename YT>
__global__ __launch_bounds__(256) void k_dconv_row(const int8_t *__restrict__ xq, const float *__restrict__ sx,
                                               const int8_t *__restrict__ wq, const float *__restrict__ sw,
                                               YT *__restrict__ y, Geo g) {
    constexpr bool K64 = G % 64 == 0;
    constexpr int KSTEPS = K64 ? G / 64 : 1;
    constexpr int SXW = 68;  // staged input columns: wo0 - pad .. wo0 + 65 - pad
    __shared__ float sw_l[9][64];      // [tap][output channel in block]
    __shared__ float sx_l[3][SXW];     // [kh][input column - (wo0 - pad)]

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int wp = wave & 1, wc = wave >> 1;
    const int nseg = (g.Wo + 63) / 64, ncb = (g.Cout + 63) / 64;
    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int cb = blk % ncb;
    int rest = blk / ncb;
    const int seg = rest % nseg;
    rest /= nseg;
    const int ho = rest % g.Ho, img = rest / g.Ho;
    const int wo0 = seg * 64, co0 = cb * 64;
    const int ng = g.Cin / G;

    const auto rX = make_rsrc(xq, (size_t)g.N * g.H * g.W * g.Cin);
    const auto rW = make_rsrc(wq, (size_t)9 * g.Cout * g.Cin);
    const bool kin = K64 || 8 * kq < G;  // K slots inside the group (G = 16: half)
    const int koff = K64 ? 16 * kq : (kin ? 8 * kq : 0);
    // A rows (output channels), clamped to a valid row: rows past Cout only
    // feed outputs that are never stored
    int coA[2];
#pragma unroll
    for (int ic = 0; ic < 2; ++ic) {
        const int co = co0 + 32 * wc + 16 * ic + r;
        coA[ic] = co < g.Cout ? co : 0;
    }
    int pxB[2];  // B columns: output pixel
#pragma unroll
    for (int ip = 0; ip < 2; ++ip) pxB[ip] = wo0 + 32 * wp + 16 * ip + r;

    float acc[2][2][4];
#pragma unroll
    for (int ic = 0; ic < 2; ++ic)
#pragma unroll
        for (int ip = 0; ip < 2; ++ip)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[ic][ip][i] = 0.0f;

    struct Ops {
        v4i a[2][K64 ? KSTEPS : 0], b[2][K64 ? KSTEPS : 0];
        long a8[2], b8[2];
    };
    auto load = [&](int gi, int tap, Ops &o) {
        const int kh = tap / 3, kw = tap % 3;
        const int h = ho + kh - g.pad;
        const bool hok = h >= 0 && h < g.H;
#pragma unroll
        for (int ip = 0; ip < 2; ++ip) {
            const int w = pxB[ip] + kw - g.pad;
            const int off = hok && w >= 0 && w < g.W
                                ? (((img * g.H + h) * g.W + w) * g.Cin + gi * G + koff) : kOob;
            if constexpr (K64) {
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    o.b[ip][ks] = __builtin_amdgcn_raw_buffer_load_b128(rX, off, 64 * ks, 0);
            } else {
                const auto q = __builtin_amdgcn_raw_buffer_load_b64(rX, off, 0, 0);
                o.b8[ip] = ((long)(uint32_t)q[1] << 32) | (uint32_t)q[0];
            }
        }
#pragma unroll
        for (int ic = 0; ic < 2; ++ic) {
            const int off = (tap * g.Cout + coA[ic]) * g.Cin + gi * G + koff;
            if constexpr (K64) {
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    o.a[ic][ks] = __builtin_amdgcn_raw_buffer_load_b128(rW, off, 64 * ks, 0);
            } else {
                const auto q = __builtin_amdgcn_raw_buffer_load_b64(rW, off, 0, 0);
                o.a8[ic] = ((long)(uint32_t)q[1] << 32) | (uint32_t)q[0];
            }
        }
    };
    auto use = [&](int tap, const Ops &o) {
        const int kh = tap / 3, kw = tap % 3;
#pragma unroll
        for (int ic = 0; ic < 2; ++ic) {
            const float4 s4 = *(const float4 *)&sw_l[tap][32 * wc + 16 * ic + 4 * kq];
            const float swv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int ip = 0; ip < 2; ++ip) {
                v4i P = {0, 0, 0, 0};
                if constexpr (K64) {
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ++ks)
                        P = __builtin_amdgcn_mfma_i32_16x16x64_i8(o.a[ic][ks], o.b[ip][ks], P, 0, 0, 0);
                } else {
                    P = __builtin_amdgcn_mfma_i32_16x16x32_i8(kin ? o.a8[ic] : 0, kin ? o.b8[ip] : 0, P, 0, 0, 0);
                }
                const float sxv = sx_l[kh][32 * wp + 16 * ip + r + kw];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[ic][ip][i] = __builtin_fmaf(sxv * swv[i], (float)P[i], acc[ic][ip][i]);
            }
        }
    };

    for (int gi = 0; gi < ng; ++gi) {
        __syncthreads();  // the previous group's scales are consumed
        for (int e = tid; e < 9 * 64; e += 256) {
            const int tap = e / 64, c = e % 64, co = co0 + c;
            sw_l[tap][c] = co < g.Cout ? sw[((size_t)tap * g.Cout + co) * ng + gi] : 0.0f;
        }
        for (int e = tid; e < 3 * SXW; e += 256) {
            const int kh = e / SXW, col = e % SXW;
            const int h = ho + kh - g.pad, w = wo0 - g.pad + col;
            sx_l[kh][col] = h >= 0 && h < g.H && w >= 0 && w < g.W
                                ? sx[(((size_t)img * g.H + h) * g.W + w) * ng + gi] : 0.0f;
        }
        __syncthreads();
        Ops buf[2];
        load(gi, 0, buf[0]);
#pragma unroll
        for (int tap = 0; tap < 9; ++tap) {
            if (tap + 1 < 9) load(gi, tap + 1, buf[(tap + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            use(tap, buf[tap & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // outputs: 16 lanes of one channel are 16 consecutive pixels of the row
#pragma unroll
    for (int ic = 0; ic < 2; ++ic)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int co = co0 + 32 * wc + 16 * ic + 4 * kq + i;
            if (co >= g.Cout) continue;
            YT *yr = y + (((size_t)img * g.Cout + co) * g.Ho + ho) * g.Wo;
#pragma unroll
            for (int ip = 0; ip < 2; ++ip)
                if (pxB[ip] < g.Wo) store_act(yr + pxB[ip], acc[ic][ip][i]);
        }
}

// ---------------------------------------------------------------- launchers
template <typename F>
static void with_group(int G, F f) {
    switch (G) {
        case 16: f(std::integral_constant<int, 16>{}); break;
        case 32: f(std::integral_constant<int, 32>{}); break;
        case 64: f(std::integral_constant<int, 64>{}); break;
        case 128: f(std::integral_constant<int, 128>{}); break;
        default: f(std::integral_constant<int, 256>{}); break;
    }
}

wq8_status launch_direct_weights(const Geo &g, const float *w, int8_t *Wq, float *sW, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    const long n = 9L * g.Cout * (g.Cin / g.G);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    with_group(g.G, [&](auto GG) {
        constexpr int G = decltype(GG)::value;
        hipLaunchKernelGGL((k_dq_w<G>), dim3(blocks), dim3(256), 0, s, w, Wq, sW, g);
    });
    return check_launch("direct-conv weight quantization");
}

wq8_status launch_direct_qx(const Geo &g, wq8_dtype xdt, const void *x, int8_t *Xq, float *sX,
                            void *stream) {
    hipStream_t s = (hipStream_t)stream;
    const long n = (long)g.N * g.H * g.W;
    const dim3 grid((unsigned)((n + 255) / 256), (unsigned)(g.Cin / g.G));
    with_group(g.G, [&](auto GG) {
        constexpr int G = decltype(GG)::value;
        if (xdt == WQ8_F32)
            hipLaunchKernelGGL((k_dq_x<G, float>), grid, dim3(256), 0, s, (const float *)x, Xq, sX, g);
        else
            hipLaunchKernelGGL((k_dq_x<G, uint16_t>), grid, dim3(256), 0, s, (const uint16_t *)x, Xq,
                               sX, g);
    });
    return check_launch("direct-conv activation quantization");
}

wq8_status launch_direct_conv(const Geo &g, wq8_dtype ydt, const int8_t *Xq, const float *sX,
                              const int8_t *Wq, const float *sW, void *y, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    // rows of at most 32 pixels would leave half or more of a row block's
    // 64 pixel columns empty: those layers take blocks of 64 consecutive
    // pixels across rows and images instead
    const bool flat = g.Wo <= 32;
    const long ncb = (g.Cout + 63) / 64;
    const unsigned blocks = flat ? (unsigned)((((long)g.N * g.Ho * g.Wo + 63) / 64) * ncb)
                                 : (unsigned)((long)g.N * g.Ho * ((g.Wo + 63) / 64) * ncb);
    with_group(g.G, [&](auto GG) {
        constexpr int G = decltype(GG)::value;
        if (flat) {
            if (ydt == WQ8_F32)
                hipLaunchKernelGGL((k_dconv_flat<G, float>), dim3(blocks), dim3(256), 0, s, Xq, sX, Wq, sW,
                                   (float *)y, g);
            else
                hipLaunchKernelGGL((k_dconv_flat<G, uint16_t>), dim3(blocks), dim3(256), 0, s, Xq, sX, Wq, sW,
                                   (uint16_t *)y, g);
        } else {
            if (ydt == WQ8_F32)
                hipLaunchKernelGGL((k_dconv_row<G, float>), dim3(blocks), dim3(256), 0, s, Xq, sX, Wq, sW,
                                   (float *)y, g);
            else
                hipLaunchKernelGGL((k_dconv_row<G, uint16_t>), dim3(blocks), dim3(256), 0, s, Xq, sX, Wq, sW,
                                   (uint16_t *)y, g);
        }
    });
    return check_launch("direct convolution");
}

}  // namespace wq8
