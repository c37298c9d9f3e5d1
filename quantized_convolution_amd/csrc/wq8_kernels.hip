// HIP kernels for group-wise fully quantized Winograd F(m,3) on gfx950.
//
//   k_weights  U = G g G^T, per-group int8 (offline weight preparation)
//   k_stage1   V = B^T d B, per-group int8 (input transform)
//   k_stage2   n*n int8 GEMMs over input channels on MFMA, group dequant
//   k_stage3   Y requant over the n*n taps of a (tile, co), A^T Yq A, crop
//
// Numerics follow the library contract bit for bit: every transform sum is an
// fp32 fma chain in index order starting from +0, the quantizer divides with
// IEEE fp32 division and rounds with rint (ties to even). Build with
// -ffp-contract=off so nothing else is fused.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq8_internal.h"

namespace wq8 {

typedef int v4i __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------- helpers
__device__ __forceinline__ float load_act(const float *p) { return *p; }
__device__ __forceinline__ float load_act(const uint16_t *p) {
    return __uint_as_float((uint32_t)(*p) << 16);  // bf16 -> f32, exact
}
__device__ __forceinline__ void store_act(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_act(uint16_t *p, float v) {
    uint32_t u = __float_as_uint(v);  // f32 -> bf16, nearest even (finite input)
    *p = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Symmetric absmax quantizer pieces (a = group absmax > 0).
__device__ __forceinline__ int quant_code(float v, float inv) {
    float r = __builtin_rintf(v * inv);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
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

template <int M, int G, typename XT>
__global__ __launch_bounds__(256) void k_stage1(const XT *__restrict__ x, int8_t *__restrict__ Vq,
                                                float *__restrict__ sV, Mats mt, Geo g) {
    constexpr int N = M + 2, NT = N * N;
    using S = GroupShape<G>;
    __shared__ float red[S::GW > 1 ? 4 : 1][NT];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * S::TPB + wave / S::GW;
    const int c = blockIdx.y * S::CPB + (wave % S::GW) * 64 + lane;
    const bool ok = t < g.T && c < g.Cin;

    float v[NT];
    {
        int img = 0, ty = 0, tx = 0;
        if (ok) {
            tx = t % g.tW;
            const int r = t / g.tW;
            ty = r % g.tH;
            img = r / g.tH;
        }
        const int h0 = ty * M - g.pad, w0 = tx * M - g.pad;
        const XT *xc = x + ((size_t)img * g.Cin + (ok ? c : 0)) * g.H * g.W;
        float d[N][N];
#pragma unroll
        for (int k = 0; k < N; ++k)
#pragma unroll
            for (int l = 0; l < N; ++l) {
                const int h = h0 + k, w = w0 + l;
                d[k][l] = (ok && h >= 0 && h < g.H && w >= 0 && w < g.W)
                              ? load_act(xc + (size_t)h * g.W + w)
                              : 0.0f;
            }
        float t1[N][N];
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int l = 0; l < N; ++l) {
                float acc = 0.0f;
#pragma unroll
                for (int k = 0; k < N; ++k) acc = __builtin_fmaf(mt.Bt[i * N + k], d[k][l], acc);
                t1[i][l] = acc;
            }
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int j = 0; j < N; ++j) {
                float acc = 0.0f;
#pragma unroll
                for (int l = 0; l < N; ++l) acc = __builtin_fmaf(t1[i][l], mt.Bt[j * N + l], acc);
                v[i * N + j] = acc;
            }
    }
    const size_t plane = (size_t)g.T * g.Cin, splane = (size_t)g.T * g.ng;
    quantize_store<NT, G>(v, ok, c, wave, Vq + (size_t)t * g.Cin + c, plane,
                          sV + (size_t)t * g.ng + c / G, splane, red);
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
// Grid (ceil(T/64), ceil(Cout/64), n*n); 4 waves in 2 x 2, each 32 x 32 of
// (tile, co) as 2 x 2 MFMA 16x16 blocks. Per group: int32 accumulation on
// MFMA, then M = fma(sV sU, P, M) in group order. KS is the MFMA K-step:
// 64 (16x16x64) when G is a multiple of 64, else 32 (16x16x32, one per group).
// MFMA operand layout (16x16xK, int8): lane l holds row (l % 16) of A / column
// (l % 16) of B, K-slice (l / 16). A and B are loaded with the same K mapping,
// so the exact int32 dot product does not depend on the order the hardware
// sums the K slots in. Result: lane l holds rows 4 (l / 16) + i, column l % 16.
template <int KS, bool I32>
__global__ __launch_bounds__(256) void k_stage2(const int8_t *__restrict__ Vq,
                                                const float *__restrict__ sV,
                                                const int8_t *__restrict__ Uq,
                                                const float *__restrict__ sU, float *__restrict__ Mo,
                                                int32_t *__restrict__ Po, Geo g) {
    const int tap = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int tb = blockIdx.x * 64 + (wave & 1) * 32;
    const int cb = blockIdx.y * 64 + (wave >> 1) * 32;
    const int8_t *Vp = Vq + (size_t)tap * g.T * g.Cin;
    const int8_t *Up = Uq + (size_t)tap * g.Cout * g.Cin;
    const float *sVp = I32 ? nullptr : sV + (size_t)tap * g.T * g.ng;
    const float *sUp = I32 ? nullptr : sU + (size_t)tap * g.Cout * g.ng;

    float acc[2][2][4];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[bi][bj][i] = 0.0f;

    for (int gi = 0; gi < g.ng; ++gi) {
        v4i p[2][2];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) p[bi][bj] = v4i{0, 0, 0, 0};
        if constexpr (KS == 64) {
            // G is a multiple of 64: G / 64 MFMA K-steps per group
            for (int k0 = gi * g.G; k0 < (gi + 1) * g.G; k0 += 64) {
                v4i a[2], b[2];
#pragma unroll
                for (int bi = 0; bi < 2; ++bi) {
                    const int row = tb + 16 * bi + r;
                    a[bi] = row < g.T ? *(const v4i *)(Vp + (size_t)row * g.Cin + k0 + 16 * kq)
                                      : v4i{0, 0, 0, 0};
                }
#pragma unroll
                for (int bj = 0; bj < 2; ++bj) {
                    const int col = cb + 16 * bj + r;
                    b[bj] = col < g.Cout ? *(const v4i *)(Up + (size_t)col * g.Cin + k0 + 16 * kq)
                                         : v4i{0, 0, 0, 0};
                }
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                    for (int bj = 0; bj < 2; ++bj)
                        p[bi][bj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[bi], b[bj], p[bi][bj], 0, 0, 0);
            }
        } else {
            // G = 16 or 32: one K = 32 step per group; K slots past the group are zero
            const int k0 = gi * g.G;
            const bool kin = 8 * kq < g.G;
            long a[2], b[2];
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) {
                const int row = tb + 16 * bi + r;
                a[bi] = (kin && row < g.T) ? *(const long *)(Vp + (size_t)row * g.Cin + k0 + 8 * kq) : 0;
            }
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                const int col = cb + 16 * bj + r;
                b[bj] = (kin && col < g.Cout) ? *(const long *)(Up + (size_t)col * g.Cin + k0 + 8 * kq) : 0;
            }
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 2; ++bj)
                    p[bi][bj] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[bi], b[bj], p[bi][bj], 0, 0, 0);
        }
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                const int col = cb + 16 * bj + r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = tb + 16 * bi + 4 * kq + i;
                    if (row >= g.T || col >= g.Cout) continue;
                    if constexpr (I32) {
                        Po[(((size_t)tap * g.ng + gi) * g.T + row) * g.Cout + col] = p[bi][bj][i];
                    } else {
                        const float s = sVp[(size_t)row * g.ng + gi] * sUp[(size_t)col * g.ng + gi];
                        acc[bi][bj][i] = __builtin_fmaf(s, (float)p[bi][bj][i], acc[bi][bj][i]);
                    }
                }
            }
    }
    if constexpr (!I32) {
        float *Mp = Mo + (size_t)tap * g.T * g.Cout;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                const int col = cb + 16 * bj + r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = tb + 16 * bi + 4 * kq + i;
                    if (row < g.T && col < g.Cout) Mp[(size_t)row * g.Cout + col] = acc[bi][bj][i];
                }
            }
    }
}

// ------------------------------------------ Y requant + output transform
// One thread per (tile, co); consecutive threads take consecutive co.
template <int M, typename YT>
__global__ __launch_bounds__(256) void k_stage3(const float *__restrict__ Mi, YT *__restrict__ y,
                                                int8_t *__restrict__ Yq, float *__restrict__ sY,
                                                Mats mt, Geo g) {
    constexpr int N = M + 2, NT = N * N;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)g.T * g.Cout) return;
    const int co = (int)(idx % g.Cout), t = (int)(idx / g.Cout);
    const size_t plane = (size_t)g.T * g.Cout;
    float mv[NT];
    float a = 0.0f;
#pragma unroll
    for (int tap = 0; tap < NT; ++tap) {
        mv[tap] = Mi[tap * plane + idx];
        a = fmaxf(a, fabsf(mv[tap]));
    }
    int q[NT];
    float s = 0.0f;
    if (a != 0.0f) {
        const float inv = 127.0f / a;
#pragma unroll
        for (int tap = 0; tap < NT; ++tap) q[tap] = quant_code(mv[tap], inv);
        s = a / 127.0f;
    } else {
#pragma unroll
        for (int tap = 0; tap < NT; ++tap) q[tap] = 0;
    }
    if (Yq)
#pragma unroll
        for (int tap = 0; tap < NT; ++tap) Yq[idx * NT + tap] = (int8_t)q[tap];
    if (sY) sY[idx] = s;

    float z[M][N];
#pragma unroll
    for (int aa = 0; aa < M; ++aa)
#pragma unroll
        for (int j = 0; j < N; ++j) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < N; ++i) acc = __builtin_fmaf(mt.At[aa * N + i], (float)q[i * N + j], acc);
            z[aa][j] = acc;
        }
    const int tx = t % g.tW, rr = t / g.tW, ty = rr % g.tH, img = rr / g.tH;
    YT *yp = y + ((size_t)img * g.Cout + co) * g.Ho * g.Wo;
#pragma unroll
    for (int aa = 0; aa < M; ++aa)
#pragma unroll
        for (int b = 0; b < M; ++b) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < N; ++j) acc = __builtin_fmaf(z[aa][j], mt.At[b * N + j], acc);
            const int h = ty * M + aa, w = tx * M + b;
            if (h < g.Ho && w < g.Wo) store_act(yp + (size_t)h * g.Wo + w, acc * s);
        }
}

// ------------------------------------------------------------- launchers
static wq8_status check_launch(const char *what) {
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

template <int M, int G, typename XT>
static void stage1_m_g(const Geo &g, const Mats &mt, const XT *x, int8_t *Vq, float *sV,
                       hipStream_t s) {
    using S = GroupShape<G>;
    dim3 grid((unsigned)((g.T + S::TPB - 1) / S::TPB), (g.Cin + S::CPB - 1) / S::CPB);
    hipLaunchKernelGGL((k_stage1<M, G, XT>), grid, dim3(256), 0, s, x, Vq, sV, mt, g);
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

template <int KS>
static void stage2_k(const Geo &g, const int8_t *Vq, const float *sV, const int8_t *Uq,
                     const float *sU, float *M, int32_t *P, hipStream_t s) {
    dim3 grid((unsigned)((g.T + 63) / 64), (g.Cout + 63) / 64, g.n * g.n);
    if (P) hipLaunchKernelGGL((k_stage2<KS, true>), grid, dim3(256), 0, s, Vq, sV, Uq, sU, M, P, g);
    else hipLaunchKernelGGL((k_stage2<KS, false>), grid, dim3(256), 0, s, Vq, sV, Uq, sU, M, P, g);
}

wq8_status launch_stage2(const Geo &g, const int8_t *Vq, const float *sV, const int8_t *Uq,
                         const float *sU, float *M, int32_t *P, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    if (g.G % 64 == 0) stage2_k<64>(g, Vq, sV, Uq, sU, M, P, s);
    else stage2_k<32>(g, Vq, sV, Uq, sU, M, P, s);
    return check_launch("Hadamard GEMM");
}

template <int M, typename YT>
static void stage3_m(const Geo &g, const Mats &mt, const float *Mi, YT *y, int8_t *Yq, float *sY,
                     hipStream_t s) {
    const int64_t work = (int64_t)g.T * g.Cout;
    dim3 grid((unsigned)((work + 255) / 256));
    hipLaunchKernelGGL((k_stage3<M, YT>), grid, dim3(256), 0, s, Mi, y, Yq, sY, mt, g);
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
