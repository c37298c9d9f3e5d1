/*
 * CPU oracle for group-wise fully quantized 8-bit Winograd convolution F(m,3)
 * with diagonal transform scales ("Data-Free Group-Wise Fully Quantized
 * Winograd Convolution via Learnable Scales", arXiv 2412.19867).
 *
 * TEST INFRASTRUCTURE ONLY: a plain, slow, obviously correct reference that
 * shares no code with the HIP library. Only tests/, the smoke check and the
 * benchmark's CPU baseline may load it. Build: see oracle/build.py
 * (gcc -O2 -ffp-contract=off -fopenmp, no fast-math).
 *
 * Contents
 *   wq8o_direct_conv_f64   exact-as-fp64 3x3 cross-correlation (ground truth)
 *   wq8o_winograd_f64      unquantized Winograd in fp64 (no quantizers)
 *   wq8o_stage2_i32        per-group int32 Hadamard partial sums
 *   wq8o_{weights,stage1,stage2,stage3}_{f32,f64}
 *                          the fixed-order quantized pipeline
 *   wq8o_{quant_bt,stage1_int}_{f32,f64}
 *                          the literal input stage (quantized B^T and input,
 *                          integer transform)
 *
 * Transform matrices (Bt, G, At) are inputs: they are built in exact rational
 * arithmetic by oracle/transforms.py and rounded once to fp32/fp64.
 *
 * Conventions (the pages do not state them; plainest readings):
 *   - stride 1, zero padding `pad`, no bias, cross-correlation
 *     y[i][co][h][w] = sum_ci sum_{a,b<3} x[i][ci][h+a-pad][w+b-pad] w[co][ci][a][b];
 *   - Ho = H + 2 pad - 2; tiles of m x m outputs, ceil(Ho/m) x ceil(Wo/m)
 *     per image; outputs past Ho/Wo are computed and discarded.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int wq8o_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count for the following calls (timing only; results do not depend on it). */
void wq8o_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Ground truth: direct 3x3 convolution with every product and sum in fp64. */
void wq8o_direct_conv_f64(int N, int Cin, int Cout, int H, int W, int pad,
                          const float *x, const float *w, double *y)
{
    const int Ho = H + 2 * pad - 2, Wo = W + 2 * pad - 2;
#pragma omp parallel for schedule(static) collapse(2)
    for (int img = 0; img < N; ++img)
        for (int co = 0; co < Cout; ++co)
            for (int h = 0; h < Ho; ++h)
                for (int ww = 0; ww < Wo; ++ww) {
                    double acc = 0.0;
                    for (int ci = 0; ci < Cin; ++ci)
                        for (int a = 0; a < 3; ++a)
                            for (int b = 0; b < 3; ++b) {
                                int hi = h + a - pad, wi = ww + b - pad;
                                if (hi < 0 || hi >= H || wi < 0 || wi >= W)
                                    continue;
                                acc += (double)x[(((size_t)img * Cin + ci) * H + hi) * W + wi] *
                                       (double)w[(((size_t)co * Cin + ci) * 3 + a) * 3 + b];
                            }
                    y[(((size_t)img * Cout + co) * Ho + h) * Wo + ww] = acc;
                }
}

/*
 * Unquantized Winograd in fp64: per tile, Y = sum_ci (Bt d Bt^T) .* (G g G^T),
 * o = At Y At^T, cropped. Written independently of the quantized pipeline;
 * equals the direct convolution up to fp64 rounding whenever
 * S_A S_B S_G = I (the scale identity of the Vandermonde factorization).
 */
void wq8o_winograd_f64(int m, int N, int Cin, int Cout, int H, int W, int pad,
                       const double *Bt, const double *Gm, const double *At,
                       const float *x, const float *w, double *y)
{
    const int n = m + 2;
    const int Ho = H + 2 * pad - 2, Wo = W + 2 * pad - 2;
    const int tH = (Ho + m - 1) / m, tW = (Wo + m - 1) / m;
    /* pre-transform every filter: Uw[co][ci][i][j] */
    double *Uw = (double *)malloc(sizeof(double) * (size_t)Cout * Cin * n * n);
    for (int co = 0; co < Cout; ++co)
        for (int ci = 0; ci < Cin; ++ci) {
            const float *g = w + ((size_t)co * Cin + ci) * 9;
            double *u = Uw + ((size_t)co * Cin + ci) * n * n;
            for (int i = 0; i < n; ++i)
                for (int j = 0; j < n; ++j) {
                    double s = 0.0;
                    for (int a = 0; a < 3; ++a)
                        for (int b = 0; b < 3; ++b)
                            s += Gm[i * 3 + a] * (double)g[a * 3 + b] * Gm[j * 3 + b];
                    u[i * n + j] = s;
                }
        }
#pragma omp parallel for schedule(static) collapse(3)
    for (int img = 0; img < N; ++img)
        for (int ty = 0; ty < tH; ++ty)
            for (int tx = 0; tx < tW; ++tx) {
                double *V = (double *)malloc(sizeof(double) * (size_t)Cin * n * n);
                for (int ci = 0; ci < Cin; ++ci) {
                    double d[16][16];
                    for (int k = 0; k < n; ++k)
                        for (int l = 0; l < n; ++l) {
                            int h = ty * m - pad + k, ww = tx * m - pad + l;
                            d[k][l] = (h >= 0 && h < H && ww >= 0 && ww < W)
                                          ? (double)x[(((size_t)img * Cin + ci) * H + h) * W + ww]
                                          : 0.0;
                        }
                    for (int i = 0; i < n; ++i)
                        for (int j = 0; j < n; ++j) {
                            double s = 0.0;
                            for (int k = 0; k < n; ++k)
                                for (int l = 0; l < n; ++l)
                                    s += Bt[i * n + k] * d[k][l] * Bt[j * n + l];
                            V[(size_t)ci * n * n + i * n + j] = s;
                        }
                }
                for (int co = 0; co < Cout; ++co) {
                    double Y[16][16];
                    for (int i = 0; i < n; ++i)
                        for (int j = 0; j < n; ++j) {
                            double s = 0.0;
                            for (int ci = 0; ci < Cin; ++ci)
                                s += V[(size_t)ci * n * n + i * n + j] *
                                     Uw[((size_t)co * Cin + ci) * n * n + i * n + j];
                            Y[i][j] = s;
                        }
                    for (int a = 0; a < m; ++a)
                        for (int b = 0; b < m; ++b) {
                            int h = ty * m + a, ww = tx * m + b;
                            if (h >= Ho || ww >= Wo)
                                continue;
                            double s = 0.0;
                            for (int i = 0; i < n; ++i)
                                for (int j = 0; j < n; ++j)
                                    s += At[a * n + i] * Y[i][j] * At[b * n + j];
                            y[(((size_t)img * Cout + co) * Ho + h) * Wo + ww] = s;
                        }
                }
                free(V);
            }
    free(Uw);
}

/* Per-group int32 partial sums P[tap][g][t][co] = sum_{ci in g} Vq * Uq. */
void wq8o_stage2_i32(int n2, long T, int Cin, int Cout, int G, const int8_t *Vq,
                     const int8_t *Uq, int32_t *P)
{
    const int ng = Cin / G;
#pragma omp parallel for schedule(static) collapse(2)
    for (int tap = 0; tap < n2; ++tap)
        for (long t = 0; t < T; ++t)
            for (int gi = 0; gi < ng; ++gi)
                for (int co = 0; co < Cout; ++co) {
                    const int8_t *v = Vq + ((size_t)tap * T + t) * Cin + (size_t)gi * G;
                    const int8_t *u = Uq + ((size_t)tap * Cout + co) * Cin + (size_t)gi * G;
                    int32_t acc = 0;
                    for (int c = 0; c < G; ++c)
                        acc += (int32_t)v[c] * (int32_t)u[c];
                    P[(((size_t)tap * ng + gi) * T + t) * Cout + co] = acc;
                }
}

/* ---- the quantized pipeline in fp32 (parity target) ---- */
#define REAL float
#define SUF(name) name##_f32
#define FMA fmaf
#define RINT rintf
#define FABS fabsf
#include "wq8_oracle_body.h"
#undef REAL
#undef SUF
#undef FMA
#undef RINT
#undef FABS

/* ---- the same loops in fp64 (for the brute-force Kronecker pin) ---- */
#define REAL double
#define SUF(name) name##_f64
#define FMA fma
#define RINT rint
#define FABS fabs
#include "wq8_oracle_body.h"
#undef REAL
#undef SUF
#undef FMA
#undef RINT
#undef FABS
