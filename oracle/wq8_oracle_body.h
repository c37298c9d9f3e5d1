/*
 * Fixed-order quantized Winograd pipeline, written once and compiled twice by
 * wq8_oracle.c: with REAL = float (the parity target, "O-C") and with
 * REAL = double (used by the brute-force Kronecker pin, where summation order
 * cannot flip a code).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link or
 * call this file; only tests/, the smoke check and the benchmark's CPU
 * baseline do.
 *
 * Method: "Data-Free Group-Wise Fully Quantized Winograd Convolution via
 * Learnable Scales" (arXiv 2412.19867). The pages describe group-wise
 * quantization at every stage of the Winograd pipeline (input transform,
 * Hadamard product, output transform; referee summary and the "Approach"
 * section of the AI summary page, Fig. 2 caption) and name the quantized
 * Winograd-domain output Y (Eq. 5) whose cross-shaped range a single scale
 * per tile cannot hold (core claim, Fig. 3 caption).
 *
 * Readings taken where the pages are silent (each also listed in the design doc):
 *  - quantization points are V (input transform), U (weight transform) and
 *    Y (Hadamard output); transform matrices stay fp32, x is not quantized
 *    before the transform;
 *  - V and U groups are G consecutive input channels inside one tap; Y has
 *    one scale per (tile, output channel) spanning all n*n taps;
 *  - symmetric absmax quantizer, codes in [-127, 127], scale = absmax/127,
 *    code = rint(x * (127/absmax)) with ties to even; an all-zero group gives
 *    codes 0 and scale 0;
 *  - every fp32 sum is a left-to-right fma chain starting from +0.
 *
 * Expects the includer to define REAL, SUF(name), FMA, RINT, FABS.
 */

/* Symmetric absmax quantizer over len values spaced `stride` apart. */
static void SUF(quantize)(const REAL *v, long stride, int len, int8_t *q,
                          long qstride, REAL *scale)
{
    REAL a = 0;
    for (int i = 0; i < len; ++i) {
        REAL mag = FABS(v[i * stride]);
        if (mag > a)
            a = mag;
    }
    if (a == 0) {
        for (int i = 0; i < len; ++i)
            q[i * qstride] = 0;
        *scale = 0;
        return;
    }
    REAL inv = (REAL)127 / a;
    for (int i = 0; i < len; ++i) {
        REAL r = RINT(v[i * stride] * inv);
        if (r > 127)
            r = 127;
        if (r < -127)
            r = -127;
        q[i * qstride] = (int8_t)r;
    }
    *scale = a / (REAL)127;
}

/*
 * Weight transform U = G g G^T for every (co, ci), then per-group
 * quantization along ci.
 *   w  : [Cout][Cin][3][3]
 *   Gm : [n][3] (already carrying S_G)
 *   Uq : [n*n][Cout][Cin] int8,  sU : [n*n][Cout][Cin/G]
 */
void SUF(wq8o_weights)(int m, int Cin, int Cout, int G, const REAL *Gm,
                       const float *w, int8_t *Uq, REAL *sU)
{
    const int n = m + 2, n2 = n * n, ng = Cin / G;
#pragma omp parallel for schedule(static)
    for (int co = 0; co < Cout; ++co) {
        REAL *U = (REAL *)malloc(sizeof(REAL) * (size_t)n2 * Cin); /* [tap][ci] */
        for (int ci = 0; ci < Cin; ++ci) {
            const float *g = w + ((size_t)co * Cin + ci) * 9;
            REAL t2[16][3];
            for (int i = 0; i < n; ++i)
                for (int b = 0; b < 3; ++b) {
                    REAL acc = 0;
                    for (int a = 0; a < 3; ++a)
                        acc = FMA(Gm[i * 3 + a], (REAL)g[a * 3 + b], acc);
                    t2[i][b] = acc;
                }
            for (int i = 0; i < n; ++i)
                for (int j = 0; j < n; ++j) {
                    REAL acc = 0;
                    for (int b = 0; b < 3; ++b)
                        acc = FMA(t2[i][b], Gm[j * 3 + b], acc);
                    U[(size_t)(i * n + j) * Cin + ci] = acc;
                }
        }
        for (int tap = 0; tap < n2; ++tap)
            for (int gi = 0; gi < ng; ++gi)
                SUF(quantize)(U + (size_t)tap * Cin + (size_t)gi * G, 1, G,
                              Uq + ((size_t)tap * Cout + co) * Cin + (size_t)gi * G, 1,
                              sU + ((size_t)tap * Cout + co) * ng + gi);
        free(U);
    }
}

/*
 * Stage 1: input tiles d (n x n, zero outside the image), V = Bt d Bt^T, then
 * per-group quantization along ci inside each (tap, tile).
 *   x  : [N][Cin][H][W]
 *   Bt : [n][n] (already carrying S_B)
 *   Vq : [n*n][T][Cin] int8,  sV : [n*n][T][Cin/G]
 * Tile t = (img*tH + ty)*tW + tx covers output rows ty*m .. ty*m+m-1 and
 * reads input rows ty*m - pad .. ty*m - pad + n - 1 (columns likewise).
 */
void SUF(wq8o_stage1)(int m, int N, int Cin, int H, int W, int pad, int G,
                      const REAL *Bt, const float *x, int8_t *Vq, REAL *sV)
{
    const int n = m + 2, n2 = n * n, ng = Cin / G;
    const int Ho = H + 2 * pad - 2, Wo = W + 2 * pad - 2;
    const int tH = (Ho + m - 1) / m, tW = (Wo + m - 1) / m;
    const long T = (long)N * tH * tW;
#pragma omp parallel for schedule(static)
    for (long t = 0; t < T; ++t) {
        const int img = (int)(t / ((long)tH * tW));
        const int ty = (int)(t / tW % tH), tx = (int)(t % tW);
        REAL *V = (REAL *)malloc(sizeof(REAL) * (size_t)n2 * Cin); /* [tap][ci] */
        for (int ci = 0; ci < Cin; ++ci) {
            REAL d[16][16], t1[16][16];
            for (int k = 0; k < n; ++k)
                for (int l = 0; l < n; ++l) {
                    int h = ty * m - pad + k, ww = tx * m - pad + l;
                    d[k][l] = (h >= 0 && h < H && ww >= 0 && ww < W)
                                  ? (REAL)x[(((size_t)img * Cin + ci) * H + h) * W + ww]
                                  : 0;
                }
            for (int i = 0; i < n; ++i)
                for (int l = 0; l < n; ++l) {
                    REAL acc = 0;
                    for (int k = 0; k < n; ++k)
                        acc = FMA(Bt[i * n + k], d[k][l], acc);
                    t1[i][l] = acc;
                }
            for (int i = 0; i < n; ++i)
                for (int j = 0; j < n; ++j) {
                    REAL acc = 0;
                    for (int l = 0; l < n; ++l)
                        acc = FMA(t1[i][l], Bt[j * n + l], acc);
                    V[(size_t)(i * n + j) * Cin + ci] = acc;
                }
        }
        for (int tap = 0; tap < n2; ++tap)
            for (int gi = 0; gi < ng; ++gi)
                SUF(quantize)(V + (size_t)tap * Cin + (size_t)gi * G, 1, G,
                              Vq + ((size_t)tap * T + t) * Cin + (size_t)gi * G, 1,
                              sV + ((size_t)tap * T + t) * ng + gi);
        free(V);
    }
}

/*
 * Literal reading of the input stage. The review page's Eqs. 14-16 survive
 * only as the combined factor "sqB sqB sqx": a scale of the transform matrix
 * on the left, the same on the right, and a scale of the input. Read plainly,
 * B^T and the input patch are both quantized, the input transform runs on
 * their integer codes, and the three scales bring the result back to real
 * values; V is then quantized per group as in wq8o_stage1.
 *
 * B^T quantization (same absmax quantizer): rows == 0 gives one scale for the
 * whole n x n matrix, rows == 1 one scale per row. sB[i] is the scale of row
 * i (all equal for rows == 0).
 *   Bt : [n][n]  ->  Bq [n][n] int8,  sB [n]
 */
void SUF(wq8o_quant_bt)(int n, int rows, const REAL *Bt, int8_t *Bq, REAL *sB)
{
    if (rows) {
        for (int i = 0; i < n; ++i)
            SUF(quantize)(Bt + (size_t)i * n, 1, n, Bq + (size_t)i * n, 1, &sB[i]);
    } else {
        REAL s;
        SUF(quantize)(Bt, 1, n * n, Bq, 1, &s);
        for (int i = 0; i < n; ++i)
            sB[i] = s;
    }
}

/*
 * Stage 1, literal reading. For every tile t and group of G input channels,
 * the n x n patches of the group's channels (zero outside the image) share
 * one scale sx[t][g] (absmax over all n*n*G values) and codes dq. Then per
 * channel
 *   W[i][j] = sum_k sum_l Bq[i][k] dq[k][l] Bq[j][l]      (exact integers)
 *   V[i][j] = float(W[i][j]) * ((sB[i] * sB[j]) * sx)     (REAL, in that order)
 * and V is quantized per (tap, t, group) as in wq8o_stage1.
 *   xq : [T][Cin][n][n] int8 patch codes and sx : [T][Cin/G], optional (NULL).
 */
void SUF(wq8o_stage1_int)(int m, int N, int Cin, int H, int W, int pad, int G,
                          const int8_t *Bq, const REAL *sB, const float *x,
                          int8_t *Vq, REAL *sV, int8_t *xq, REAL *sx)
{
    const int n = m + 2, n2 = n * n, ng = Cin / G;
    const int Ho = H + 2 * pad - 2, Wo = W + 2 * pad - 2;
    const int tH = (Ho + m - 1) / m, tW = (Wo + m - 1) / m;
    const long T = (long)N * tH * tW;
#pragma omp parallel for schedule(static)
    for (long t = 0; t < T; ++t) {
        const int img = (int)(t / ((long)tH * tW));
        const int ty = (int)(t / tW % tH), tx = (int)(t % tW);
        REAL *V = (REAL *)malloc(sizeof(REAL) * (size_t)n2 * Cin);     /* [tap][ci] */
        REAL *d = (REAL *)malloc(sizeof(REAL) * (size_t)G * n2);       /* [c][k][l] */
        int8_t *dq = (int8_t *)malloc((size_t)G * n2);
        for (int gi = 0; gi < ng; ++gi) {
            for (int c = 0; c < G; ++c) {
                const int ci = gi * G + c;
                for (int k = 0; k < n; ++k)
                    for (int l = 0; l < n; ++l) {
                        int h = ty * m - pad + k, ww = tx * m - pad + l;
                        d[(size_t)c * n2 + k * n + l] =
                            (h >= 0 && h < H && ww >= 0 && ww < W)
                                ? (REAL)x[(((size_t)img * Cin + ci) * H + h) * W + ww]
                                : 0;
                    }
            }
            REAL s;
            SUF(quantize)(d, 1, G * n2, dq, 1, &s);
            if (sx)
                sx[t * ng + gi] = s;
            if (xq)
                memcpy(xq + ((size_t)t * Cin + (size_t)gi * G) * n2, dq, (size_t)G * n2);
            for (int c = 0; c < G; ++c) {
                const int8_t *p = dq + (size_t)c * n2;
                long t1[16][16];
                for (int i = 0; i < n; ++i)
                    for (int l = 0; l < n; ++l) {
                        long acc = 0;
                        for (int k = 0; k < n; ++k)
                            acc += (long)Bq[i * n + k] * p[k * n + l];
                        t1[i][l] = acc;
                    }
                for (int i = 0; i < n; ++i)
                    for (int j = 0; j < n; ++j) {
                        long acc = 0;
                        for (int l = 0; l < n; ++l)
                            acc += t1[i][l] * Bq[j * n + l];
                        const REAL cij = (sB[i] * sB[j]) * s;
                        V[(size_t)(i * n + j) * Cin + gi * G + c] = (REAL)acc * cij;
                    }
            }
        }
        for (int tap = 0; tap < n2; ++tap)
            for (int gi = 0; gi < ng; ++gi)
                SUF(quantize)(V + (size_t)tap * Cin + (size_t)gi * G, 1, G,
                              Vq + ((size_t)tap * T + t) * Cin + (size_t)gi * G, 1,
                              sV + ((size_t)tap * T + t) * ng + gi);
        free(dq);
        free(d);
        free(V);
    }
}

/*
 * Stage 2: Hadamard product summed over input channels (Eq. 5), per tap:
 *   P_g = sum_{ci in group g} Vq * Uq            (exact int32)
 *   M   = fma(sV_g * sU_g, P_g, M) for g = 0, 1, ...  starting from +0
 *   M  : [n*n][T][Cout]
 */
void SUF(wq8o_stage2)(int n2, long T, int Cin, int Cout, int G, const int8_t *Vq,
                      const REAL *sV, const int8_t *Uq, const REAL *sU, REAL *M)
{
    const int ng = Cin / G;
#pragma omp parallel for schedule(static) collapse(2)
    for (int tap = 0; tap < n2; ++tap)
        for (long t = 0; t < T; ++t)
            for (int co = 0; co < Cout; ++co) {
                const int8_t *v = Vq + ((size_t)tap * T + t) * Cin;
                const int8_t *u = Uq + ((size_t)tap * Cout + co) * Cin;
                REAL acc = 0;
                for (int gi = 0; gi < ng; ++gi) {
                    int32_t P = 0;
                    for (int c = gi * G; c < (gi + 1) * G; ++c)
                        P += (int32_t)v[c] * (int32_t)u[c];
                    REAL s = sV[((size_t)tap * T + t) * ng + gi] *
                             sU[((size_t)tap * Cout + co) * ng + gi];
                    acc = FMA(s, (REAL)P, acc);
                }
                M[((size_t)tap * T + t) * Cout + co] = acc;
            }
}

/*
 * Stage 3: Y = M for one (tile, co) over all n*n taps, quantized with a single
 * scale; output o = sY * (At Yq At^T), cropped to the image.
 *   M  : [n*n][T][Cout],  At : [m][n] (already carrying S_A)
 *   y  : [N][Cout][Ho][Wo]
 *   Yq : [T][Cout][n*n] (optional),  sY : [T][Cout] (optional)
 */
void SUF(wq8o_stage3)(int m, int N, int Cout, int H, int W, int pad, const REAL *At,
                      const REAL *M, REAL *y, int8_t *Yq_out, REAL *sY_out)
{
    const int n = m + 2, n2 = n * n;
    const int Ho = H + 2 * pad - 2, Wo = W + 2 * pad - 2;
    const int tH = (Ho + m - 1) / m, tW = (Wo + m - 1) / m;
    const long T = (long)N * tH * tW;
#pragma omp parallel for schedule(static) collapse(2)
    for (long t = 0; t < T; ++t)
        for (int co = 0; co < Cout; ++co) {
            const int img = (int)(t / ((long)tH * tW));
            const int ty = (int)(t / tW % tH), tx = (int)(t % tW);
            int8_t yq[256];
            REAL sy, z[16][16];
            SUF(quantize)(M + (size_t)t * Cout + co, (long)T * Cout, n2, yq, 1, &sy);
            for (int a = 0; a < m; ++a)
                for (int j = 0; j < n; ++j) {
                    REAL acc = 0;
                    for (int i = 0; i < n; ++i)
                        acc = FMA(At[a * n + i], (REAL)yq[i * n + j], acc);
                    z[a][j] = acc;
                }
            for (int a = 0; a < m; ++a)
                for (int b = 0; b < m; ++b) {
                    REAL acc = 0;
                    for (int j = 0; j < n; ++j)
                        acc = FMA(z[a][j], At[b * n + j], acc);
                    int h = ty * m + a, ww = tx * m + b;
                    if (h < Ho && ww < Wo)
                        y[(((size_t)img * Cout + co) * Ho + h) * Wo + ww] = acc * sy;
                }
            if (Yq_out)
                for (int k = 0; k < n2; ++k)
                    Yq_out[((size_t)t * Cout + co) * n2 + k] = yq[k];
            if (sY_out)
                sY_out[(size_t)t * Cout + co] = sy;
        }
}

/*
 * Stages 2 and 3 evaluated only at chosen (tile, co) pairs, for checks at
 * sizes where the full Hadamard stage is too slow on the CPU. Same
 * definitions as wq8o_stage2 / wq8o_stage3, one pair at a time:
 *   pairs : [S][2] (t, co)
 *   Ms    : [S][n*n]   M over every tap of the pair
 *   Yqs   : [S][n*n],  sYs : [S]
 *   ys    : [S][m][m]  the output tile (uncropped)
 */
void SUF(wq8o_sampled)(int m, long T, int Cin, int Cout, int G, const int8_t *Vq,
                       const REAL *sV, const int8_t *Uq, const REAL *sU, const REAL *At,
                       int S, const long *pairs, REAL *Ms, int8_t *Yqs, REAL *sYs, REAL *ys)
{
    const int n = m + 2, n2 = n * n, ng = Cin / G;
#pragma omp parallel for schedule(static)
    for (int s = 0; s < S; ++s) {
        const long t = pairs[2 * s];
        const int co = (int)pairs[2 * s + 1];
        REAL *Mv = Ms + (size_t)s * n2;
        for (int tap = 0; tap < n2; ++tap) {
            const int8_t *v = Vq + ((size_t)tap * T + t) * Cin;
            const int8_t *u = Uq + ((size_t)tap * Cout + co) * Cin;
            REAL acc = 0;
            for (int gi = 0; gi < ng; ++gi) {
                int32_t P = 0;
                for (int c = gi * G; c < (gi + 1) * G; ++c)
                    P += (int32_t)v[c] * (int32_t)u[c];
                REAL sc = sV[((size_t)tap * T + t) * ng + gi] *
                          sU[((size_t)tap * Cout + co) * ng + gi];
                acc = FMA(sc, (REAL)P, acc);
            }
            Mv[tap] = acc;
        }
        int8_t *yq = Yqs + (size_t)s * n2;
        REAL sy, z[16][16];
        SUF(quantize)(Mv, 1, n2, yq, 1, &sy);
        sYs[s] = sy;
        for (int a = 0; a < m; ++a)
            for (int j = 0; j < n; ++j) {
                REAL acc = 0;
                for (int i = 0; i < n; ++i)
                    acc = FMA(At[a * n + i], (REAL)yq[i * n + j], acc);
                z[a][j] = acc;
            }
        for (int a = 0; a < m; ++a)
            for (int b = 0; b < m; ++b) {
                REAL acc = 0;
                for (int j = 0; j < n; ++j)
                    acc = FMA(z[a][j], At[b * n + j], acc);
                ys[((size_t)s * m + a) * m + b] = acc * sy;
            }
    }
}

/* ------------------------------------------------------------------------
 * Group-wise W8A8 direct 3x3 convolution: the non-Winograd baseline the pages
 * compare against (group-quantized direct kernels, summary page, Fig. 6
 * caption; "W8A8 without Winograd" in the review page's results). Same
 * quantizer as above. Readings: activations are quantized per (image, pixel,
 * group of G consecutive input channels); weights per (kernel tap, output
 * channel, group of G input channels); the output is one fp32 fma chain per
 * (image, co, pixel) over groups ascending and, inside each group, taps
 * kh*3+kw ascending, of fl(sx * sw) * P with P the exact int32 group dot
 * product (the pages fix no order; group-major lets an implementation hold
 * one group's scales at a time); taps that fall outside the image contribute
 * nothing (zero codes).
 * Layouts: xq [N][H][W][Cin], sx [N][H][W][Cin/G]; wq [9][Cout][Cin],
 * sw [9][Cout][Cin/G]; y [N][Cout][Ho][Wo].
 */
void SUF(wq8o_w8a8_quant_x)(int N, int Cin, int H, int W, int G, const float *x,
                              int8_t *xq, REAL *sx)
{
    const int ng = Cin / G;
#pragma omp parallel for schedule(static) collapse(2)
    for (int img = 0; img < N; ++img)
        for (int h = 0; h < H; ++h) {
            REAL buf[256];
            for (int w = 0; w < W; ++w) {
                const size_t px = ((size_t)img * H + h) * W + w;
                for (int gi = 0; gi < ng; ++gi) {
                    for (int c = 0; c < G; ++c)
                        buf[c] = (REAL)x[(((size_t)img * Cin + gi * G + c) * H + h) * W + w];
                    SUF(quantize)(buf, 1, G, xq + px * Cin + (size_t)gi * G, 1, sx + px * ng + gi);
                }
            }
        }
}

void SUF(wq8o_w8a8_quant_w)(int Cin, int Cout, int G, const float *w, int8_t *wq, REAL *sw)
{
    const int ng = Cin / G;
#pragma omp parallel for schedule(static)
    for (int co = 0; co < Cout; ++co) {
        REAL buf[256];
        for (int tap = 0; tap < 9; ++tap)
            for (int gi = 0; gi < ng; ++gi) {
                for (int c = 0; c < G; ++c)
                    buf[c] = (REAL)w[((size_t)co * Cin + gi * G + c) * 9 + tap];
                SUF(quantize)(buf, 1, G, wq + ((size_t)tap * Cout + co) * Cin + (size_t)gi * G, 1,
                              sw + ((size_t)tap * Cout + co) * ng + gi);
            }
    }
}

void SUF(wq8o_w8a8_conv)(int N, int Cin, int Cout, int H, int W, int pad, int G,
                           const int8_t *xq, const REAL *sx, const int8_t *wq, const REAL *sw,
                           REAL *y)
{
    const int Ho = H + 2 * pad - 2, Wo = W + 2 * pad - 2, ng = Cin / G;
#pragma omp parallel for schedule(static) collapse(2)
    for (int img = 0; img < N; ++img)
        for (int co = 0; co < Cout; ++co)
            for (int ho = 0; ho < Ho; ++ho)
                for (int wo = 0; wo < Wo; ++wo) {
                    REAL acc = 0;
                    for (int gi = 0; gi < ng; ++gi)
                        for (int kh = 0; kh < 3; ++kh)
                            for (int kw = 0; kw < 3; ++kw) {
                                const int h = ho + kh - pad, w = wo + kw - pad;
                                if (h < 0 || h >= H || w < 0 || w >= W)
                                    continue;
                                const int tap = kh * 3 + kw;
                                const size_t px = ((size_t)img * H + h) * W + w;
                                const int8_t *a = xq + px * Cin;
                                const int8_t *b = wq + ((size_t)tap * Cout + co) * Cin;
                                int32_t P = 0;
                                for (int c = gi * G; c < (gi + 1) * G; ++c)
                                    P += (int32_t)a[c] * (int32_t)b[c];
                                const REAL s = sx[px * ng + gi] * sw[((size_t)tap * Cout + co) * ng + gi];
                                acc = FMA(s, (REAL)P, acc);
                            }
                    y[(((size_t)img * Cout + co) * Ho + ho) * Wo + wo] = acc;
                }
}

/* Stage 3 with one Y scale per row of taps: for each (t, co) and row i of
 * the n x n Winograd-domain tile, quantize M[i*n + j] over j; dequantize
 * Y^[i][j] = sy_i * Yq[i][j]; then O = A^T Y^ A as fp32 fma chains in index
 * order (the scales vary by row, so they enter before the transform). The
 * review page's core claim names "a single or per-row scale" as the two
 * granularities that cannot hold the cross-shaped range of Y.
 * sY_out: [T][Cout][n]. */
void SUF(wq8o_stage3_rows)(int m, int N, int Cout, int H, int W, int pad, const REAL *At,
                           const REAL *M, REAL *y, int8_t *Yq_out, REAL *sY_out)
{
    const int n = m + 2, n2 = n * n;
    const int Ho = H + 2 * pad - 2, Wo = W + 2 * pad - 2;
    const int tH = (Ho + m - 1) / m, tW = (Wo + m - 1) / m;
    const long T = (long)N * tH * tW;
#pragma omp parallel for schedule(static) collapse(2)
    for (long t = 0; t < T; ++t)
        for (int co = 0; co < Cout; ++co) {
            const int img = (int)(t / ((long)tH * tW));
            const int ty = (int)(t / tW % tH), tx = (int)(t % tW);
            int8_t yq[256];
            REAL sy[16], yd[16][16], z[16][16];
            for (int i = 0; i < n; ++i) {
                SUF(quantize)(M + ((size_t)i * n * T + t) * Cout + co, (long)T * Cout, n, yq + i * n, 1,
                              &sy[i]);
                for (int j = 0; j < n; ++j)
                    yd[i][j] = sy[i] * (REAL)yq[i * n + j];
            }
            for (int a = 0; a < m; ++a)
                for (int j = 0; j < n; ++j) {
                    REAL acc = 0;
                    for (int i = 0; i < n; ++i)
                        acc = FMA(At[a * n + i], yd[i][j], acc);
                    z[a][j] = acc;
                }
            for (int a = 0; a < m; ++a)
                for (int b = 0; b < m; ++b) {
                    REAL acc = 0;
                    for (int j = 0; j < n; ++j)
                        acc = FMA(z[a][j], At[b * n + j], acc);
                    int h = ty * m + a, ww = tx * m + b;
                    if (h < Ho && ww < Wo)
                        y[(((size_t)img * Cout + co) * Ho + h) * Wo + ww] = acc;
                }
            if (Yq_out)
                for (int k = 0; k < n2; ++k)
                    Yq_out[((size_t)t * Cout + co) * n2 + k] = yq[k];
            if (sY_out)
                for (int i = 0; i < n; ++i)
                    sY_out[((size_t)t * Cout + co) * n + i] = sy[i];
        }
}
