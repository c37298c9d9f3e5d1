/*
 * wino_q8_conv — group-wise fully quantized 8-bit Winograd convolution F(m,3)
 * with diagonal transform scales, for AMD Instinct MI355X (gfx950).
 *
 * Method: "Data-Free Group-Wise Fully Quantized Winograd Convolution via
 * Learnable Scales" (arXiv 2412.19867).
 *   - Transforms from the Vandermonde factorization with diagonal scales,
 *     B^T = S_B V^-T, G = S_G V, A^T = V^T S_A, S_A S_B S_G = I; only S_B and
 *     S_G are free ("What carries the argument" on the review page). V is
 *     built from homogeneous polynomial points, V[i][j] = f_i^j g_i^(b-1-j)
 *     (appendix 7.1, "Standard Winograd transforms").
 *   - Group-wise int8 quantization at every stage: input transform, Hadamard
 *     product, output transform (referee summary; Fig. 2 caption).
 *   - The Winograd-domain output Y (Eq. 5) is quantized with one scale that
 *     spans all taps of a tile, the granularity whose cross-shaped range the
 *     learned scales even out (core claim; Fig. 3 caption).
 * The scales are inputs: learning them (the paper's Algorithm 1) is offline.
 *
 * Computation (n = m + 2, T tiles, tile t = (img*tH + ty)*tW + tx,
 * tH = ceil(Ho/m), tW = ceil(Wo/m), Ho = H + 2 pad - 2, Wo likewise):
 *   U  = G g G^T per (co, ci); codes/scales per group of G input channels
 *        inside one tap:         Uq [n*n][Cout][Cin] int8, sU [n*n][Cout][Cin/G] f32
 *   V  = B^T d B per (t, ci), d the n x n input patch (zero outside the
 *        image):                  Vq [n*n][T][Cin] int8,   sV [n*n][T][Cin/G] f32
 *   P_g = sum_{ci in g} Vq Uq (int32, exact)
 *   M  = sum_g (sV_g sU_g) P_g as an fp32 fma chain over g: M [n*n][T][Cout] f32
 *   Y  = M over the n*n taps of one (t, co), one scale: Yq [T][Cout][n*n], sY [T][Cout]
 *   y  = sY * (A^T Yq A), cropped to Ho x Wo:  y [N][Cout][Ho][Wo]
 * Quantizer: a = max|v| over the group; a == 0 -> codes 0, scale 0; otherwise
 * code = clamp(rint(v * (127/a)), -127, 127) (ties to even), scale = a/127.
 * All transform sums up to the Y codes are fp32 fma chains in index order,
 * so codes and scales are reproducible bit for bit (see wq8_algo for the
 * output transform).
 *
 * Convolution semantics: 3x3 cross-correlation, stride 1, zero padding `pad`
 * (0..2), no bias, NCHW activations.
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned allocations on the current HIP device;
 *     the library never allocates device memory at run time (the workspace of
 *     wq8_conv_forward_noalloc is a module-scope array) and never synchronises.
 *     All work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *     and completes asynchronously; device faults surface at the caller's
 *     next synchronisation.
 *   - Device pointers must be 16-byte aligned. Arguments are checked before
 *     anything is enqueued; on error nothing is launched and the status says
 *     why (details in wq8_last_error()).
 *   - Inputs must be finite; behaviour for NaN/Inf data is unspecified.
 *   - A plan is immutable after creation and may be used from several host
 *     threads on different streams, each with its own workspace.
 */
#ifndef WINO_Q8_CONV_H
#define WINO_Q8_CONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WQ8_OK = 0,
    WQ8_ERR_INVALID_ARG = -1,      /* a size, pointer or enum is out of range */
    WQ8_ERR_UNSUPPORTED = -2,      /* valid, but not a configuration the library runs */
    WQ8_ERR_SINGULAR_POINTS = -3,  /* points not distinct: V is singular */
    WQ8_ERR_WORKSPACE_TOO_SMALL = -4,
    WQ8_ERR_MISALIGNED = -5,       /* a device pointer is not 16-byte aligned */
    WQ8_ERR_HIP = -6,              /* a HIP launch failed; see wq8_last_error() */
    WQ8_ERR_NO_MEMORY = -7         /* host allocation for the plan failed */
} wq8_status;

typedef enum { WQ8_F32 = 0, WQ8_BF16 = 1 } wq8_dtype;

/* How wq8_conv_forward runs stages 2 and 3. Both give bit-identical M, Y
 * scales and Y codes; they differ only in how A^T Yq A is evaluated:
 *   STAGED: an int8 GEMM kernel writes M (fp32) to the workspace and a second
 *           kernel requantizes it and applies the output transform as fp32
 *           fma chains in index order (bit-identical to that definition);
 *   FUSED:  one kernel keeps M on chip (registers) per block of 16 or 32
 *           tiles x 16 or 32 output channels, re-reading the prepared
 *           weights per tile block,
 *           and evaluates vec(O) = (A^T kron A^T) vec(Yq) on fp16 matrix
 *           cores with the Kronecker matrix split into two fp16 parts
 *           (fp32 accumulation): outputs within ~1e-5 of their RMS of the
 *           fp32 evaluation;
 *   AUTO:   FUSED when the weight codes are at most 2 MiB, or re-reading
 *           them once per 16-tile block moves fewer bytes than writing and
 *           reading M; else STAGED. */
typedef enum { WQ8_ALGO_AUTO = 0, WQ8_ALGO_STAGED = 1, WQ8_ALGO_FUSED = 2 } wq8_algo;

/* Granularity of the Y (Winograd-domain output) scales. TILE: one scale per
 * (tile, output channel) spanning all n*n taps (the default; the
 * tap-spanning scale whose cross-shaped range the learned S_B, S_G even out;
 * core claim and Fig. 3 caption of the review page). ROW: one scale per row
 * of taps (the other granularity the core claim names); the dequantized
 * Y^[i][j] = sy_i Yq[i][j] then enters A^T Y^ A. ROW runs the staged
 * schedule only. */
typedef enum { WQ8_YGROUP_TILE = 0, WQ8_YGROUP_ROW = 1 } wq8_ygroup;

/* What the input transform quantizes. The review page's Eqs. 14-16 survive
 * only as the combined factor "sqB sqB sqx" (a B^T scale on each side and an
 * input scale; minor comments), so two readings are offered:
 *   FP32:       V = B^T d B in fp32 fma chains (the default; no quantizer
 *               before the transform);
 *   INT_TENSOR: B^T quantized with one scale for the matrix (codes Bq, row
 *               scale sq_i all equal), the n x n input patches of a (tile,
 *               group of G input channels) with one scale sx over all n*n*G
 *               values (zero padding included; codes dq). The transform then
 *               runs exactly on integers and is scaled back:
 *                 Wi[i][j] = sum_k sum_l Bq[i][k] dq[k][l] Bq[j][l]  (int32)
 *                 V[i][j]  = float(Wi[i][j]) * ((sq_i * sq_j) * sx)  (fp32, RNE)
 *               after which V is quantized per group exactly as for FP32;
 *   INT_ROW:    as INT_TENSOR with one scale per row of B^T.
 * Only stage 1 changes; stages 2 and 3 and every layout stay as they are. */
typedef enum { WQ8_INQ_FP32 = 0, WQ8_INQ_INT_TENSOR = 1, WQ8_INQ_INT_ROW = 2 } wq8_inq;

typedef struct wq8_plan wq8_plan; /* opaque */

typedef struct {
    int m;                 /* output tile size: 4 or 6 (r = 3 fixed) */
    const double *points;  /* n = m + 2 distinct points; +INFINITY is the point
                              at infinity (homogeneous (1, 0)). NULL selects the
                              standard points 0, 1, -1, 2, -2, [1/2, -1/2,] inf */
    const float *s_B;      /* n diagonal entries of S_B, finite, non-zero; NULL = 1 */
    const float *s_G;      /* n diagonal entries of S_G; S_A = (S_B S_G)^-1 */
    int group;             /* G: 16, 32, 64, 128 or 256; Cin % G == 0 */
    int N, Cin, Cout, H, W;
    int pad;               /* 0, 1 or 2 */
    wq8_dtype x_dtype;     /* activations in */
    wq8_dtype y_dtype;     /* activations out */
    wq8_algo algo;         /* stage 2 + 3 schedule for wq8_conv_forward */
    wq8_ygroup y_group;    /* Y scale granularity (TILE unless stated) */
    wq8_inq in_quant;      /* input-stage reading (FP32 unless stated) */
    /* Kernel shapes, for tests and tuning; 0 lets the library choose (by block
     * count against the device's compute units, at launch). Every shape
     * performs the same operations per output in the same order, so results
     * do not depend on the choice. A value out of range is
     * WQ8_ERR_INVALID_ARG; a shape not built for the layer is
     * WQ8_ERR_UNSUPPORTED. */
    int stage1_rows;       /* input-transform LDS window: 1 all n input rows,
                              2 half of them at a time (FP32 input stage) */
    int fused_waves;       /* waves of a 16 x 16 fused block: 4; 8 or 16 for F(6,3) */
    int fused_block;       /* fused block: 1 16 tiles x 16 output channels;
                              F(6,3) with G <= 64 also 2 32 x 32, 3 32 tiles x
                              16 channels, 4 16 tiles x 32 channels (these
                              wide blocks hold at most that many tiles: the
                              launch spreads the tiles evenly over the
                              compute units) */
    int stage2_rows;       /* staged Hadamard GEMM: 1 the LDS-pipelined kernel
                              (64 tiles x 64 channels per block); 4, 5, 6 or 8
                              the register-streamed kernel with that many
                              16-tile rows per block */
    int stage2_cols;       /* staged Hadamard GEMM: output channels per wave
                              in units of 16: 1, or 2 for stage2_rows 4 or 5 */
    int stage2_waves;      /* staged Hadamard GEMM: waves per block, 2 or 4 */
    int stage3_lanes;      /* staged output transform: lanes per (tile, output
                              channel) pair, 1 or 2 */
} wq8_desc;

/* Validates the descriptor and builds the scaled transforms on the host (exact
 * rational arithmetic, each entry rounded once to fp32, ties to even). No
 * device work. The caller owns *out and frees it with wq8_plan_destroy. */
wq8_status wq8_plan_create(const wq8_desc *desc, wq8_plan **out);
void wq8_plan_destroy(wq8_plan *plan);

/* Sizes in bytes of the forward workspace (for the schedule the plan chose)
 * and of the prepared weights, the tile count T, and the schedule itself
 * (WQ8_ALGO_STAGED or WQ8_ALGO_FUSED, never AUTO). Any output pointer may be
 * NULL. */
wq8_status wq8_plan_query(const wq8_plan *plan, size_t *workspace_bytes,
                          size_t *u_code_bytes, size_t *u_scale_bytes, int64_t *tiles,
                          wq8_algo *algo);

/* Host copies of the fp32 matrices the kernels use: Bt [n][n] (carries S_B),
 * G [n][3] (carries S_G), At [m][n] (carries S_A). Any pointer may be NULL. */
wq8_status wq8_plan_matrices(const wq8_plan *plan, float *Bt, float *G, float *At);

/* Host copies of the quantized B^T used by the INT_TENSOR / INT_ROW input
 * stage: Bq [n][n] int8 and its row scales sq [n] (fp32 absmax quantizer as
 * above, over the whole matrix or per row). WQ8_ERR_INVALID_ARG for an FP32
 * plan. Either pointer may be NULL. */
wq8_status wq8_plan_bt_codes(const wq8_plan *plan, int8_t *Bq, float *sq);

/* Offline weight transform and quantization (U = G g G^T; per-group int8).
 *   w  [Cout][Cin][3][3] f32 (device), Uq [n*n][Cout][Cin] int8 (device),
 *   sU [n*n][Cout][Cin/G] f32 (device). */
wq8_status wq8_weights_prepare(const wq8_plan *plan, const float *w, int8_t *Uq,
                               float *sU, void *stream);

/* The hot path: input transform + quantization, int8 Hadamard GEMMs with group
 * dequantization, Y requantization + output transform + crop.
 *   x [N][Cin][H][W] (x_dtype), y [N][Cout][Ho][Wo] (y_dtype), Uq/sU from
 *   wq8_weights_prepare, workspace of at least the queried size (device,
 *   256-byte aligned recommended). x and y must not overlap. */
wq8_status wq8_conv_forward(const wq8_plan *plan, const void *x, const int8_t *Uq,
                            const float *sU, void *y, void *workspace,
                            size_t workspace_bytes, void *stream);

/* wq8_conv_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The workspace is a device array built into
 * the library, WQ8_NOALLOC_MAX_WORKSPACE bytes on every GPU the library runs
 * on, held from module load until the process ends; this call allocates
 * nothing. Its device address is looked up once per device, on the first call
 * with that device current. Plans whose forward needs a larger workspace
 * (wq8_plan_query) get WQ8_ERR_WORKSPACE_TOO_SMALL and nothing is launched.
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (different streams, or several host threads) race and give wrong
 * results; serialise them. The array keeps the last call's contents; no stage
 * reads workspace bytes it has not written in the same call. Results are bit
 * for bit those of wq8_conv_forward. */
#define WQ8_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
wq8_status wq8_conv_forward_noalloc(const wq8_plan *plan, const void *x, const int8_t *Uq,
                                    const float *sU, void *y, void *stream);

/* Individual stages with the layouts above (for parity checks and profiling). */
wq8_status wq8_stage1(const wq8_plan *plan, const void *x, int8_t *Vq, float *sV,
                      void *stream);
wq8_status wq8_stage2(const wq8_plan *plan, const int8_t *Vq, const float *sV,
                      const int8_t *Uq, const float *sU, float *M, void *stream);
/* int32 partial sums P [n*n][Cin/G][T][Cout], one per quantization group. */
wq8_status wq8_stage2_i32(const wq8_plan *plan, const int8_t *Vq, const int8_t *Uq,
                          int32_t *P, void *stream);
/* Y requantization + output transform. Yq [T][Cout][n*n] and sY ([T][Cout],
 * or [T][Cout][n] for WQ8_YGROUP_ROW) are optional outputs (NULL to skip). */
wq8_status wq8_stage3(const wq8_plan *plan, const float *M, void *y, int8_t *Yq,
                      float *sY, void *stream);

/* Stages 2 and 3 as the single fused kernel (M stays on chip): the same Y
 * codes as wq8_stage2 followed by wq8_stage3; y as described for FUSED.
 * WQ8_ERR_UNSUPPORTED for a WQ8_YGROUP_ROW plan. */
wq8_status wq8_stage23(const wq8_plan *plan, const int8_t *Vq, const float *sV,
                       const int8_t *Uq, const float *sU, void *y, void *stream);

/* ---- Group-wise W8A8 direct 3x3 convolution: the non-Winograd baseline the
 * method is compared against (group-quantized direct kernels; summary page,
 * Fig. 6 caption, and the review page's "W8A8 without Winograd" results).
 * Uses the plan's N, Cin, Cout, H, W, pad, group and dtypes; the Winograd
 * fields are not used. Same quantizer as above:
 *   x codes per (image, pixel, group of G input channels):
 *     Xq [N][H][W][Cin] int8, sX [N][H][W][Cin/G] f32;
 *   weights per (kernel tap kh*3+kw, output channel, group):
 *     Wq [9][Cout][Cin] int8, sW [9][Cout][Cin/G] f32;
 *   y[img][co][ho][wo] = fp32 fma chain over groups ascending, then taps
 *     ascending, of fl(sX * sW) * P (P the int32 group dot product of the
 *     codes; taps outside the image contribute nothing). */

/* Workspace bytes of wq8_direct_forward (Xq | sX) and sizes of Wq and sW. */
wq8_status wq8_direct_query(const wq8_plan *plan, size_t *workspace_bytes, size_t *w_code_bytes,
                            size_t *w_scale_bytes);
/* w [Cout][Cin][3][3] f32 -> Wq, sW (device). */
wq8_status wq8_direct_weights_prepare(const wq8_plan *plan, const float *w, int8_t *Wq, float *sW,
                                      void *stream);
/* x (x_dtype, NCHW) -> Xq, sX. */
wq8_status wq8_direct_quantize_x(const wq8_plan *plan, const void *x, int8_t *Xq, float *sX,
                                 void *stream);
/* Xq, sX, Wq, sW -> y (y_dtype, NCHW). */
wq8_status wq8_direct_conv(const wq8_plan *plan, const int8_t *Xq, const float *sX,
                           const int8_t *Wq, const float *sW, void *y, void *stream);
/* wq8_direct_quantize_x then wq8_direct_conv, with Xq and sX in the workspace. */
wq8_status wq8_direct_forward(const wq8_plan *plan, const void *x, const int8_t *Wq,
                              const float *sW, void *y, void *workspace, size_t workspace_bytes,
                              void *stream);

const char *wq8_status_string(wq8_status status);
/* Detail of the last error on the calling host thread ("" if none). */
const char *wq8_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WINO_Q8_CONV_H */
