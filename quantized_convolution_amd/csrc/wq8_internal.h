// Internal declarations shared by the host plan, the C ABI and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/wino_q8_conv.h"

namespace wq8 {

constexpr int kMaxN = 8;  // n = m + 2 for m = 6

// Transform matrices passed by value to the kernels (row-major).
struct Mats {
    float Bt[kMaxN * kMaxN];  // [n][n]  carries S_B
    float G[kMaxN * 3];       // [n][3]  carries S_G
    float At[6 * kMaxN];      // [m][n]  carries S_A
    float kscale, oscale;     // 2^-s and 2^s with max |A^T (x) A^T| * 2^-s <= 2^14
    int Bq[kMaxN * kMaxN];    // [n][n] int8 codes of B^T (integer input stage only)
    float sqb[kMaxN];         // their row scales
};

// Problem geometry shared by every kernel.
struct Geo {
    int m, n, G, ng;          // tile size, n = m + 2, group size, groups per Cin
    int N, Cin, Cout, H, W, pad;
    int Ho, Wo, tH, tW;
    int64_t T;                // tiles
    int bt_std, at_std;       // 1 if B^T / A^T vanish wherever the standard
                              // points' matrices do (zero terms may be skipped)
    int co_major;             // fused kernel: 1 = output-channel blocks outermost
                              // (weights larger than the activation codes)
    int fused_waves;          // fused kernel: waves per 16 x 16 block (4, 8 or 16), 0 chosen at launch
    int fused_wide;           // fused kernel, F(6,3): -1 chosen at launch; 0 16 x 16 blocks; 1 32 x 32,
                              // 2 32 tiles x 16 channels, 3 16 x 32
    int fused_ntb;            // wide fused kernel: tile blocks (set at launch); block b takes
                              // tiles [b T / ntb, (b + 1) T / ntb)
    int y_rows;               // 1: one Y scale per row of taps (staged only)
    int in_quant;             // wq8_inq: 0 fp32 input transform, 1/2 integer
    int s1_rows;              // stage-1 window: 0 chosen at launch, 1 all rows, 2 half the rows
    int s2_rows;              // stage-2 block tiles / 16 (4, 5, 6, 8), 0 chosen at launch
    int s2_cols;              // stage-2 channels per wave / 16 (1, 2), 0 chosen at launch
    int s2_waves;             // stage-2 waves per block (2 or 4), 0 chosen at launch
    int s3_lanes;             // stage-3 lanes per (tile, co) pair (1 or 2), 0 chosen at launch
};

// Nonzero patterns of B^T [n][n] and A^T [m][n] for the standard points
// 0, 1, -1, 2, -2, (1/2, -1/2,) infinity: bit (row * n + col) is set where the
// entry is nonzero. Diagonal scales never change these patterns.
constexpr uint64_t kBtPattern4 = 0xa9e79e795ull;
constexpr uint64_t kBtPattern6 = 0xaa7e7e7e7e7e7e55ull;
constexpr uint64_t kAtPattern4 = 0xf9e79full;
constexpr uint64_t kAtPattern6 = 0xfe7e7e7e7e7full;

// Set the thread-local error detail (printf-style) and return `st`.
wq8_status fail(wq8_status st, const char *fmt, ...);
void clear_error();

// Compute units of the current HIP device (cached per device; 256 if the
// query fails). Host code, for choosing launch shapes.
int device_cus();

// WQ8_OK, or WQ8_ERR_HIP with the pending launch error as detail.
wq8_status check_launch(const char *what);

// Kernel launchers (wq8_kernels.hip). Each returns WQ8_OK or WQ8_ERR_HIP.
wq8_status launch_weights(const Geo &g, const Mats &mt, const float *w, int8_t *Uq, float *sU,
                          void *stream);
wq8_status launch_stage1(const Geo &g, const Mats &mt, wq8_dtype xdt, const void *x,
                         int8_t *Vq, float *sV, void *stream);
wq8_status launch_stage2(const Geo &g, const int8_t *Vq, const float *sV, const int8_t *Uq,
                         const float *sU, float *M, int32_t *P, void *stream);
wq8_status launch_hgemm(const Geo &g, const int8_t *Vq, const float *sV, const int8_t *Uq,
                        const float *sU, float *M, int32_t *P, void *stream);
wq8_status launch_stage3(const Geo &g, const Mats &mt, wq8_dtype ydt, const float *M, void *y,
                         int8_t *Yq, float *sY, void *stream);
wq8_status launch_fused23(const Geo &g, const Mats &mt, wq8_dtype ydt, const int8_t *Vq,
                          const float *sV, const int8_t *Uq, const float *sU, void *y,
                          void *stream);

// The forward's kernels on a workspace laid out as the plan says (Vq | sV |
// M); arguments already checked.
wq8_status forward_launch(const wq8_plan *p, const void *x, const int8_t *Uq, const float *sU,
                          void *y, void *workspace, void *stream);
// The forward's pointer checks (null, 16-byte alignment, x != y).
wq8_status check_forward_args(const wq8_plan *p, const void *x, const int8_t *Uq, const float *sU,
                              const void *y);

// Group-wise W8A8 direct convolution (wq8_direct.hip), the non-Winograd
// baseline: weights Wq [9][Cout][Cin] / sW [9][Cout][Cin/G], activation codes
// Xq [N][H][W][Cin] / sX [N][H][W][Cin/G].
wq8_status launch_direct_weights(const Geo &g, const float *w, int8_t *Wq, float *sW, void *stream);
wq8_status launch_direct_qx(const Geo &g, wq8_dtype xdt, const void *x, int8_t *Xq, float *sX,
                            void *stream);
wq8_status launch_direct_conv(const Geo &g, wq8_dtype ydt, const int8_t *Xq, const float *sX,
                              const int8_t *Wq, const float *sW, void *y, void *stream);

}  // namespace wq8

struct wq8_plan {
    wq8::Geo geo;
    wq8::Mats mats;
    wq8_dtype xdt, ydt;
    double points[wq8::kMaxN];
    float sB[wq8::kMaxN], sG[wq8::kMaxN];
    int fused;  // stage 2 + 3 schedule chosen for the forward
    // forward workspace layout (bytes); M is only used by the staged schedule
    size_t off_vq, off_sv, off_m, ws_bytes;
    size_t u_code_bytes, u_scale_bytes;
    // W8A8 direct convolution: workspace Xq | sX, weight sizes
    size_t d_off_sx, d_ws_bytes, d_w_code_bytes, d_w_scale_bytes;
};
