// C ABI entry points: synchronous argument checks, then kernel launches on the
// caller's stream. Nothing is enqueued when a check fails.
#include <stdint.h>

#include "wq8_internal.h"

using namespace wq8;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

wq8_status need(const void *p, const char *name) {
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(WQ8_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
    return WQ8_OK;
}

#define WQ8_NEED(p)                                  \
    do {                                             \
        wq8_status _st = need((const void *)(p), #p); \
        if (_st != WQ8_OK) return _st;               \
    } while (0)

#define WQ8_TRY(expr)                  \
    do {                               \
        wq8_status _st = (expr);       \
        if (_st != WQ8_OK) return _st; \
    } while (0)

}  // namespace

namespace wq8 {

wq8_status forward_launch(const wq8_plan *p, const void *x, const int8_t *Uq, const float *sU,
                          void *y, void *workspace, void *stream) {
    char *ws = (char *)workspace;
    int8_t *Vq = (int8_t *)(ws + p->off_vq);
    float *sV = (float *)(ws + p->off_sv);
    float *M = (float *)(ws + p->off_m);
    WQ8_TRY(launch_stage1(p->geo, p->mats, p->xdt, x, Vq, sV, stream));
    if (p->fused) return launch_fused23(p->geo, p->mats, p->ydt, Vq, sV, Uq, sU, y, stream);
    WQ8_TRY(launch_stage2(p->geo, Vq, sV, Uq, sU, M, nullptr, stream));
    return launch_stage3(p->geo, p->mats, p->ydt, M, y, nullptr, nullptr, stream);
}

wq8_status check_forward_args(const wq8_plan *p, const void *x, const int8_t *Uq, const float *sU,
                              const void *y) {
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(x);
    WQ8_NEED(Uq);
    WQ8_NEED(sU);
    WQ8_NEED(y);
    if (x == y) return fail(WQ8_ERR_INVALID_ARG, "x and y must not overlap");
    return WQ8_OK;
}

}  // namespace wq8

extern "C" {

wq8_status wq8_weights_prepare(const wq8_plan *p, const float *w, int8_t *Uq, float *sU,
                               void *stream) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(w);
    WQ8_NEED(Uq);
    WQ8_NEED(sU);
    return launch_weights(p->geo, p->mats, w, Uq, sU, stream);
}

wq8_status wq8_conv_forward(const wq8_plan *p, const void *x, const int8_t *Uq, const float *sU,
                            void *y, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(x);
    WQ8_NEED(Uq);
    WQ8_NEED(sU);
    WQ8_NEED(y);
    WQ8_NEED(workspace);
    if (workspace_bytes < p->ws_bytes)
        return fail(WQ8_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                    p->ws_bytes);
    if (x == y) return fail(WQ8_ERR_INVALID_ARG, "x and y must not overlap");
    return forward_launch(p, x, Uq, sU, y, workspace, stream);
}

wq8_status wq8_stage1(const wq8_plan *p, const void *x, int8_t *Vq, float *sV, void *stream) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(x);
    WQ8_NEED(Vq);
    WQ8_NEED(sV);
    return launch_stage1(p->geo, p->mats, p->xdt, x, Vq, sV, stream);
}

wq8_status wq8_stage2(const wq8_plan *p, const int8_t *Vq, const float *sV, const int8_t *Uq,
                      const float *sU, float *M, void *stream) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(Vq);
    WQ8_NEED(sV);
    WQ8_NEED(Uq);
    WQ8_NEED(sU);
    WQ8_NEED(M);
    return launch_stage2(p->geo, Vq, sV, Uq, sU, M, nullptr, stream);
}

wq8_status wq8_stage2_i32(const wq8_plan *p, const int8_t *Vq, const int8_t *Uq, int32_t *P,
                          void *stream) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(Vq);
    WQ8_NEED(Uq);
    WQ8_NEED(P);
    return launch_stage2(p->geo, Vq, nullptr, Uq, nullptr, nullptr, P, stream);
}

wq8_status wq8_stage3(const wq8_plan *p, const float *M, void *y, int8_t *Yq, float *sY,
                      void *stream) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(M);
    WQ8_NEED(y);
    if (Yq) WQ8_NEED(Yq);
    if (sY) WQ8_NEED(sY);
    return launch_stage3(p->geo, p->mats, p->ydt, M, y, Yq, sY, stream);
}

wq8_status wq8_stage23(const wq8_plan *p, const int8_t *Vq, const float *sV, const int8_t *Uq,
                       const float *sU, void *y, void *stream) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(Vq);
    WQ8_NEED(sV);
    WQ8_NEED(Uq);
    WQ8_NEED(sU);
    WQ8_NEED(y);
    if (p->geo.y_rows) return fail(WQ8_ERR_UNSUPPORTED, "per-row Y scales run the staged schedule only");
    return launch_fused23(p->geo, p->mats, p->ydt, Vq, sV, Uq, sU, y, stream);
}

wq8_status wq8_direct_query(const wq8_plan *p, size_t *workspace_bytes, size_t *w_code_bytes,
                            size_t *w_scale_bytes) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    if (workspace_bytes) *workspace_bytes = p->d_ws_bytes;
    if (w_code_bytes) *w_code_bytes = p->d_w_code_bytes;
    if (w_scale_bytes) *w_scale_bytes = p->d_w_scale_bytes;
    return WQ8_OK;
}

wq8_status wq8_direct_weights_prepare(const wq8_plan *p, const float *w, int8_t *Wq, float *sW,
                                      void *stream) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(w);
    WQ8_NEED(Wq);
    WQ8_NEED(sW);
    return launch_direct_weights(p->geo, w, Wq, sW, stream);
}

wq8_status wq8_direct_quantize_x(const wq8_plan *p, const void *x, int8_t *Xq, float *sX,
                                 void *stream) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(x);
    WQ8_NEED(Xq);
    WQ8_NEED(sX);
    return launch_direct_qx(p->geo, p->xdt, x, Xq, sX, stream);
}

wq8_status wq8_direct_conv(const wq8_plan *p, const int8_t *Xq, const float *sX, const int8_t *Wq,
                           const float *sW, void *y, void *stream) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(Xq);
    WQ8_NEED(sX);
    WQ8_NEED(Wq);
    WQ8_NEED(sW);
    WQ8_NEED(y);
    return launch_direct_conv(p->geo, p->ydt, Xq, sX, Wq, sW, y, stream);
}

wq8_status wq8_direct_forward(const wq8_plan *p, const void *x, const int8_t *Wq, const float *sW,
                              void *y, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    if (!p) return fail(WQ8_ERR_INVALID_ARG, "null plan");
    WQ8_NEED(x);
    WQ8_NEED(Wq);
    WQ8_NEED(sW);
    WQ8_NEED(y);
    WQ8_NEED(workspace);
    if (workspace_bytes < p->d_ws_bytes)
        return fail(WQ8_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                    p->d_ws_bytes);
    if (x == y) return fail(WQ8_ERR_INVALID_ARG, "x and y must not overlap");
    char *ws = (char *)workspace;
    int8_t *Xq = (int8_t *)ws;
    float *sX = (float *)(ws + p->d_off_sx);
    WQ8_TRY(launch_direct_qx(p->geo, p->xdt, x, Xq, sX, stream));
    return launch_direct_conv(p->geo, p->ydt, Xq, sX, Wq, sW, y, stream);
}

}  // extern "C"
