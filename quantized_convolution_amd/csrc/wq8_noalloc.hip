// The forward without a caller-supplied workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). Its workspace (activation codes and
// scales, and M for the staged schedule) lives in one file-scope device array
// of fixed size; every GPU the library runs on holds its own copy of that
// array from module load until the process ends.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "wq8_internal.h"

namespace {

// Every forward of the benchmark layers fits (the largest, the staged 56 x 56
// ResNet-18 layer, needs 66.4 MB); larger plans are rejected.
constexpr size_t kScratchBytes = WQ8_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of `scratch` per device. In host code the array's name is
// only a stand-in: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current.
constexpr int kMaxDevices = 64;
std::atomic<char *> g_scratch[kMaxDevices];
std::mutex g_scratch_lock;

wq8_status scratch_of_current_device(char **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return wq8::fail(WQ8_ERR_HIP, "no current HIP device (or device index >= %d)", kMaxDevices);
    }
    char *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_lock);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *addr = nullptr;
            const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !addr) {
                (void)hipGetLastError();
                return wq8::fail(WQ8_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                                 hipGetErrorString(e));
            }
            p = (char *)addr;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return WQ8_OK;
}

}  // namespace

extern "C" {

wq8_status wq8_conv_forward_noalloc(const wq8_plan *p, const void *x, const int8_t *Uq,
                                    const float *sU, void *y, void *stream) {
    wq8::clear_error();
    wq8_status st = wq8::check_forward_args(p, x, Uq, sU, y);
    if (st != WQ8_OK) return st;
    if (p->ws_bytes > kScratchBytes)
        return wq8::fail(WQ8_ERR_WORKSPACE_TOO_SMALL,
                         "the forward needs %zu bytes of workspace; the built-in one holds %zu",
                         p->ws_bytes, kScratchBytes);
    char *ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != WQ8_OK) return st;
    // No stage reads workspace bytes it has not written in the same call, so
    // the array needs no clearing between calls.
    return wq8::forward_launch(p, x, Uq, sU, y, ws, stream);
}

}  // extern "C"
