// lora_apply_packed without a caller workspace: the calls' scratch (segments,
// split-K partial sums, the buffer, the single-launch K-split decode's
// zero-on-entry region) lives in one file-scope device array per GPU, so the
// entry point allocates nothing.  For callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// Layout of the array.  lora_apply_packed keeps every region but one from the
// start of its workspace and the K-split decode region (plus the error word's
// line) at its end.  Here the array is passed as a workspace of
// kStaticScratchBytes, and a call is taken only when its start regions fit in
// the lower half and its end region in the upper half: then no call's start
// regions reach another call's end region, whatever their shapes.
//
// Every call on a device shares that device's array and leaves it as the
// K-split decode needs it (that region zero; the others are written before
// they are read within each call), so calls that overlap in time on one GPU
// race.
#include <mutex>

#include "../../include/adapter_apply.h"
#include "common.hpp"

using namespace aa;

// One per GPU the library runs on, held until the process ends.
static __device__ __align__(256) char scratch[LORA_STATIC_SCRATCH_BYTES];

namespace {

constexpr size_t kStaticScratchBytes = (size_t)LORA_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

struct DeviceScratch {
    void *ptr = nullptr;    // device address of `scratch` on this device
    bool zeroed = false;    // zero-filled by an eager (not captured) call
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

int current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    return dev;
}

// The array's device address on the current device: hipGetSymbolAddress once
// per device (its return code checked), kept per device; the array's name in
// host code is only a host-side stand-in, so every use below goes through
// this address.  Enqueues nothing.
lora_status_t scratch_address(int dev, void **out) {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch &d = g_dev[dev];
    if (!d.ptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LORA_E_RUNTIME;
        d.ptr = p;
    }
    *out = d.ptr;
    return LORA_OK;
}

// Zero-fills the device's array on `st` until an eager call has done it: a
// fill recorded into a graph under capture runs at each replay, so the device
// counts as zeroed only once a call outside capture has filled it.
lora_status_t ensure_zeroed(int dev, hipStream_t st) {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch &d = g_dev[dev];
    if (d.zeroed) return LORA_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return LORA_E_RUNTIME;
    if (launch_fill_zero(d.ptr, kStaticScratchBytes, st) != hipSuccess) return LORA_E_LAUNCH;
    if (cs == hipStreamCaptureStatusNone) d.zeroed = true;
    return LORA_OK;
}

}  // namespace

namespace aa {

// lora_workspace_check(NULL, 0, stream): the current device's array.
int32_t static_scratch_check(hipStream_t st) {
    const int dev = current_device();
    if (dev < 0) return LORA_E_RUNTIME;
    void *p = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        p = g_dev[dev].ptr;
    }
    if (!p) return LORA_OK;            // no call has used it on this device
    int32_t word = 0;
    const char *e = static_cast<const char *>(p) + err_word_offset(kStaticScratchBytes);
    if (hipMemcpyAsync(&word, e, sizeof(word), hipMemcpyDeviceToHost, st) != hipSuccess)
        return LORA_E_RUNTIME;
    if (hipStreamSynchronize(st) != hipSuccess) return LORA_E_RUNTIME;
    if (word == 0) return LORA_OK;
    if (launch_fill_zero(p, kStaticScratchBytes, st) != hipSuccess) return LORA_E_LAUNCH;
    if (hipStreamSynchronize(st) != hipSuccess) return LORA_E_RUNTIME;
    return LORA_E_TIMEOUT;
}

}  // namespace aa

extern "C" {

lora_status_t lora_apply_packed_noalloc(void *y, int64_t ldy, int64_t y_col_offset,
                                        const void *x, int64_t ldx, int32_t T, int32_t K,
                                        const void *const *A, const void *const *B,
                                        const int64_t *N, int32_t S, int32_t L, int32_t R,
                                        const int32_t *idx, const int32_t *slot_rank,
                                        const float *scale, int32_t dtype, int32_t path,
                                        uint32_t flags, void *stream) {
    // the sizes lora_apply_packed checks first, so ws_layout below is defined
    if (dtype != LORA_DT_F32 && dtype != LORA_DT_BF16) return LORA_E_DTYPE;
    if (T < 0 || L < 1 || L > LORA_MAX_SLOTS || K < 1) return LORA_E_SHAPE;
    if (R < 1 || R > LORA_MAX_RANK) return LORA_E_RANK;
    if (S < 1 || S > LORA_MAX_SLICES) return LORA_E_SLICES;
    const WsLayout wl = ws_layout(T, K, S, R, L);
    const size_t half = kStaticScratchBytes / 2;
    if (wl.end - wl.relay - 256 > half || wl.relay + 256 > half) return LORA_E_SCRATCH;
    const int dev = current_device();
    if (dev < 0) return LORA_E_RUNTIME;
    void *ws = nullptr;
    lora_status_t e = scratch_address(dev, &ws);
    if (e != LORA_OK) return e;
    // segments in the array are another call's: every call builds its own
    flags &= ~LORA_FLAG_SEGMENTS_READY;
    PackedPlan p;
    e = packed_plan(y, ldy, y_col_offset, x, ldx, T, K, A, B, N, S, L, R, idx, slot_rank, scale,
                    dtype, path, flags, ws, kStaticScratchBytes, &p);
    if (e != LORA_OK || p.noop) return e;
    hipStream_t st = static_cast<hipStream_t>(stream);
    e = ensure_zeroed(dev, st);
    if (e != LORA_OK) return e;
    return packed_run(p, y, ldy, y_col_offset, x, ldx, T, K, A, B, N, S, L, R, idx, slot_rank,
                      scale, dtype, flags, ws, kStaticScratchBytes, st);
}

}  // extern "C"
