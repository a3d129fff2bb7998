// The backward without a caller-supplied workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// fa_bwd's only scratch is two fp32 row statistics per query row (D_i / c
// and -lse_i log2 e, written by its first stage before the later stages read
// them).  Here they live in a file-scope device array of fixed size, one copy
// per device, held until the process ends; the entry point checks the
// problem against that size, looks the array's device address up once per
// device and then runs fa_bwd on it.  Nothing is allocated and nothing needs
// clearing: the first stage overwrites every entry the later ones read.
// All calls on one device share its copy, so calls that overlap on one
// device (on different streams or host threads) race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>

#include "../../include/fa.h"

namespace fa {
// Records a status and message for fa_last_error (fa_api.cpp).
fa_status_t record_error(fa_status_t s, const char *msg);
}  // namespace fa

constexpr size_t kScratchBytes = size_t(32) << 20;   // 4,194,304 query rows

// The device array.  In host code this name only identifies the symbol for
// hipGetSymbolAddress; the host never passes it to a kernel or a copy.
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::atomic<void *> g_scratch[kMaxDevices];   // device address of each device's copy
std::mutex g_scratch_mu;

// Device address of the current device's copy, looked up on the first call
// on that device (with it current).
fa_status_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        char msg[160];
        snprintf(msg, sizeof msg, "fa_bwd_noalloc: hipGetDevice: %s (%d)", hipGetErrorString(e), (int)e);
        return fa::record_error(FA_EHIP, msg);
    }
    if (dev < 0 || dev >= kMaxDevices) return fa::record_error(FA_EHIP, "fa_bwd_noalloc: device index out of range");
    void *ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !ptr) {
                char msg[160];
                snprintf(msg, sizeof msg, "fa_bwd_noalloc: hipGetSymbolAddress: %s (%d)",
                         hipGetErrorString(e), (int)e);
                return fa::record_error(FA_EHIP, msg);
            }
            g_scratch[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return FA_OK;
}

bool ptr_ok(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" size_t fa_bwd_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

extern "C" fa_status_t fa_bwd_noalloc(const fa_params_t *p, const void *q, const void *k,
                                      const void *v, const void *o, const float *lse,
                                      const void *dout, void *dq, void *dk, void *dv,
                                      void *stream) {
    const size_t need = fa_bwd_workspace_bytes(p);
    // Invalid parameters or an empty problem: fa_bwd reports them (or
    // returns FA_OK) before it looks at the workspace.
    if (need == (size_t)-1 || need == 0)
        return fa_bwd(p, q, k, v, o, lse, dout, dq, dk, dv, nullptr, 0, stream);
    const void *ptrs[9] = {q, k, v, o, lse, dout, dq, dk, dv};
    static const char *names[9] = {"q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv"};
    for (int i = 0; i < 9; ++i) {
        if (!ptr_ok(ptrs[i])) {
            char msg[96];
            snprintf(msg, sizeof msg, "%s is NULL or not 16-byte aligned", names[i]);
            return fa::record_error(FA_EINVAL, msg);
        }
    }
    if (need > kScratchBytes) {
        char msg[200];
        snprintf(msg, sizeof msg,
                 "fa_bwd_noalloc: the row statistics need %zu bytes, beyond the static scratch of "
                 "%zu bytes (B*H*N <= 4194304); use fa_bwd with a workspace",
                 need, kScratchBytes);
        return fa::record_error(FA_EINVAL, msg);
    }
    void *ws = nullptr;
    const fa_status_t s = scratch_address(&ws);
    if (s != FA_OK) return s;
    return fa_bwd(p, q, k, v, o, lse, dout, dq, dk, dv, ws, kScratchBytes, stream);
}
