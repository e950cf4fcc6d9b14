// noalloc.hip -- the fused decode -> matrix-vector products for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// wc_decode_gemv_async takes its work buffer (the per-group partial dot
// products and the first group of every row) from the caller.  This entry
// point uses a file-scope device array instead, `scratch`, of kScratchBytes:
// every GPU the library runs on holds its own copy until the process ends.
// Its device address is looked up once per device, with that device current,
// on the entry point's first call there (hipGetSymbolAddress); after that
// only that address is used.  The call itself allocates nothing.
//
// Every call on one GPU shares that GPU's array, which keeps the last call's
// contents.  Nothing in it has to start at zero: each call writes every
// partial and every row's first group before its second kernel reads them.
// Calls that overlap on one GPU (for instance on two streams) race on the
// array; a caller must order them.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/wc.h"
#include "kernels.h"

namespace {

constexpr uint64_t kScratchBytes = WC_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` on each device, once looked up

// The address of this device's `scratch` (the current device must be `dev`).
int scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return WC_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WC_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return WC_OK;
}

}  // namespace

extern "C" int wc_decode_gemv_noalloc_async(const wc_plan_t* plan, const void* blob_dev, const wc_gemv_operand* ops,
                                            uint32_t n_ops, void* stream) {
    uint64_t need = 0;
    const int st = wc_decode_gemv_work_bytes(plan, ops, n_ops, &need);
    if (st != WC_OK) return st;
    if (need == 0) return WC_OK;                 // every tensor empty: nothing to do
    if (need > kScratchBytes) return WC_ERR_SCRATCH;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return WC_ERR_HIP;
    if (cur != wc::plan_device(plan)) return WC_ERR_INVALID_ARG;
    void* work = nullptr;
    const int sa = scratch_address(cur, &work);
    if (sa != WC_OK) return sa;
    return wc_decode_gemv_async(plan, blob_dev, ops, n_ops, work, need, stream);
}
