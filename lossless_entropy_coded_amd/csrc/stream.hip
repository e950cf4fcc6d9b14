// stream.hip -- the streaming yardstick the decode kernels are measured
// against: the simplest kernel that reads R bytes from HBM once and writes
// W >= R bytes, as a decode of a container of R bytes into W bytes of weights
// does.  It does no decoding: each 16-byte item of the output is the bitwise
// NOT of one 16-byte item of the input, and every input item is read.
//
// Its launch shape is the fastest measured on MI355X for such a mix of reads
// and writes: one workgroup of 256 lanes per 4 KiB of output, each lane one
// non-temporal 16-byte load and one non-temporal 16-byte store.  Workgroups
// are dispatched in index order and retire quickly, so the accesses in flight
// always lie in a narrow, advancing window of both buffers; persistent
// workgroups that each stream a long range (or walk strided units) leave more
// DRAM rows open at once and were measurably slower, most of all for the
// writes.
//
// Mapping: with ns input items and nd >= ns output items, output item j takes
// input item floor(j * r / 2^32), r = ceil(ns * 2^32 / nd) <= 2^32.  Adjacent
// j map to the same or the next input item, so no input item is skipped, and
// the last output item maps to input item ns - 1 (clamped against rounding).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/wc.h"

namespace wc {
namespace {

constexpr uint32_t kStreamLanes = 256;   // lanes per workgroup: 4 KiB of output

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kStreamLanes) void stream_reference_kernel(const u32x4* __restrict__ src, uint64_t ns,
                                                                        u32x4* __restrict__ dst, uint64_t nd,
                                                                        uint64_t r) {
    const uint64_t j = (uint64_t)blockIdx.x * kStreamLanes + threadIdx.x;
    if (j >= nd) return;
    uint64_t i = (j * r) >> 32;   // j < 2^39 and r <= 2^32: no overflow
    i = i < ns - 1 ? i : ns - 1;
    const u32x4 v = __builtin_nontemporal_load(src + i);
    __builtin_nontemporal_store(~v, dst + j);
}

}  // namespace
}  // namespace wc

extern "C" int wc_stream_reference_async(const void* src, uint64_t src_bytes, void* dst, uint64_t dst_bytes,
                                         void* stream) {
    if (dst_bytes == 0 && src_bytes == 0) return WC_OK;
    if (!src || !dst || src_bytes == 0 || src_bytes % 16 || dst_bytes % 16 || src_bytes > dst_bytes)
        return WC_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u))
        return WC_ERR_INVALID_ARG;
    const uint64_t ns = src_bytes / 16, nd = dst_bytes / 16;
    const uint64_t grid = (nd + wc::kStreamLanes - 1) / wc::kStreamLanes;
    if (nd >= (1ull << 39) || grid > 0x7FFFFFFFull) return WC_ERR_INVALID_ARG;
    // r = ceil(ns * 2^32 / nd) without overflow: ns <= nd < 2^39
    const uint64_t q = ns / nd, rem = ns % nd;   // q is 1 when ns == nd, else 0
    const uint64_t r = (q << 32) + (((unsigned __int128)rem << 32) + nd - 1) / nd;
    hipLaunchKernelGGL(wc::stream_reference_kernel, dim3((uint32_t)grid), dim3(wc::kStreamLanes), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<const wc::u32x4*>(src), ns,
                       reinterpret_cast<wc::u32x4*>(dst), nd, r);
    return hipGetLastError() == hipSuccess ? WC_OK : WC_ERR_HIP;
}
