// Host stand-ins for the GPU side of libwc, for the sanitizer build of the
// encoder and planner (tests/test_host_sanitizers.py): the HIP runtime calls
// the planner makes (device memory is host memory here) and the kernel-side
// entry points of kernels.h.  Every launch entry point checks that the
// parameters it was handed point inside the container the test passed as
// the "device" copy, and counts the launch; nothing is decoded.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../lossless_entropy_coded_amd/csrc/kernels.h"
#include "stub_state.h"

StubState g_stub;

namespace {

bool inside(const void* p, uint64_t bytes) {
    const uint8_t* b = static_cast<const uint8_t*>(p);
    return b >= g_stub.lo && b <= g_stub.hi && bytes <= (uint64_t)(g_stub.hi - b);
}

void fail(const char* what) {
    std::fprintf(stderr, "stub check failed: %s\n", what);
    std::abort();
}

void check_common(const wc::DecodeParams& p, uint32_t waves, uint32_t grid) {
    g_stub.last_no_long = p.no_long;
    g_stub.last_one_code = p.one_code;
    g_stub.last_status = p.status;
    if (!wc::supported_waves(waves)) fail("waves");
    if (grid == 0) fail("empty grid");
    if (p.u_begin >= p.u_end) fail("empty group range");
    if (!g_stub.lo) return;   // no container range to check against
    // the group table: entries u_begin .. u_end (16 bytes each)
    if (!inside(p.groups + 2 * p.u_begin, 16 * (p.u_end - p.u_begin + 1))) fail("group table outside the container");
    if (!inside(p.stream, 0) || !inside(p.gap, 0)) fail("stream or gap section outside the container");
    // the last group's bits lie inside the stream section
    const uint64_t end_bit = p.groups[2 * p.u_end + 1];
    if (!inside(p.stream, (end_bit + 7) / 8)) fail("stream bits outside the container");
}

}  // namespace

extern "C" {
hipError_t hipSetDevice(int d) { return d == 0 ? hipSuccess : hipErrorInvalidDevice; }
hipError_t hipGetDevice(int* d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t a, int d) {
    if (d != 0) return hipErrorInvalidDevice;
    *v = a == hipDeviceAttributeMultiprocessorCount ? 256 : 160 * 1024;
    return hipSuccess;
}
hipError_t hipMalloc(void** p, size_t n) {
    *p = std::malloc(n ? n : 1);
    ++g_stub.live_allocs;
    return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* p) {
    if (p) --g_stub.live_allocs;
    std::free(p);
    return hipSuccess;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
    std::memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipMemset(void* dst, int v, size_t n) {
    std::memset(dst, v, n);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipDeviceSynchronize() { return hipSuccess; }
}

namespace wc {

uint32_t decode_dyn_lds_bytes(uint32_t waves, uint32_t ebuf_bytes, uint32_t l2_cap) {
    return waves * (ebuf_bytes + 64) + (l2_cap << kL2Bits) * 2;
}
uint32_t decode_lds_bytes(uint32_t count_bits, uint32_t decode_bits, uint32_t waves, uint32_t ebuf_bytes,
                          uint32_t l2_cap) {
    return table_words(count_bits, decode_bits) * 4 + decode_dyn_lds_bytes(waves, ebuf_bytes, l2_cap);
}
int decode_blocks_per_cu(uint32_t, uint32_t, uint32_t waves, uint32_t, uint32_t) { return waves == 4 ? 3 : 2; }
hipError_t launch_build_tables(const CodeLens&, uint32_t count_bits, uint32_t decode_bits, uint32_t* d_tables,
                               hipStream_t) {
    std::memset(d_tables, 0, (size_t)table_words(count_bits, decode_bits) * 4);
    return hipSuccess;
}
hipError_t launch_decode(const DecodeParams& p, uint32_t, uint32_t, uint32_t waves, uint32_t grid, bool dot,
                         hipStream_t) {
    check_common(p, waves, grid);
    ++g_stub.launches;
    g_stub.dot_launches += dot;
    return hipSuccess;
}
uint32_t decode_lanes_dyn_lds_bytes(uint32_t waves, uint32_t l2_cap, LaneLds layout) {
    return waves * lane_wave_bytes(layout) + (l2_cap << kL2Bits) * 2;
}
uint32_t decode_lanes_lds_bytes(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap, LaneLds layout) {
    return ((2u << decode_bits) + kLongWords) * 4 + decode_lanes_dyn_lds_bytes(waves, l2_cap, layout);
}
int decode_lanes_blocks_per_cu(uint32_t, uint32_t waves, uint32_t, bool, LaneLds) { return waves == 4 ? 3 : 2; }
hipError_t launch_decode_lanes(const DecodeParams& p, uint32_t, uint32_t waves, uint32_t grid, LanesOut mode,
                               bool, hipStream_t) {
    check_common(p, waves, grid);
    ++g_stub.launches;
    g_stub.dot_launches += mode == kLanesToDot;
    return hipSuccess;
}
uint32_t decode_lanes_dot_lds_bytes(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap) {
    return decode_lanes_lds_bytes(decode_bits, waves, l2_cap, kLdsSlots);
}
int decode_lanes_dot_blocks_per_cu(uint32_t, uint32_t, uint32_t) { return 3; }
hipError_t launch_decode_lanes_dot(const DecodeParams& p, uint32_t, uint32_t waves, uint32_t grid, hipStream_t) {
    check_common(p, waves, grid);
    ++g_stub.launches;
    ++g_stub.dot_launches;
    return hipSuccess;
}
hipError_t launch_gemv_rows(const DecodeParams& p, hipStream_t) {
    if (p.dot.n_mats == 0 || p.dot.n_mats > kMaxDotMats) fail("matrix count");
    for (uint32_t k = 0; k < p.dot.n_mats; ++k) {
        if (p.dot.bounds[k] >= p.dot.bounds[k + 1] || p.dot.bounds[k + 1] > p.n_elems) fail("matrix bounds");
        if (p.dot.cols[k] == 0 || p.dot.cols[k] % 8 || (p.dot.bounds[k + 1] - p.dot.bounds[k]) % p.dot.cols[k])
            fail("matrix shape");
        if (p.dot.row_base[k + 1] - p.dot.row_base[k] != (p.dot.bounds[k + 1] - p.dot.bounds[k]) / p.dot.cols[k])
            fail("row bases");
    }
    if (p.dot.rows != p.dot.row_base[p.dot.n_mats]) fail("total rows");
    ++g_stub.launches;
    return hipSuccess;
}

}  // namespace wc
