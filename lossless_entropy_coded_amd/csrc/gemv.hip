// gemv.hip -- batch-1 bf16 matrix-vector product on gfx950, the consumer that
// decoded weights feed: the pages decode weights on demand for the compute
// kernels that read them (DFloat11 page, abstract: GPU inference on the
// decompressed weights; LazyWeights review, "Truck packing": weights are
// unpacked right before the compute units use them).
//
// y[r] = sum_c W[r][c] * x[c] for a row-major bf16 W (rows x cols), a bf16 x
// and an fp32 y.  A batch-1 product reads every weight once and does two
// flops per weight: it is bound by HBM bandwidth, so it runs on the vector ALUs
// (a matrix-core tile would leave 15 of its 16 columns empty).
//
// Work decomposition: a wave64 owns kRowsPerWave consecutive rows.  Lane l
// takes the 16-byte column chunks l, l + 64, l + 128, ... of those rows (the
// wave's loads of one row cover 1 KB of contiguous memory) and accumulates
// each row in fp32 with fused multiply-adds in a fixed order: chunk by chunk,
// eight columns per chunk in column order.  The 64 lane partials of a row are
// then added by a fixed butterfly (xor 32, 16, 8, 4, 2, 1).  The result is a
// deterministic function of W and x: the same bits decoded from a container
// and read from an uncompressed copy give bit-identical y.  A product of two
// bf16 values is exact in fp32, so only the additions round.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/wc.h"

namespace wc {
namespace {

constexpr uint32_t kGemvLanes = 64;
constexpr uint32_t kRowsPerWave = 4;
constexpr uint32_t kGemvWaves = 4;   // wave64s per workgroup
constexpr uint32_t kUnroll = 2;      // column chunks per lane and step

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// acc += W chunk (8 bf16) . x chunk (8 bf16), column order
__device__ __forceinline__ float dot8(const u32x4& w, const u32x4& x, float acc) {
    acc = __builtin_fmaf(bf16_lo(w.x), bf16_lo(x.x), acc);
    acc = __builtin_fmaf(bf16_hi(w.x), bf16_hi(x.x), acc);
    acc = __builtin_fmaf(bf16_lo(w.y), bf16_lo(x.y), acc);
    acc = __builtin_fmaf(bf16_hi(w.y), bf16_hi(x.y), acc);
    acc = __builtin_fmaf(bf16_lo(w.z), bf16_lo(x.z), acc);
    acc = __builtin_fmaf(bf16_hi(w.z), bf16_hi(x.z), acc);
    acc = __builtin_fmaf(bf16_lo(w.w), bf16_lo(x.w), acc);
    acc = __builtin_fmaf(bf16_hi(w.w), bf16_hi(x.w), acc);
    return acc;
}

__global__ __launch_bounds__(kGemvLanes * kGemvWaves) void gemv_bf16_kernel(const uint16_t* __restrict__ W,
                                                                           const uint16_t* __restrict__ x,
                                                                           float* __restrict__ y, uint32_t rows,
                                                                           uint32_t cols) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint64_t r0 = ((uint64_t)blockIdx.x * kGemvWaves + wave) * kRowsPerWave;
    if (r0 >= rows) return;
    const uint32_t chunks = cols / 8;   // 16-byte column chunks per row
    const u32x4* const xv = reinterpret_cast<const u32x4*>(x);
    const u32x4* wrow[kRowsPerWave];
#pragma unroll
    for (uint32_t i = 0; i < kRowsPerWave; ++i) {
        const uint64_t r = r0 + i < rows ? r0 + i : rows - 1;   // rows past the end repeat the last (not stored)
        wrow[i] = reinterpret_cast<const u32x4*>(W + r * cols);
    }
    float acc[kRowsPerWave];
#pragma unroll
    for (uint32_t i = 0; i < kRowsPerWave; ++i) acc[i] = 0.0f;

    const uint32_t step = kGemvLanes * kUnroll;
    uint32_t c = lane;
    for (; c + (kUnroll - 1) * kGemvLanes < chunks; c += step) {
        u32x4 xs[kUnroll], ws[kUnroll][kRowsPerWave];
#pragma unroll
        for (uint32_t u = 0; u < kUnroll; ++u) {
            xs[u] = xv[c + u * kGemvLanes];
#pragma unroll
            for (uint32_t i = 0; i < kRowsPerWave; ++i)
                ws[u][i] = __builtin_nontemporal_load(wrow[i] + c + u * kGemvLanes);
        }
#pragma unroll
        for (uint32_t u = 0; u < kUnroll; ++u)
#pragma unroll
            for (uint32_t i = 0; i < kRowsPerWave; ++i) acc[i] = dot8(ws[u][i], xs[u], acc[i]);
    }
    for (; c < chunks; c += kGemvLanes) {
        const u32x4 xs = xv[c];
#pragma unroll
        for (uint32_t i = 0; i < kRowsPerWave; ++i)
            acc[i] = dot8(__builtin_nontemporal_load(wrow[i] + c), xs, acc[i]);
    }
#pragma unroll
    for (uint32_t i = 0; i < kRowsPerWave; ++i) {
        float v = acc[i];
#pragma unroll
        for (uint32_t m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, (int)m, 64);
        if (lane == 0 && r0 + i < rows) y[r0 + i] = v;
    }
}

}  // namespace
}  // namespace wc

extern "C" int wc_gemv_bf16_async(const uint16_t* W, uint32_t rows, uint32_t cols, const uint16_t* x, float* y,
                                  void* stream) {
    if (rows == 0) return WC_OK;
    if (!W || !x || !y || cols == 0 || cols % 8 != 0) return WC_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(W) & 15u) || (reinterpret_cast<uintptr_t>(x) & 15u) ||
        (reinterpret_cast<uintptr_t>(y) & 3u))
        return WC_ERR_INVALID_ARG;
    const uint64_t rows_per_block = (uint64_t)wc::kRowsPerWave * wc::kGemvWaves;
    const uint64_t grid = (rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL(wc::gemv_bf16_kernel, dim3((uint32_t)grid), dim3(wc::kGemvLanes * wc::kGemvWaves), 0,
                       static_cast<hipStream_t>(stream), W, x, y, rows, cols);
    return hipGetLastError() == hipSuccess ? WC_OK : WC_ERR_HIP;
}
