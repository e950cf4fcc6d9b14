// kernels.h -- internal interface between the planner (plan.cpp) and the
// gfx950 kernels (decode.hip).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace wc {

constexpr uint32_t kDecodeThreads = 256;   // one 64-bit chunk per lane, G = 256 chunks per group
constexpr uint32_t kMinLutBits = 10;
constexpr uint32_t kMaxLutBits = 12;

// Decode tables, as 32-bit words, for a first-level index of K bits:
//   [0, 2^K)            single-codeword table, one entry per K-bit window:
//                         bits 0..4  (32 - len) & 31   (the funnel-shift amount)
//                         bits 8..12 len
//                         bits 16..23 symbol
//                         bit 31      set when the window starts a code longer than K
//   [2^K, 2^(K+1))      codeword-start table for the counting phase:
//                         bits 0..4  (32 - adv) & 31, bits 8..12 adv,
//                         bits 16..16+K-1 mask of codeword starts inside the window
//                         (adv = bits covered by the codewords that fit; 0 when none fits)
//   then 32 words count[L], 32 words first[L] (canonical first code of length L),
//   32 words base[L] (rank of the first symbol of length L), 64 words holding the
//   256 symbols sorted by (length, symbol).
inline uint32_t table_words(uint32_t lut_bits) { return (2u << lut_bits) + 160u; }

struct CodeLens {
    uint8_t len[256];
};

struct DecodeParams {
    const uint8_t* stream;
    const uint8_t* gap;
    const uint64_t* group_start;
    const uint8_t* sm;
    uint16_t* out;
    const uint32_t* tables;
    uint64_t n_chunks;
    uint64_t stream_bits;
    uint64_t n_groups;
    uint32_t ebuf_bytes;
    uint32_t pad;
};

// Dynamic LDS bytes of one decode workgroup.
uint32_t decode_lds_bytes(uint32_t lut_bits, uint32_t ebuf_bytes);

// Resident decode workgroups per compute unit for that LDS size (0 on error).
int decode_blocks_per_cu(uint32_t lut_bits, uint32_t lds_bytes);

// Build the decode tables of `lens` into d_tables (table_words(lut_bits) words) on `stream`.
hipError_t launch_build_tables(const CodeLens& lens, uint32_t lut_bits, uint32_t* d_tables, hipStream_t stream);

// One launch decoding every group of a container.
hipError_t launch_decode(const DecodeParams& p, uint32_t lut_bits, uint32_t grid, uint32_t lds_bytes,
                         hipStream_t stream);

}  // namespace wc
