// kernels.h -- internal interface between the planner (plan.cpp) and the
// gfx950 kernels (decode.hip).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

struct wc_plan_s;

namespace wc {

constexpr uint32_t kWaveLanes = 64;        // lanes of a wavefront
constexpr uint32_t kChunksPerLane = 2;     // each lane decodes two adjacent 64-bit chunks
constexpr uint32_t kGroupChunks = kWaveLanes * kChunksPerLane;   // chunks per group G: one wave's unit
constexpr uint32_t kSingleBits = 12;       // width of the build-time single-codeword table
constexpr uint32_t kEbufSlack = 3;         // bytes a chain may write past its range (then rewritten)
constexpr uint32_t kHeadBytes = 3;         // leading bytes of a chain that a left neighbour may overwrite
constexpr uint32_t kMergeElems = 8;        // elements per lane per merge step (one 16-byte bf16 store)
constexpr uint32_t kMergeSteps = 8;        // merge steps per lane and group
constexpr uint32_t kGroupMaxElems = kWaveLanes * kMergeSteps * kMergeElems;   // 4096 elements per group at most

// Device decode tables, as 32-bit words, for index widths KC (counting) and KD (decoding):
//   [0, 2^KC)                codeword-start table: for a KC-bit window,
//                              bits 0..4   (32 - adv) & 31      (funnel-shift amount)
//                              bits 8..15  adv = bits covered by the whole codewords in the window
//                              bits 16..31 mask of the offsets where those codewords start
//                            0 when the first codeword is longer than KC bits;
//   [2^KC, 2^KC + 2*2^KD)    multi-codeword table, two words per KD-bit window, up to four
//                            whole codewords:
//                              word 0: bits 0..4 (32 - nbits) & 31, bits 8..15 number of
//                                      symbols n (1..4), bits 16..23 nbits
//                              word 1: the n symbols, first in the lowest byte
//                            word 0 is 0 when the first codeword is longer than KD bits;
//   then 32 words count[L], 32 words first[L] (canonical first code of length L),
//   32 words base[L] (rank of the first symbol of length L), 64 words holding the
//   256 symbols sorted by (length, symbol) -- used for codes longer than the index;
//   then F (the KD-bit prefix of the first code longer than KD), np (the number of
//   long-code prefixes the second level covers, at most kL2Prefixes) and two zero
//   words; then the second level: kL2Prefixes * 2^kL2Bits u16 entries, entry
//   (p - F) * 2^kL2Bits + b for the (KD + kL2Bits)-bit window (p, b) holding
//   (length << 8) | rotated symbol of its first codeword, or 0 when that code is
//   longer than KD + kL2Bits bits.
// Symbols in the multi-codeword and sorted tables are stored rotated right by one
// bit, e' = (e >> 1) | (e & 1) << 7: e' & 0x7F is the exponent's part of the bf16
// high byte and e' & 0x80 its part of the low byte.
constexpr uint32_t kLongWords = 164;       // count, first, base, sorted symbols, then F, np, 0, 0
constexpr uint32_t kL2Bits = 8;            // second-level index: bits after the KD-bit prefix
constexpr uint32_t kL2Prefixes = 3;        // long-code prefixes the second level covers
inline uint32_t table_words(uint32_t count_bits, uint32_t decode_bits) {
    return (1u << count_bits) + (2u << decode_bits) + kLongWords + (kL2Prefixes << kL2Bits) / 2;
}
inline bool supported_table_bits(uint32_t count_bits, uint32_t decode_bits) {
    return (count_bits == 12 && (decode_bits == 11 || decode_bits == 10)) ||
           (count_bits == 11 && (decode_bits == 11 || decode_bits == 10)) ||
           (count_bits == 10 && decode_bits == 10);
}

struct CodeLens {
    uint8_t len[256];
};

// Fused decode -> matrix-vector products over consecutive matrices of a
// container (one launch for all of them): the elements [bounds[0],
// bounds[n_mats]) are the matrices back to back, matrix k in rows of cols[k]
// starting at element bounds[k]; its rows are the global rows row_base[k] ..
// Every cols[k] is a multiple of 8 and at least the largest group, so a group
// touches at most two consecutive global rows: the row holding its first
// element inside the range and the next.
constexpr uint32_t kMaxDotMats = 16;

// Division by an invariant divisor 1 < d < 2^31 through a multiply (the
// round-up method of Granlund and Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994, section 4): with l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1 and t = floor(m n / 2^32),
// floor(n / d) = (t + ((n - t) >> 1)) >> (l - 1) for every n < 2^32.
inline void div_magic_params(uint32_t d, uint32_t& magic, uint32_t& shift) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    magic = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    shift = l - 1;
}
struct DotParams {
    uint64_t bounds[kMaxDotMats + 1];
    uint64_t row_base[kMaxDotMats + 1];   // row_base[n_mats] = total rows
    const uint16_t* x[kMaxDotMats];       // cols[k] bf16 each, 16-byte aligned
    float* y[kMaxDotMats];                // rows of matrix k, fp32
    uint32_t cols[kMaxDotMats];           // < 2^31; every matrix holds < 2^32 elements
    uint32_t magic[kMaxDotMats];          // e / cols[k] = div_magic(e, magic[k], shift[k]) for e < 2^32
    uint32_t shift[kMaxDotMats];
    uint32_t n_mats;
    uint32_t rows;                        // total rows
    float* part;        // per group g: part[2(g - u_begin)] for its first row, part[2(g - u_begin) + 1] for the next
    uint32_t* row_group;  // per global row r: the first group (minus u_begin) whose first row is r
};

struct DecodeParams {
    const uint8_t* stream;
    const uint8_t* gap;
    const uint64_t* groups;  // {first element, first bit} per group, n_groups + 1 entries
    const uint8_t* sm;
    uint16_t* out;           // decoded bf16 (decode launches)
    uint8_t* out8;           // decoded bytes (u8-kind lanes launches)
    const uint32_t* tables;
    uint64_t n_elems;
    uint64_t u_begin;        // groups [u_begin, u_end) are decoded, one per wave
    uint64_t u_end;
    uint32_t ebuf_bytes;     // exponent staging bytes per wave
    uint32_t l2_cap;         // long-code prefixes staged in LDS (0 .. kL2Prefixes)
    uint32_t gap_packed;     // chunks layout: gaps stored in 5 bits (else one byte each)
    uint32_t one_code;       // lanes layout, Huffman: one code per table entry at most, all <= 16 bits
    uint32_t no_long;        // Huffman: no code is longer than the multi-codeword table's index
    uint32_t* status;        // debug plans: invariant failures are OR-ed in here (else null)
    DotParams dot;           // fused matrix-vector launches only
};

// Interleaved-lane containers (version 3): each wave stages a segment's
// stream window (its bits, the first bit's 16-byte alignment and 8 bytes of
// lookahead) in kLaneStageBytes of LDS, then the exponent bytes, one
// kLaneSlotBytes slot per lane (its at most 64 symbols and the up to three
// bytes a four-symbol lookup may write past them: 68 bytes, 17 dwords, an odd
// stride, so that lanes at equal offsets use 64 different banks; slots are
// accessed as bytes and dwords); a segment therefore holds at most
// kLanesMaxSegBits stream bits.
constexpr uint32_t kLaneStageBytes = 2048;
constexpr uint32_t kLaneSlotBytes = 68;
// Each wave's region starts with kLanePadBytes that nothing writes: a window
// read at bit position 0 takes the word before the staging (and discards it).
constexpr uint32_t kLanePadBytes = 16;
constexpr uint32_t kLaneWaveBytes = kLanePadBytes + kLaneStageBytes + kWaveLanes * kLaneSlotBytes;
// Code planes with one code per table entry write their bytes straight to
// memory and need no slots: a wave's region is the pad, the staging and 128
// bytes a lane's last 64-bit windows may read past the staging.  Other code
// planes take the wide table (up to three codes per lookup, up to four
// lookups per window) in two phases of 32 symbols sharing a 36-byte slot (9
// dwords, odd): a lookup starts below its phase's 32nd symbol, so it stores
// up to byte 35.
constexpr uint32_t kLaneCompactWaveBytes = kLanePadBytes + kLaneStageBytes + 128;
constexpr uint32_t kWidePhase = 32;                 // symbols per lane and phase on the wide table
constexpr uint32_t kLaneWideSlotBytes = kWidePhase + 4;
constexpr uint32_t kLaneWideWaveBytes = kLanePadBytes + kLaneStageBytes + kWaveLanes * kLaneWideSlotBytes;
enum LaneLds : uint32_t { kLdsSlots = 0, kLdsCompact = 1, kLdsWide = 2 };
inline uint32_t lane_wave_bytes(LaneLds layout) {
    return layout == kLdsCompact ? kLaneCompactWaveBytes : layout == kLdsWide ? kLaneWideWaveBytes : kLaneWaveBytes;
}
constexpr uint32_t kLanesMaxSegBits = 15872;

// Wavefronts per decode workgroup the kernels are built for.
inline bool supported_waves(uint32_t waves) { return waves == 4 || waves == 8; }

// LDS bytes of one decode workgroup of `waves` wavefronts: static tables plus
// the dynamic part (each wave's exponent staging and l2_cap second-level prefixes).
uint32_t decode_dyn_lds_bytes(uint32_t waves, uint32_t ebuf_bytes, uint32_t l2_cap);
uint32_t decode_lds_bytes(uint32_t count_bits, uint32_t decode_bits, uint32_t waves, uint32_t ebuf_bytes,
                          uint32_t l2_cap);

// Resident decode workgroups per compute unit by the runtime's estimate (0 on error).
int decode_blocks_per_cu(uint32_t count_bits, uint32_t decode_bits, uint32_t waves, uint32_t ebuf_bytes,
                         uint32_t l2_cap);

// Build the decode tables of `lens` into d_tables (table_words(...) words) on `stream`.
hipError_t launch_build_tables(const CodeLens& lens, uint32_t count_bits, uint32_t decode_bits, uint32_t* d_tables,
                               hipStream_t stream);

// One launch decoding groups [p.u_begin, p.u_end) (p.ebuf_bytes and p.l2_cap set
// the dynamic LDS): to bf16 in p.out, or (dot) to partial dot products in p.work.
hipError_t launch_decode(const DecodeParams& p, uint32_t count_bits, uint32_t decode_bits, uint32_t waves,
                         uint32_t grid, bool dot, hipStream_t stream);

// Interleaved-lane decode: LDS bytes of one workgroup (decode table index
// width decode_bits, 11 or 10), resident workgroups per CU, and one launch
// decoding segments [p.u_begin, p.u_end) to bf16 in p.out, or (dot) to
// partial dot products in p.dot; p.gap points at the lane offsets and
// p.tables at the multi-codeword table of the plan's tables.
// What a lanes launch produces: bf16 words in p.out (the exponent coded,
// joined with the sign+mantissa plane), partial dot products in p.dot, or
// the decoded bytes themselves in p.out8 (u8-kind containers).
// With rans, the lanes are rANS streams and p.tables holds the 2^12-entry
// slot table in the multi-codeword table's place (decode_bits must be 11):
// entry t = rotated symbol | (f mod 2^12) << 8 | (t - cum) << 20 (f = 2^12,
// stored as 0, only when one symbol has every slot).
enum LanesOut : uint32_t { kLanesToBf16 = 0, kLanesToDot = 1, kLanesToU8 = 2 };
// layout: the per-wave LDS region (kLdsSlots for bf16, rANS and the fused
// product; kLdsCompact or kLdsWide for Huffman code planes).
uint32_t decode_lanes_dyn_lds_bytes(uint32_t waves, uint32_t l2_cap, LaneLds layout = kLdsSlots);
uint32_t decode_lanes_lds_bytes(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap, LaneLds layout = kLdsSlots);
int decode_lanes_blocks_per_cu(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap, bool rans,
                               LaneLds layout = kLdsSlots);
hipError_t launch_decode_lanes(const DecodeParams& p, uint32_t decode_bits, uint32_t waves, uint32_t grid,
                               LanesOut mode, bool rans, hipStream_t stream);

// The HIP device a plan was made for.
int plan_device(const wc_plan_s* plan);

// The fused product of a Huffman lanes container: LDS bytes of one workgroup,
// resident workgroups per CU, and one launch over segments [p.u_begin,
// p.u_end) leaving partial dot products in p.dot (p.gap at the lane offsets,
// p.tables at the multi-codeword table, as for launch_decode_lanes).
uint32_t decode_lanes_dot_lds_bytes(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap);
int decode_lanes_dot_blocks_per_cu(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap);
hipError_t launch_decode_lanes_dot(const DecodeParams& p, uint32_t decode_bits, uint32_t waves, uint32_t grid,
                                   hipStream_t stream);

// One launch adding, for every global row of p.dot, the partial dot products
// of the groups covering it, in group order, into the row's y.
hipError_t launch_gemv_rows(const DecodeParams& p, hipStream_t stream);

}  // namespace wc
