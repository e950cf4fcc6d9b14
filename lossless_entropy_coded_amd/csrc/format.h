// format.h -- container layouts shared by the host encoder, the planner and
// the device decoder of libwc: version 2 (per-chunk gaps and a group table)
// and version 3 (interleaved lanes).  (The CPU oracle keeps its own
// restatement.)
#pragma once

#include <cstdint>
#include <cstring>

namespace wc {

constexpr uint32_t kMagic = 0x46424357u;   // bytes "WCBF"
constexpr uint16_t kVersion = 2;
constexpr uint32_t kHeaderBytes = 256;
constexpr uint32_t kAlign = 256;
constexpr uint32_t kMaxCodeLen = 24;       // longest code the format allows
constexpr uint32_t kChunkBits = 64;        // one 8-byte chunk per decoding lane
constexpr uint32_t kDefaultGroup = 128;    // chunks per group: one wave64 unit, two chunks per lane
constexpr uint32_t kDefaultAlign = 128;    // elements per block: groups start at multiples of it
constexpr uint32_t kDefaultMaxElems = 4096; // elements a group may hold at most
constexpr uint32_t kStreamSlack = 16;      // zero bytes after the last chunk
// Version 2 gap widths: one byte per chunk, or 5 bits per chunk (every gap is
// below the longest code, at most 23): gap c in bits 5c .. 5c + 4 of the
// section read as a little-endian bit string; header byte 10 holds 0 or 5.
constexpr uint32_t kGapBitsByte = 8;
constexpr uint32_t kGapBitsPacked = 5;

// Version 3, the interleaved-lane layout: per segment (a run of whole blocks),
// 8-element lane blocks are dealt to 64 lanes (lane j: lane blocks j, j + 64,
// ...); each lane's codewords are contiguous, lanes follow each other, and a
// u16 per lane gives its first bit relative to the segment's.
constexpr uint16_t kVersionLanes = 3;
constexpr uint32_t kLanes = 64;
constexpr uint32_t kLaneBlock = 8;
constexpr uint32_t kLanesSlack = 64;       // zero bytes after the 8-byte-padded stream
constexpr uint32_t kDefaultSegBits = 15872;   // stream bits per segment at most (1984 bytes)
// Element kinds of a version-3 container: bf16 words (the exponent coded, the
// sign+mantissa byte raw) or bytes (each byte coded, no raw plane: planes of
// quantized integer codes).
constexpr uint32_t kKindBf16 = 0;
constexpr uint32_t kKindU8 = 1;
// Default code length limit of u8-kind (code plane) containers: the GPU
// decoder's table index width, so that no code takes its slower long-code
// path.  Wide alphabets of quantized codes have many long codes otherwise
// (about 0.4% of int8 codes of spread 20 exceed 11 bits); the limit costs
// them 0.3-0.6% in size.  bf16 exponents keep kMaxCodeLen.
constexpr uint32_t kDefaultCodeLenU8 = 11;
// Coders of a version-3 container: the canonical Huffman code, or rANS
// (Llama2-7B page, abstract: ANS; the LazyWeights page compares the two).
// rANS: kRansBits-bit quantized frequencies (u16[256] in place of the code
// lengths, summing to 2^kRansBits), a 32-bit state kept in [kRansLow, 2^32),
// 16-bit renormalisation words; a lane's string is its final state (two
// words, high first) followed by the words its decoder reads, each
// big-endian, and is empty for a lane with no symbols.
constexpr uint32_t kCoderHuffman = 0;
constexpr uint32_t kCoderRans = 1;
constexpr uint32_t kRansBits = 12;
constexpr uint32_t kRansLow = 1u << 16;
constexpr uint32_t kRansStateBits = 32;    // the final state every non-empty lane string starts with

// Header field offsets (little-endian).
struct HeaderOffsets {
    static constexpr int magic = 0, version = 4, flags = 6, max_code_len = 8, chunk_bits = 9,
                         gap_bits = 10, reserved0 = 11, chunks_per_group = 12, n_tensors = 16, group_align = 20,
                         n_elems = 24, stream_bits = 32, n_chunks = 40, n_groups = 48,
                         off_code_len = 56, off_tensors = 64, off_groups = 72, off_gap = 80,
                         off_stream = 88, stream_bytes = 96, off_sm = 104, total_bytes = 112,
                         group_max_elems = 120, elem_kind = 124, coder = 125, reserved_tail = 126;
    // version 3 reuses the positions: lanes at 9, lane block at 10, the
    // segment bit cap at 12, the lane offsets at off_gap; n_chunks is 0
    static constexpr int lanes = 9, lane_block = 10, seg_max_bits = 12;
};

struct Header {
    uint32_t version = kVersion;   // kVersion or kVersionLanes
    uint32_t seg_max_bits = 0;     // version 3
    uint32_t elem_kind = kKindBf16;   // version 3: kKindBf16 or kKindU8
    uint32_t coder = kCoderHuffman;   // version 3: kCoderHuffman or kCoderRans
    uint32_t gap_bits = kGapBitsByte;  // version 2: kGapBitsByte or kGapBitsPacked
    uint32_t max_code_len = 0, chunks_per_group = 0, n_tensors = 0, group_align = 0, group_max_elems = 0;
    uint64_t n_elems = 0, stream_bits = 0, n_chunks = 0, n_groups = 0;
    uint64_t off_code_len = 0, off_tensors = 0, off_groups = 0, off_gap = 0, off_stream = 0,
             stream_bytes = 0, off_sm = 0, total_bytes = 0;
};

inline uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
inline uint64_t div_up(uint64_t x, uint64_t a) { return (x + a - 1) / a; }

template <typename T>
inline T load_le(const uint8_t* p) {
    T v;
    std::memcpy(&v, p, sizeof(T));   // x86-64 and gfx950 hosts are little-endian
    return v;
}
template <typename T>
inline void store_le(uint8_t* p, T v) {
    std::memcpy(p, &v, sizeof(T));
}

// Bytes of one entry of the groups section: u64 first element, u64 its bit.
constexpr uint32_t kGroupEntryBytes = 16;

// Bytes of a version-2 gap section.
inline uint64_t gap_section_bytes(uint64_t n_chunks, uint32_t gap_bits) {
    return gap_bits == kGapBitsPacked ? div_up(5 * n_chunks, 8) : n_chunks;
}

// Chunks touched by the stream bits [p, q), q > p.
inline uint64_t chunk_span(uint64_t p, uint64_t q) { return (q - 1) / kChunkBits - p / kChunkBits + 1; }

// Section placement for a container with the given sizes.
inline Header layout(uint64_t n_elems, uint64_t stream_bits, uint32_t n_tensors, uint32_t max_code_len,
                     uint32_t group, uint32_t align, uint32_t max_elems, uint64_t n_groups,
                     uint32_t gap_bits = kGapBitsByte) {
    Header h;
    h.gap_bits = gap_bits;
    h.max_code_len = max_code_len;
    h.chunks_per_group = group;
    h.group_align = align;
    h.group_max_elems = max_elems;
    h.n_tensors = n_tensors;
    h.n_elems = n_elems;
    h.stream_bits = stream_bits;
    h.n_chunks = div_up(stream_bits, kChunkBits);
    h.n_groups = n_groups;
    h.stream_bytes = h.n_chunks * 8 + kStreamSlack;
    h.off_code_len = kHeaderBytes;
    h.off_tensors = round_up(h.off_code_len + 256, kAlign);
    h.off_groups = round_up(h.off_tensors + 16ull * n_tensors, kAlign);
    h.off_gap = round_up(h.off_groups + kGroupEntryBytes * (h.n_groups + 1), kAlign);
    h.off_stream = round_up(h.off_gap + gap_section_bytes(h.n_chunks, gap_bits), kAlign);
    h.off_sm = round_up(h.off_stream + h.stream_bytes, kAlign);
    h.total_bytes = round_up(h.off_sm + n_elems, kAlign);
    return h;
}

// Bytes of the code section: code lengths (u8) or rANS frequencies (u16).
inline uint64_t code_section_bytes(uint32_t coder) { return coder == kCoderRans ? 512 : 256; }

// Section placement of a version-3 (interleaved-lane) container; the lane
// offsets take the place of the gaps (off_gap).  For rANS, max_code_len is
// kRansBits.
inline Header layout_lanes(uint64_t n_elems, uint64_t stream_bits, uint32_t n_tensors, uint32_t max_code_len,
                           uint32_t align, uint32_t max_elems, uint32_t seg_max_bits, uint64_t n_segs,
                           uint32_t elem_kind = kKindBf16, uint32_t coder = kCoderHuffman) {
    Header h;
    h.version = kVersionLanes;
    h.elem_kind = elem_kind;
    h.coder = coder;
    h.seg_max_bits = seg_max_bits;
    h.max_code_len = max_code_len;
    h.group_align = align;
    h.group_max_elems = max_elems;
    h.n_tensors = n_tensors;
    h.n_elems = n_elems;
    h.stream_bits = stream_bits;
    h.n_chunks = 0;
    h.n_groups = n_segs;
    h.stream_bytes = round_up(div_up(stream_bits, 8), 8) + kLanesSlack;
    h.off_code_len = kHeaderBytes;
    h.off_tensors = round_up(h.off_code_len + code_section_bytes(coder), kAlign);
    h.off_groups = round_up(h.off_tensors + 16ull * n_tensors, kAlign);
    h.off_gap = round_up(h.off_groups + kGroupEntryBytes * (n_segs + 1), kAlign);
    h.off_stream = round_up(h.off_gap + 2ull * kLanes * n_segs, kAlign);
    h.off_sm = round_up(h.off_stream + h.stream_bytes, kAlign);
    h.total_bytes = round_up(h.off_sm + (elem_kind == kKindBf16 ? n_elems : 0), kAlign);
    return h;
}

inline void write_header(uint8_t* p, const Header& h) {
    using O = HeaderOffsets;
    std::memset(p, 0, kHeaderBytes);
    store_le<uint32_t>(p + O::magic, kMagic);
    store_le<uint16_t>(p + O::version, (uint16_t)h.version);
    store_le<uint8_t>(p + O::max_code_len, (uint8_t)h.max_code_len);
    if (h.version == kVersionLanes) {
        store_le<uint8_t>(p + O::lanes, (uint8_t)kLanes);
        store_le<uint16_t>(p + O::lane_block, (uint16_t)kLaneBlock);
        store_le<uint32_t>(p + O::seg_max_bits, h.seg_max_bits);
        store_le<uint8_t>(p + O::elem_kind, (uint8_t)h.elem_kind);
        store_le<uint8_t>(p + O::coder, (uint8_t)h.coder);
    } else {
        store_le<uint8_t>(p + O::chunk_bits, (uint8_t)kChunkBits);
        store_le<uint8_t>(p + O::gap_bits, (uint8_t)(h.gap_bits == kGapBitsPacked ? kGapBitsPacked : 0));
        store_le<uint32_t>(p + O::chunks_per_group, h.chunks_per_group);
    }
    store_le<uint32_t>(p + O::n_tensors, h.n_tensors);
    store_le<uint32_t>(p + O::group_align, h.group_align);
    store_le<uint32_t>(p + O::group_max_elems, h.group_max_elems);
    store_le<uint64_t>(p + O::n_elems, h.n_elems);
    store_le<uint64_t>(p + O::stream_bits, h.stream_bits);
    store_le<uint64_t>(p + O::n_chunks, h.n_chunks);
    store_le<uint64_t>(p + O::n_groups, h.n_groups);
    store_le<uint64_t>(p + O::off_code_len, h.off_code_len);
    store_le<uint64_t>(p + O::off_tensors, h.off_tensors);
    store_le<uint64_t>(p + O::off_groups, h.off_groups);
    store_le<uint64_t>(p + O::off_gap, h.off_gap);
    store_le<uint64_t>(p + O::off_stream, h.off_stream);
    store_le<uint64_t>(p + O::stream_bytes, h.stream_bytes);
    store_le<uint64_t>(p + O::off_sm, h.off_sm);
    store_le<uint64_t>(p + O::total_bytes, h.total_bytes);
}

}  // namespace wc
