// plan.cpp -- container validation, decode planning and the decode entry point
// of libwc.
//
// wc_plan checks every field and section of a container before any kernel
// sees it, so that the decode kernel can trust the auxiliary variables it
// reads (DFloat11 page, abstract, design point (ii)): group starts are
// monotone and end at n, gaps are shorter than the longest code, and the code
// lengths form a complete prefix code.  It then builds the compact decode
// tables on the device (design point (i)) and sizes one persistent launch
// that covers a whole multi-tensor container (design point (iii)).  For an
// rANS container (the Llama2-7B page's ANS) the checks are on the quantized
// frequencies and 16-bit word alignment instead, and the decode table maps
// each of the 2^12 slots to its symbol, frequency and offset.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "format.h"
#include "kernels.h"
#include "../../include/wc.h"

struct wc_plan_s {
    int device = 0;
    wc::Header h;
    std::vector<uint64_t> tensor_offsets, tensor_numels;
    std::vector<uint64_t> tensor_g0, tensor_g1;   // groups [g0, g1) cover tensor k's elements
    uint64_t max_group_elems = 0;   // elements of the largest group (one wave's unit)
    uint32_t count_bits = 12;    // index width of the codeword-start table
    uint32_t decode_bits = 11;   // index width of the multi-codeword table
    // Launch shapes: the plain bf16 decode is bound by HBM and runs best with
    // 4-wave workgroups (3 per CU); the code-plane decode and the fused
    // product are bound by the decode's own latency and instructions and run
    // best with more waves in flight, 8-wave workgroups (2 per CU).
    // WC_WAVES sets both.
    struct Shape {
        uint32_t waves = 4;      // wavefronts per workgroup
        uint32_t grid = 0;       // persistent workgroups of a whole-container decode
        uint32_t slots = 0;      // co-resident workgroups on the device
        uint32_t lds_bytes = 0;
    };
    Shape plain, busy;
    Shape dot;                   // fused product of a Huffman lanes container (its own kernel)
    uint32_t grid = 0;           // of the container's decode entry point (stats)
    uint32_t lds_bytes = 0;
    uint32_t ebuf_bytes = 0;
    uint32_t l2_cap = 0;         // long-code prefixes whose second-level entries are staged in LDS
    bool lanes = false;          // container version 3 (interleaved lanes)
    bool rans = false;           // coder rANS (version 3)
    bool one_code = false;       // Huffman: one code per table entry at most, none longer than 16 bits
    bool single_table = false;   // code planes: the first-code table in the multi-codeword table's place
    bool no_long = false;        // Huffman: no code longer than decode_bits
    uint32_t launch_rounds = 0;  // plain decode: segment rounds per launch at most (0: one launch)
    uint32_t* d_tables = nullptr;
    uint32_t* d_status = nullptr;   // WC_DEBUG plans: the debug status word
};

namespace {

using wc::Header;
using wc::HeaderOffsets;
using wc::load_le;

int parse_and_validate(const uint8_t* b, uint64_t bytes, Header& h, std::vector<uint64_t>& toff,
                       std::vector<uint64_t>& tnum, uint64_t& max_group_elems) {
    using O = HeaderOffsets;
    if (bytes < wc::kHeaderBytes) return WC_ERR_TRUNCATED;
    if (load_le<uint32_t>(b + O::magic) != wc::kMagic || load_le<uint16_t>(b + O::flags) != 0)
        return WC_ERR_BAD_MAGIC;
    h.version = load_le<uint16_t>(b + O::version);
    const bool lanes = h.version == wc::kVersionLanes;
    if (lanes) {
        if (b[O::lanes] != wc::kLanes || load_le<uint16_t>(b + O::lane_block) != wc::kLaneBlock ||
            load_le<uint64_t>(b + O::n_chunks) != 0)
            return WC_ERR_BAD_MAGIC;
    } else if (h.version != wc::kVersion || b[O::chunk_bits] != wc::kChunkBits || b[O::reserved0] != 0 ||
               (b[O::gap_bits] != 0 && b[O::gap_bits] != wc::kGapBitsPacked)) {
        return WC_ERR_BAD_MAGIC;
    }
    h.gap_bits = !lanes && b[O::gap_bits] == wc::kGapBitsPacked ? wc::kGapBitsPacked : wc::kGapBitsByte;
    for (uint32_t k = O::reserved_tail; k < wc::kHeaderBytes; ++k)
        if (b[k]) return WC_ERR_BAD_MAGIC;
    h.elem_kind = b[O::elem_kind];
    if (h.elem_kind != wc::kKindBf16 && (!lanes || h.elem_kind != wc::kKindU8)) return WC_ERR_BAD_MAGIC;
    h.coder = b[O::coder];
    if (h.coder != wc::kCoderHuffman && (!lanes || h.coder != wc::kCoderRans)) return WC_ERR_BAD_MAGIC;
    const bool rans = h.coder == wc::kCoderRans;
    h.max_code_len = b[O::max_code_len];
    h.chunks_per_group = lanes ? 0u : load_le<uint32_t>(b + O::chunks_per_group);
    h.seg_max_bits = lanes ? load_le<uint32_t>(b + O::seg_max_bits) : 0u;
    h.n_tensors = load_le<uint32_t>(b + O::n_tensors);
    h.group_align = load_le<uint32_t>(b + O::group_align);
    h.group_max_elems = load_le<uint32_t>(b + O::group_max_elems);
    h.n_elems = load_le<uint64_t>(b + O::n_elems);
    h.stream_bits = load_le<uint64_t>(b + O::stream_bits);
    h.n_chunks = load_le<uint64_t>(b + O::n_chunks);
    h.n_groups = load_le<uint64_t>(b + O::n_groups);
    h.off_code_len = load_le<uint64_t>(b + O::off_code_len);
    h.off_tensors = load_le<uint64_t>(b + O::off_tensors);
    h.off_groups = load_le<uint64_t>(b + O::off_groups);
    h.off_gap = load_le<uint64_t>(b + O::off_gap);
    h.off_stream = load_le<uint64_t>(b + O::off_stream);
    h.stream_bytes = load_le<uint64_t>(b + O::stream_bytes);
    h.off_sm = load_le<uint64_t>(b + O::off_sm);
    h.total_bytes = load_le<uint64_t>(b + O::total_bytes);
    if (h.max_code_len < 1 || h.max_code_len > wc::kMaxCodeLen || h.group_align < 1 ||
        h.group_max_elems < h.group_align || h.group_max_elems % h.group_align)
        return WC_ERR_BAD_MAGIC;
    if (!lanes && h.chunks_per_group < 1) return WC_ERR_BAD_MAGIC;
    if (lanes && !rans && (h.seg_max_bits > 65535u || (uint64_t)h.group_align * h.max_code_len > h.seg_max_bits))
        return WC_ERR_BAD_MAGIC;
    // rANS: P = 12, and one block always fits a segment (at most 97 eighths
    // of a bit per symbol besides the 64 final states)
    constexpr uint32_t kStates = wc::kLanes * wc::kRansStateBits;
    if (rans && (h.max_code_len != wc::kRansBits || h.seg_max_bits > 65535u || h.seg_max_bits < kStates ||
                 97ull * h.group_align > 8ull * (h.seg_max_bits - kStates)))
        return WC_ERR_BAD_MAGIC;
    if (h.total_bytes > bytes) return WC_ERR_TRUNCATED;

    // size fields (rANS: at most 13 bits per symbol and a final state per lane,
    // whole 16-bit words)
    if (h.n_elems > (1ull << 40) || h.n_groups > h.n_elems || (h.n_groups == 0) != (h.n_elems == 0))
        return WC_ERR_STREAM_BITS;
    if (rans ? h.stream_bits % 16 || h.stream_bits > h.n_elems * (wc::kRansBits + 1) + kStates * h.n_groups
             : h.stream_bits > h.n_elems * (uint64_t)h.max_code_len || h.stream_bits < h.n_elems)
        return WC_ERR_STREAM_BITS;
    if (lanes ? h.stream_bytes != wc::round_up(wc::div_up(h.stream_bits, 8), 8) + wc::kLanesSlack
              : (h.n_chunks != wc::div_up(h.stream_bits, wc::kChunkBits) ||
                 h.stream_bytes != h.n_chunks * 8 + wc::kStreamSlack))
        return WC_ERR_STREAM_BITS;

    // sections: 256-byte aligned, in order, non-overlapping, inside total_bytes
    if (h.n_tensors > (1u << 24)) return WC_ERR_SECTION_BOUNDS;
    const uint64_t off[6] = {h.off_code_len, h.off_tensors, h.off_groups, h.off_gap, h.off_stream, h.off_sm};
    const uint64_t len[6] = {wc::code_section_bytes(h.coder), 16ull * h.n_tensors,
                             wc::kGroupEntryBytes * (h.n_groups + 1),
                             lanes ? 2ull * wc::kLanes * h.n_groups : wc::gap_section_bytes(h.n_chunks, h.gap_bits),
                             h.stream_bytes,
                             h.elem_kind == wc::kKindBf16 ? h.n_elems : 0};
    uint64_t lo = wc::kHeaderBytes;
    for (int k = 0; k < 6; ++k) {
        if (off[k] % wc::kAlign || off[k] < lo || off[k] > h.total_bytes || len[k] > h.total_bytes - off[k])
            return WC_ERR_SECTION_BOUNDS;
        lo = off[k] + len[k];
    }
    // the decoder reads the sign+mantissa plane in 16-byte blocks
    if (h.elem_kind == wc::kKindBf16 && wc::round_up(h.n_elems, 16) > h.total_bytes - h.off_sm)
        return WC_ERR_SECTION_BOUNDS;

    // tensor table
    toff.resize(h.n_tensors);
    tnum.resize(h.n_tensors);
    uint64_t acc = 0;
    for (uint32_t t = 0; t < h.n_tensors; ++t) {
        toff[t] = load_le<uint64_t>(b + h.off_tensors + 16ull * t);
        tnum[t] = load_le<uint64_t>(b + h.off_tensors + 16ull * t + 8);
        if (toff[t] != acc || tnum[t] > h.n_elems - acc) return WC_ERR_TENSOR_TABLE;
        acc += tnum[t];
    }
    if (acc != h.n_elems) return WC_ERR_TENSOR_TABLE;

    if (rans) {
        // frequencies: each at most 2^12, summing to 2^12 (all 0 for no elements)
        uint32_t sum = 0;
        for (int s = 0; s < 256; ++s) {
            const uint32_t f = load_le<uint16_t>(b + h.off_code_len + 2 * s);
            if (f > (1u << wc::kRansBits)) return WC_ERR_CODE_LENGTHS;
            sum += f;
        }
        if (sum != (h.n_elems ? 1u << wc::kRansBits : 0u)) return WC_ERR_KRAFT;
    }
    // code lengths: complete prefix code (Kraft sum exactly 1), or one 1-bit code
    const uint8_t* cl = b + h.off_code_len;
    uint64_t kraft = 0;
    uint32_t present = 0, longest = 0;
    for (int s = 0; s < 256 && !rans; ++s) {
        if (!cl[s]) continue;
        if (cl[s] > h.max_code_len) return WC_ERR_CODE_LENGTHS;
        kraft += 1ull << (wc::kMaxCodeLen - cl[s]);
        ++present;
        longest = std::max<uint32_t>(longest, cl[s]);
    }
    if (!rans && present == 0 && h.n_elems) return WC_ERR_CODE_LENGTHS;
    if (present >= 2 && kraft != (1ull << wc::kMaxCodeLen)) return WC_ERR_KRAFT;
    if (present == 1 && longest != 1) return WC_ERR_KRAFT;

    // gaps: a codeword reaches at most max_code_len - 1 bits into the next chunk
    const uint8_t* gap = b + h.off_gap;
    for (uint64_t c = 0; !lanes && c < h.n_chunks; ++c) {
        uint32_t g = gap[c];
        if (h.gap_bits == wc::kGapBitsPacked) {
            const uint64_t bit = 5 * c;
            g = (uint32_t)((gap[bit >> 3] | (uint32_t)gap[(bit >> 3) + 1] << 8) >> (bit & 7)) & 31u;
        }
        if (g >= h.max_code_len || 64 * c + g > h.stream_bits) return WC_ERR_GAP;
    }

    // groups: start at {0, 0}, strictly increasing, first elements on block
    // boundaries, at most G chunks, at most group_max_elems elements and at
    // least one bit per element each, ending at {n, stream_bits}
    const uint8_t* gt = b + h.off_groups;
    if (load_le<uint64_t>(gt) != 0 || load_le<uint64_t>(gt + 8) != 0) return WC_ERR_GROUP_START;
    max_group_elems = 0;
    for (uint64_t g = 1; g <= h.n_groups; ++g) {
        const uint64_t e0 = load_le<uint64_t>(gt + wc::kGroupEntryBytes * (g - 1));
        const uint64_t p0 = load_le<uint64_t>(gt + wc::kGroupEntryBytes * (g - 1) + 8);
        const uint64_t e1 = load_le<uint64_t>(gt + wc::kGroupEntryBytes * g);
        const uint64_t p1 = load_le<uint64_t>(gt + wc::kGroupEntryBytes * g + 8);
        if (e1 <= e0 || p1 <= p0 || e1 > h.n_elems || p1 > h.stream_bits) return WC_ERR_GROUP_START;
        if (g < h.n_groups && e1 % h.group_align) return WC_ERR_GROUP_START;
        if ((!rans && e1 - e0 > p1 - p0) || e1 - e0 > h.group_max_elems) return WC_ERR_GROUP_START;
        if (rans && p1 % 16) return WC_ERR_GROUP_START;
        if (lanes ? p1 - p0 > h.seg_max_bits : wc::chunk_span(p0, p1) > h.chunks_per_group)
            return WC_ERR_GROUP_START;
        if (lanes) {
            // lane offsets: lane 0 at the segment's first bit, non-decreasing,
            // inside the segment
            const uint8_t* lo = gap + 2ull * wc::kLanes * (g - 1);
            if (load_le<uint16_t>(lo) != 0) return WC_ERR_GAP;
            for (uint32_t j = 1; j < wc::kLanes; ++j)
                if (load_le<uint16_t>(lo + 2 * j) < load_le<uint16_t>(lo + 2 * (j - 1)) ||
                    (rans && load_le<uint16_t>(lo + 2 * j) % 16))
                    return WC_ERR_GAP;
            if (load_le<uint16_t>(lo + 2 * (wc::kLanes - 1)) > p1 - p0) return WC_ERR_GAP;
        }
        max_group_elems = std::max(max_group_elems, e1 - e0);
    }
    if (load_le<uint64_t>(gt + wc::kGroupEntryBytes * h.n_groups) != h.n_elems ||
        load_le<uint64_t>(gt + wc::kGroupEntryBytes * h.n_groups + 8) != h.stream_bits)
        return WC_ERR_GROUP_START;

    // stream padding past stream_bits must be zero (so that it cannot be
    // mistaken for codewords by a reader that ignores stream_bits)
    const uint8_t* st = b + h.off_stream;
    if (h.stream_bits & 7) {
        uint8_t tail = st[h.stream_bits >> 3];
        if (tail & (0xFFu >> (h.stream_bits & 7))) return WC_ERR_STREAM_BITS;
    }
    for (uint64_t k = wc::div_up(h.stream_bits, 8); k < h.stream_bytes; ++k)
        if (st[k]) return WC_ERR_STREAM_BITS;
    return WC_OK;
}

uint32_t env_u32(const char* name, uint32_t dflt) {
    const char* v = std::getenv(name);
    if (!v || !*v) return dflt;
    return (uint32_t)std::strtoul(v, nullptr, 10);
}

struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) return;
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

}  // namespace

// For each `bits`-bit window, the code it starts with, as symbol | length
// << 8, or 0 when that code is longer than the window.  Codes are canonical
// (shorter codes numerically smaller, equal lengths in symbol order).
static std::vector<uint32_t> first_codes(const uint8_t* lens, uint32_t bits) {
    std::vector<uint32_t> first(1u << bits, 0u);
    uint32_t count[wc::kMaxCodeLen + 2] = {0};
    for (int s = 0; s < 256; ++s) count[lens[s]] += lens[s] != 0;
    uint32_t next[wc::kMaxCodeLen + 2] = {0};
    for (uint32_t L = 1, code = 0; L <= wc::kMaxCodeLen; ++L) {
        code = (code + count[L - 1] * (L > 1)) << 1;
        next[L] = code;
    }
    for (uint32_t L = 1; L <= std::min<uint32_t>(bits, wc::kMaxCodeLen); ++L)
        for (int s = 0; s < 256; ++s) {
            if (lens[s] != L) continue;
            const uint32_t code = next[L]++;
            const uint32_t lo = code << (bits - L), hi = (code + 1) << (bits - L);
            for (uint32_t w = lo; w < hi; ++w) first[w] = (uint32_t)s | L << 8;
        }
    return first;
}

// The wide decode table of Huffman code planes: for each `bits`-bit window,
// up to three whole codes from its start, as total bits | count << 5 |
// symbols << 8 (first code in the low byte), or 0 when the window's first
// code is longer than the window.
static void build_wide_table(const uint8_t* lens, uint32_t bits, uint32_t* out) {
    const uint32_t size = 1u << bits;
    const std::vector<uint32_t> first = first_codes(lens, bits);
    for (uint32_t w = 0; w < size; ++w) {
        uint32_t pos = 0, n = 0, syms = 0;
        while (n < 3 && pos < bits) {
            const uint32_t f = first[(w << pos) & (size - 1)];
            const uint32_t L = f >> 8;
            if (f == 0 || L > bits - pos) break;
            syms |= (f & 0xFFu) << (8 * n);
            ++n;
            pos += L;
        }
        out[w] = n ? pos | n << 5 | syms << 8 : 0u;
    }
}

// The first-code table: the multi-codeword table's entry format (two words
// per `bits`-bit window: (32 - length) | count << 8 | length << 16, then the
// symbols rotated right by one bit) with each window's first code alone, or
// 0 when it is longer than the window.
static void build_single_table(const uint8_t* lens, uint32_t bits, uint32_t* out) {
    const std::vector<uint32_t> first = first_codes(lens, bits);
    for (uint32_t w = 0; w < first.size(); ++w) {
        const uint32_t L = first[w] >> 8, sym = first[w] & 0xFFu;
        out[2 * w] = first[w] ? ((32u - L) & 31u) | 1u << 8 | L << 16 : 0u;
        out[2 * w + 1] = first[w] ? ((sym >> 1) | (sym & 1u) << 7) : 0u;
    }
}

extern "C" int wc_plan(const uint8_t* blob_host, uint64_t blob_bytes, int hip_device, wc_plan_t** out) {
    if (!out) return WC_ERR_INVALID_ARG;
    *out = nullptr;
    if (!blob_host) return WC_ERR_INVALID_ARG;
    wc_plan_t* p = new (std::nothrow) wc_plan_t;
    if (!p) return WC_ERR_NOMEM;
    int st = parse_and_validate(blob_host, blob_bytes, p->h, p->tensor_offsets, p->tensor_numels, p->max_group_elems);
    const bool lanes = st == WC_OK && p->h.version == wc::kVersionLanes;
    if (st == WC_OK && (p->h.group_align % wc::kMergeElems || p->h.group_max_elems > wc::kGroupMaxElems))
        st = WC_ERR_UNSUPPORTED;
    // (any chunks_per_group: a group spanning more than 128 chunks is decoded
    // in passes of 128)
    if (st == WC_OK && lanes && p->h.seg_max_bits > wc::kLanesMaxSegBits) st = WC_ERR_UNSUPPORTED;
    if (st != WC_OK) {
        delete p;
        return st;
    }
    p->device = hip_device;
    // groups covering each tensor: from the last group starting at or before
    // its first element to the last group starting before its end
    {
        const uint8_t* gt = blob_host + p->h.off_groups;
        const uint64_t ng = p->h.n_groups;
        auto first_elem = [&](uint64_t g) { return load_le<uint64_t>(gt + wc::kGroupEntryBytes * g); };
        auto groups_le = [&](uint64_t e) {   // number of groups whose first element is <= e
            uint64_t lo = 0, hi = ng;
            while (lo < hi) {
                const uint64_t mid = lo + (hi - lo) / 2;
                if (first_elem(mid) <= e) lo = mid + 1; else hi = mid;
            }
            return lo;
        };
        const size_t nt = p->tensor_offsets.size();
        p->tensor_g0.assign(nt, 0);
        p->tensor_g1.assign(nt, 0);
        for (size_t k = 0; k < nt; ++k) {
            if (p->tensor_numels[k] == 0) continue;
            const uint64_t a = p->tensor_offsets[k], e = a + p->tensor_numels[k];
            p->tensor_g0[k] = groups_le(a) - 1;
            p->tensor_g1[k] = groups_le(e - 1);
        }
    }
    p->rans = p->h.coder == wc::kCoderRans;
    p->count_bits = env_u32("WC_COUNT_BITS", 12);
    p->decode_bits = env_u32("WC_DECODE_BITS", 11);
    if (!wc::supported_table_bits(p->count_bits, p->decode_bits) || p->rans) {
        p->count_bits = 12;   // rANS: the 2^12-slot table takes the place of the 11-bit multi-codeword table
        p->decode_bits = 11;
    }
    if (!p->rans) {
        uint32_t shortest = 0, longest = 0, present = 0;
        for (int s = 0; s < 256; ++s) {
            const uint32_t L = blob_host[p->h.off_code_len + s];
            if (L && (!shortest || L < shortest)) shortest = L;
            longest = std::max(longest, L);
            present += L != 0;
        }
        // Without the long-code lookup every table entry must decode at least
        // one code, i.e. the code must be complete: a single symbol's code
        // "0" leaves the windows that start with 1 undecodable, and a lookup
        // there would not advance (the long-code lookup always does).
        p->no_long = present >= 2 && longest <= p->decode_bits;
        // One code per lookup: no multi-codeword table entry holds two whole
        // codes when the shortest code is longer than half the table index
        // (four codes of at most 16 bits fit one 64-bit window).  Code planes
        // whose codes all fit the index take one code per lookup whatever
        // their shortest code, from the first-code table: on int4 pairs
        // (shortest codes of 4 bits) eight codes per 96-bit window decode
        // faster than the wide table's up to three per lookup.
        // WC_FIRST_CODE_TABLE=0 keeps the wide table for them.
        const bool single = p->h.elem_kind == wc::kKindU8 && p->no_long && env_u32("WC_FIRST_CODE_TABLE", 1) != 0;
        p->one_code = shortest && longest <= 16 && (2 * shortest > p->decode_bits || single);
        p->single_table = p->one_code && 2 * shortest <= p->decode_bits;
    }
    {
        const uint32_t forced_waves = env_u32("WC_WAVES", 0);
        const bool ok = wc::supported_waves(forced_waves);
        p->plain.waves = ok ? forced_waves : 4u;
        p->busy.waves = ok ? forced_waves : 8u;
    }
    // each wave's staging of one group's exponents: a chain may write
    // kEbufSlack bytes past the end, and the merge reads whole blocks
    p->ebuf_bytes =
        (uint32_t)wc::round_up(p->max_group_elems + (wc::kMergeElems - 1) + wc::kEbufSlack, 16);
    // Long codes: canonical codes longer than the decode-table index all have
    // index-bit prefixes >= F = (first code of length decode_bits + 1) / 2; the
    // second-level table is staged for min(2^decode_bits - F, kL2Prefixes) of them.
    if (!p->rans) {
        const uint8_t* len = blob_host + p->h.off_code_len;
        uint64_t count[33] = {0};
        for (int sym = 0; sym < 256; ++sym)
            if (len[sym] >= 1 && len[sym] <= 32) ++count[len[sym]];
        uint64_t code = 0;
        uint64_t first_next = 0;   // first code of length decode_bits + 1
        for (uint32_t L = 1; L <= p->decode_bits + 1; ++L) {
            code = (code + (L > 1 ? count[L - 1] : 0)) << 1;
            if (L == p->decode_bits + 1) first_next = code;
        }
        const uint64_t F = first_next >> 1;
        const uint64_t span = 1ull << p->decode_bits;
        p->l2_cap = F < span ? (uint32_t)std::min<uint64_t>(span - F, wc::kL2Prefixes) : 0u;
    }
    p->lanes = lanes;

    DeviceGuard guard(hip_device);
    if (!guard.ok) {
        delete p;
        return WC_ERR_HIP;
    }
    int n_cu = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, hip_device) != hipSuccess || n_cu <= 0) {
        delete p;
        return WC_ERR_HIP;
    }
    int lds_cu = 0;
    if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, hip_device) != hipSuccess ||
        lds_cu <= 0)
        lds_cu = 160 * 1024;
    const uint32_t forced_grid = env_u32("WC_GRID", 0);
    // The plain decode of a large container runs as launches of at most 40
    // rounds of the persistent grid (a 70B-shape block: two launches of 34):
    // over many rounds the waves drift apart and spread their accesses over
    // more memory; a launch boundary brings them back together (measured
    // 1.8% faster for the 70B-shape block; for the 8B-shape block's 17 rounds
    // splitting only costs).  WC_LAUNCH_ROUNDS overrides it (0: one launch).
    p->launch_rounds = env_u32("WC_LAUNCH_ROUNDS", 40);
    // Huffman code planes: no slots with one code per table entry, else the
    // wide table's larger slots
    const bool u8_huffman = lanes && !p->rans && p->h.elem_kind == wc::kKindU8;
    const wc::LaneLds layout = !u8_huffman ? wc::kLdsSlots : p->one_code ? wc::kLdsCompact : wc::kLdsWide;
    auto size_shape = [&](wc_plan_s::Shape& sh, bool fused_lanes) {
        sh.lds_bytes = fused_lanes ? wc::decode_lanes_dot_lds_bytes(p->decode_bits, sh.waves, p->l2_cap)
                       : lanes     ? wc::decode_lanes_lds_bytes(p->decode_bits, sh.waves, p->l2_cap, layout)
                                   : wc::decode_lds_bytes(p->count_bits, p->decode_bits, sh.waves, p->ebuf_bytes,
                                                          p->l2_cap);
        int per_cu = fused_lanes ? wc::decode_lanes_dot_blocks_per_cu(p->decode_bits, sh.waves, p->l2_cap)
                     : lanes     ? wc::decode_lanes_blocks_per_cu(p->decode_bits, sh.waves, p->l2_cap, p->rans, layout)
                                 : wc::decode_blocks_per_cu(p->count_bits, p->decode_bits, sh.waves, p->ebuf_bytes,
                                                            p->l2_cap);
        // The persistent grid must be co-resident.  LDS is handed out in
        // granules of 1/128 of a compute unit's LDS (1,280 bytes of 160 KiB on
        // gfx950), which the runtime's occupancy estimate does not round for:
        // count the granules.
        const uint32_t granule = std::max<uint32_t>(1, (uint32_t)lds_cu / 128);
        const uint32_t granules = (uint32_t)wc::div_up(sh.lds_bytes, granule);
        per_cu = std::min<int>(per_cu, (int)(128 / std::max<uint32_t>(granules, 1)));
        if (per_cu <= 0) return false;
        // One persistent workgroup per resident slot (all of them: every
        // extra wave helps the decode more than an even last round of groups
        // would), and no more workgroups than there are groups to give their
        // waves.
        uint64_t want = (uint64_t)n_cu * (uint64_t)per_cu;
        sh.slots = (uint32_t)want;
        if (forced_grid) want = forced_grid;
        const uint64_t need = std::max<uint64_t>(1, wc::div_up(p->h.n_groups, sh.waves));
        sh.grid = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(want, need));
        return true;
    };
    p->dot.waves = p->busy.waves;
    const bool fused_lanes = lanes && !p->rans && p->h.elem_kind == wc::kKindBf16;
    if (!size_shape(p->plain, false) || !size_shape(p->busy, false) || (fused_lanes && !size_shape(p->dot, true))) {
        delete p;
        return WC_ERR_UNSUPPORTED;
    }
    {
        const wc_plan_s::Shape& own = p->h.elem_kind == wc::kKindU8 ? p->busy : p->plain;
        p->grid = own.grid;
        p->lds_bytes = own.lds_bytes;
    }

    const size_t tbytes = (size_t)wc::table_words(p->count_bits, p->decode_bits) * 4;
    if (hipMalloc(reinterpret_cast<void**>(&p->d_tables), tbytes) != hipSuccess) {
        delete p;
        return WC_ERR_NOMEM;
    }
    hipError_t te;
    if (p->rans) {
        // slot t of [0, 2^12): the symbol s with cum[s] <= t < cum[s] + f[s],
        // stored rotated as the Huffman tables store it, | (f mod 2^12) << 8 |
        // (t - cum[s]) << 20; at the multi-codeword table's place
        std::vector<uint32_t> host(tbytes / 4, 0u);
        uint32_t* entries = host.data() + (1u << p->count_bits);
        for (uint32_t sym = 0, t = 0; sym < 256; ++sym) {
            const uint32_t f = load_le<uint16_t>(blob_host + p->h.off_code_len + 2 * sym);
            const uint32_t rot = ((sym >> 1) | (sym << 7)) & 0xFFu;
            for (uint32_t r = 0; r < f; ++r, ++t) entries[t] = rot | (f & 0xFFFu) << 8 | r << 20;
        }
        te = hipMemcpy(p->d_tables, host.data(), tbytes, hipMemcpyHostToDevice);
    } else {
        wc::CodeLens lens;
        std::memcpy(lens.len, blob_host + p->h.off_code_len, 256);
        te = wc::launch_build_tables(lens, p->count_bits, p->decode_bits, p->d_tables, nullptr);
        if (te == hipSuccess && p->single_table) {
            // in the multi-codeword table's place, after its build
            std::vector<uint32_t> single(2u << p->decode_bits);
            build_single_table(lens.len, p->decode_bits, single.data());
            te = hipStreamSynchronize(nullptr);
            if (te == hipSuccess)
                te = hipMemcpy(p->d_tables + (1u << p->count_bits), single.data(), single.size() * 4,
                               hipMemcpyHostToDevice);
        }
        if (te == hipSuccess && layout == wc::kLdsWide) {
            // the wide table of code planes, at the multi-codeword table's
            // place (2^(decode_bits + 1) 4-byte entries: the same bytes)
            std::vector<uint32_t> wide(2u << p->decode_bits);
            build_wide_table(lens.len, p->decode_bits + 1, wide.data());
            te = hipStreamSynchronize(nullptr);
            if (te == hipSuccess)
                te = hipMemcpy(p->d_tables + (1u << p->count_bits), wide.data(), wide.size() * 4,
                               hipMemcpyHostToDevice);
        }
    }
    if (te == hipSuccess && env_u32("WC_DEBUG", 0)) {
        te = hipMalloc(reinterpret_cast<void**>(&p->d_status), 4);
        if (te == hipSuccess) te = hipMemset(p->d_status, 0, 4);
    }
    if (te != hipSuccess || hipStreamSynchronize(nullptr) != hipSuccess) {
        (void)hipFree(p->d_tables);
        if (p->d_status) (void)hipFree(p->d_status);
        delete p;
        return WC_ERR_HIP;
    }
    *out = p;
    return WC_OK;
}

extern "C" int wc_plan_info(const wc_plan_t* p, uint64_t* n_elems, uint32_t* n_tensors, uint64_t* tensor_offsets,
                            uint64_t* tensor_numels) {
    if (!p) return WC_ERR_INVALID_ARG;
    if (n_elems) *n_elems = p->h.n_elems;
    if (n_tensors) *n_tensors = p->h.n_tensors;
    if (tensor_offsets) std::copy(p->tensor_offsets.begin(), p->tensor_offsets.end(), tensor_offsets);
    if (tensor_numels) std::copy(p->tensor_numels.begin(), p->tensor_numels.end(), tensor_numels);
    return WC_OK;
}

extern "C" int wc_plan_stats(const wc_plan_t* p, uint64_t* container_bytes, uint64_t* stream_bits, uint64_t* n_groups,
                             uint32_t* count_bits, uint32_t* decode_bits, uint32_t* grid, uint32_t* lds_bytes) {
    if (!p) return WC_ERR_INVALID_ARG;
    if (container_bytes) *container_bytes = p->h.total_bytes;
    if (stream_bits) *stream_bits = p->h.stream_bits;
    if (n_groups) *n_groups = p->h.n_groups;
    if (count_bits) *count_bits = p->count_bits;
    if (decode_bits) *decode_bits = p->decode_bits;
    if (grid) *grid = p->grid;
    if (lds_bytes) *lds_bytes = p->lds_bytes;
    return WC_OK;
}

// The plain decode's split: launches of at most launch_rounds rounds of the
// persistent grid each, cut into equal spans of whole rounds; the segments per
// launch (the last launch takes what is left).
static uint64_t plain_span(const wc_plan_t* p) {
    const uint64_t per_round = (uint64_t)p->plain.grid * p->plain.waves;
    const uint64_t rounds = wc::div_up(p->h.n_groups, per_round);
    const uint64_t n_launch = p->launch_rounds ? wc::div_up(rounds, p->launch_rounds) : 1;
    return std::max<uint64_t>(1, wc::div_up(rounds, n_launch) * per_round);
}

extern "C" int wc_plan_decode_shape(const wc_plan_t* p, uint32_t* waves_per_group, uint32_t* grid,
                                    uint32_t* launches) {
    if (!p) return WC_ERR_INVALID_ARG;
    const bool u8 = p->h.elem_kind == wc::kKindU8;
    const wc_plan_s::Shape& own = u8 ? p->busy : p->plain;
    if (waves_per_group) *waves_per_group = own.waves;
    if (grid) *grid = own.grid;
    if (launches)
        *launches = p->h.n_groups == 0 ? 0u : u8 ? 1u : (uint32_t)wc::div_up(p->h.n_groups, plain_span(p));
    return WC_OK;
}

extern "C" int wc_decode_async(const wc_plan_t* p, const void* blob_dev, uint16_t* out_dev, void* stream) {
    if (!p || p->h.elem_kind != wc::kKindBf16) return WC_ERR_INVALID_ARG;
    if (p->h.n_elems == 0) return WC_OK;
    if (!blob_dev || !out_dev) return WC_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(blob_dev) & 255u) || (reinterpret_cast<uintptr_t>(out_dev) & 15u))
        return WC_ERR_INVALID_ARG;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return WC_ERR_HIP;
    if (cur != p->device) return WC_ERR_INVALID_ARG;
    const uint8_t* b = static_cast<const uint8_t*>(blob_dev);
    wc::DecodeParams d;
    d.stream = b + p->h.off_stream;
    d.gap = b + p->h.off_gap;
    d.groups = reinterpret_cast<const uint64_t*>(b + p->h.off_groups);
    d.sm = b + p->h.off_sm;
    d.out = out_dev;
    d.out8 = nullptr;
    d.tables = p->d_tables;
    d.n_elems = p->h.n_elems;
    d.u_begin = 0;
    d.u_end = p->h.n_groups;
    d.ebuf_bytes = p->ebuf_bytes;
    d.l2_cap = p->l2_cap;
    d.gap_packed = p->h.gap_bits == wc::kGapBitsPacked ? 1u : 0u;
    d.one_code = p->one_code ? 1u : 0u;
    d.no_long = p->no_long ? 1u : 0u;
    d.status = p->d_status;
    hipError_t e = hipSuccess;
    const uint64_t span = plain_span(p);
    if (p->lanes) d.tables = p->d_tables + (1u << p->count_bits);   // from the multi-codeword table on
    for (uint64_t u0 = 0; u0 < p->h.n_groups && e == hipSuccess; u0 += span) {
        d.u_begin = u0;
        d.u_end = std::min<uint64_t>(u0 + span, p->h.n_groups);
        if (p->lanes) {
            // the lane offsets sit where the gaps do
            e = wc::launch_decode_lanes(d, p->decode_bits, p->plain.waves, p->plain.grid, wc::kLanesToBf16, p->rans,
                                        static_cast<hipStream_t>(stream));
        } else {
            e = wc::launch_decode(d, p->count_bits, p->decode_bits, p->plain.waves, p->plain.grid, false,
                                  static_cast<hipStream_t>(stream));
        }
    }
    return e == hipSuccess ? WC_OK : WC_ERR_HIP;
}

extern "C" int wc_decode_u8_async(const wc_plan_t* p, const void* blob_dev, uint8_t* out_dev, void* stream) {
    if (!p || p->h.elem_kind != wc::kKindU8) return WC_ERR_INVALID_ARG;
    if (p->h.n_elems == 0) return WC_OK;
    if (!blob_dev || !out_dev) return WC_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(blob_dev) & 255u) || (reinterpret_cast<uintptr_t>(out_dev) & 15u))
        return WC_ERR_INVALID_ARG;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return WC_ERR_HIP;
    if (cur != p->device) return WC_ERR_INVALID_ARG;
    const uint8_t* b = static_cast<const uint8_t*>(blob_dev);
    wc::DecodeParams d;
    d.stream = b + p->h.off_stream;
    d.gap = b + p->h.off_gap;
    d.groups = reinterpret_cast<const uint64_t*>(b + p->h.off_groups);
    d.sm = nullptr;
    d.out = nullptr;
    d.out8 = out_dev;
    d.tables = p->d_tables + (1u << p->count_bits);
    d.n_elems = p->h.n_elems;
    d.u_begin = 0;
    d.u_end = p->h.n_groups;
    d.ebuf_bytes = p->ebuf_bytes;
    d.l2_cap = p->l2_cap;
    d.gap_packed = p->h.gap_bits == wc::kGapBitsPacked ? 1u : 0u;
    d.one_code = p->one_code ? 1u : 0u;
    d.no_long = p->no_long ? 1u : 0u;
    d.status = p->d_status;
    const hipError_t e = wc::launch_decode_lanes(d, p->decode_bits, p->busy.waves, p->busy.grid, wc::kLanesToU8,
                                                 p->rans, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? WC_OK : WC_ERR_HIP;
}

extern "C" int wc_plan_format(const wc_plan_t* p, uint32_t* version, uint32_t* elem_kind, uint32_t* coder) {
    if (!p) return WC_ERR_INVALID_ARG;
    if (version) *version = p->h.version;
    if (elem_kind) *elem_kind = p->h.elem_kind;
    if (coder) *coder = p->h.coder;
    return WC_OK;
}

namespace {

// The fused product's launch parameters for ops[0 .. n_ops): checks every
// operand, drops empty matrices, and sizes the work buffer (the group
// partials, then the per-row first groups, each 256-byte aligned).
int prepare_gemv(const wc_plan_t* p, const wc_gemv_operand* ops, uint32_t n_ops, wc::DotParams& q,
                 uint64_t& u_begin, uint64_t& u_end, uint64_t& work_bytes, uint64_t& rows_off) {
    if (!p || !ops || n_ops == 0 || n_ops > wc::kMaxDotMats || p->h.elem_kind != wc::kKindBf16)
        return WC_ERR_INVALID_ARG;
    std::memset(&q, 0, sizeof(q));
    uint64_t rows = 0;
    for (uint32_t i = 0; i < n_ops; ++i) {
        const wc_gemv_operand& o = ops[i];
        if (o.tensor >= p->h.n_tensors || o.tensor != ops[0].tensor + i) return WC_ERR_INVALID_ARG;
        if (o.cols == 0 || o.cols % wc::kMergeElems || o.cols > 0x7FFFFFFFu) return WC_ERR_INVALID_ARG;
        const uint64_t off = p->tensor_offsets[o.tensor], numel = p->tensor_numels[o.tensor];
        if (numel == 0) continue;
        if (numel % o.cols || off % wc::kMergeElems || o.cols < p->max_group_elems || numel > 0xFFFFFFFFull)
            return WC_ERR_INVALID_ARG;
        if (!o.x || !o.y || (reinterpret_cast<uintptr_t>(o.x) & 15u) || (reinterpret_cast<uintptr_t>(o.y) & 3u))
            return WC_ERR_INVALID_ARG;
        const uint32_t k = q.n_mats++;
        if (k == 0) u_begin = p->tensor_g0[o.tensor];
        u_end = p->tensor_g1[o.tensor];
        q.bounds[k] = off;
        q.bounds[k + 1] = off + numel;
        q.row_base[k] = rows;
        q.cols[k] = o.cols;
        wc::div_magic_params(o.cols, q.magic[k], q.shift[k]);
        q.x[k] = o.x;
        q.y[k] = o.y;
        rows += numel / o.cols;
    }
    q.row_base[q.n_mats] = rows;
    if (rows > 0xFFFFFFFFull) return WC_ERR_INVALID_ARG;
    q.rows = (uint32_t)rows;
    if (q.n_mats == 0) {
        u_begin = u_end = 0;
        work_bytes = rows_off = 0;
        return WC_OK;
    }
    if (u_end - u_begin > 0xFFFFFFFFull) return WC_ERR_INVALID_ARG;
    rows_off = wc::round_up(8 * (u_end - u_begin), 256);
    work_bytes = rows_off + 4 * rows;
    return WC_OK;
}

}  // namespace

extern "C" int wc_decode_gemv_work_bytes(const wc_plan_t* p, const wc_gemv_operand* ops, uint32_t n_ops,
                                         uint64_t* work_bytes) {
    if (!work_bytes) return WC_ERR_INVALID_ARG;
    wc::DotParams q;
    uint64_t ub = 0, ue = 0, wb = 0, ro = 0;
    const int st = prepare_gemv(p, ops, n_ops, q, ub, ue, wb, ro);
    if (st == WC_OK) *work_bytes = wb;
    return st;
}

extern "C" int wc_decode_gemv_async(const wc_plan_t* p, const void* blob_dev, const wc_gemv_operand* ops,
                                    uint32_t n_ops, void* work_dev, uint64_t work_bytes, void* stream) {
    wc::DecodeParams d;
    uint64_t need = 0, rows_off = 0;
    const int st = prepare_gemv(p, ops, n_ops, d.dot, d.u_begin, d.u_end, need, rows_off);
    if (st != WC_OK) return st;
    if (d.dot.n_mats == 0) return WC_OK;
    if (!blob_dev || !work_dev || work_bytes < need || (reinterpret_cast<uintptr_t>(blob_dev) & 255u) ||
        (reinterpret_cast<uintptr_t>(work_dev) & 255u))
        return WC_ERR_INVALID_ARG;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return WC_ERR_HIP;
    if (cur != p->device) return WC_ERR_INVALID_ARG;
    const uint8_t* b = static_cast<const uint8_t*>(blob_dev);
    d.stream = b + p->h.off_stream;
    d.gap = b + p->h.off_gap;
    d.groups = reinterpret_cast<const uint64_t*>(b + p->h.off_groups);
    d.sm = b + p->h.off_sm;
    d.out = nullptr;
    d.out8 = nullptr;
    d.tables = p->d_tables;
    d.n_elems = p->h.n_elems;
    d.ebuf_bytes = p->ebuf_bytes;
    d.l2_cap = p->l2_cap;
    d.gap_packed = p->h.gap_bits == wc::kGapBitsPacked ? 1u : 0u;
    d.one_code = p->one_code ? 1u : 0u;
    d.no_long = p->no_long ? 1u : 0u;
    d.status = p->d_status;
    d.dot.part = static_cast<float*>(work_dev);
    d.dot.row_group = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(work_dev) + rows_off);
    // Huffman lanes containers have a fused kernel of their own (its own
    // launch shape); rANS lanes and chunks containers use their decode
    // kernel's fused mode
    const bool own = p->lanes && !p->rans;
    const wc_plan_s::Shape& sh = own ? p->dot : p->busy;
    const uint64_t groups = wc::div_up(d.u_end - d.u_begin, sh.waves);
    const uint32_t grid = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(sh.slots, groups));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (own) {
        d.tables = p->d_tables + (1u << p->count_bits);
        e = wc::launch_decode_lanes_dot(d, p->decode_bits, sh.waves, grid, s);
    } else if (p->lanes) {
        d.tables = p->d_tables + (1u << p->count_bits);
        e = wc::launch_decode_lanes(d, p->decode_bits, sh.waves, grid, wc::kLanesToDot, p->rans, s);
    } else {
        e = wc::launch_decode(d, p->count_bits, p->decode_bits, p->busy.waves, grid, true, s);
    }
    if (e == hipSuccess) e = wc::launch_gemv_rows(d, s);
    return e == hipSuccess ? WC_OK : WC_ERR_HIP;
}

int wc::plan_device(const wc_plan_s* p) { return p->device; }

extern "C" void wc_plan_destroy(wc_plan_t* p) {
    if (!p) return;
    if (p->d_tables || p->d_status) {
        DeviceGuard guard(p->device);
        if (p->d_tables) (void)hipFree(p->d_tables);
        if (p->d_status) (void)hipFree(p->d_status);
    }
    delete p;
}

extern "C" int wc_plan_debug_status(const wc_plan_t* p, uint32_t* status, int reset) {
    if (!p || !status || !p->d_status) return WC_ERR_INVALID_ARG;
    DeviceGuard guard(p->device);
    if (!guard.ok || hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(status, p->d_status, 4, hipMemcpyDeviceToHost) != hipSuccess)
        return WC_ERR_HIP;
    if (reset && (hipMemset(p->d_status, 0, 4) != hipSuccess || hipDeviceSynchronize() != hipSuccess))
        return WC_ERR_HIP;
    return WC_OK;
}

extern "C" const char* wc_status_str(int s) {
    switch (s) {
        case WC_OK: return "ok";
        case WC_ERR_INVALID_ARG: return "invalid argument";
        case WC_ERR_NOMEM: return "out of memory";
        case WC_ERR_HIP: return "HIP runtime error";
        case WC_ERR_UNSUPPORTED: return "unsupported container parameters";
        case WC_ERR_SCRATCH: return "work exceeds the static scratch of the no-allocation entry point";
        case WC_ERR_BAD_MAGIC: return "bad magic, version or fixed header field";
        case WC_ERR_TRUNCATED: return "container truncated";
        case WC_ERR_SECTION_BOUNDS: return "section misaligned, out of order or out of bounds";
        case WC_ERR_CODE_LENGTHS: return "code length out of range";
        case WC_ERR_KRAFT: return "code lengths do not form a complete prefix code";
        case WC_ERR_GAP: return "per-chunk gap out of range";
        case WC_ERR_GROUP_START: return "group output starts invalid";
        case WC_ERR_STREAM_BITS: return "stream size fields inconsistent";
        case WC_ERR_TENSOR_TABLE: return "tensor table is not a partition of the elements";
        default: return "unknown status";
    }
}
