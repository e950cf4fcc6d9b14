// encode.cpp -- host-side container writer of libwc (offline weight preparation).
//
// Steps (pages: DFloat11 abstract -- entropy coding of the bf16 representation
// by symbol frequency; LazyWeights review -- Huffman codes, shorter for common
// values; "From a Lossless (~1.5:1) Compression Algorithm for Llama2 7B
// Weights ...", abstract -- lossless coding of bf16 weights):
//   1. split every bf16 word into its exponent byte and its sign+mantissa byte;
//   2. histogram the exponents over all tensors of the block (one codebook);
//   3. optimal code lengths limited to max_code_len (package-merge);
//   4. canonical codes;
//   5. cut the elements into groups: runs of whole blocks of `align` elements,
//      each run as long as its codewords touch at most G 64-bit chunks and it
//      holds at most `max_elems` elements; every group records its first
//      element and the stream bit where that element's codeword starts;
//   6. pack the codes MSB-first in parallel over element ranges, recording for
//      every 64-bit chunk the offset of its first codeword (with the group
//      table, the auxiliary variables of the DFloat11 abstract, design point
//      (ii)).
// The interleaved-lane layout (container v3; the LazyWeights page stores
// Huffman codes in interleaved lanes) shares steps 1-4, cuts segments by a
// bit cap instead of a chunk cap in step 5, and in step 6 writes each
// segment lane by lane: lane j's lane blocks j, j + 64, ... of 8 elements,
// with a u16 offset per lane.
// The rANS coder (coder 1; the Llama2-7B page's abstract names ANS) replaces
// steps 3-4 by quantized frequencies, cuts segments by a proven upper bound
// of their encoded size, and makes every lane one rANS stream.
#include <algorithm>
#include <array>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "format.h"
#include "../../include/wc.h"

namespace wc {
namespace {

inline uint8_t exponent_of(uint16_t b) { return (uint8_t)(b >> 7); }   // bits 14..7 (bit 15 shifted out)
inline uint8_t sign_mantissa_of(uint16_t b) { return (uint8_t)(((b >> 8) & 0x80u) | (b & 0x7Fu)); }
// The coded symbol of an element: a bf16 word's exponent, or a code byte itself.
inline uint8_t symbol_of(uint16_t b) { return exponent_of(b); }
inline uint8_t symbol_of(uint8_t b) { return b; }

// ---------------------------------------------------------------------------
// Optimal length-limited code: package-merge over a node pool.  A node is a
// leaf (one symbol) or a package of two nodes of the next-deeper list; the
// length of a symbol is the number of times its leaf is reached from the
// first 2m-2 nodes of the shallowest list.
// ---------------------------------------------------------------------------
struct PMNode {
    uint64_t weight;
    int32_t left, right;   // -1 for a leaf
    int32_t symbol;        // leaf symbol
};

int limited_code_lengths(const uint64_t hist[256], uint32_t max_len, uint8_t len[256]) {
    std::memset(len, 0, 256);
    std::vector<int> present;
    for (int s = 0; s < 256; ++s)
        if (hist[s]) present.push_back(s);
    const int m = (int)present.size();
    if (m == 0) return WC_OK;
    if (m == 1) { len[present[0]] = 1; return WC_OK; }
    if ((uint64_t)m > (1ull << max_len)) return WC_ERR_INVALID_ARG;
    std::stable_sort(present.begin(), present.end(),
                     [&](int a, int b) { return hist[a] < hist[b]; });
    std::vector<PMNode> pool;
    pool.reserve((size_t)2 * m * (max_len + 1));
    std::vector<int32_t> leaves(m);
    for (int k = 0; k < m; ++k) {
        leaves[k] = (int32_t)pool.size();
        pool.push_back({hist[present[k]], -1, -1, present[k]});
    }
    std::vector<int32_t> cur = leaves, merged;
    for (uint32_t depth = max_len; depth > 1; --depth) {
        merged.clear();
        size_t li = 0, pi = 0, npk = cur.size() / 2;
        while (li < leaves.size() || pi < npk) {
            bool take_leaf;
            if (pi >= npk) take_leaf = true;
            else if (li >= leaves.size()) take_leaf = false;
            else {
                uint64_t pw = pool[cur[2 * pi]].weight + pool[cur[2 * pi + 1]].weight;
                take_leaf = pool[leaves[li]].weight <= pw;
            }
            if (take_leaf) {
                merged.push_back(leaves[li++]);
            } else {
                int32_t a = cur[2 * pi], b = cur[2 * pi + 1];
                merged.push_back((int32_t)pool.size());
                pool.push_back({pool[a].weight + pool[b].weight, a, b, -1});
                ++pi;
            }
        }
        cur.swap(merged);
    }
    std::vector<int32_t> stack;
    for (int j = 0; j < 2 * m - 2; ++j) {
        stack.push_back(cur[j]);
        while (!stack.empty()) {
            int32_t v = stack.back();
            stack.pop_back();
            if (pool[v].left < 0) ++len[pool[v].symbol];
            else { stack.push_back(pool[v].left); stack.push_back(pool[v].right); }
        }
    }
    return WC_OK;
}

// Canonical code assignment by per-length counters (shorter codes are
// numerically smaller; equal lengths follow symbol order).
void canonical_codes(const uint8_t len[256], uint32_t code[256]) {
    uint32_t count[kMaxCodeLen + 2] = {0}, next[kMaxCodeLen + 2] = {0};
    for (int s = 0; s < 256; ++s)
        if (len[s]) ++count[len[s]];
    uint32_t c = 0;
    for (uint32_t L = 1; L <= kMaxCodeLen; ++L) {
        c = (c + count[L - 1]) << 1;
        next[L] = c;
    }
    for (int s = 0; s < 256; ++s) code[s] = len[s] ? next[len[s]]++ : 0;
}

// Global element index space over several tensors.
template <typename T>
struct SourceT {
    std::vector<const T*> ptr;
    std::vector<uint64_t> begin;   // global index of each tensor's first element
    std::vector<uint64_t> size;

    template <typename F>
    void for_range(uint64_t i0, uint64_t i1, F&& f) const {   // f(global_index, const T* p, count)
        size_t t = std::upper_bound(begin.begin(), begin.end(), i0) - begin.begin() - 1;
        uint64_t i = i0;
        while (i < i1) {
            while (i >= begin[t] + size[t]) ++t;
            uint64_t k = std::min(i1, begin[t] + size[t]) - i;
            f(i, ptr[t] + (i - begin[t]), k);
            i += k;
        }
    }
    T at(uint64_t i) const {
        size_t t = std::upper_bound(begin.begin(), begin.end(), i) - begin.begin() - 1;
        while (size[t] == 0 || i >= begin[t] + size[t]) ++t;
        return ptr[t][i - begin[t]];
    }
};

template <typename F>
void parallel_for(unsigned nthreads, F&& f) {
    if (nthreads <= 1) { f(0u); return; }
    std::vector<std::thread> th;
    th.reserve(nthreads);
    for (unsigned t = 0; t < nthreads; ++t) th.emplace_back([&f, t] { f(t); });
    for (auto& x : th) x.join();
}

// MSB-first bit writer over a byte range whose first and last bytes may be
// shared with a neighbouring writer (those two are OR-ed in atomically).
struct BitWriter {
    uint8_t* stream;
    uint64_t wbyte;
    uint32_t acc = 0;
    int nacc;
    bool shared_head;
    BitWriter(uint8_t* s, uint64_t pos) : stream(s), wbyte(pos >> 3), nacc((int)(pos & 7)), shared_head(nacc != 0) {}
    void put_code(uint32_t code, int L) {   // L <= 24
        acc = (acc << L) | code;
        nacc += L;
        while (nacc >= 8) {
            nacc -= 8;
            const uint8_t v = (uint8_t)(acc >> nacc);
            if (shared_head) {
                __atomic_fetch_or(stream + wbyte, v, __ATOMIC_RELAXED);
                shared_head = false;
            } else {
                stream[wbyte] = v;
            }
            ++wbyte;
        }
        acc &= (1u << nacc) - 1u;
    }
    void finish() {
        if (nacc) __atomic_fetch_or(stream + wbyte, (uint8_t)(acc << (8 - nacc)), __ATOMIC_RELAXED);
    }
};

// Container v3: segments of whole blocks (at most max_elems elements and
// seg_bits stream bits), each written lane by lane; bf16 elements also write
// their sign+mantissa plane, code bytes have none.
template <typename T>
int write_lanes(const SourceT<T>& src, uint64_t n, uint32_t n_tensors, const uint8_t len[256], const uint32_t code[256],
                uint32_t max_len, uint32_t align, uint32_t max_elems, uint32_t seg_bits,
                const std::vector<uint64_t>& block_bit, uint64_t stream_bits, unsigned nthreads, uint8_t** blob,
                uint64_t* blob_bytes) {
    const uint64_t n_blocks = block_bit.size() - 1;
    std::vector<uint64_t> s_elem{0}, s_bit{0};
    for (uint64_t k0 = 0; k0 < n_blocks;) {
        uint64_t k1 = k0 + 1;
        const uint64_t k_cap = k0 + max_elems / align;
        while (k1 < n_blocks && k1 < k_cap && block_bit[k1 + 1] - block_bit[k0] <= seg_bits) ++k1;
        s_elem.push_back(std::min<uint64_t>(k1 * align, n));
        s_bit.push_back(block_bit[k1]);
        k0 = k1;
    }
    const uint64_t n_segs = s_elem.size() - 1;
    uint64_t seg_max = 0;   // the largest segment: each thread's staging buffer
    for (uint64_t g = 0; g < n_segs; ++g) seg_max = std::max<uint64_t>(seg_max, s_elem[g + 1] - s_elem[g]);
    constexpr bool kBf16 = sizeof(T) == 2;
    const Header h = layout_lanes(n, stream_bits, n_tensors, max_len, align, max_elems, seg_bits, n_segs,
                                  kBf16 ? kKindBf16 : kKindU8);
    const uint64_t sm_bytes = kBf16 ? n : 0;
    uint8_t* out = (uint8_t*)std::aligned_alloc(kAlign, h.total_bytes);
    if (!out) return WC_ERR_NOMEM;
    std::memset(out, 0, h.off_sm);
    std::memset(out + h.off_sm + sm_bytes, 0, h.total_bytes - h.off_sm - sm_bytes);
    write_header(out, h);
    std::memcpy(out + h.off_code_len, len, 256);
    for (uint32_t k = 0; k < n_tensors; ++k) {
        store_le<uint64_t>(out + h.off_tensors + 16ull * k, src.begin[k]);
        store_le<uint64_t>(out + h.off_tensors + 16ull * k + 8, src.size[k]);
    }
    for (uint64_t g = 0; g <= n_segs; ++g) {
        store_le<uint64_t>(out + h.off_groups + kGroupEntryBytes * g, s_elem[g]);
        store_le<uint64_t>(out + h.off_groups + kGroupEntryBytes * g + 8, s_bit[g]);
    }
    uint8_t* stream = out + h.off_stream;
    uint8_t* lane_off = out + h.off_gap;
    uint8_t* sm = out + h.off_sm;
    const unsigned nt = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(nthreads, n_segs));
    parallel_for(nt, [&](unsigned t) {
        const uint64_t g0 = n_segs * t / nt, g1 = n_segs * (t + 1) / nt;
        if (g0 == g1) return;
        BitWriter bw(stream, s_bit[g0]);
        uint64_t pos = s_bit[g0];
        std::vector<T> seg(seg_max);
        for (uint64_t g = g0; g < g1; ++g) {
            const uint64_t e0 = s_elem[g], m = s_elem[g + 1] - e0;
            src.for_range(e0, e0 + m, [&](uint64_t gi, const T* p, uint64_t k) {
                std::memcpy(seg.data() + (gi - e0), p, k * sizeof(T));
            });
            if constexpr (kBf16)
                for (uint64_t i = 0; i < m; ++i) sm[e0 + i] = sign_mantissa_of(seg[i]);
            const uint64_t nb8 = div_up(m, kLaneBlock);
            for (uint32_t j = 0; j < kLanes; ++j) {
                store_le<uint16_t>(lane_off + 2 * (kLanes * g + j), (uint16_t)(pos - s_bit[g]));
                for (uint64_t b = j; b < nb8; b += kLanes) {
                    const uint64_t i1 = std::min<uint64_t>(m, kLaneBlock * (b + 1));
                    for (uint64_t i = kLaneBlock * b; i < i1; ++i) {
                        const uint8_t e = symbol_of(seg[i]);
                        bw.put_code(code[e], len[e]);
                        pos += len[e];
                    }
                }
            }
        }
        bw.finish();
    });
    *blob = out;
    *blob_bytes = h.total_bytes;
    return WC_OK;
}

// ---------------------------------------------------------------------------
// rANS in the lane layout.
// ---------------------------------------------------------------------------
// Quantized frequencies summing to 2^12: every present symbol first gets
// max(1, floor(count * 2^12 / n)); an excess is then removed one unit at a
// time from the largest frequency above 1 (the lowest symbol among equal
// ones), a shortfall is added to the most frequent symbol (the lowest among
// equal counts).
void rans_frequencies(const uint64_t hist[256], uint64_t n, uint32_t freq[256]) {
    constexpr uint32_t kTotal = 1u << kRansBits;
    int top = -1;
    uint32_t sum = 0;
    for (int s = 0; s < 256; ++s) {
        freq[s] = hist[s] ? (uint32_t)std::max<uint64_t>(1, (hist[s] << kRansBits) / n) : 0u;
        sum += freq[s];
        if (hist[s] && (top < 0 || hist[s] > hist[top])) top = s;
    }
    if (top < 0) return;
    while (sum > kTotal) {
        int big = -1;
        for (int s = 0; s < 256; ++s)
            if (freq[s] > 1 && (big < 0 || freq[s] > freq[big])) big = s;
        --freq[big];
        --sum;
    }
    freq[top] += kTotal - sum;
}

// Upper bound, in eighths of a bit, of the growth of a lane's string per
// symbol of frequency f: encoding multiplies the state by at most
// 2^12 / f * (1 + f / x) with x >= 2^16, so it adds less than 12 - log2 f +
// 0.0875 bits, and ceil(8 (12 - log2 f)) + 1 eighths bound it.  With
// v = f^8 <= 2^96 of bit length b, the ceiling is the least q with
// v 2^q >= 2^96, which is 97 - b whether or not v is a power of two.
uint32_t rans_cost8(uint32_t f) {
    unsigned __int128 v = 1;
    for (int i = 0; i < 8; ++i) v *= f;
    const uint64_t hi = (uint64_t)(v >> 64), lo = (uint64_t)v;
    const uint32_t b = hi ? 128u - (uint32_t)__builtin_clzll(hi) : 64u - (uint32_t)__builtin_clzll(lo);
    return 97u - b + 1u;
}

// One segment of m symbols: every lane's string appended to `words` (lane
// order), lane j's bit offset from the segment's first bit in loff[j].  A
// lane encodes its symbols last to first from the state 2^16; a word is
// pushed out when the state would leave [2^16, 2^32) (x >= f 2^20 before
// the step), so one push always suffices.
void rans_encode_segment(const uint8_t* sym, uint64_t m, const uint32_t freq[256], const uint32_t cum[256],
                         std::vector<uint16_t>& words, std::vector<uint16_t>& pushed, uint16_t* loff) {
    const uint64_t start = words.size();
    const uint64_t nb8 = div_up(m, kLaneBlock);
    for (uint32_t j = 0; j < kLanes; ++j) {
        loff[j] = (uint16_t)(16 * (words.size() - start));
        if (j >= nb8) continue;
        pushed.clear();
        uint32_t x = kRansLow;
        const uint64_t last = j + (nb8 - 1 - j) / kLanes * kLanes;   // the lane's last lane block
        for (uint64_t b = last + kLanes; b > j;) {
            b -= kLanes;
            const uint64_t i0 = kLaneBlock * b, i1 = std::min<uint64_t>(m, i0 + kLaneBlock);
            for (uint64_t i = i1; i-- > i0;) {
                const uint32_t f = freq[sym[i]];
                if (x >= ((uint64_t)f << 20)) {
                    pushed.push_back((uint16_t)x);
                    x >>= 16;
                }
                x = ((x / f) << kRansBits) + x % f + cum[sym[i]];
            }
        }
        words.push_back((uint16_t)(x >> 16));
        words.push_back((uint16_t)x);
        words.insert(words.end(), pushed.rbegin(), pushed.rend());   // the order the decoder reads them
    }
}

template <typename T>
int write_lanes_rans(const SourceT<T>& src, uint64_t n, uint32_t n_tensors, const uint64_t hist[256],
                     uint32_t align, uint32_t max_elems, uint32_t seg_bits, unsigned nthreads, uint8_t** blob,
                     uint64_t* blob_bytes) {
    constexpr bool kBf16 = sizeof(T) == 2;
    uint32_t freq[256], cum[256], cost8[256];
    rans_frequencies(hist, n, freq);
    for (uint32_t s = 0, acc = 0; s < 256; ++s) {
        cum[s] = acc;
        acc += freq[s];
        cost8[s] = freq[s] ? rans_cost8(freq[s]) : 0u;
    }
    // segments: the longest runs of whole blocks with at most max_elems
    // elements whose bound (64 final states plus the symbols' cost8) fits
    const uint64_t n_blocks = div_up(n, align);
    std::vector<uint64_t> cost_before(n_blocks + 1, 0);
    parallel_for(nthreads, [&](unsigned t) {
        const uint64_t k0 = n_blocks * t / nthreads, k1 = n_blocks * (t + 1) / nthreads;
        for (uint64_t k = k0; k < k1; ++k) {
            uint64_t c = 0;
            src.for_range(k * align, std::min<uint64_t>(n, (k + 1) * align), [&](uint64_t, const T* p, uint64_t cnt) {
                for (uint64_t i = 0; i < cnt; ++i) c += cost8[symbol_of(p[i])];
            });
            cost_before[k + 1] = c;
        }
    });
    for (uint64_t k = 0; k < n_blocks; ++k) cost_before[k + 1] += cost_before[k];
    const uint64_t fixed8 = 8ull * kLanes * kRansStateBits;
    std::vector<uint64_t> s_elem{0};
    for (uint64_t k0 = 0; k0 < n_blocks;) {
        uint64_t k1 = k0 + 1;
        const uint64_t k_cap = k0 + max_elems / align;
        while (k1 < n_blocks && k1 < k_cap && fixed8 + cost_before[k1 + 1] - cost_before[k0] <= 8ull * seg_bits) ++k1;
        s_elem.push_back(std::min<uint64_t>(k1 * align, n));
        k0 = k1;
    }
    const uint64_t n_segs = s_elem.size() - 1;
    uint64_t seg_max = 0;   // the largest segment: each thread's staging buffer
    for (uint64_t g = 0; g < n_segs; ++g) seg_max = std::max<uint64_t>(seg_max, s_elem[g + 1] - s_elem[g]);

    // encode: each thread a run of segments into its own words
    const unsigned nt = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(nthreads, n_segs));
    std::vector<std::vector<uint16_t>> words(nt);
    std::vector<uint64_t> seg_words(n_segs + 1, 0);
    std::vector<uint16_t> loff(kLanes * n_segs);
    std::atomic<bool> too_long{false};
    parallel_for(nt, [&](unsigned t) {
        const uint64_t g0 = n_segs * t / nt, g1 = n_segs * (t + 1) / nt;
        std::vector<uint8_t> sym(seg_max);
        std::vector<uint16_t> pushed;
        for (uint64_t g = g0; g < g1; ++g) {
            const uint64_t e0 = s_elem[g], m = s_elem[g + 1] - e0;
            src.for_range(e0, e0 + m, [&](uint64_t gi, const T* p, uint64_t k) {
                for (uint64_t i = 0; i < k; ++i) sym[gi - e0 + i] = symbol_of(p[i]);
            });
            const uint64_t before = words[t].size();
            rans_encode_segment(sym.data(), m, freq, cum, words[t], pushed, loff.data() + kLanes * g);
            seg_words[g + 1] = words[t].size() - before;
            if (16 * seg_words[g + 1] > seg_bits) too_long = true;   // excluded by the bound
        }
    });
    if (too_long) return WC_ERR_INVALID_ARG;
    for (uint64_t g = 0; g < n_segs; ++g) seg_words[g + 1] += seg_words[g];
    const uint64_t stream_bits = 16 * seg_words[n_segs];

    const Header h = layout_lanes(n, stream_bits, n_tensors, kRansBits, align, max_elems, seg_bits, n_segs,
                                  kBf16 ? kKindBf16 : kKindU8, kCoderRans);
    const uint64_t sm_bytes = kBf16 ? n : 0;
    uint8_t* out = (uint8_t*)std::aligned_alloc(kAlign, h.total_bytes);
    if (!out) return WC_ERR_NOMEM;
    std::memset(out, 0, h.off_sm);
    std::memset(out + h.off_sm + sm_bytes, 0, h.total_bytes - h.off_sm - sm_bytes);
    write_header(out, h);
    for (int s = 0; s < 256; ++s) store_le<uint16_t>(out + h.off_code_len + 2 * s, (uint16_t)freq[s]);
    for (uint32_t k = 0; k < n_tensors; ++k) {
        store_le<uint64_t>(out + h.off_tensors + 16ull * k, src.begin[k]);
        store_le<uint64_t>(out + h.off_tensors + 16ull * k + 8, src.size[k]);
    }
    for (uint64_t g = 0; g <= n_segs; ++g) {
        store_le<uint64_t>(out + h.off_groups + kGroupEntryBytes * g, s_elem[g]);
        store_le<uint64_t>(out + h.off_groups + kGroupEntryBytes * g + 8, 16 * seg_words[g]);
    }
    for (uint64_t i = 0; i < kLanes * n_segs; ++i) store_le<uint16_t>(out + h.off_gap + 2 * i, loff[i]);
    uint8_t* stream = out + h.off_stream;
    uint8_t* sm = out + h.off_sm;
    parallel_for(nt, [&](unsigned t) {
        const uint64_t g0 = n_segs * t / nt, g1 = n_segs * (t + 1) / nt;
        uint8_t* dst = stream + 2 * seg_words[g0];
        for (const uint16_t w : words[t]) {   // big-endian words
            *dst++ = (uint8_t)(w >> 8);
            *dst++ = (uint8_t)w;
        }
        if constexpr (kBf16)
            src.for_range(s_elem[g0], s_elem[g1], [&](uint64_t gi, const T* p, uint64_t k) {
                for (uint64_t i = 0; i < k; ++i) sm[gi + i] = sign_mantissa_of(p[i]);
            });
    });
    *blob = out;
    *blob_bytes = h.total_bytes;
    return WC_OK;
}

// The whole encoder for bf16 words (T = uint16_t) or code bytes (T = uint8_t).
template <typename T>
int encode_impl(const T* const* tensors, const uint64_t* numels, uint32_t n_tensors, const wc_encode_opts* opts,
                uint8_t** blob, uint64_t* blob_bytes) {
    constexpr bool kBf16 = sizeof(T) == 2;
    if (!blob || !blob_bytes) return WC_ERR_INVALID_ARG;
    *blob = nullptr;
    *blob_bytes = 0;
    if (n_tensors && (!tensors || !numels)) return WC_ERR_INVALID_ARG;
    uint32_t max_len = kBf16 ? kMaxCodeLen : kDefaultCodeLenU8, group = kDefaultGroup, align = kDefaultAlign,
             max_elems = kDefaultMaxElems;
    uint32_t nthreads = 0, kind = WC_LAYOUT_LANES, seg_bits = kDefaultSegBits, coder = WC_CODER_HUFFMAN;
    uint32_t gap_bits = kGapBitsByte;
    if (opts) {
        if (opts->max_code_len) max_len = opts->max_code_len;
        if (opts->chunk_bytes && opts->chunk_bytes != 8) return WC_ERR_INVALID_ARG;
        if (opts->chunks_per_group) group = opts->chunks_per_group;
        if (opts->group_align) align = opts->group_align;
        if (opts->group_max_elems) max_elems = opts->group_max_elems;
        nthreads = opts->n_threads;
        kind = opts->layout;
        if (opts->seg_max_bits) seg_bits = opts->seg_max_bits;
        coder = opts->coder;
        if (opts->gap_bits) gap_bits = opts->gap_bits;
    }
    // The containers this library writes are the ones its GPU decoder takes:
    // blocks of a positive multiple of 8 elements (each lane writes whole
    // 8-element blocks), at most 4096 elements per group or segment (one
    // wave's eight merge steps), and for the lanes layout at most 15872 bits
    // per segment (one wave's 2 KB staging window).  The oracle's writer also
    // accepts other values of these fields; the GPU decoder refuses those
    // containers with WC_ERR_UNSUPPORTED.
    if (max_len < 1 || max_len > kMaxCodeLen || group < 1 || group > (1u << 20) || align < 8 || align % 8 ||
        max_elems < align || max_elems % align || max_elems > kDefaultMaxElems)
        return WC_ERR_INVALID_ARG;
    if (kind == WC_LAYOUT_CHUNKS) {
        // every block must fit in one group whatever its codes: align codewords of
        // up to max_len bits, starting anywhere in a chunk, touch at most G chunks
        if ((uint64_t)align * max_len + (kChunkBits - 1) > (uint64_t)kChunkBits * group) return WC_ERR_INVALID_ARG;
    } else if (kind == WC_LAYOUT_LANES) {
        // a segment's lane offsets are u16 bit counts; one block always fits
        // (rANS: A symbols cost at most 97 eighths each besides the 64 final states)
        if (seg_bits > kDefaultSegBits) return WC_ERR_INVALID_ARG;
        if (coder == WC_CODER_RANS ? seg_bits < kLanes * kRansStateBits ||
                                         97ull * align > 8ull * (seg_bits - kLanes * kRansStateBits)
                                   : (uint64_t)align * max_len > seg_bits)
            return WC_ERR_INVALID_ARG;
    } else {
        return WC_ERR_INVALID_ARG;
    }
    if (!kBf16 && kind != WC_LAYOUT_LANES) return WC_ERR_INVALID_ARG;   // code planes: lanes layout only
    if (coder != WC_CODER_HUFFMAN && (coder != WC_CODER_RANS || kind != WC_LAYOUT_LANES)) return WC_ERR_INVALID_ARG;
    if (gap_bits != kGapBitsByte && (gap_bits != kGapBitsPacked || kind != WC_LAYOUT_CHUNKS)) return WC_ERR_INVALID_ARG;

    SourceT<T> src;
    uint64_t n = 0;
    for (uint32_t k = 0; k < n_tensors; ++k) {
        if (numels[k] && !tensors[k]) return WC_ERR_INVALID_ARG;
        if (numels[k] > (1ull << 40) || n + numels[k] > (1ull << 40)) return WC_ERR_INVALID_ARG;
        src.ptr.push_back(tensors[k]);
        src.begin.push_back(n);
        src.size.push_back(numels[k]);
        n += numels[k];
    }
    if (nthreads == 0) nthreads = std::max(1u, std::thread::hardware_concurrency());
    nthreads = (unsigned)std::min<uint64_t>(nthreads, std::max<uint64_t>(1, n / 65536));
    nthreads = std::min(nthreads, 64u);
    // element ranges of the threads, on block boundaries
    const uint64_t n_blocks = div_up(n, align);
    std::vector<uint64_t> r0(nthreads + 1);
    for (unsigned t = 0; t <= nthreads; ++t) r0[t] = std::min<uint64_t>(n, n_blocks * t / nthreads * align);

    // 1-2. exponent histogram
    std::vector<std::array<uint64_t, 256>> hist_t(nthreads);
    parallel_for(nthreads, [&](unsigned t) {
        auto& h = hist_t[t];
        h.fill(0);
        src.for_range(r0[t], r0[t + 1], [&](uint64_t, const T* p, uint64_t k) {
            for (uint64_t j = 0; j < k; ++j) ++h[symbol_of(p[j])];
        });
    });
    uint64_t hist[256] = {0};
    for (auto& h : hist_t)
        for (int s = 0; s < 256; ++s) hist[s] += h[s];
    if (coder == WC_CODER_RANS)
        return write_lanes_rans(src, n, n_tensors, hist, align, max_elems, seg_bits, nthreads, blob, blob_bytes);

    // 3-4. code lengths and canonical codes
    uint8_t len[256];
    uint32_t code[256];
    int st = limited_code_lengths(hist, max_len, len);
    if (st != WC_OK) return st;
    canonical_codes(len, code);

    // bit offset of every thread's first codeword
    std::vector<uint64_t> tbits(nthreads + 1, 0);
    for (unsigned t = 0; t < nthreads; ++t) {
        uint64_t b = 0;
        for (int s = 0; s < 256; ++s) b += hist_t[t][s] * len[s];
        tbits[t + 1] = tbits[t] + b;
    }
    const uint64_t stream_bits = tbits[nthreads];

    // 5. groups: bit offset of every block, then the longest runs of blocks
    // whose codewords touch at most G chunks, of at most max_elems elements
    std::vector<uint64_t> block_bit(n_blocks + 1, 0);
    parallel_for(nthreads, [&](unsigned t) {
        uint64_t pos = tbits[t];
        src.for_range(r0[t], r0[t + 1], [&](uint64_t gi, const T* p, uint64_t k) {
            for (uint64_t j = 0; j < k; ++j) {
                if ((gi + j) % align == 0) block_bit[(gi + j) / align] = pos;
                pos += len[symbol_of(p[j])];
            }
        });
    });
    block_bit[n_blocks] = stream_bits;
    if (kind == WC_LAYOUT_LANES)
        return write_lanes(src, n, n_tensors, len, code, max_len, align, max_elems, seg_bits, block_bit, stream_bits,
                           nthreads, blob, blob_bytes);
    std::vector<uint64_t> g_elem{0}, g_bit{0};
    for (uint64_t k0 = 0; k0 < n_blocks;) {
        uint64_t k1 = k0 + 1;
        const uint64_t k_cap = k0 + max_elems / align;
        while (k1 < n_blocks && k1 < k_cap && chunk_span(block_bit[k0], block_bit[k1 + 1]) <= group) ++k1;
        g_elem.push_back(std::min<uint64_t>(k1 * align, n));
        g_bit.push_back(block_bit[k1]);
        k0 = k1;
    }
    const uint64_t n_groups = g_elem.size() - 1;
    Header h = layout(n, stream_bits, n_tensors, max_len, group, align, max_elems, n_groups, gap_bits);

    uint8_t* out = (uint8_t*)std::aligned_alloc(kAlign, h.total_bytes);
    if (!out) return WC_ERR_NOMEM;
    {   // zero everything but the sm plane (written in full below)
        const uint64_t zero_end = h.off_sm;
        parallel_for(nthreads, [&](unsigned t) {
            uint64_t a = zero_end * t / nthreads, b = zero_end * (t + 1) / nthreads;
            std::memset(out + a, 0, b - a);
        });
        std::memset(out + h.off_sm + n, 0, h.total_bytes - h.off_sm - n);
    }
    write_header(out, h);
    std::memcpy(out + h.off_code_len, len, 256);
    for (uint32_t k = 0; k < n_tensors; ++k) {
        store_le<uint64_t>(out + h.off_tensors + 16ull * k, src.begin[k]);
        store_le<uint64_t>(out + h.off_tensors + 16ull * k + 8, src.size[k]);
    }
    for (uint64_t g = 0; g <= n_groups; ++g) {
        store_le<uint64_t>(out + h.off_groups + kGroupEntryBytes * g, g_elem[g]);
        store_le<uint64_t>(out + h.off_groups + kGroupEntryBytes * g + 8, g_bit[g]);
    }
    uint8_t* stream = out + h.off_stream;
    // packed gaps are collected one byte per chunk, then packed
    std::vector<uint8_t> gap_bytes(gap_bits == kGapBitsPacked ? h.n_chunks : 0);
    uint8_t* gap = gap_bits == kGapBitsPacked ? gap_bytes.data() : out + h.off_gap;
    uint8_t* sm = out + h.off_sm;

    // 6. pack, plane split and per-chunk gaps, per element range
    parallel_for(nthreads, [&](unsigned t) {
        const uint64_t i0 = r0[t], i1 = r0[t + 1];
        if (i0 == i1) return;
        uint64_t pos = tbits[t];                                     // start bit of element i0
        uint64_t prev = i0 ? pos - len[exponent_of(src.at(i0 - 1))] : 0;
        bool first_elem = (i0 == 0);
        uint64_t wbyte = pos >> 3;                                   // next byte to write
        uint32_t acc = 0;
        int nacc = (int)(pos & 7);                                   // leading bits belong to the previous range
        bool shared_head = nacc != 0;
        auto put = [&](uint8_t v) {
            if (shared_head) {
                __atomic_fetch_or(stream + wbyte, v, __ATOMIC_RELAXED);
                shared_head = false;
            } else {
                stream[wbyte] = v;
            }
            ++wbyte;
        };
        src.for_range(i0, i1, [&](uint64_t gi, const T* p, uint64_t k) {
            for (uint64_t j = 0; j < k; ++j) {
                const uint16_t b = p[j];
                const uint8_t e = exponent_of(b);
                sm[gi + j] = sign_mantissa_of(b);
                if (first_elem || (prev >> 6) != (pos >> 6)) gap[pos >> 6] = (uint8_t)(pos & 63);
                first_elem = false;
                const int L = len[e];
                acc = (acc << L) | code[e];
                nacc += L;
                while (nacc >= 8) {
                    nacc -= 8;
                    put((uint8_t)(acc >> nacc));
                }
                acc &= (1u << nacc) - 1u;
                prev = pos;
                pos += L;
            }
        });
        if (nacc) __atomic_fetch_or(stream + wbyte, (uint8_t)(acc << (8 - nacc)), __ATOMIC_RELAXED);
        if (t + 1 == nthreads) {
            // chunks after the last codeword start point at the stream end
            for (uint64_t c = (prev >> 6) + 1; c < h.n_chunks; ++c) gap[c] = (uint8_t)(stream_bits - 64 * c);
        }
    });
    if (gap_bits == kGapBitsPacked) {
        // 8 gaps fill 5 bytes: threads take runs of whole 8-chunk groups
        uint8_t* packed = out + h.off_gap;
        const uint64_t n8 = div_up(h.n_chunks, 8);
        parallel_for(nthreads, [&](unsigned t) {
            for (uint64_t q = n8 * t / nthreads; q < n8 * (t + 1) / nthreads; ++q) {
                uint64_t v = 0;
                for (uint64_t c = 8 * q; c < std::min<uint64_t>(8 * q + 8, h.n_chunks); ++c)
                    v |= (uint64_t)(gap_bytes[c] & 31u) << (5 * (c - 8 * q));
                for (uint64_t k = 5 * q; k < std::min<uint64_t>(5 * q + 5, div_up(5 * h.n_chunks, 8)); ++k)
                    packed[k] = (uint8_t)(v >> (8 * (k - 5 * q)));
            }
        });
    }

    *blob = out;
    *blob_bytes = h.total_bytes;
    return WC_OK;
}

}  // namespace
}  // namespace wc

extern "C" int wc_encode_host(const uint16_t* const* tensors, const uint64_t* numels, uint32_t n_tensors,
                              const wc_encode_opts* opts, uint8_t** blob, uint64_t* blob_bytes) {
    return wc::encode_impl<uint16_t>(tensors, numels, n_tensors, opts, blob, blob_bytes);
}

extern "C" int wc_encode_u8_host(const uint8_t* const* tensors, const uint64_t* numels, uint32_t n_tensors,
                                 const wc_encode_opts* opts, uint8_t** blob, uint64_t* blob_bytes) {
    return wc::encode_impl<uint8_t>(tensors, numels, n_tensors, opts, blob, blob_bytes);
}

extern "C" void wc_free_host(uint8_t* blob) { std::free(blob); }
