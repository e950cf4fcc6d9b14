// decode.hip -- gfx950 kernels of libwc: decode-table construction and the
// block-level decode of an exponent-Huffman bf16 container.
//
// Design points taken from the DFloat11 page ("70% Size, 100% Accuracy:
// Lossless LLM Compression for Efficient GPU Inference via Dynamic-Length
// Float", abstract): (i) the big code lookup is split into compact tables
// that live in on-chip memory (here: LDS of each workgroup); (ii) a two-phase
// kernel coordinates where each thread reads and writes through small
// auxiliary variables (here: a per-chunk bit offset `gap` and a per-group
// first output index `group_start`); (iii) a whole transformer block is
// decoded by one launch (here: every group of a multi-tensor container).
//
// Work decomposition on CDNA4: one workgroup of 256 lanes (4 wave64s) owns a
// group of 256 chunks of 64 stream bits; lane t owns chunk t of the group.
//   phase 1  each lane counts the codewords that START in its chunk, several
//            per lookup of a codeword-start table;
//   scan     wave64 inclusive scan with DPP row shifts and row broadcasts,
//            then across the 4 waves through LDS -> each lane's first output;
//   phase 2  each lane decodes its codewords again, up to three per lookup of
//            a multi-codeword table, and stages the exponent bytes in LDS at
//            their final group-relative place.  A lookup always writes three
//            bytes; the ones past the lane's range are rewritten afterwards by
//            the lane that owns them (its first two symbols are kept aside);
//   merge    the workgroup joins the group's sign+mantissa bytes (prefetched
//            with 16-byte loads while the phases run) with the staged
//            exponents in integer registers and writes bf16 with 16-byte stores.
// Workgroups are persistent: each stages the tables once and loops over
// groups, loading the next group's chunk while it works on the current one.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace wc {
namespace {

constexpr uint32_t kCodeLimit = 24;
constexpr uint32_t kWaves = kDecodeThreads / 64;

struct LongTables {
    const uint32_t* count;
    const uint32_t* first;
    const uint32_t* base;
    const uint8_t* sorted;
};

// Canonical decode of a codeword longer than the table index.  `win` holds at
// least 24 valid stream bits, MSB-aligned.  Returns the length; the symbol
// goes to *sym.  A window that matches no code (only in a corrupted stream)
// decodes as a 24-bit codeword of the first sorted symbol.
__device__ __forceinline__ uint32_t decode_long(uint32_t win, uint32_t first_len, const LongTables& t,
                                                uint32_t* sym) {
    uint32_t L = first_len;
    uint32_t idx = 0;
#pragma unroll 1
    for (; L <= kCodeLimit; ++L) {
        const uint32_t code = win >> (32u - L);
        const uint32_t off = code - t.first[L];
        if (off < t.count[L]) {
            idx = t.base[L] + off;
            break;
        }
    }
    if (L > kCodeLimit) L = kCodeLimit;
    *sym = t.sorted[idx & 255u];
    return L;
}

// Shift a 96-bit MSB-first register left by (32 - (s & 31)) bits.
__device__ __forceinline__ void consume(uint32_t& w0, uint32_t& w1, uint32_t& w2, uint32_t s) {
    w0 = __builtin_amdgcn_alignbit(w0, w1, s);
    w1 = __builtin_amdgcn_alignbit(w1, w2, s);
    w2 = __builtin_amdgcn_alignbit(w2, 0u, s);
}

// Inclusive prefix sum over a wave64 with DPP: row_shr 1/2/4/8 inside rows of
// 16 lanes, then row_bcast:15 (rows 1, 3) and row_bcast:31 (rows 2, 3).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);
    return x;
}

__device__ __forceinline__ uint64_t min_u64(uint64_t a, uint64_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Four bf16 words from four sign+mantissa bytes `s` and four exponent bytes `e`
// (byte k of each belongs to element k).  The bf16 word is
// (sm & 0x80) << 8 | e << 7 | (sm & 0x7F): a byte permute builds
// [sm_k, sign-extension of sm_k] per 16-bit half, which already holds the sign
// at bit 15 and the mantissa at bits 6..0; a bit-field insert then puts the
// exponent into bits 14..7.
__device__ __forceinline__ void join4(uint32_t s, uint32_t e, uint32_t& lo, uint32_t& hi) {
    const uint32_t s8 = s << 8;
    const uint32_t x01 = __builtin_amdgcn_perm(s8, s, 0x08010A00u);   // sm0, sext0, sm1, sext1
    const uint32_t x23 = __builtin_amdgcn_perm(s8, s, 0x09030B02u);   // sm2, sext2, sm3, sext3
    const uint32_t e02 = __builtin_amdgcn_perm(e, e, 0x03010200u);    // e0, e2, e1, e3
    lo = (0x7F807F80u & (e02 << 7)) | (~0x7F807F80u & x01);
    hi = (0x7F807F80u & (e02 >> 1)) | (~0x7F807F80u & x23);
}

struct Chunk {
    uint32_t d0, d1, d2, gap;   // raw little-endian stream words and the first-codeword offset
    uint64_t A, B;              // group output range [A, B)
};

__device__ __forceinline__ Chunk load_chunk(const DecodeParams& p, uint64_t g, uint32_t tid) {
    Chunk k;
    const uint64_t c = g * kDecodeThreads + tid;
    k.d0 = k.d1 = k.d2 = k.gap = 0;
    if (c < p.n_chunks) {
        const uint2 d01 = *reinterpret_cast<const uint2*>(p.stream + 8 * c);
        k.d0 = d01.x;
        k.d1 = d01.y;
        k.d2 = *reinterpret_cast<const uint32_t*>(p.stream + 8 * c + 8);
        k.gap = p.gap[c];
    }
    // group bounds through the vector memory path (waited on with the chunk)
    const uint2 a = *reinterpret_cast<const uint2*>(p.group_start + g);
    const uint2 b = *reinterpret_cast<const uint2*>(p.group_start + g + 1);
    k.A = ((uint64_t)a.y << 32) | a.x;
    k.B = ((uint64_t)b.y << 32) | b.x;
    return k;
}

// A lane's chunk ready for decoding: 96 stream bits MSB-first, shifted so that
// the first codeword starting in the chunk is at the top; `bits` is the number
// of bits after it in which further codewords may start.  Also the group range.
struct State {
    uint32_t w0, w1, w2;
    int32_t bits;
    uint64_t A, B;
};

__device__ __forceinline__ State make_state(const DecodeParams& p, const Chunk& k, uint64_t g, uint32_t tid) {
    State s;
    const uint64_t c = g * kDecodeThreads + tid;
    uint32_t w0 = __builtin_bswap32(k.d0), w1 = __builtin_bswap32(k.d1), w2 = __builtin_bswap32(k.d2);
    uint32_t end = 0;
    if (c < p.n_chunks) {
        const uint64_t left = p.stream_bits - 64 * c;
        end = left < 64 ? (uint32_t)left : 64u;
    }
    const uint64_t h01 = ((uint64_t)w0 << 32 | w1) << k.gap;
    const uint64_t h12 = ((uint64_t)w1 << 32 | w2) << k.gap;
    s.w0 = (uint32_t)(h01 >> 32);
    s.w1 = (uint32_t)(h12 >> 32);
    s.w2 = w2 << k.gap;
    s.bits = (int32_t)end - (int32_t)k.gap;
    s.A = uniform64(k.A);
    s.B = uniform64(k.B);
    return s;
}

template <int KC, int KD>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeParams p) {
    __shared__ __attribute__((aligned(16))) uint32_t s_cnt[1u << KC];
    __shared__ __attribute__((aligned(16))) uint32_t s_dec[1u << KD];
    __shared__ __attribute__((aligned(16))) uint32_t s_long[160];
    __shared__ uint32_t s_wave[kWaves];
    extern __shared__ __attribute__((aligned(16))) uint8_t ebuf[];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;

    // stage the decode tables (built once per container) into LDS
    {
        const uint4* src = reinterpret_cast<const uint4*>(p.tables);
        for (uint32_t i = tid; i < (1u << KC) / 4; i += kDecodeThreads)
            reinterpret_cast<uint4*>(s_cnt)[i] = src[i];
        src += (1u << KC) / 4;
        for (uint32_t i = tid; i < (1u << KD) / 4; i += kDecodeThreads)
            reinterpret_cast<uint4*>(s_dec)[i] = src[i];
        src += (1u << KD) / 4;
        if (tid < 40) reinterpret_cast<uint4*>(s_long)[tid] = src[tid];
    }
    LongTables lt;
    lt.count = s_long;
    lt.first = s_long + 32;
    lt.base = s_long + 64;
    lt.sorted = reinterpret_cast<const uint8_t*>(s_long + 96);
    __syncthreads();

    uint64_t g = blockIdx.x;
    if (g >= p.n_groups) return;
    State cur = make_state(p, load_chunk(p, g, tid), g, tid);

    for (;;) {
        // no register read below waits on memory until the next group's chunk
        // is consumed, after phase 2: the loads issued here stay in flight
        const uint64_t A = cur.A;
        const uint64_t B = cur.B;
        const uint64_t A0 = A & ~15ull;
        const uint32_t nblk = (uint32_t)((B - A0 + 15) >> 4);
        uint32_t w0 = cur.w0, w1 = cur.w1, w2 = cur.w2;

        // sign+mantissa bytes of this lane's first two merge blocks (block indexes
        // past the group are clamped to the plane's last block: loaded, never used)
        const uint4 sm0 = *reinterpret_cast<const uint4*>(p.sm + min_u64(A0 + 16ull * tid, p.sm_last));
        const uint4 sm1 = *reinterpret_cast<const uint4*>(p.sm + min_u64(A0 + 16ull * (tid + kDecodeThreads), p.sm_last));

        // next group's chunk and bounds
        const uint64_t gn = g + gridDim.x;
        const bool more = gn < p.n_groups;
        Chunk nxt;
        if (more) nxt = load_chunk(p, gn, tid);

        // phase 1: count the codewords starting in [start, end)
        uint32_t count = 0;
        {
            uint32_t a0 = w0, a1 = w1, a2 = w2;
            int32_t r = cur.bits;
            while (r > 0) {
                uint32_t e = s_cnt[a0 >> (32 - KC)];
                if (e == 0) {                                   // a code longer than KC bits (rare)
                    uint32_t sym;
                    const uint32_t L = decode_long(a0, KC + 1, lt, &sym);
                    e = ((32u - L) & 31u) | (L << 8) | (1u << 16);
                }
                count += __popc(__builtin_amdgcn_ubfe(e, 16, (uint32_t)(r < 16 ? r : 16)));
                r -= (int32_t)((e >> 8) & 0xFFu);
                consume(a0, a1, a2, e);
            }
        }

        // block-wide exclusive scan of the counts
        const uint32_t incl = wave_inclusive_scan(count);
        if (lane == 63) s_wave[wave] = incl;
        __syncthreads();
        uint32_t before = 0;
#pragma unroll
        for (uint32_t w = 0; w < kWaves; ++w) before += (w < wave) ? s_wave[w] : 0u;
        const uint32_t pos = before + incl - count;

        // phase 2: decode again and stage the exponent bytes; never past the
        // group's element range, even for a corrupted stream
        const uint32_t n_group = (uint32_t)(B - A);
        const uint32_t room = pos < n_group ? n_group - pos : 0u;
        const uint32_t todo = count < room ? count : room;
        const uint32_t o_first = (uint32_t)(A & 15u) + pos;
        const uint32_t o_end = o_first + todo;
        uint8_t* q = ebuf + o_first;          // LDS address of the next symbol
        uint8_t* const q_end = ebuf + o_end;
        auto lookup = [&]() {
            uint32_t e = s_dec[w0 >> (32 - KD)];
            if (e == 0) {                                       // a code longer than KD bits (rare)
                uint32_t sym;
                const uint32_t L = decode_long(w0, KD + 1, lt, &sym);
                e = ((32u - L) & 31u) | (1u << 5) | (sym << 8);
            }
            const uint32_t t = __builtin_amdgcn_alignbit(e, e, 8);   // symbols in bytes 0, 1, 2
            q[0] = (uint8_t)t;
            q[1] = (uint8_t)(e >> 16);
            q[2] = (uint8_t)(t >> 16);
            q += (e >> 5) & 3u;
            consume(w0, w1, w2, e);
            return e;
        };
        // the first two symbols are kept aside: the left neighbour's last
        // three-byte write may land on them
        uint32_t head = 0;
        if (q < q_end) {
            const uint32_t e = lookup();
            head = (e >> 8) & 0xFFFFu;
            if (((e >> 5) & 3u) == 1u && q < q_end) head = (head & 0xFFu) | (lookup() & 0xFF00u);
        }
        while (q < q_end) lookup();
        __syncthreads();
        if (todo >= 1) ebuf[o_first] = (uint8_t)head;
        if (todo >= 2) ebuf[o_first + 1] = (uint8_t)(head >> 8);
        // consume the next group's chunk now, before the merge issues its stores
        State next = cur;
        if (more) next = make_state(p, nxt, gn, tid);
        __syncthreads();

        // merge: 16 elements per lane per step, 16-byte loads and stores
        auto merge_block = [&](uint32_t b, const uint4& s4) {
            const uint4 e4 = *reinterpret_cast<const uint4*>(ebuf + 16 * b);
            uint32_t o8[8];
            join4(s4.x, e4.x, o8[0], o8[1]);
            join4(s4.y, e4.y, o8[2], o8[3]);
            join4(s4.z, e4.z, o8[4], o8[5]);
            join4(s4.w, e4.w, o8[6], o8[7]);
            const uint64_t base = A0 + 16ull * b;
            if (base >= A && base + 16 <= B) {
                uint4* dst4 = reinterpret_cast<uint4*>(p.out + base);
                dst4[0] = make_uint4(o8[0], o8[1], o8[2], o8[3]);
                dst4[1] = make_uint4(o8[4], o8[5], o8[6], o8[7]);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint64_t idx = base + i;
                    if (idx >= A && idx < B) p.out[idx] = (uint16_t)(o8[i >> 1] >> (16 * (i & 1)));
                }
            }
        };
        if (tid < nblk) merge_block(tid, sm0);
        if (tid + kDecodeThreads < nblk) merge_block(tid + kDecodeThreads, sm1);
        for (uint32_t b = tid + 2 * kDecodeThreads; b < nblk; b += kDecodeThreads)
            merge_block(b, *reinterpret_cast<const uint4*>(p.sm + A0 + 16ull * b));
        if (!more) break;
        __syncthreads();   // ebuf and s_wave are reused by the next group
        g = gn;
        cur = next;
    }
}

// Decode tables from the 256 code lengths (one workgroup, once per plan).
template <int KC, int KD>
__global__ __launch_bounds__(1024) void build_tables_kernel(CodeLens lens, uint32_t* tables) {
    constexpr uint32_t kS = kSingleBits;
    static_assert(KC <= (int)kSingleBits && KD <= (int)kSingleBits, "index wider than the single table");
    __shared__ uint32_t count[32], first[32], base[32];
    __shared__ uint8_t sorted[256];
    __shared__ uint32_t single[1u << kS];   // symbol | length << 8, or ~0 for a longer code
    const uint32_t tid = threadIdx.x;
    if (tid == 0) {
        for (int L = 0; L < 32; ++L) count[L] = 0;
        for (int s = 0; s < 256; ++s) {
            sorted[s] = 0;
            if (lens.len[s] >= 1 && lens.len[s] <= kCodeLimit) ++count[lens.len[s]];
        }
        uint32_t code = 0, rank = 0;
        for (uint32_t L = 1; L < 32; ++L) {
            code = (code + (L > 1 ? count[L - 1] : 0u)) << 1;
            first[L] = code;             // first code of length L (canonical)
            base[L] = rank;
            for (int s = 0; s < 256; ++s)
                if (lens.len[s] == L) sorted[rank++] = (uint8_t)s;
        }
        first[0] = 0;
        base[0] = 0;
    }
    __syncthreads();
    for (uint32_t w = tid; w < (1u << kS); w += blockDim.x) {
        uint32_t entry = 0xFFFFFFFFu;
        for (uint32_t L = 1; L <= kS; ++L) {
            const uint32_t off = (w >> (kS - L)) - first[L];
            if (off < count[L]) {
                entry = (uint32_t)sorted[(base[L] + off) & 255u] | (L << 8);
                break;
            }
        }
        single[w] = entry;
    }
    __syncthreads();
    // codeword-start table
    for (uint32_t w = tid; w < (1u << KC); w += blockDim.x) {
        uint32_t at = 0, mask = 0;
        while (at < (uint32_t)KC) {
            const uint32_t x = ((w << at) & ((1u << KC) - 1u)) << (kS - KC);
            const uint32_t s = single[x];
            if (s == 0xFFFFFFFFu) break;
            const uint32_t L = s >> 8;
            if (at + L > (uint32_t)KC) break;
            mask |= 1u << at;
            at += L;
        }
        tables[w] = at ? (((32u - at) & 31u) | (at << 8) | (mask << 16)) : 0u;
    }
    // multi-codeword table
    for (uint32_t w = tid; w < (1u << KD); w += blockDim.x) {
        uint32_t at = 0, n = 0, syms = 0;
        while (n < 3) {
            const uint32_t x = ((w << at) & ((1u << KD) - 1u)) << (kS - KD);
            const uint32_t s = single[x];
            if (s == 0xFFFFFFFFu) break;
            const uint32_t L = s >> 8;
            if (at + L > (uint32_t)KD) break;
            syms |= (s & 0xFFu) << (8 * n);
            ++n;
            at += L;
        }
        tables[(1u << KC) + w] = n ? (((32u - at) & 31u) | (n << 5) | (syms << 8)) : 0u;
    }
    uint32_t* tail = tables + (1u << KC) + (1u << KD);
    if (tid < 32) {
        tail[tid] = count[tid];
        tail[32 + tid] = first[tid];
        tail[64 + tid] = base[tid];
    }
    if (tid < 64) {
        tail[96 + tid] = (uint32_t)sorted[4 * tid] | ((uint32_t)sorted[4 * tid + 1] << 8) |
                         ((uint32_t)sorted[4 * tid + 2] << 16) | ((uint32_t)sorted[4 * tid + 3] << 24);
    }
}

template <int KC, int KD>
struct Variant {
    static hipError_t launch(const DecodeParams& p, uint32_t grid, uint32_t ebuf, hipStream_t stream) {
        hipLaunchKernelGGL((decode_kernel<KC, KD>), dim3(grid), dim3(kDecodeThreads), ebuf, stream, p);
        return hipGetLastError();
    }
    static int blocks_per_cu(uint32_t ebuf) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<KC, KD>, kDecodeThreads, ebuf) !=
            hipSuccess)
            return 0;
        return n;
    }
    static hipError_t build(const CodeLens& lens, uint32_t* d_tables, hipStream_t stream) {
        hipLaunchKernelGGL((build_tables_kernel<KC, KD>), dim3(1), dim3(1024), 0, stream, lens, d_tables);
        return hipGetLastError();
    }
};

template <typename F>
auto dispatch(uint32_t kc, uint32_t kd, F&& f) {
    if (kc == 12 && kd == 12) return f(Variant<12, 12>{});
    if (kc == 12 && kd == 11) return f(Variant<12, 11>{});
    if (kc == 12 && kd == 10) return f(Variant<12, 10>{});
    if (kc == 11 && kd == 11) return f(Variant<11, 11>{});
    return f(Variant<10, 10>{});
}

}  // namespace

uint32_t decode_lds_bytes(uint32_t count_bits, uint32_t decode_bits, uint32_t ebuf_bytes) {
    return table_words(count_bits, decode_bits) * 4u + kWaves * 4u + ebuf_bytes;
}

int decode_blocks_per_cu(uint32_t count_bits, uint32_t decode_bits, uint32_t ebuf_bytes) {
    if (!supported_table_bits(count_bits, decode_bits)) return 0;
    return dispatch(count_bits, decode_bits, [&](auto v) { return decltype(v)::blocks_per_cu(ebuf_bytes); });
}

hipError_t launch_build_tables(const CodeLens& lens, uint32_t count_bits, uint32_t decode_bits, uint32_t* d_tables,
                               hipStream_t stream) {
    if (!supported_table_bits(count_bits, decode_bits)) return hipErrorInvalidValue;
    return dispatch(count_bits, decode_bits, [&](auto v) { return decltype(v)::build(lens, d_tables, stream); });
}

hipError_t launch_decode(const DecodeParams& p, uint32_t count_bits, uint32_t decode_bits, uint32_t grid,
                         uint32_t ebuf_bytes, hipStream_t stream) {
    if (!supported_table_bits(count_bits, decode_bits)) return hipErrorInvalidValue;
    return dispatch(count_bits, decode_bits,
                    [&](auto v) { return decltype(v)::launch(p, grid, ebuf_bytes, stream); });
}

}  // namespace wc
