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
// Work decomposition on CDNA4: a workgroup of 256 lanes (4 wave64s) owns two
// adjacent groups (512 chunks of 64 stream bits, one contiguous output range);
// lane t owns chunks 2t and 2t+1 of that range and decodes them as two
// independent chains, so two table lookups are in flight per lane.
//   phase 1  each chain counts the codewords that START in its chunk, several
//            per lookup of a codeword-start table;
//   scan     wave64 inclusive scan with DPP row shifts and row broadcasts,
//            then across the 4 waves through LDS -> each lane's first output;
//   phase 2  each chain decodes its codewords again, up to four per lookup of
//            a multi-codeword table, and stages the exponent bytes in LDS at
//            their final place (four byte stores per lookup; unaligned dword
//            LDS stores stall on CDNA4).  Bytes written past a chain's range
//            land on the next chain's first three bytes, which that chain
//            keeps aside and rewrites after a barrier; writes of a finished
//            chain go to a per-lane dummy slot;
//   merge    the workgroup joins the sign+mantissa bytes (prefetched while
//            the phases run) with the staged exponents in integer registers,
//            8 elements per lane and step, and writes bf16 with 16-byte stores
//            that are contiguous across the lanes of a wave.
// Workgroups are persistent: each stages the tables once and loops over its
// units, loading the next unit's chunks while it works on the current one.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace wc {
namespace {

constexpr uint32_t kCodeLimit = 24;
constexpr uint32_t kWaves = kDecodeThreads / 64;
constexpr uint32_t kUnitChunks = kDecodeThreads * kChunksPerLane;   // chunks per workgroup unit
// bf16 output is written with non-temporal 16-byte stores: it is not read
// again by this kernel and streams past the caches
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kPrefetchBlocks = 8;                            // merge blocks per lane loaded ahead

struct LongTables {
    const uint32_t* count;
    const uint32_t* first;
    const uint32_t* base;
    const uint8_t* sorted;
    const uint16_t* l2;   // second level: (length << 8) | rotated symbol, or 0
    uint32_t l2_first;    // KD-bit prefix of the first code longer than KD
    uint32_t l2_n;        // long-code prefixes the second level covers (at most kL2Prefixes)
};

// Canonical decode of a codeword longer than the table index.  `win` holds at
// least 24 valid stream bits, MSB-aligned.  Returns the length; the (rotated)
// symbol goes to *sym.  A window that matches no code (only in a corrupted
// stream) decodes as a 24-bit codeword of the first sorted symbol.
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

// Four bf16 words from four sign+mantissa bytes `s` and four rotated exponent
// bytes `e` (byte k of each belongs to element k).  With e' = ror8(e, 1), the
// bf16 low byte is (e' & 0x80) | (sm & 0x7F) and the high byte is
// (sm & 0x80) | (e' & 0x7F); two bit-field inserts build all low and all high
// bytes, two byte permutes interleave them.
__device__ __forceinline__ void join4(uint32_t s, uint32_t e, uint32_t& lo, uint32_t& hi) {
    const uint32_t lows = (0x80808080u & e) | (~0x80808080u & s);
    const uint32_t highs = (0x80808080u & s) | (~0x80808080u & e);
    lo = __builtin_amdgcn_perm(highs, lows, 0x05010400u);
    hi = __builtin_amdgcn_perm(highs, lows, 0x07030602u);
}

// Raw loads for one lane of one unit: 20 stream bytes covering its two chunks
// plus the halo, both gaps, and the unit's output range.
struct Raw {
    uint4 d;        // stream bytes [8a, 8a + 16)
    uint32_t d4;    // stream bytes [8a + 16, 8a + 20)
    uint32_t gaps;  // gap[a] | gap[a + 1] << 8 (the second byte is not used when a + 1 is past the end)
    uint64_t A;     // first element of the unit
    uint32_t B;     // low 32 bits of its end (B - A < 2^32: a unit holds at most 2^15 codewords)
};

__device__ __forceinline__ Raw load_raw(const DecodeParams& p, uint64_t u, uint32_t tid) {
    Raw r;
    const uint64_t a = u * kUnitChunks + kChunksPerLane * tid;
    r.d = make_uint4(0, 0, 0, 0);
    r.d4 = 0;
    r.gaps = 0;
    if (a < p.n_chunks) {
        // a is even: the stream load is 16-byte aligned and the gap pair 2-byte
        // aligned; gap[a + 1] lies inside the container even when a + 1 ==
        // n_chunks (the next section follows), and is then ignored.
        r.d = *reinterpret_cast<const uint4*>(p.stream + 8 * a);
        r.d4 = *reinterpret_cast<const uint32_t*>(p.stream + 8 * a + 16);
        r.gaps = *reinterpret_cast<const uint16_t*>(p.gap + a);
    }
    const uint64_t g0 = u * kGroupsPerBlock;
    const uint64_t g1 = min_u64(g0 + kGroupsPerBlock, p.n_groups);
    const uint2 x = *reinterpret_cast<const uint2*>(p.group_start + g0);
    r.A = ((uint64_t)x.y << 32) | x.x;
    r.B = *reinterpret_cast<const uint32_t*>(p.group_start + g1);   // little-endian low word
    return r;
}

// A chain ready for decoding: 96 stream bits MSB-first, shifted so that the
// first codeword starting in the chunk is at the top; `bits` counts the bits
// after that point in which further codewords may start.
struct Chain {
    uint32_t w0, w1, w2;
    int32_t bits;
};

__device__ __forceinline__ Chain make_chain(const DecodeParams& p, uint64_t c, uint32_t d0, uint32_t d1, uint32_t d2,
                                            uint32_t gap) {
    Chain h;
    const uint32_t w0 = __builtin_bswap32(d0), w1 = __builtin_bswap32(d1), w2 = __builtin_bswap32(d2);
    uint32_t end = 0;
    if (c < p.n_chunks) {
        const uint64_t left = p.stream_bits - 64 * c;
        end = left < 64 ? (uint32_t)left : 64u;
    } else {
        gap = 0;
    }
    const uint64_t h01 = ((uint64_t)w0 << 32 | w1) << gap;
    const uint64_t h12 = ((uint64_t)w1 << 32 | w2) << gap;
    h.w0 = (uint32_t)(h01 >> 32);
    h.w1 = (uint32_t)(h12 >> 32);
    h.w2 = w2 << gap;
    h.bits = (int32_t)end - (int32_t)gap;
    return h;
}

struct Unit {
    Chain a, b;
    uint64_t A;
    uint32_t B;
};

__device__ __forceinline__ Unit make_unit(const DecodeParams& p, const Raw& r, uint64_t u, uint32_t tid) {
    Unit x;
    const uint64_t c = u * kUnitChunks + kChunksPerLane * tid;
    x.a = make_chain(p, c, r.d.x, r.d.y, r.d.z, r.gaps & 0xFFu);
    x.b = make_chain(p, c + 1, r.d.z, r.d.w, r.d4, (r.gaps >> 8) & 0xFFu);
    x.A = uniform64(r.A);
    x.B = __builtin_amdgcn_readfirstlane(r.B);
    return x;
}

// First codeword of a window whose first codeword is longer than KD bits:
// (length << 8) | rotated symbol.  Canonical codes longer than KD bits all
// have KD-bit prefixes >= l2_first; the second-level table, indexed by such a
// prefix and the kL2Bits bits after it, resolves every code of at most
// KD + kL2Bits bits with one lookup.  Longer codes, and prefixes past the
// table, take the length-by-length canonical search.
template <int KD>
__device__ __forceinline__ uint32_t long_code(uint32_t win, uint32_t first_len, const LongTables& t) {
    const uint32_t idx = (win >> (32 - KD - kL2Bits)) - (t.l2_first << kL2Bits);
    if (idx < (t.l2_n << kL2Bits)) {
        const uint32_t e = t.l2[idx];
        if (e != 0) return e;
    }
    uint32_t sym;
    const uint32_t L = decode_long(win, first_len, t, &sym);
    return (L << 8) | sym;
}

// Entry of the codeword-start table for a code longer than the index: one
// codeword start at offset 0, covering its L bits.
template <int KD>
__device__ __forceinline__ uint32_t long_count_entry(uint32_t win, uint32_t first_len, const LongTables& lt) {
    const uint32_t L = long_code<KD>(win, first_len, lt) >> 8;
    return ((32u - L) & 31u) | (L << 8) | (1u << 16);
}

// Entry of the multi-codeword table for a code longer than the index: one symbol.
template <int KD>
__device__ __forceinline__ uint2 long_decode_entry(uint32_t win, uint32_t first_len, const LongTables& lt) {
    const uint32_t c = long_code<KD>(win, first_len, lt);
    const uint32_t L = c >> 8;
    return make_uint2(((32u - L) & 31u) | (1u << 8) | (L << 16), c & 0xFFu);
}

// Store the (up to four) symbol bytes of entry e at q, or at the chain's
// dummy slot once it is past its end, and advance q by the entry's symbol
// count.  Byte stores: ds_write_b8 takes bits 7..0 of a register and the d16_hi
// form bits 23..16, so one byte permute feeds all four.
__device__ __forceinline__ void put4(uint8_t*& q, const uint8_t* q_end, uint8_t* dummy, const uint2& e) {
    uint8_t* dst = q < q_end ? q : dummy;
    const uint32_t odd = __builtin_amdgcn_perm(e.y, e.y, 0x0C030C01u);   // [s1, 0, s3, 0]
    dst[0] = (uint8_t)e.y;
    dst[1] = (uint8_t)odd;
    dst[2] = (uint8_t)(e.y >> 16);
    dst[3] = (uint8_t)(odd >> 16);
    q += (e.x >> 8) & 0xFFu;
}

template <int KC, int KD>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeParams p) {
    __shared__ __attribute__((aligned(16))) uint32_t s_cnt[1u << KC];
    __shared__ __attribute__((aligned(16))) uint2 s_dec[1u << KD];
    __shared__ __attribute__((aligned(16))) uint32_t s_long[kLongWords];
    __shared__ uint32_t s_wave[kWaves];
    __shared__ __attribute__((aligned(16))) uint8_t s_dummy[4 * kDecodeThreads];
    // dynamic: the unit's exponent staging (ebuf_bytes), then the second-level
    // table for the long-code prefixes this container has (l2_cap * 2^kL2Bits u16)
    extern __shared__ __attribute__((aligned(16))) uint8_t ebuf[];
    uint16_t* const s_l2 = reinterpret_cast<uint16_t*>(ebuf + p.ebuf_bytes);

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    uint8_t* const dummy = s_dummy + 4 * tid;

    // stage the decode tables (built once per container) into LDS
    {
        const uint4* src = reinterpret_cast<const uint4*>(p.tables);
        for (uint32_t i = tid; i < (1u << KC) / 4; i += kDecodeThreads)
            reinterpret_cast<uint4*>(s_cnt)[i] = src[i];
        src += (1u << KC) / 4;
        for (uint32_t i = tid; i < (2u << KD) / 4; i += kDecodeThreads)
            reinterpret_cast<uint4*>(s_dec)[i] = src[i];
        src += (2u << KD) / 4;
        if (tid < kLongWords / 4) reinterpret_cast<uint4*>(s_long)[tid] = src[tid];
        src += kLongWords / 4;
        for (uint32_t i = tid; i < (p.l2_cap << kL2Bits) / 8; i += kDecodeThreads)
            reinterpret_cast<uint4*>(s_l2)[i] = src[i];
    }
    __syncthreads();
    LongTables lt;
    lt.count = s_long;
    lt.first = s_long + 32;
    lt.base = s_long + 64;
    lt.sorted = reinterpret_cast<const uint8_t*>(s_long + 96);
    lt.l2 = s_l2;
    lt.l2_first = __builtin_amdgcn_readfirstlane(s_long[160]);
    lt.l2_n = min(__builtin_amdgcn_readfirstlane(s_long[161]), p.l2_cap);

    uint64_t u = blockIdx.x;
    if (u >= p.n_blocks) return;
    Unit cur = make_unit(p, load_raw(p, u, tid), u, tid);

    for (;;) {
        // Nothing below waits on memory until the next unit's loads are
        // consumed after phase 2, so the loads issued here stay in flight.
        // The unit's elements [A, B) are merged in blocks of 8 counted from
        // A0 = A rounded down to 64, so that the wave-wide accesses cover
        // whole cache lines; offsets inside the unit fit 32 bits, so every
        // global access is a uniform base plus a 32-bit lane offset.
        const uint64_t A = cur.A;
        const uint64_t A0 = A & ~(uint64_t)(kMergeAlign - 1);
        const uint32_t lo_rel = (uint32_t)(A - A0);
        const uint32_t hi_rel = cur.B - (uint32_t)A0;
        const uint32_t nblk = (hi_rel + kMergeElems - 1) / kMergeElems;

        // sign+mantissa bytes of this lane's first merge blocks; block indexes
        // past the unit are clamped to its last block (an L2 hit, never used).
        // With nblk >= 1 every block lies inside round_up(n, 8) <= the plane's
        // padded size; a unit with no block reads the plane's last piece.
        const uint32_t last_blk = nblk ? nblk - 1 : 0u;
        const uint8_t* const smu = p.sm + min_u64(A0, p.sm_last);
        uint16_t* const outu = p.out + A0;
        uint2 smv[kPrefetchBlocks];
#pragma unroll
        for (uint32_t k = 0; k < kPrefetchBlocks; ++k)
            smv[k] = *reinterpret_cast<const uint2*>(smu + kMergeElems * min(tid + k * kDecodeThreads, last_blk));

        const uint64_t un = u + gridDim.x;
        const bool more = un < p.n_blocks;
        Raw nxt;
        if (more) nxt = load_raw(p, un, tid);

        // phase 1: count the codewords starting in each chunk
        uint32_t ca = 0, cb = 0;
        {
            uint32_t a0 = cur.a.w0, a1 = cur.a.w1, a2 = cur.a.w2;
            uint32_t b0 = cur.b.w0, b1 = cur.b.w1, b2 = cur.b.w2;
            int32_t ra = cur.a.bits, rb = cur.b.bits;
            while (ra > 0 || rb > 0) {
                // both lookups are issued before the (rare) long-code branch
                uint32_t ea = s_cnt[a0 >> (32 - KC)];
                uint32_t eb = s_cnt[b0 >> (32 - KC)];
                if ((ea == 0) | (eb == 0)) {
                    if (ea == 0) ea = long_count_entry<KD>(a0, KC + 1, lt);
                    if (eb == 0) eb = long_count_entry<KD>(b0, KC + 1, lt);
                }
                ca += __popc(__builtin_amdgcn_ubfe(ea, 16, (uint32_t)min(max(ra, 0), 16)));
                cb += __popc(__builtin_amdgcn_ubfe(eb, 16, (uint32_t)min(max(rb, 0), 16)));
                ra -= (int32_t)((ea >> 8) & 0xFFu);
                rb -= (int32_t)((eb >> 8) & 0xFFu);
                consume(a0, a1, a2, ea);
                consume(b0, b1, b2, eb);
            }
        }

        // block-wide exclusive scan of the lane counts
        const uint32_t count = ca + cb;
        const uint32_t incl = wave_inclusive_scan(count);
        if (lane == 63) s_wave[wave] = incl;
        __syncthreads();
        uint32_t before = 0;
#pragma unroll
        for (uint32_t w = 0; w < kWaves; ++w) before += (w < wave) ? s_wave[w] : 0u;
        const uint32_t pos_a = before + incl - count;
        const uint32_t pos_b = pos_a + ca;

        // phase 2: decode again and stage the exponent bytes; a chain never
        // writes past the unit's element range, even for a corrupted stream
        const uint32_t n_unit = hi_rel - lo_rel;
        const uint32_t base = lo_rel;
        const uint32_t todo_a = min(ca, pos_a < n_unit ? n_unit - pos_a : 0u);
        const uint32_t todo_b = min(cb, pos_b < n_unit ? n_unit - pos_b : 0u);
        uint8_t* qa = ebuf + base + pos_a;
        uint8_t* qb = ebuf + base + pos_b;
        uint8_t* const qa_end = qa + todo_a;
        uint8_t* const qb_end = qb + todo_b;
        {
            uint32_t a0 = cur.a.w0, a1 = cur.a.w1, a2 = cur.a.w2;
            uint32_t b0 = cur.b.w0, b1 = cur.b.w1, b2 = cur.b.w2;
            auto step_a = [&]() {
                uint2 e = s_dec[a0 >> (32 - KD)];
                if (e.x == 0) e = long_decode_entry<KD>(a0, KD + 1, lt);
                put4(qa, qa_end, dummy, e);
                consume(a0, a1, a2, e.x);
                return e;
            };
            auto step_b = [&]() {
                uint2 e = s_dec[b0 >> (32 - KD)];
                if (e.x == 0) e = long_decode_entry<KD>(b0, KD + 1, lt);
                put4(qb, qb_end, dummy, e);
                consume(b0, b1, b2, e.x);
                return e;
            };
            // first lookups: each chain keeps its first three symbols aside
            uint32_t head_a, head_b, na, nb;
            {
                uint2 ea = s_dec[a0 >> (32 - KD)];
                uint2 eb = s_dec[b0 >> (32 - KD)];
                if ((ea.x == 0) | (eb.x == 0)) {
                    if (ea.x == 0) ea = long_decode_entry<KD>(a0, KD + 1, lt);
                    if (eb.x == 0) eb = long_decode_entry<KD>(b0, KD + 1, lt);
                }
                put4(qa, qa_end, dummy, ea);
                put4(qb, qb_end, dummy, eb);
                consume(a0, a1, a2, ea.x);
                consume(b0, b1, b2, eb.x);
                head_a = ea.y;
                head_b = eb.y;
                na = (ea.x >> 8) & 0xFFu;
                nb = (eb.x >> 8) & 0xFFu;
            }
            while (na < kHeadBytes && qa < qa_end) {   // rare: the first lookup held fewer symbols
                const uint2 e = step_a();
                head_a = (head_a & ((1u << (8 * na)) - 1u)) | (e.y << (8 * na));
                na += (e.x >> 8) & 0xFFu;
            }
            while (nb < kHeadBytes && qb < qb_end) {
                const uint2 e = step_b();
                head_b = (head_b & ((1u << (8 * nb)) - 1u)) | (e.y << (8 * nb));
                nb += (e.x >> 8) & 0xFFu;
            }
            while (qa < qa_end || qb < qb_end) {
                // both lookups are issued before the (rare) long-code branch
                uint2 ea = s_dec[a0 >> (32 - KD)];
                uint2 eb = s_dec[b0 >> (32 - KD)];
                if ((ea.x == 0) | (eb.x == 0)) {
                    if (ea.x == 0) ea = long_decode_entry<KD>(a0, KD + 1, lt);
                    if (eb.x == 0) eb = long_decode_entry<KD>(b0, KD + 1, lt);
                }
                put4(qa, qa_end, dummy, ea);
                put4(qb, qb_end, dummy, eb);
                consume(a0, a1, a2, ea.x);
                consume(b0, b1, b2, eb.x);
            }
            __syncthreads();
            uint8_t* ha = ebuf + base + pos_a;
            uint8_t* hb = ebuf + base + pos_b;
#pragma unroll
            for (uint32_t k = 0; k < kHeadBytes; ++k) {
                if (todo_a > k) ha[k] = (uint8_t)(head_a >> (8 * k));
                if (todo_b > k) hb[k] = (uint8_t)(head_b >> (8 * k));
            }
        }
        // consume the next unit's loads now, before the merge issues its stores
        Unit next = cur;
        if (more) next = make_unit(p, nxt, un, tid);
        __syncthreads();

        // Every prefetched block is consumed here, before any store of this
        // unit: a load still counted as pending at the next iteration (where
        // its registers are reloaded) would make that point wait for all
        // outstanding memory operations, the merge stores included.
#pragma unroll
        for (uint32_t k = 0; k < kPrefetchBlocks; ++k)
            asm volatile("" ::"v"(smv[k].x), "v"(smv[k].y));

        // merge: 8 elements per lane per step; consecutive lanes take
        // consecutive blocks, so each wave-wide 8-byte load and 16-byte store
        // covers one contiguous range (whole 64-byte segments)
        // (whole blocks inside [A, B) only: the block holding A and the one
        // holding B may be shared with the neighbouring units and are written
        // element by element below)
        const uint32_t full_lo = (lo_rel + kMergeElems - 1) / kMergeElems;
        const uint32_t full_hi = hi_rel / kMergeElems;
        auto merge_block = [&](uint32_t blk, const uint2& s2) {
            const uint2 e2 = *reinterpret_cast<const uint2*>(ebuf + kMergeElems * blk);
            uint32_t o0, o1, o2, o3;
            join4(s2.x, e2.x, o0, o1);
            join4(s2.y, e2.y, o2, o3);
            u32x4 v;
            v.x = o0;
            v.y = o1;
            v.z = o2;
            v.w = o3;
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(outu + kMergeElems * blk));
        };
#pragma unroll
        for (uint32_t k = 0; k < kPrefetchBlocks; ++k) {
            const uint32_t blk = tid + k * kDecodeThreads;
            if (blk >= full_lo && blk < full_hi) merge_block(blk, smv[k]);
        }
        for (uint32_t blk = tid + kPrefetchBlocks * kDecodeThreads; blk < full_hi; blk += kDecodeThreads)
            merge_block(blk, *reinterpret_cast<const uint2*>(smu + kMergeElems * blk));
        // partial edge blocks: lane 0 takes the one holding A, lane 1 the one
        // holding B unless it is the same block
        {
            const uint32_t blk = tid == 0 ? lo_rel / kMergeElems : nblk - 1;
            const bool partial =
                tid == 0 ? (lo_rel % kMergeElems) != 0 : (tid == 1 && full_hi < nblk && nblk - 1 >= full_lo);
            if (partial) {
                const uint32_t rel = kMergeElems * blk;
                const uint2 s2 = *reinterpret_cast<const uint2*>(smu + rel);
                const uint2 e2 = *reinterpret_cast<const uint2*>(ebuf + rel);
                uint32_t o[4];
                join4(s2.x, e2.x, o[0], o[1]);
                join4(s2.y, e2.y, o[2], o[3]);
#pragma unroll
                for (uint32_t i = 0; i < kMergeElems; ++i) {
                    const uint32_t idx = rel + i;
                    if (idx >= lo_rel && idx < hi_rel) outu[idx] = (uint16_t)(o[i >> 1] >> (16 * (i & 1)));
                }
            }
        }

        if (!more) break;
        __syncthreads();   // ebuf and s_wave are reused by the next unit
        u = un;
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
    __shared__ uint32_t single[1u << kS];   // rotated symbol | length << 8, or ~0 for a longer code
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
                if (lens.len[s] == L) sorted[rank++] = (uint8_t)((s >> 1) | ((s & 1) << 7));
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
    // multi-codeword table: up to four whole codewords per window
    for (uint32_t w = tid; w < (1u << KD); w += blockDim.x) {
        uint32_t at = 0, n = 0, syms = 0;
        while (n < 4) {
            const uint32_t x = ((w << at) & ((1u << KD) - 1u)) << (kS - KD);
            const uint32_t s = single[x];
            if (s == 0xFFFFFFFFu) break;
            const uint32_t L = s >> 8;
            if (at + L > (uint32_t)KD) break;
            syms |= (s & 0xFFu) << (8 * n);
            ++n;
            at += L;
        }
        tables[(1u << KC) + 2 * w] = n ? (((32u - at) & 31u) | (n << 8) | (at << 16)) : 0u;
        tables[(1u << KC) + 2 * w + 1] = syms;
    }
    uint32_t* tail = tables + (1u << KC) + (2u << KD);
    if (tid < 32) {
        tail[tid] = count[tid];
        tail[32 + tid] = first[tid];
        tail[64 + tid] = base[tid];
    }
    if (tid < 64) {
        tail[96 + tid] = (uint32_t)sorted[4 * tid] | ((uint32_t)sorted[4 * tid + 1] << 8) |
                         ((uint32_t)sorted[4 * tid + 2] << 16) | ((uint32_t)sorted[4 * tid + 3] << 24);
    }
    // second level for codes longer than KD: the KD-bit windows >= F hold a
    // longer first codeword, F = (first code of length KD + 1) / 2
    const uint32_t F = first[KD + 1] >> 1;
    const uint32_t np = F < (1u << KD) ? min((1u << KD) - F, kL2Prefixes) : 0u;
    if (tid < 4) tail[160 + tid] = tid == 0 ? F : (tid == 1 ? np : 0u);
    uint16_t* l2 = reinterpret_cast<uint16_t*>(tail + kLongWords);
    for (uint32_t w = tid; w < (kL2Prefixes << kL2Bits); w += blockDim.x) {
        uint32_t e = 0;
        if (w < (np << kL2Bits)) {
            const uint32_t win = (F << kL2Bits) + w;   // a (KD + kL2Bits)-bit window
            for (uint32_t L = KD + 1; L <= KD + kL2Bits; ++L) {
                const uint32_t off = (win >> (KD + kL2Bits - L)) - first[L];
                if (off < count[L]) {
                    e = (L << 8) | sorted[(base[L] + off) & 255u];
                    break;
                }
            }
        }
        l2[w] = (uint16_t)e;
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
    if (kc == 12 && kd == 11) return f(Variant<12, 11>{});
    if (kc == 12 && kd == 10) return f(Variant<12, 10>{});
    if (kc == 11 && kd == 11) return f(Variant<11, 11>{});
    if (kc == 11 && kd == 10) return f(Variant<11, 10>{});
    return f(Variant<10, 10>{});
}

}  // namespace

uint32_t decode_dyn_lds_bytes(uint32_t ebuf_bytes, uint32_t l2_cap) {
    return ebuf_bytes + (l2_cap << kL2Bits) * 2u;
}

uint32_t decode_lds_bytes(uint32_t count_bits, uint32_t decode_bits, uint32_t ebuf_bytes, uint32_t l2_cap) {
    return ((1u << count_bits) + (2u << decode_bits) + kLongWords) * 4u + kWaves * 4u + 4u * kDecodeThreads +
           decode_dyn_lds_bytes(ebuf_bytes, l2_cap);
}

int decode_blocks_per_cu(uint32_t count_bits, uint32_t decode_bits, uint32_t ebuf_bytes, uint32_t l2_cap) {
    if (!supported_table_bits(count_bits, decode_bits)) return 0;
    const uint32_t dyn = decode_dyn_lds_bytes(ebuf_bytes, l2_cap);
    return dispatch(count_bits, decode_bits, [&](auto v) { return decltype(v)::blocks_per_cu(dyn); });
}

hipError_t launch_build_tables(const CodeLens& lens, uint32_t count_bits, uint32_t decode_bits, uint32_t* d_tables,
                               hipStream_t stream) {
    if (!supported_table_bits(count_bits, decode_bits)) return hipErrorInvalidValue;
    return dispatch(count_bits, decode_bits, [&](auto v) { return decltype(v)::build(lens, d_tables, stream); });
}

hipError_t launch_decode(const DecodeParams& p, uint32_t count_bits, uint32_t decode_bits, uint32_t grid,
                         hipStream_t stream) {
    if (!supported_table_bits(count_bits, decode_bits) || p.l2_cap > kL2Prefixes) return hipErrorInvalidValue;
    const uint32_t dyn = decode_dyn_lds_bytes(p.ebuf_bytes, p.l2_cap);
    return dispatch(count_bits, decode_bits, [&](auto v) { return decltype(v)::launch(p, grid, dyn, stream); });
}

}  // namespace wc
