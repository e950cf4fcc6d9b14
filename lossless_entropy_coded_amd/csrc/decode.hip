// decode.hip -- gfx950 kernels of libwc: decode-table construction and the
// block-level decode of an exponent-Huffman bf16 container.
//
// Design points taken from the DFloat11 page ("70% Size, 100% Accuracy:
// Lossless LLM Compression for Efficient GPU Inference via Dynamic-Length
// Float", abstract): (i) the big code lookup is split into compact tables
// that live in on-chip memory (here: LDS of each workgroup); (ii) a two-phase
// kernel coordinates where each thread reads and writes through small
// auxiliary variables (here: a per-chunk bit offset `gap` and a group table
// of first elements and their stream bits); (iii) a whole transformer block
// is decoded by one launch (here: every group of a multi-tensor container).
//
// Work decomposition on CDNA4: one wave64 decodes one group (at most 128
// chunks of 64 stream bits, at most 4096 elements, output starting on a
// 128-element boundary); lane t owns the group's chunks c0 + 2t and c0 + 2t + 1
// and decodes them as two independent chains, so two table lookups are in
// flight per lane.  Waves never wait for each other after the table staging.
//   phase 1  each chain counts the codewords that START in its part of the
//            group's bits, several per lookup of a codeword-start table;
//   scan     wave64 inclusive scan with DPP row shifts and row broadcasts ->
//            each chain's first output inside the group;
//   phase 2  each chain decodes its codewords again, up to four per lookup of
//            a multi-codeword table, and stages the exponent bytes in the
//            wave's LDS buffer at their final place (four byte stores per
//            lookup; unaligned dword LDS stores stall on CDNA4).  Bytes
//            written past a chain's range land on the next chain's first
//            three bytes, which that chain keeps aside and rewrites once the
//            whole wave has left the loop; writes of a finished chain go to a
//            per-lane dummy slot;
//   merge    the wave joins the sign+mantissa bytes (prefetched while the
//            phases run) with the staged exponents in integer registers, 8
//            elements per lane and step, and writes bf16 with 16-byte stores
//            that are contiguous across the lanes: whole cache lines, none of
//            them shared with another group.
// Workgroups are persistent: each stages the tables once and its waves loop
// over their groups, loading the next group's chunks while they work on the
// current one.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>

#include "../../include/wc.h"
#include "decode_common.h"
#include "kernels.h"

namespace wc {
namespace {

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

// Raw loads of one lane for one group: the stream bytes of its two chunks
// a = c0 + 2t and a + 1 plus the lookahead of the second (20 bytes from 8a),
// and both gaps (packed gaps: the three bytes holding bits 5a .. 5a + 9).
// The group's chunks c0 .. c1 (c0 = p0 / 64, c1 = (p1 - 1) / 64) start at
// any chunk, so the 20 bytes are taken from two aligned 16-byte
// loads at 8 * (a rounded down to even) (of 16 and 12 bytes); the parity of a
// is that of c0, the same for every lane.  Both loads stay inside the
// container: they end at most 4 bytes past the stream section, which is
// followed by the sm section.  Every loaded word is used: a load whose
// register is partly dead lets that register be reused while the load is in
// flight, which costs a wait for it.
struct Raw {
    uint4 q0;
    uint3 q1;
    uint32_t ga, gb;
};

__device__ __forceinline__ Raw load_raw(const DecodeParams& p, const Meta& m, uint32_t lane, uint32_t pass = 0) {
    Raw r;
    const uint64_t a = (m.p0 >> 6) + kGroupChunks * pass + kChunksPerLane * lane;
    const uint64_t c1 = (m.p1 - 1) >> 6;
    r.q0 = make_uint4(0, 0, 0, 0);
    r.q1 = make_uint3(0, 0, 0);
    r.ga = r.gb = 0;
    if (a <= c1) {
        const uint8_t* q = p.stream + 8 * (a & ~(uint64_t)1);
        r.q0 = *reinterpret_cast<const uint4*>(q);
        r.q1 = *reinterpret_cast<const uint3*>(q + 16);
        if (p.gap_packed) {
            // at most 2 bytes past the section: the stream section follows
            const uint8_t* g = p.gap + ((5 * a) >> 3);
            const uint32_t v = ((uint32_t)g[0] | (uint32_t)g[1] << 8 | (uint32_t)g[2] << 16) >> ((5 * a) & 7u);
            r.ga = v & 31u;
            r.gb = (v >> 5) & 31u;
        } else {
            r.ga = p.gap[a];
            r.gb = p.gap[a + 1];   // gap[n_chunks] lies in the padding after the gap section
        }
    }
    return r;
}

// A chain ready for decoding: 96 stream bits MSB-first, shifted so that the
// first codeword it owns is at the top; `bits` counts the bits after that
// point in which further codewords it owns may start.
struct Chain {
    uint32_t w0, w1, w2;
    int32_t bits;
};

// Chain of chunk c of a group whose codewords start in [p0, p1): it owns the
// codewords starting in [max(64c, p0), min(64(c + 1), p1)).  gap is gap[c];
// the group's first chunk starts at p0 instead.  A chunk past the group owns
// nothing.
__device__ __forceinline__ Chain make_chain(uint64_t c, uint64_t p0, uint64_t p1, uint32_t d0, uint32_t d1,
                                            uint32_t d2, uint32_t gap) {
    Chain h;
    const uint32_t w0 = __builtin_bswap32(d0), w1 = __builtin_bswap32(d1), w2 = __builtin_bswap32(d2);
    const uint64_t lo = 64 * c, hi = lo + 64;
    int32_t end = 0;
    if (lo < p1) {
        if (lo <= p0) gap = (uint32_t)(p0 - lo);
        end = (int32_t)((hi < p1 ? hi : p1) - lo);
    } else {
        gap = 0;
    }
    // shift the 96 bits left by gap (0..63): whole words first, then the rest
    const bool far = gap >= 32;
    const uint32_t x0 = far ? w1 : w0, x1 = far ? w2 : w1, x2 = far ? 0u : w2;
    const uint32_t sh = gap & 31u;
    const uint64_t h01 = ((uint64_t)x0 << 32 | x1) << sh;
    const uint64_t h12 = ((uint64_t)x1 << 32 | x2) << sh;
    h.w0 = (uint32_t)(h01 >> 32);
    h.w1 = (uint32_t)(h12 >> 32);
    h.w2 = x2 << sh;
    h.bits = end - (int32_t)gap;
    return h;
}

struct Unit {
    Chain a, b;
    uint64_t A;       // first element of the group
    uint32_t n;       // its elements (at most kGroupMaxElems)
    uint32_t passes;  // passes of 128 chunks its codewords span (1 unless chunks_per_group > 128)
};

// The chains of pass `pass` of a group: lane t takes its chunks
// c0 + 128 pass + 2t and the next (the pass's first chunk has the parity of
// c0, so the same window cut serves every pass).
__device__ __forceinline__ Unit make_unit(const Raw& r, const Meta& m, uint32_t lane, uint32_t pass = 0) {
    Unit x;
    const bool odd = (m.p0 >> 6) & 1;
    const uint32_t d0 = odd ? r.q0.z : r.q0.x, d1 = odd ? r.q0.w : r.q0.y;
    const uint32_t d2 = odd ? r.q1.x : r.q0.z, d3 = odd ? r.q1.y : r.q0.w;
    const uint32_t d4 = odd ? r.q1.z : r.q1.x;
    const uint64_t c = (m.p0 >> 6) + kGroupChunks * pass + kChunksPerLane * lane;
    x.a = make_chain(c, m.p0, m.p1, d0, d1, d2, r.ga);
    x.b = make_chain(c + 1, m.p0, m.p1, d2, d3, d4, r.gb);
    x.A = m.e0;
    x.n = (uint32_t)min_u64(m.e1 - m.e0, kGroupMaxElems);   // kept 64-bit: every loaded word is used
    const uint64_t span = ((m.p1 - 1) >> 6) - (m.p0 >> 6) + 1;   // chunks the group's codewords touch
    x.passes = (uint32_t)((span + kGroupChunks - 1) / kGroupChunks);
    return x;
}

// Entry of the codeword-start table for a code longer than the index: one
// codeword start at offset 0, covering its L bits.
template <int KD>
__device__ __forceinline__ uint32_t long_count_entry(uint32_t win, uint32_t first_len, const LongTables& lt) {
    const uint32_t L = long_code<KD>(win, first_len, lt) >> 8;
    return ((32u - L) & 31u) | (L << 8) | (1u << 16);
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

// kDot = false: decode the groups to bf16 in p.out.  kDot = true (fused
// decode -> matrix-vector product): the decoded weights of each group never
// leave the chip; the wave multiplies them by x and leaves its partial dot
// products in p.work.
// The fused product runs 8-wave workgroups, two per CU: at most 128 VGPRs (4
// waves per SIMD).
template <int KC, int KD, int W, bool kDot, bool kCheck>
__global__ __launch_bounds__(kWaveLanes * W, kDot ? 4 : 1) void decode_kernel(DecodeParams p) {
    constexpr uint32_t kThreads = kWaveLanes * W;
    // decode tables, in the order of the plan's device buffer: codeword-start
    // table, multi-codeword table, the canonical arrays for long codes
    constexpr uint32_t kCntVec = (1u << KC) / 4, kDecVec = (2u << KD) / 4, kLongVec = kLongWords / 4;
    constexpr uint32_t kTabVec = kCntVec + kDecVec + kLongVec;
    __shared__ __attribute__((aligned(16))) uint4 s_tab[kTabVec];
    __shared__ __attribute__((aligned(16))) uint8_t s_dummy[4 * kThreads];
    uint32_t* const s_cnt = reinterpret_cast<uint32_t*>(s_tab);
    uint2* const s_dec = reinterpret_cast<uint2*>(s_tab + kCntVec);
    uint32_t* const s_long = reinterpret_cast<uint32_t*>(s_tab + kCntVec + kDecVec);
    // dynamic: W exponent staging buffers of ebuf_bytes (one per wave), then the
    // second-level table for the long-code prefixes of this container
    // (l2_cap * 2^kL2Bits u16)
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    uint16_t* const s_l2 = reinterpret_cast<uint16_t*>(dyn + W * p.ebuf_bytes);

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint8_t* const dummy = s_dummy + 4 * tid;
    uint8_t* const ebuf = dyn + wave * p.ebuf_bytes;

    // Wave w of workgroup b takes groups b*W + w, then every (grid * W)-th
    // one after it: the groups in flight at any time form one contiguous
    // stretch of the stream and of the output, and neighbouring groups run in
    // the same workgroup.
    //
    // Pipeline of one wave, per group u: at the top, the stream and gap loads
    // of the next group (its table entries arrived one iteration earlier),
    // the sm loads of u and the table entries of the group after next are
    // issued; the phases run on u from LDS only; then the next group's loads
    // are consumed, and u is merged with eight fixed store steps.  Every
    // iteration issues the same vector memory instructions, so each wait
    // covers exactly the loads it needs.
    const uint64_t stride = (uint64_t)gridDim.x * W;
    uint64_t u = p.u_begin + (uint64_t)blockIdx.x * W + wave;
    const uint64_t last_u = p.u_end - 1;
    const bool active = u < p.u_end;

    // Prologue: the first group's table entries, then every table load of the
    // workgroup's staging, are in flight together; the first group's stream
    // loads are issued before the tables are written to LDS.  The barrier
    // after the staging is the only point where the waves of a workgroup wait
    // for each other.  Group table entries come through the scalar data
    // cache (measured faster here than vector loads that every lane takes;
    // the lanes kernel's plain decode measured the other way).
    const Meta m_first = load_meta_scalar(p, min_u64(u, last_u));
    constexpr uint32_t kFull = kTabVec / kThreads;          // staging rounds every lane takes part in
    constexpr uint32_t kTail = kTabVec - kFull * kThreads;  // pieces of the last, partial round
    const u32x4* const tsrc = reinterpret_cast<const u32x4*>(p.tables);
    u32x4* const tdst = reinterpret_cast<u32x4*>(s_tab);
    u32x4 stage[kFull];
#pragma unroll
    for (uint32_t k = 0; k < kFull; ++k) stage[k] = tsrc[tid + k * kThreads];
    u32x4 stage_tail = {0, 0, 0, 0};
    if (kTail && tid < kTail) stage_tail = tsrc[kFull * kThreads + tid];
    const Meta& m0 = m_first;
    const Raw r0 = load_raw(p, m0, lane);
    Meta m_next = load_meta_scalar(p, min_u64(u + stride, last_u));
#pragma unroll
    for (uint32_t k = 0; k < kFull; ++k) tdst[tid + k * kThreads] = stage[k];
    if (kTail && tid < kTail) tdst[kFull * kThreads + tid] = stage_tail;
    {
        const uint4* src = reinterpret_cast<const uint4*>(p.tables) + kTabVec;
        for (uint32_t i = tid; i < (p.l2_cap << kL2Bits) / 8; i += kThreads)
            reinterpret_cast<uint4*>(s_l2)[i] = src[i];
    }
    __syncthreads();
    if (!active) return;
    LongTables lt;
    lt.count = s_long;
    lt.first = s_long + 32;
    lt.base = s_long + 64;
    lt.sorted = reinterpret_cast<const uint8_t*>(s_long + 96);
    lt.l2 = s_l2;
    lt.l2_first = __builtin_amdgcn_readfirstlane(s_long[160]);
    lt.l2_n = min(__builtin_amdgcn_readfirstlane(s_long[161]), p.l2_cap);

    Unit cur = make_unit(r0, m0, lane);
    Meta cur_meta = m0;
    uint32_t dot_mat = 0;   // fused product: matrix of the wave's current group

    for (;;) {
        const uint64_t un = u + stride;
        const bool more = un < p.u_end;
        const Raw nxt = load_raw(p, m_next, lane);

        // sign+mantissa bytes of the group (non-temporal: read once); block
        // indexes past the group are clamped to its last block (a cache hit,
        // never used).  Every block lies inside round_up(n, 8) <= the
        // plane's padded size.
        const uint64_t A = cur.A;
        const uint32_t n_unit = cur.n;
        const uint32_t last_blk = (n_unit - 1) / kMergeElems;
        const uint8_t* const smu = p.sm + A;
        uint16_t* const outu = p.out + A;
        uint2 smv[kMergeSteps];
#pragma unroll
        for (uint32_t k = 0; k < kMergeSteps; ++k)
            smv[k] = load_nt8(smu + kMergeElems * min(lane + k * kWaveLanes, last_blk));
        // fused product: the x entries of the group's blocks, loaded with the
        // sm bytes so that they have arrived by the merge (blocks outside the
        // multiplied range load x0[0..7], never used)
        DotRows dr;
        uint4 xv[kDot ? kMergeSteps : 1];
        if constexpr (kDot) {
            dr = dot_rows(p.dot, A, n_unit, dot_mat);
            load_dot_x(dr, n_unit, lane, 0, xv);
        }

        const Meta m_after = load_meta_scalar(p, min_u64(un + stride, last_u));

        // The phases over one pass of chains: lane t's chains are the pass's
        // chunks 2t and 2t + 1; their output starts at `base` inside the
        // group.  Returns the pass's codeword count (the same for every lane).
        auto run_pass = [&](const Chain& ch_a, const Chain& ch_b, uint32_t base) -> uint32_t {
            // phase 1: count the codewords starting in each chunk
            uint32_t ca = 0, cb = 0;
            {
                uint32_t a0 = ch_a.w0, a1 = ch_a.w1, a2 = ch_a.w2;
                uint32_t b0 = ch_b.w0, b1 = ch_b.w1, b2 = ch_b.w2;
                int32_t ra = ch_a.bits, rb = ch_b.bits;
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

            // wave-wide exclusive scan of the lane counts: each chain's first
            // output index inside the unit
            const uint32_t count = ca + cb;
            const uint32_t incl = wave_inclusive_scan(count);
            const uint32_t pos_a = base + incl - count;
            const uint32_t pos_b = pos_a + ca;

            // phase 2: decode again and stage the exponent bytes; a chain never
            // writes past the group's element range, even for a corrupted stream
            const uint32_t todo_a = min(ca, pos_a < n_unit ? n_unit - pos_a : 0u);
            const uint32_t todo_b = min(cb, pos_b < n_unit ? n_unit - pos_b : 0u);
            uint8_t* qa = ebuf + pos_a;
            uint8_t* qb = ebuf + pos_b;
            uint8_t* const qa_end = qa + todo_a;
            uint8_t* const qb_end = qb + todo_b;
            {
                uint32_t a0 = ch_a.w0, a1 = ch_a.w1, a2 = ch_a.w2;
                uint32_t b0 = ch_b.w0, b1 = ch_b.w1, b2 = ch_b.w2;
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
                // The staging belongs to this wave alone, and the LDS executes a
                // wave's accesses in issue order: once every lane has left the
                // loop, the head bytes overwrite whatever a left neighbour's last
                // four-byte store put there.
                wave_lds_order();
                uint8_t* ha = ebuf + pos_a;
                uint8_t* hb = ebuf + pos_b;
    #pragma unroll
                for (uint32_t k = 0; k < kHeadBytes; ++k) {
                    if (todo_a > k) ha[k] = (uint8_t)(head_a >> (8 * k));
                    if (todo_b > k) hb[k] = (uint8_t)(head_b >> (8 * k));
                }
            }
            return (uint32_t)__builtin_amdgcn_readlane((int)incl, kWaveLanes - 1);
        };
        uint32_t done = run_pass(cur.a, cur.b, 0);
        // a group whose codewords span more than one pass of 128 chunks
        // (chunks_per_group above 128): the further passes load their chunks
        // here and continue at the count decoded so far
        for (uint32_t pass = 1; pass < cur.passes; ++pass) {
            const Unit w = make_unit(load_raw(p, cur_meta, lane, pass), cur_meta, lane, pass);
            done += run_pass(w.a, w.b, done);
        }
        // debug plans (kernels compiled with the check): the codewords that
        // start in the group's bits are its elements, one each (a corrupted
        // stream or group bit offset, which the host checks cannot see,
        // breaks this); a vector-memory atomic OR into the status word
        if constexpr (kCheck) {
            if (done != n_unit && lane == 0) atomicOr(p.status, WC_DEBUG_GROUP_COUNT);
        }

        // consume every load of this iteration now, before the merge issues
        // its stores: the next group's chains and table entries, and the sm
        // bytes (a load still pending at the next iteration's top would make
        // the wait there cover the merge stores as well)
        const Unit next = make_unit(nxt, m_next, lane);
        const Meta next_meta = m_next;
        m_next = m_after;
        wave_lds_order();
#pragma unroll
        for (uint32_t k = 0; k < kMergeSteps; ++k)
            asm volatile("" ::"v"(smv[k].x), "v"(smv[k].y));

        // merge: 8 elements per lane per step; consecutive lanes take
        // consecutive blocks, so each wave-wide 8-byte load and 16-byte store
        // covers one contiguous range of whole cache lines.  A group holds at
        // most kMergeSteps blocks per lane.  Only the container's very last
        // block can be partial; it is written after the loop.
        const uint32_t full = n_unit / kMergeElems;
        if constexpr (kDot) {
            dot_group(p.dot, dr, full, lane, smv, xv, u - p.u_begin, [&](uint32_t k) {
                // blocks past the group read its last block: inside the staging
                return *reinterpret_cast<const uint2*>(ebuf + kMergeElems * min(lane + k * kWaveLanes, last_blk));
            });
        } else {
#pragma unroll
        for (uint32_t k = 0; k < kMergeSteps; ++k) {
            const uint32_t blk = lane + k * kWaveLanes;
            if (blk < full) {
                const uint2 e2 = *reinterpret_cast<const uint2*>(ebuf + kMergeElems * blk);
                uint32_t o0, o1, o2, o3;
                join4(smv[k].x, e2.x, o0, o1);
                join4(smv[k].y, e2.y, o2, o3);
                u32x4 v;
                v.x = o0;
                v.y = o1;
                v.z = o2;
                v.w = o3;
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(outu + kMergeElems * blk));
            }
        }
        }

        if (!more) break;
        wave_lds_order();   // the staging is rewritten by the next group
        u = un;
        cur = next;
        cur_meta = next_meta;
    }

    // the container's last block, when it holds fewer than 8 elements (a
    // matrix for the fused product never ends in a partial block)
    const uint32_t full = cur.n / kMergeElems;
    if (!kDot && full * kMergeElems < cur.n && lane == 0) {
        const uint32_t rel = kMergeElems * full;
        const uint2 s2 = load_nt8(p.sm + cur.A + rel);
        const uint2 e2 = *reinterpret_cast<const uint2*>(ebuf + rel);
        uint32_t o[4];
        join4(s2.x, e2.x, o[0], o[1]);
        join4(s2.y, e2.y, o[2], o[3]);
#pragma unroll
        for (uint32_t i = 0; i < kMergeElems; ++i)
            if (rel + i < cur.n) p.out[cur.A + rel + i] = (uint16_t)(o[i >> 1] >> (16 * (i & 1)));
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

template <int KC, int KD, int W>
struct Variant {
    // plans with a status word run the kernels compiled with the per-group
    // check; the others pay nothing for it
    template <bool kDot, bool kCheck>
    static void go(const DecodeParams& p, uint32_t grid, uint32_t dyn, hipStream_t stream) {
        hipLaunchKernelGGL((decode_kernel<KC, KD, W, kDot, kCheck>), dim3(grid), dim3(kWaveLanes * W), dyn, stream,
                           p);
    }
    static hipError_t launch(const DecodeParams& p, uint32_t grid, uint32_t dyn, bool dot, hipStream_t stream) {
        const bool check = p.status != nullptr;
        if (dot)
            check ? go<true, true>(p, grid, dyn, stream) : go<true, false>(p, grid, dyn, stream);
        else
            check ? go<false, true>(p, grid, dyn, stream) : go<false, false>(p, grid, dyn, stream);
        return hipGetLastError();
    }
    static int blocks_per_cu(uint32_t dyn) {
        int least = 1 << 30;
        for (const void* k : {reinterpret_cast<const void*>(decode_kernel<KC, KD, W, false, false>),
                              reinterpret_cast<const void*>(decode_kernel<KC, KD, W, true, false>),
                              reinterpret_cast<const void*>(decode_kernel<KC, KD, W, false, true>),
                              reinterpret_cast<const void*>(decode_kernel<KC, KD, W, true, true>)}) {
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kWaveLanes * W, dyn) != hipSuccess) return 0;
            least = n < least ? n : least;
        }
        return least;
    }
    static hipError_t build(const CodeLens& lens, uint32_t* d_tables, hipStream_t stream) {
        hipLaunchKernelGGL((build_tables_kernel<KC, KD>), dim3(1), dim3(1024), 0, stream, lens, d_tables);
        return hipGetLastError();
    }
};

template <int W, typename F>
auto dispatch_bits(uint32_t kc, uint32_t kd, F&& f) {
    if (kc == 12 && kd == 11) return f(Variant<12, 11, W>{});
    if (kc == 12 && kd == 10) return f(Variant<12, 10, W>{});
    if (kc == 11 && kd == 11) return f(Variant<11, 11, W>{});
    if (kc == 11 && kd == 10) return f(Variant<11, 10, W>{});
    return f(Variant<10, 10, W>{});
}

template <typename F>
auto dispatch(uint32_t kc, uint32_t kd, uint32_t waves, F&& f) {
    if (waves == 4) return dispatch_bits<4>(kc, kd, f);
    return dispatch_bits<8>(kc, kd, f);
}

}  // namespace

uint32_t decode_dyn_lds_bytes(uint32_t waves, uint32_t ebuf_bytes, uint32_t l2_cap) {
    return waves * ebuf_bytes + (l2_cap << kL2Bits) * 2u;
}

uint32_t decode_lds_bytes(uint32_t count_bits, uint32_t decode_bits, uint32_t waves, uint32_t ebuf_bytes,
                          uint32_t l2_cap) {
    return ((1u << count_bits) + (2u << decode_bits) + kLongWords) * 4u + 4u * kWaveLanes * waves +
           decode_dyn_lds_bytes(waves, ebuf_bytes, l2_cap);
}

int decode_blocks_per_cu(uint32_t count_bits, uint32_t decode_bits, uint32_t waves, uint32_t ebuf_bytes,
                         uint32_t l2_cap) {
    if (!supported_table_bits(count_bits, decode_bits) || !supported_waves(waves)) return 0;
    const uint32_t dyn = decode_dyn_lds_bytes(waves, ebuf_bytes, l2_cap);
    return dispatch(count_bits, decode_bits, waves, [&](auto v) { return decltype(v)::blocks_per_cu(dyn); });
}

hipError_t launch_build_tables(const CodeLens& lens, uint32_t count_bits, uint32_t decode_bits, uint32_t* d_tables,
                               hipStream_t stream) {
    if (!supported_table_bits(count_bits, decode_bits)) return hipErrorInvalidValue;
    return dispatch(count_bits, decode_bits, 8, [&](auto v) { return decltype(v)::build(lens, d_tables, stream); });
}

hipError_t launch_decode(const DecodeParams& p, uint32_t count_bits, uint32_t decode_bits, uint32_t waves,
                         uint32_t grid, bool dot, hipStream_t stream) {
    if (!supported_table_bits(count_bits, decode_bits) || !supported_waves(waves) || p.l2_cap > kL2Prefixes)
        return hipErrorInvalidValue;
    const uint32_t dyn = decode_dyn_lds_bytes(waves, p.ebuf_bytes, p.l2_cap);
    return dispatch(count_bits, decode_bits, waves,
                    [&](auto v) { return decltype(v)::launch(p, grid, dyn, dot, stream); });
}

namespace {

// y of global row r = the second partial of the last group whose first row
// is r - 1 (zero when that group ends before row r), then the first partials
// of the groups whose first row is r, in group order: a fixed order, so y is
// reproducible.  One lane per row.
__global__ __launch_bounds__(256) void gemv_rows_kernel(DecodeParams p) {
    const DotParams& q = p.dot;
    const uint32_t r = blockIdx.x * 256 + threadIdx.x;
    if (r >= q.rows) return;
    const uint32_t g0 = q.row_group[r];
    const uint32_t g1 = r + 1 < q.rows ? q.row_group[r + 1] : (uint32_t)(p.u_end - p.u_begin);
    float sum = r > 0 ? q.part[2 * (uint64_t)g0 - 1] : 0.0f;
    for (uint32_t g = g0; g < g1; ++g) sum += q.part[2 * (uint64_t)g];
    uint32_t k = 0;
    for (uint32_t j = 1; j < q.n_mats; ++j) k = q.row_base[j] <= r ? j : k;
    q.y[k][r - q.row_base[k]] = sum;
}

}  // namespace

hipError_t launch_gemv_rows(const DecodeParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(gemv_rows_kernel, dim3((p.dot.rows + 255) / 256), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace wc
