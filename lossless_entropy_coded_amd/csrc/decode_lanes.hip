// decode_lanes.hip -- gfx950 decode kernel of libwc for the interleaved-lane
// container (version 3).
//
// The LazyWeights page (analogy section) stores Huffman codes in interleaved
// lanes that are decoded on demand.  Here a segment (at most 4096 elements and
// 15872 stream bits) is one wave64's unit, and lane j of the wave owns the
// segment's 8-element lane blocks j, j + 64, ..., whose codewords are stored
// contiguously from the lane's own offset.  So every lane knows where its bits
// start and how many symbols it decodes: no per-chunk gaps, no counting pass
// and no scan.  Lane j's lane blocks are exactly the blocks it writes in the
// merge (block j + 64k in step k), so the exponent bytes go from the lane's
// registers to its own 8-byte LDS slots and back, never across lanes.
//
// Per segment and wave:
//   stage   the segment's stream bytes (at most 1984, plus the alignment and
//           the lookahead) arrive one iteration early as two 16-byte loads per
//           lane and are written byte-swapped to the wave's LDS words, so that
//           word k holds stream bits 32k .. 32k + 31 MSB-first;
//   decode  each lane looks up the multi-codeword table (up to four symbols
//           per lookup, as the chunked kernel) with a 32-bit window of its
//           bits: for the plain decode from a 64-bit register window refilled
//           one LDS word at a time; for the fused product and code planes,
//           whose instructions bound them, re-read from the staged words at
//           every lookup (no per-lane refill branch).  The symbols go to the
//           lane's own LDS slot at the count decoded so far (code planes:
//           gathered into aligned words);
//   merge   as the chunked kernel: the sign+mantissa bytes (loaded while the
//           lanes decode) and the staged exponents (lane i's k-th 8 bytes
//           are block i + 64k) become bf16 in registers, written with
//           16-byte non-temporal stores, whole cache lines.
//
// rANS containers (the Llama2-7B page's abstract names ANS; the LazyWeights
// review compares a Huffman and an rANS decoder) use the same segments,
// staging and merge; a lane is then one rANS stream: the staged bytes are
// swapped within 16-bit halves so that half-word q is the stream's q-th
// big-endian word, and each step takes one symbol from the 2^12-slot table
// (x = f (x >> 12) + x mod 2^12 - cum, then one word in when x < 2^16).
// The state chain allows one symbol per table read where a Huffman lookup
// yields up to four.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "decode_common.h"
#include "format.h"
#include "kernels.h"

namespace wc {
namespace {

constexpr uint32_t kStageWords = kLaneStageBytes / 4;
constexpr uint32_t kRansSlots = 1u << kRansBits;

// One lane's loads for one segment: its two 16-byte pieces of the segment's
// stream window (pieces past the bytes the segment needs are not loaded) and
// the offset of its own bits.
struct LaneRaw {
    uint4 q0, q1;
    uint32_t off;
};

__device__ __forceinline__ LaneRaw load_lane_raw(const DecodeParams& p, const Meta& m, uint64_t g, uint32_t lane) {
    LaneRaw r;
    const uint64_t base = (m.p0 >> 7) << 4;                    // 16-byte aligned first byte
    const uint64_t need = ((m.p1 + 7) >> 3) + 8 - base;        // bytes up to the last bit, plus the lookahead
    const uint8_t* q = p.stream + base;
    r.q0 = make_uint4(0, 0, 0, 0);
    r.q1 = make_uint4(0, 0, 0, 0);
    if (16u * lane < need) r.q0 = *reinterpret_cast<const uint4*>(q + 16u * lane);
    if (16u * (lane + kWaveLanes) < need) r.q1 = *reinterpret_cast<const uint4*>(q + 16u * (lane + kWaveLanes));
    r.off = reinterpret_cast<const uint16_t*>(p.gap)[kLanes * g + lane];
    return r;
}

__device__ __forceinline__ uint4 bswap4(const uint4& v) {
    return make_uint4(__builtin_bswap32(v.x), __builtin_bswap32(v.y), __builtin_bswap32(v.z),
                      __builtin_bswap32(v.w));
}

// Each 16-bit half of each word byte-swapped: LDS half-word q of the staged
// window is the stream's big-endian 16-bit word q.
__device__ __forceinline__ uint4 swap16x8(const uint4& v) {
    return make_uint4(__builtin_amdgcn_perm(v.x, v.x, 0x02030001u), __builtin_amdgcn_perm(v.y, v.y, 0x02030001u),
                      __builtin_amdgcn_perm(v.z, v.z, 0x02030001u), __builtin_amdgcn_perm(v.w, v.w, 0x02030001u));
}

// Eight bytes of a lane slot (4-byte aligned: slots are 17 dwords apart) as
// two dwords.
__device__ __forceinline__ uint2 load_slot8(const uint8_t* q) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(q);
    return make_uint2(w[0], w[1]);
}
__device__ __forceinline__ void store_slot8(uint8_t* q, uint2 v) {
    uint32_t* w = reinterpret_cast<uint32_t*>(q);
    w[0] = v.x;
    w[1] = v.y;
}

// Undo the one-bit rotation the decode tables store symbols with, in each
// byte of a word (e = rol8(e', 1)).
__device__ __forceinline__ uint32_t unrotate4(uint32_t x) {
    return ((x << 1) & 0xFEFEFEFEu) | ((x >> 7) & 0x01010101u);
}

// kMode kLanesToBf16: decode bf16 segments into p.out.  kLanesToDot (fused
// decode -> matrix-vector product): the decoded weights never leave the chip;
// each wave multiplies its segment by x and leaves its partial dot products
// in p.dot.part.  kLanesToU8: decode a plane of code bytes into p.out8 (no
// sign+mantissa plane).  kRans: rANS lanes (KD = 11: the slot table fills
// the multi-codeword table's 16 KiB).
template <int KD, int W, uint32_t kMode, bool kRans>
__global__ __launch_bounds__(kWaveLanes * W) void decode_lanes_kernel(DecodeParams p) {
    static_assert(!kRans || (2u << KD) == kRansSlots, "the rANS slot table takes the multi-codeword table's place");
    constexpr bool kDot = kMode == kLanesToDot;
    constexpr bool kU8 = kMode == kLanesToU8;
    constexpr uint32_t kThreads = kWaveLanes * W;
    // multi-codeword table, then the canonical arrays for long codes (the
    // plan's tables from the multi-codeword table on)
    constexpr uint32_t kDecVec = (2u << KD) / 4, kLongVec = kLongWords / 4;
    constexpr uint32_t kTabVec = kDecVec + kLongVec;
    __shared__ __attribute__((aligned(16))) uint4 s_tab[kTabVec];
    const uint2* const s_dec = reinterpret_cast<const uint2*>(s_tab);
    const uint32_t* const s_long = reinterpret_cast<const uint32_t*>(s_tab + kDecVec);
    // dynamic: per wave, kLaneStageBytes of stream words then one
    // kLaneSlotBytes exponent slot per lane; then the second-level table
    // (l2_cap * 2^kL2Bits u16)
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    uint16_t* const s_l2 = reinterpret_cast<uint16_t*>(dyn + W * kLaneWaveBytes);

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t* const sbuf = reinterpret_cast<uint32_t*>(dyn + wave * kLaneWaveBytes + kLanePadBytes);
    uint8_t* const ebuf = dyn + wave * kLaneWaveBytes + kLanePadBytes + kLaneStageBytes;
    uint8_t* const slot = ebuf + kLaneSlotBytes * lane;   // this lane's exponents, in its symbol order

    // wave w of workgroup b takes segments b*W + w, then every (grid * W)-th
    const uint64_t stride = (uint64_t)gridDim.x * W;
    uint64_t u = p.u_begin + (uint64_t)blockIdx.x * W + wave;
    const uint64_t last_u = p.u_end - 1;
    const bool active = u < p.u_end;

    // prologue: the first segment's table entries and loads are in flight
    // while the workgroup stages the tables
    const Meta m_first = load_meta(p, min_u64(u, last_u));
    constexpr uint32_t kFull = kTabVec / kThreads;
    constexpr uint32_t kTail = kTabVec - kFull * kThreads;
    const u32x4* const tsrc = reinterpret_cast<const u32x4*>(p.tables);
    u32x4* const tdst = reinterpret_cast<u32x4*>(s_tab);
    u32x4 stage[kFull > 0 ? kFull : 1];
#pragma unroll
    for (uint32_t k = 0; k < kFull; ++k) stage[k] = tsrc[tid + k * kThreads];
    u32x4 stage_tail = {0, 0, 0, 0};
    if (kTail && tid < kTail) stage_tail = tsrc[kFull * kThreads + tid];
    Meta cur_m = uniform_meta(m_first);
    LaneRaw cur_r = load_lane_raw(p, cur_m, min_u64(u, last_u), lane);
    Meta m_next = load_meta(p, min_u64(u + stride, last_u));
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
    m_next = uniform_meta(m_next);
    uint32_t dot_mat = 0;   // fused product: matrix of the wave's current segment
    // rANS with one symbol: its frequency 2^12 is stored as 0
    const bool rans_single =
        kRans && ((__builtin_amdgcn_readfirstlane(reinterpret_cast<const uint32_t*>(s_tab)[0]) >> 8) & 0xFFFu) == 0;
    // code planes: each multi-codeword table entry holds one code at most
    const bool one_code = kU8 && !kRans && p.one_code != 0;

    for (;;) {
        const uint64_t un = u + stride;
        const bool more = un < p.u_end;

        // the segment's stream words, byte-swapped (word k = bits 32k.. MSB-first;
        // rANS: half-word q = big-endian word q)
        if constexpr (kRans) {
            reinterpret_cast<uint4*>(sbuf)[lane] = swap16x8(cur_r.q0);
            reinterpret_cast<uint4*>(sbuf)[lane + kWaveLanes] = swap16x8(cur_r.q1);
        } else {
            reinterpret_cast<uint4*>(sbuf)[lane] = bswap4(cur_r.q0);
            reinterpret_cast<uint4*>(sbuf)[lane + kWaveLanes] = bswap4(cur_r.q1);
        }
        const uint32_t off = cur_r.off;

        // next segment's loads, this segment's sign+mantissa bytes, the table
        // entries of the segment after next
        const LaneRaw nxt = load_lane_raw(p, m_next, min_u64(un, last_u), lane);
        const uint64_t A = cur_m.e0;
        const uint32_t n = (uint32_t)min_u64(cur_m.e1 - cur_m.e0, kGroupMaxElems);
        const uint32_t last_blk = (n - 1) / kMergeElems;
        const uint8_t* const smu = p.sm + A;
        uint16_t* const outu = p.out + A;
        uint2 smv[kMergeSteps];
        if constexpr (!kU8) {
#pragma unroll
            for (uint32_t k = 0; k < kMergeSteps; ++k)
                smv[k] = load_nt8(smu + kMergeElems * min(lane + k * kWaveLanes, last_blk));
        }
        // fused product: the x entries of the segment's blocks, loaded with
        // the sm bytes so that they have arrived by the merge
        DotRows dr;
        uint4 xv[kDot ? kMergeSteps : 1];
        if constexpr (kDot) {
            dr = dot_rows(p.dot, A, n, dot_mat);
            load_dot_x(dr, n, lane, xv);
        }
        const Meta m_after = load_meta(p, min_u64(un + stride, last_u));
        wave_lds_order();

        // decode: this lane's symbols (8 per lane block it owns; the
        // container's last block may be shorter)
        {
            const uint32_t nb8 = (n + kLaneBlock - 1) / kLaneBlock;
            const uint32_t cnt = lane < nb8 ? (nb8 - 1 - lane) / kWaveLanes + 1 : 0u;
            uint32_t nsym = kLaneBlock * cnt;
            if (cnt && lane == (nb8 - 1) % kWaveLanes) nsym -= kLaneBlock * nb8 - n;
            const uint32_t pos = (uint32_t)(cur_m.p0 & 127u) + off;   // first bit in the staged words
            if constexpr (kRans) {
                // the final state, then one symbol per step, eight per slot
                // store (a lane whose count is not a multiple of eight decodes
                // up to seven more into the slot's unused bytes).  Reads stay
                // in the wave's LDS region unclamped: the planner bounds every
                // lane offset by the segment's bits (<= 15872), so the first
                // half-word is at most 999, and a lane takes at most 64 steps
                // and one word per step: at most half-word 1065, byte 2131 of
                // the wave's 2048 staging and 4352 slot bytes.
                const uint16_t* const s16 = reinterpret_cast<const uint16_t*>(sbuf);
                const uint32_t* const s_slot = reinterpret_cast<const uint32_t*>(s_tab);
                if (rans_single) {
                    // one symbol of frequency 2^12: the state never moves
                    const uint32_t v = (s_slot[0] & 0xFFu) * 0x01010101u;
                    for (uint32_t p = 0; p < nsym; p += kMergeElems)
                        store_slot8(slot + p, make_uint2(v, v));
                } else {
                    uint32_t q = pos >> 4;
                    uint32_t x = (uint32_t)s16[q] << 16 | s16[q + 1];
                    q += 2;
                    for (uint32_t p = 0; p < nsym; p += kMergeElems) {
                        uint32_t e[kMergeElems];
#pragma unroll
                        for (uint32_t i = 0; i < kMergeElems; ++i) {
                            const uint32_t w = s16[q];
                            e[i] = s_slot[x & (kRansSlots - 1)];
                            // f (x >> 12) + slot - cum
                            x = __umul24((e[i] >> 8) & 0xFFFu, x >> kRansBits) + (e[i] >> 20);
                            const bool in = x < kRansLow;
                            x = in ? x << 16 | w : x;
                            q += in ? 1u : 0u;
                        }
                        // the symbols are the entries' low bytes
                        const uint32_t s0 = __builtin_amdgcn_perm(e[1], e[0], 0x0C0C0400u) |
                                            __builtin_amdgcn_perm(e[3], e[2], 0x04000C0Cu);
                        const uint32_t s1 = __builtin_amdgcn_perm(e[5], e[4], 0x0C0C0400u) |
                                            __builtin_amdgcn_perm(e[7], e[6], 0x04000C0Cu);
                        store_slot8(slot + p, make_uint2(s0, s1));
                    }
                }
            } else if constexpr (kMode == kLanesToBf16) {
                // plain decode (bound by HBM): a 64-bit MSB-first register
                // window of the lane's bits, at least 32 valid before a
                // lookup, refilled one staged word at a time (index clamped
                // to the staging).  A lookup's symbols past the lane's last
                // one (they belong to the next lane) land in the slot's spare
                // bytes: p < nsym <= 64 before the store, so it ends by byte 67
                uint32_t wi = pos >> 5;
                uint64_t win = (((uint64_t)sbuf[wi] << 32) | sbuf[wi + 1]) << (pos & 31u);
                int32_t valid = 64 - (int32_t)(pos & 31u);
                wi += 2;
                uint32_t p = 0;
                while (p < nsym) {
                    const uint32_t top = (uint32_t)(win >> 32);
                    uint2 e = s_dec[top >> (32 - KD)];
                    if (e.x == 0) e = long_decode_entry<KD>(top, KD + 1, lt);
                    uint8_t* const dst = slot + p;
                    const uint32_t odd = __builtin_amdgcn_perm(e.y, e.y, 0x0C030C01u);   // [s1, 0, s3, 0]
                    dst[0] = (uint8_t)e.y;
                    dst[1] = (uint8_t)odd;
                    dst[2] = (uint8_t)(e.y >> 16);
                    dst[3] = (uint8_t)(odd >> 16);
                    p += (e.x >> 8) & 0xFFu;
                    const uint32_t nbits = (e.x >> 16) & 0xFFu;
                    win <<= nbits;
                    valid -= (int32_t)nbits;
                    if (valid < 32) {
                        win |= (uint64_t)sbuf[min(wi, kStageWords - 1)] << (32 - valid);
                        ++wi;
                        valid += 32;
                    }
                }
            } else {
                // fused product and code planes (bound by the decode's
                // instructions and LDS): no register window; each lookup
                // re-reads its 32-bit window from the staged
                // words: t = (bit position) - 1, words t >> 5 (arithmetic:
                // -1 at position 0, the last word of the wave's pad, shifted
                // out) and the next, shifted right by -position mod 32
                // (always below 32).
                // A lookup's symbols past the lane's last one (they belong
                // to the next lane) land in the slot's spare bytes: p < nsym
                // <= 64 before the store, so it ends by byte 67.  The words
                // stay in the wave's LDS region unclamped: the planner bounds
                // every lane offset by the segment's bits (<= 15872), and a
                // lane makes at most 64 lookups of at most 24 bits (at most
                // word 548, byte 2195 of the wave's staging and slots).
                int32_t t = (int32_t)pos - 1;
                if (one_code) {
                    // code planes whose shortest code is longer than half the
                    // table index and whose codes are at most 16 bits: every
                    // lookup yields exactly one code (the entry's other
                    // symbol bytes are 0), and four of them fit one 64-bit
                    // window, read from three staged words.  Four lookups
                    // fill one aligned word.  A lane whose count is not a
                    // multiple of four decodes up to three more, into the
                    // slot's unused bytes; it still makes at most 64 lookups
                    // of at most 16 bits (at most word 530 of the wave's
                    // staging and slots) and stores below byte 64.
                    for (uint32_t q = 0; q < nsym; q += 4) {
                        const int32_t k = t >> 5;
                        const uint32_t w1 = sbuf[k + 1];
                        uint64_t win = (uint64_t)__builtin_amdgcn_alignbit(sbuf[k], w1, ~(uint32_t)t) << 32 |
                                       __builtin_amdgcn_alignbit(w1, sbuf[k + 2], ~(uint32_t)t);
                        uint32_t w = 0, used = 0;
#pragma unroll
                        for (uint32_t i = 0; i < 4; ++i) {
                            const uint32_t top = (uint32_t)(win >> 32);
                            uint2 e = s_dec[top >> (32 - KD)];
                            if (e.x == 0) e = long_decode_entry<KD>(top, KD + 1, lt);
                            w |= e.y << (8 * i);
                            const uint32_t len = (e.x >> 16) & 0xFFu;
                            win <<= len;
                            used += len;
                        }
                        t += (int32_t)used;
                        *reinterpret_cast<uint32_t*>(slot + q) = w;
                    }
                } else {
                    uint32_t p = 0;
                    // code planes (about one symbol per lookup): the symbols are
                    // gathered in a register and written as aligned words (the
                    // table's bytes past a lookup's symbols are 0); the last word
                    // ends by byte 67.  bf16 exponents for the fused product (two
                    // to three symbols per lookup): four byte stores at the count
                    // decoded so far.
                    uint32_t acc = 0;
                    while (p < nsym) {
                        const int32_t k = t >> 5;
                        const uint32_t top = __builtin_amdgcn_alignbit(sbuf[k], sbuf[k + 1], ~(uint32_t)t);
                        uint2 e = s_dec[top >> (32 - KD)];
                        if (e.x == 0) e = long_decode_entry<KD>(top, KD + 1, lt);
                        const uint32_t pn = p + ((e.x >> 8) & 0xFFu);
                        if constexpr (kU8) {
                            const uint64_t comb = ((uint64_t)e.y << ((p & 3u) << 3)) | acc;
                            if ((p ^ pn) >= 4u) {   // a word is complete
                                *reinterpret_cast<uint32_t*>(slot + (p & ~3u)) = (uint32_t)comb;
                                acc = (uint32_t)(comb >> 32);
                            } else {
                                acc = (uint32_t)comb;
                            }
                        } else {
                            uint8_t* const dst = slot + p;
                            const uint32_t odd = __builtin_amdgcn_perm(e.y, e.y, 0x0C030C01u);   // [s1, 0, s3, 0]
                            dst[0] = (uint8_t)e.y;
                            dst[1] = (uint8_t)odd;
                            dst[2] = (uint8_t)(e.y >> 16);
                            dst[3] = (uint8_t)(odd >> 16);
                        }
                        p = pn;
                        t += (int32_t)((e.x >> 16) & 0xFFu);
                    }
                    if (kU8 && (p & 3u)) *reinterpret_cast<uint32_t*>(slot + (p & ~3u)) = acc;
                }
            }
        }

        const LaneRaw next_r = nxt;
        const Meta next_m = m_next;
        m_next = uniform_meta(m_after);
        wave_lds_order();

        // merge: step k of lane i is block 64k + i, bytes 8k.. of the lane's slot
        const uint32_t full = n / kMergeElems;
        if constexpr (kDot) {
            dot_group(p.dot, dr, full, lane, smv, xv, u - p.u_begin,
                      [&](uint32_t k) { return load_slot8(slot + kMergeElems * k); });
        } else if constexpr (kU8) {
            uint8_t* const outb = p.out8 + A;
#pragma unroll
            for (uint32_t k = 0; k < kMergeSteps; ++k) {
                const uint32_t blk = lane + k * kWaveLanes;
                if (blk < full) {
                    const uint2 e2 = load_slot8(slot + kMergeElems * k);
                    u32x2 v;
                    v.x = unrotate4(e2.x);
                    v.y = unrotate4(e2.y);
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(outb + kMergeElems * blk));
                }
            }
        } else {
#pragma unroll
        for (uint32_t k = 0; k < kMergeSteps; ++k) {
            const uint32_t blk = lane + k * kWaveLanes;
            if (blk < full) {
                const uint2 e2 = load_slot8(slot + kMergeElems * k);
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
        // the container's last block, when it holds fewer than 8 elements (a
        // matrix for the fused product never ends in a partial block); block
        // `full` is the (full / 64)-th of lane full % 64
        if (kU8 && full * kMergeElems < n && lane == 0) {
            const uint32_t rel = kMergeElems * full;
            const uint2 e2 = load_slot8(ebuf + kLaneSlotBytes * (full % kWaveLanes) + kMergeElems * (full / kWaveLanes));
            const uint32_t o[2] = {unrotate4(e2.x), unrotate4(e2.y)};
#pragma unroll
            for (uint32_t i = 0; i < kMergeElems; ++i)
                if (rel + i < n) p.out8[A + rel + i] = (uint8_t)(o[i >> 2] >> (8 * (i & 3)));
        }
        if (kMode == kLanesToBf16 && full * kMergeElems < n && lane == 0) {
            const uint32_t rel = kMergeElems * full;
            const uint2 s2 = load_nt8(p.sm + A + rel);
            const uint2 e2 = load_slot8(ebuf + kLaneSlotBytes * (full % kWaveLanes) + kMergeElems * (full / kWaveLanes));
            uint32_t o[4];
            join4(s2.x, e2.x, o[0], o[1]);
            join4(s2.y, e2.y, o[2], o[3]);
#pragma unroll
            for (uint32_t i = 0; i < kMergeElems; ++i)
                if (rel + i < n) p.out[A + rel + i] = (uint16_t)(o[i >> 1] >> (16 * (i & 1)));
        }

        if (!more) break;
        wave_lds_order();   // the staging is rewritten by the next segment
        u = un;
        cur_m = next_m;
        cur_r = next_r;
    }
}

template <int KD, int W, bool kRans>
struct LanesVariant {
    static hipError_t launch(const DecodeParams& p, uint32_t grid, uint32_t dyn, LanesOut mode, hipStream_t stream) {
        const dim3 g(grid), b(kWaveLanes * W);
        if (mode == kLanesToDot)
            hipLaunchKernelGGL((decode_lanes_kernel<KD, W, kLanesToDot, kRans>), g, b, dyn, stream, p);
        else if (mode == kLanesToU8)
            hipLaunchKernelGGL((decode_lanes_kernel<KD, W, kLanesToU8, kRans>), g, b, dyn, stream, p);
        else
            hipLaunchKernelGGL((decode_lanes_kernel<KD, W, kLanesToBf16, kRans>), g, b, dyn, stream, p);
        return hipGetLastError();
    }
    static int blocks_per_cu(uint32_t dyn) {
        int n[3] = {0, 0, 0};
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[0], decode_lanes_kernel<KD, W, kLanesToBf16, kRans>,
                                                         kWaveLanes * W, dyn) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[1], decode_lanes_kernel<KD, W, kLanesToDot, kRans>,
                                                         kWaveLanes * W, dyn) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[2], decode_lanes_kernel<KD, W, kLanesToU8, kRans>,
                                                         kWaveLanes * W, dyn) != hipSuccess)
            return 0;
        return std::min(n[0], std::min(n[1], n[2]));
    }
};

template <typename F>
hipError_t dispatch_lanes(uint32_t decode_bits, uint32_t waves, bool rans, F&& f) {
    if (rans) return waves == 8 ? f(LanesVariant<11, 8, true>{}) : f(LanesVariant<11, 4, true>{});
    if (decode_bits == 11) return waves == 8 ? f(LanesVariant<11, 8, false>{}) : f(LanesVariant<11, 4, false>{});
    return waves == 8 ? f(LanesVariant<10, 8, false>{}) : f(LanesVariant<10, 4, false>{});
}

}  // namespace

uint32_t decode_lanes_dyn_lds_bytes(uint32_t waves, uint32_t l2_cap) {
    return waves * kLaneWaveBytes + (l2_cap << kL2Bits) * 2;
}

uint32_t decode_lanes_lds_bytes(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap) {
    return ((2u << decode_bits) + kLongWords) * 4 + decode_lanes_dyn_lds_bytes(waves, l2_cap);
}

int decode_lanes_blocks_per_cu(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap, bool rans) {
    if ((decode_bits != 11 && decode_bits != 10) || (rans && decode_bits != 11) || !supported_waves(waves)) return 0;
    const uint32_t dyn = decode_lanes_dyn_lds_bytes(waves, l2_cap);
    int n = 0;
    (void)dispatch_lanes(decode_bits, waves, rans, [&](auto v) {
        n = decltype(v)::blocks_per_cu(dyn);
        return hipSuccess;
    });
    return n;
}

hipError_t launch_decode_lanes(const DecodeParams& p, uint32_t decode_bits, uint32_t waves, uint32_t grid,
                               LanesOut mode, bool rans, hipStream_t stream) {
    if ((decode_bits != 11 && decode_bits != 10) || (rans && (decode_bits != 11 || p.l2_cap)) ||
        !supported_waves(waves) || p.l2_cap > kL2Prefixes)
        return hipErrorInvalidValue;
    const uint32_t dyn = decode_lanes_dyn_lds_bytes(waves, p.l2_cap);
    return dispatch_lanes(decode_bits, waves, rans,
                          [&](auto v) { return decltype(v)::launch(p, grid, dyn, mode, stream); });
}

}  // namespace wc
