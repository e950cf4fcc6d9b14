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
#include <type_traits>

#include "../../include/wc.h"
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
    // bytes up to the last bit, plus the lookahead (at most 2,008: the
    // planner bounds a segment's bits)
    const uint32_t need = (uint32_t)(((m.p1 + 7) >> 3) + 8 - base);
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
// the multi-codeword table's 16 KiB).  kCheck (debug plans; the plain bf16
// decode, and the fused product of rANS lanes): every lane checks that its
// decode ends its own string where the next lane's begins, and a failure ORs
// WC_DEBUG_LANE_BITS into p.status.
template <int KD, int W, uint32_t kMode, bool kRans, bool kCheck = false>
__global__ __launch_bounds__(kWaveLanes * W, kMode == kLanesToU8 ? 6 : 1) void decode_lanes_kernel(DecodeParams p) {
    static_assert(!kCheck || kMode == kLanesToBf16 || (kMode == kLanesToDot && kRans),
                  "the lane-end check is compiled into the plain bf16 decode and the rANS fused product only");
    static_assert(!kRans || (2u << KD) == kRansSlots, "the rANS slot table takes the multi-codeword table's place");
    static_assert(kMode != kLanesToDot || kRans, "the fused product of Huffman lanes is decode_lanes_dot_kernel");
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
    const uint16_t* const s_c16 = reinterpret_cast<const uint16_t*>(s_tab);   // code planes, one code per entry
    // dynamic: per wave, kLaneStageBytes of stream words then one
    // kLaneSlotBytes exponent slot per lane (code planes with one code per
    // table entry: no slots, kLaneCompactWaveBytes per wave); then the
    // second-level table (l2_cap * 2^kL2Bits u16)
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    const bool one_code = kU8 && !kRans && p.one_code != 0;
    const bool wide = kU8 && !kRans && !one_code;   // code planes with the wide table
    const uint32_t slot_bytes = wide ? kLaneWideSlotBytes : kLaneSlotBytes;
    const uint32_t wave_bytes = one_code ? kLaneCompactWaveBytes : wide ? kLaneWideWaveBytes : kLaneWaveBytes;
    uint16_t* const s_l2 = reinterpret_cast<uint16_t*>(dyn + W * wave_bytes);

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t* const sbuf = reinterpret_cast<uint32_t*>(dyn + wave * wave_bytes + kLanePadBytes);
    uint8_t* const ebuf = dyn + wave * wave_bytes + kLanePadBytes + kLaneStageBytes;
    uint8_t* const slot = ebuf + slot_bytes * lane;   // this lane's symbols, in its symbol order

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
    // code planes (Huffman) with one code per entry: the multi-codeword
    // table is staged as 16-bit entries ((32 - length) | un-rotated symbol <<
    // 8, 0 for a code longer than the index) packed into the first 2^KD / 2
    // words of the table's place, a quarter of the LDS bytes per lookup.  The
    // low bits are the alignbit shift that drops the code from a window.  (Other
    // Huffman code planes find the wide table, built by the planner, in the
    // multi-codeword table's place and stage it as it is.)
    if constexpr (kU8 && !kRans) {
        const bool compact = p.one_code != 0;
        auto put = [&](uint32_t i, u32x4 v) {
            if (compact && i < kDecVec) {
                auto c16 = [](uint32_t x, uint32_t y) {
                    return x == 0 ? 0u : ((32u - ((x >> 16) & 0xFFu)) & 31u) | (unrotate4(y) & 0xFFu) << 8;
                };
                reinterpret_cast<uint32_t*>(s_tab)[i] = c16(v.x, v.y) | c16(v.z, v.w) << 16;
                return;
            }
            tdst[i] = v;
        };
#pragma unroll
        for (uint32_t k = 0; k < kFull; ++k) put(tid + k * kThreads, stage[k]);
        if (kTail && tid < kTail) put(kFull * kThreads + tid, stage_tail);
    } else {
#pragma unroll
        for (uint32_t k = 0; k < kFull; ++k) tdst[tid + k * kThreads] = stage[k];
        if (kTail && tid < kTail) tdst[kFull * kThreads + tid] = stage_tail;
    }
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
            load_dot_x(dr, n, lane, 0, xv);
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
            // debug plans: where this lane's string ends in the staged words,
            // the next lane's first bit (the last lane's: the segment's end)
            uint32_t lane_end = 0;
            bool lane_bad = false;
            if constexpr (kCheck) {
                const uint32_t off_next = (uint32_t)__shfl_down((int)off, 1);
                lane_end = (uint32_t)(cur_m.p0 & 127u) +
                           (lane == kWaveLanes - 1 ? (uint32_t)(cur_m.p1 - cur_m.p0) : off_next);
                lane_bad = nsym == 0 && lane_end != pos;   // an empty lane has an empty string
            }
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
                    // (debug: the lane's string is its final state alone)
                    if constexpr (kCheck) lane_bad |= nsym != 0 && lane_end != pos + 32u;
                } else {
                    uint32_t q = pos >> 4;
                    uint32_t x = (uint32_t)s16[q] << 16 | s16[q + 1];
                    q += 2;
                    // debug: the state and next half-word after the lane's
                    // last symbol (the loop decodes up to seven more)
                    uint32_t x_end = kRansLow, q_end = q;
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
                            if constexpr (kCheck) {
                                if (p + i + 1 == nsym) {
                                    x_end = x;
                                    q_end = q;
                                }
                            }
                        }
                        // the symbols are the entries' low bytes
                        const uint32_t s0 = __builtin_amdgcn_perm(e[1], e[0], 0x0C0C0400u) |
                                            __builtin_amdgcn_perm(e[3], e[2], 0x04000C0Cu);
                        const uint32_t s1 = __builtin_amdgcn_perm(e[5], e[4], 0x0C0C0400u) |
                                            __builtin_amdgcn_perm(e[7], e[6], 0x04000C0Cu);
                        store_slot8(slot + p, make_uint2(s0, s1));
                    }
                    // debug: a lane ends in the encoder's initial state,
                    // exactly where the next lane's string begins
                    if constexpr (kCheck) lane_bad |= nsym != 0 && (x_end != kRansLow || 16u * q_end != lane_end);
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
                uint32_t last_bits = 0;   // debug: the bits of the lane's last lookup
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
                    if constexpr (kCheck) last_bits = nbits;
                    win <<= nbits;
                    valid -= (int32_t)nbits;
                    if (valid < 32) {
                        win |= (uint64_t)sbuf[min(wi, kStageWords - 1)] << (32 - valid);
                        ++wi;
                        valid += 32;
                    }
                }
                // debug: the window starts at staged bit 32 wi - valid; the
                // lane's last symbol ends inside its last lookup (whose
                // further symbols, if any, belong to the next lane)
                if constexpr (kCheck) {
                    const uint32_t at = 32u * wi - (uint32_t)valid;
                    lane_bad |= nsym != 0 && !(at - last_bits < lane_end && lane_end <= at);
                }
            } else {
                // code planes (bound by the decode's instructions and LDS):
                // no register window; each lookup
                // re-reads its 32-bit window from the staged
                // words: t = (bit position) - 1, words t >> 5 (arithmetic:
                // -1 at position 0, the last word of the wave's pad, shifted
                // out) and the next, shifted right by -position mod 32
                // (always below 32).
                // A lookup's symbols past the lane's last one (they belong
                // to the next lane) land in the slot's spare bytes: c < nsym
                // <= 64 before the store, so it ends by byte 67.  The words
                // stay in the wave's LDS region unclamped: the planner bounds
                // every lane offset by the segment's bits (<= 15872), and a
                // lane makes at most 64 lookups of at most 24 bits (at most
                // word 548, byte 2195 of the wave's staging and slots).
                // The long-code lookup is compiled in only for codebooks with
                // codes longer than the table index.
                int32_t t = (int32_t)pos - 1;
                auto run = [&](auto has_long) {
                    constexpr bool kLong = decltype(has_long)::value;
                    if (one_code) {
                        // the shortest code is longer than half the table
                        // index and no code exceeds 16 bits: every lookup
                        // yields exactly one code; eight of them fit one
                        // 96-bit window of four staged words when no code
                        // exceeds the index, else four fit one 64-bit
                        // window of three.
                        // Eight lookups make one lane block, stored straight
                        // to memory (block 64k + lane is the lane's k-th: a
                        // wave's store covers 512 contiguous bytes); the
                        // container's last, partial block byte by byte.  A
                        // lane whose count is not a multiple of eight
                        // decodes up to seven more symbols, never stored; it
                        // still makes at most 64 lookups of at most 16 bits,
                        // so it reads at most word 533 past the pad (byte
                        // 2136 of the wave's region of 2192; with codes of
                        // at most 11 bits, the 96-bit windows end by word
                        // 522).
                        uint8_t* const outb = p.out8 + A;
                        const uint32_t full = n / kMergeElems;
                        for (uint32_t q = 0; q < nsym; q += 8) {
                            uint32_t w[2];
                            if constexpr (!kLong) {
                                // no code exceeds the table index (KD <=
                                // 11 bits): the eight codes (at most 88
                                // bits) come from one 96-bit window of four
                                // staged words, held in three registers;
                                // each lookup's entry shifts them by its
                                // code (its low bits are 32 - length,
                                // alignbit's shift).  The sum of the eight
                                // entries' low bytes is that of their
                                // 32 - length (each at most 26: at most 208).
                                const int32_t k = t >> 5;
                                const uint32_t s1 = sbuf[k + 1], s2 = sbuf[k + 2];
                                uint32_t hi = __builtin_amdgcn_alignbit(sbuf[k], s1, ~(uint32_t)t);
                                uint32_t mid = __builtin_amdgcn_alignbit(s1, s2, ~(uint32_t)t);
                                uint32_t lo = __builtin_amdgcn_alignbit(s2, sbuf[k + 3], ~(uint32_t)t);
                                uint32_t e[8];
#pragma unroll
                                for (uint32_t i = 0; i < 8; ++i) {
                                    e[i] = s_c16[hi >> (32 - KD)];
                                    hi = __builtin_amdgcn_alignbit(hi, mid, e[i]);
                                    mid = __builtin_amdgcn_alignbit(mid, lo, e[i]);
                                    lo = __builtin_amdgcn_alignbit(lo, 0u, e[i]);
                                }
                                // the symbols are the entries' second bytes
                                w[0] = __builtin_amdgcn_perm(e[1], e[0], 0x0C0C0501u) |
                                       __builtin_amdgcn_perm(e[3], e[2], 0x05010C0Cu);
                                w[1] = __builtin_amdgcn_perm(e[5], e[4], 0x0C0C0501u) |
                                       __builtin_amdgcn_perm(e[7], e[6], 0x05010C0Cu);
                                const uint32_t sum = e[0] + e[1] + e[2] + e[3] + e[4] + e[5] + e[6] + e[7];
                                t += (int32_t)(256u - (sum & 0xFFu));
                            } else {
#pragma unroll
                                for (uint32_t h = 0; h < 2; ++h) {
                                    const int32_t k = t >> 5;
                                    const uint32_t w1 = sbuf[k + 1];
                                    uint64_t win =
                                        (uint64_t)__builtin_amdgcn_alignbit(sbuf[k], w1, ~(uint32_t)t) << 32 |
                                        __builtin_amdgcn_alignbit(w1, sbuf[k + 2], ~(uint32_t)t);
                                    uint32_t acc = 0, used = 0;
#pragma unroll
                                    for (uint32_t i = 0; i < 4; ++i) {
                                        const uint32_t top = (uint32_t)(win >> 32);
                                        uint32_t e = s_c16[top >> (32 - KD)];
                                        if (e == 0) {
                                            const uint2 l = long_decode_entry<KD>(top, KD + 1, lt);
                                            e = ((32u - ((l.x >> 16) & 0xFFu)) & 31u) | (unrotate4(l.y) & 0xFFu) << 8;
                                        }
                                        acc |= (e >> 8) << (8 * i);
                                        const uint32_t len = 32u - (e & 31u);
                                        win <<= len;
                                        used += len;
                                    }
                                    t += (int32_t)used;
                                    w[h] = acc;
                                }
                            }
                            const uint32_t blk = lane + kWaveLanes * (q / kMergeElems);
                            if (blk < full) {
                                u32x2 v;
                                v.x = w[0];
                                v.y = w[1];
                                __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(outb + kMergeElems * blk));
                            } else if (blk == full) {
#pragma unroll
                                for (uint32_t i = 0; i < kMergeElems; ++i)
                                    if (kMergeElems * full + i < n)
                                        outb[kMergeElems * full + i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
                            }
                        }
                    } else {
                        // the wide table: a (KD + 1)-bit index, 4-byte entries
                        // of up to three whole codes (total bits | count << 5
                        // | symbols << 8, first in the low byte; 0 when the
                        // first code is longer than the index).  Symbols go
                        // to the slot as aligned words, one store per
                        // lookup: `acc` holds the bytes [c & ~3, c) decoded
                        // so far (its other bytes 0); a lookup's symbols,
                        // shifted to c & 3, join it, the word at c & ~3 is
                        // stored and the part past that word carries over.
                        // Two phases of 32 symbols (the lane's blocks 0..3,
                        // then 4..7), each stored to memory right after it,
                        // share a 36-byte slot (symbol c of phase h at byte
                        // c - 32h), so that three 8-wave workgroups fit a
                        // compute unit.  A lookup starts only below its
                        // phase's end and adds at most three symbols, so a
                        // phase's stores end by byte 35; the bytes it carries
                        // past 32 go on in `acc` (32 is a multiple of 4).
                        // With the phase's end a multiple of 4, every symbol
                        // below it is stored once the phase ends.
                        const uint32_t* const s_wide = reinterpret_cast<const uint32_t*>(s_tab);
                        constexpr uint32_t KW = KD + 1;
                        // (sh = 8 (c & 3), kept in a register of its own)
                        int32_t c = 0;
                        uint32_t acc = 0, sh = 0;
                        auto put = [&](uint32_t e) {
                            const uint32_t ns = (e >> 5) & 3u;
                            const uint64_t w = (uint64_t)(e >> 8) << sh;
                            const uint32_t lo = (uint32_t)w | acc;
                            *reinterpret_cast<uint32_t*>(slot + (c & ~3)) = lo;
                            const uint32_t s2 = sh + 8u * ns;
                            acc = s2 >= 32u ? (uint32_t)(w >> 32) : lo;
                            sh = s2 & 24u;
                            c += (int32_t)ns;
                        };
                        uint8_t* const outb = p.out8 + A;
                        const uint32_t full = n / kMergeElems;
#pragma unroll
                        for (uint32_t h = 0; h < 2; ++h) {
                            const int32_t end = (int32_t)min(nsym, kWidePhase * (h + 1)) - (int32_t)(kWidePhase * h);
                            if constexpr (!kLong) {
                                // every code fits the index (and the code is
                                // complete, so every entry holds one at
                                // least): up to four lookups of at most KW
                                // bits per 64-bit window, read from three
                                // staged words.  A lane makes at most 64
                                // lookups of at most 12 bits (at most word
                                // 524 of the wave's staging and slots).
                                while (c < end) {
                                    const int32_t k = t >> 5;
                                    const uint32_t w1 = sbuf[k + 1];
                                    uint64_t win =
                                        (uint64_t)__builtin_amdgcn_alignbit(sbuf[k], w1, ~(uint32_t)t) << 32 |
                                        __builtin_amdgcn_alignbit(w1, sbuf[k + 2], ~(uint32_t)t);
                                    uint32_t used = 0;
#pragma unroll
                                    for (uint32_t i = 0; i < 4; ++i) {
                                        if (i == 0 || c < end) {
                                            const uint32_t e = s_wide[(uint32_t)(win >> 32) >> (32 - KW)];
                                            put(e);
                                            const uint32_t nb = e & 31u;
                                            win <<= nb;
                                            used += nb;
                                        }
                                    }
                                    t += (int32_t)used;
                                }
                            } else {
                                // codes longer than the index: one lookup
                                // per window, re-read at every lookup (a
                                // long code takes up to 24 bits).
                                while (c < end) {
                                    const int32_t k = t >> 5;
                                    const uint32_t top =
                                        __builtin_amdgcn_alignbit(sbuf[k], sbuf[k + 1], ~(uint32_t)t);
                                    uint32_t e = s_wide[top >> (32 - KW)];
                                    if (e == 0) {
                                        const uint2 l = long_decode_entry<KD>(top, KD + 1, lt);
                                        e = ((l.x >> 16) & 31u) | 1u << 5 | (unrotate4(l.y) & 0xFFu) << 8;
                                    }
                                    put(e);
                                    t += (int32_t)(e & 31u);
                                }
                            }
                            // the container's last, partial block may end
                            // inside a word still held in acc (a lane with
                            // no symbols in this phase has c <= 0 and
                            // nothing to add: its slot offset would be
                            // negative)
                            if (c > 0 && (c & 3)) *reinterpret_cast<uint32_t*>(slot + (c & ~3)) = acc;
                            wave_lds_order();
#pragma unroll
                            for (uint32_t i = 0; i < kMergeSteps / 2; ++i) {
                                const uint32_t blk = lane + kWaveLanes * (kMergeSteps / 2 * h + i);
                                if (blk < full) {
                                    const uint2 e2 = load_slot8(slot + kMergeElems * i);
                                    u32x2 v;
                                    v.x = e2.x;
                                    v.y = e2.y;
                                    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(outb + kMergeElems * blk));
                                }
                            }
                            if (h == 0) {
                                c -= (int32_t)kWidePhase;
                                wave_lds_order();   // the second phase rewrites the slot
                            }
                        }
                    }
                };
                if (p.no_long)
                    run(std::false_type{});
                else
                    run(std::true_type{});
            }
            // debug plans: one vector-memory atomic OR per wave whose lanes
            // found a string that does not end where the next one begins (a
            // corrupted stream or lane offset, which wc_plan cannot see)
            if constexpr (kCheck) {
                if (__ballot(lane_bad) != 0 && lane == 0) atomicOr(p.status, WC_DEBUG_LANE_BITS);
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
                if (kRans && blk < full) {   // Huffman code planes: stored by the decode
                    const uint2 e2 = load_slot8(slot + kMergeElems * k);
                    u32x2 v;
                    v.x = kRans ? unrotate4(e2.x) : e2.x;
                    v.y = kRans ? unrotate4(e2.y) : e2.y;
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
        if (kU8 && !one_code && full * kMergeElems < n && lane == 0) {
            const uint32_t rel = kMergeElems * full;
            // (the wide table's slots hold one phase of four blocks)
            const uint32_t at = wide ? (full / kWaveLanes) % (kMergeSteps / 2) : full / kWaveLanes;
            const uint2 e2 = load_slot8(ebuf + slot_bytes * (full % kWaveLanes) + kMergeElems * at);
            const uint32_t o[2] = {kRans ? unrotate4(e2.x) : e2.x, kRans ? unrotate4(e2.y) : e2.y};
#pragma unroll
            for (uint32_t i = 0; i < kMergeElems; ++i)
                if (rel + i < n) p.out8[A + rel + i] = (uint8_t)(o[i >> 2] >> (8 * (i & 3)));
        }
        if (kMode == kLanesToBf16 && full * kMergeElems < n && lane == 0) {
            const uint32_t rel = kMergeElems * full;
            const uint2 s2 = load_nt8(p.sm + A + rel);
            const uint2 e2 =
                load_slot8(ebuf + kLaneSlotBytes * (full % kWaveLanes) + kMergeElems * (full / kWaveLanes));
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

// ---- fused decode -> matrix-vector product of Huffman lanes -----------------
//
// The fused product reads only the container, so the decode's own latency and
// instructions bound it, not HBM: it runs with as many waves in flight as the
// LDS and the register file allow.  Each lane decodes its (at most 64)
// symbols in two phases of 32, its lane blocks 0..3 and then 4..7, into a
// 36-byte slot, and the wave multiplies the phase's four blocks right after
// it.  A wave's LDS region is 4,368 bytes instead of 6,416, so three 8-wave
// workgroups fit a compute unit (24 waves instead of 16), and only one
// phase's x entries are held in registers at a time.
// The symbols go to the slot as aligned dwords, one store per lookup: `acc`
// holds the bytes [c & ~3, c) decoded but not yet stored (its other bytes are
// 0); a lookup's up to four symbols, shifted to c & 3, join it, the dword at
// c & ~3 is stored and the part past that dword carries over, also from one
// phase into the next (the second phase stores symbol c at slot byte c - 32).
// The shift 8 (c & 3) is kept in a register of its own and advanced by the
// entry's 8 * (symbol count), which the staging adds to each multi-codeword
// entry's top byte: that sum, past 31, is also the carry test.
// Every byte a merge reads lies below the phase's end, in a dword that the
// last lookup reaching it stored whole; bytes past the lane's symbols are
// never multiplied.
constexpr uint32_t kDotHalf = 32;                 // symbols per lane and phase
constexpr uint32_t kDotSlotBytes = kDotHalf + 4;  // 9 dwords: an odd stride across the LDS banks
constexpr uint32_t kDotSteps = kMergeSteps / 2;   // merge steps per phase
constexpr uint32_t kDotWaveBytes = kLanePadBytes + kLaneStageBytes + kWaveLanes * kDotSlotBytes;

// kCheck (debug plans): the lane-end check of the plain decode, with a failure
// ORed into p.status as WC_DEBUG_LANE_BITS.
template <int KD, int W, bool kCheck = false>
__global__ __launch_bounds__(kWaveLanes * W, 6) void decode_lanes_dot_kernel(DecodeParams p) {
    constexpr uint32_t kThreads = kWaveLanes * W;
    constexpr uint32_t kDecVec = (2u << KD) / 4, kLongVec = kLongWords / 4;
    constexpr uint32_t kTabVec = kDecVec + kLongVec;
    __shared__ __attribute__((aligned(16))) uint4 s_tab[kTabVec];
    const uint2* const s_dec = reinterpret_cast<const uint2*>(s_tab);
    const uint32_t* const s_long = reinterpret_cast<const uint32_t*>(s_tab + kDecVec);
    // dynamic: per wave the 16-byte pad, kLaneStageBytes of stream words and
    // one kDotSlotBytes slot per lane; then the second-level table
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    uint16_t* const s_l2 = reinterpret_cast<uint16_t*>(dyn + W * kDotWaveBytes);

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t* const sbuf = reinterpret_cast<uint32_t*>(dyn + wave * kDotWaveBytes + kLanePadBytes);
    uint8_t* const slot = dyn + wave * kDotWaveBytes + kLanePadBytes + kLaneStageBytes + kDotSlotBytes * lane;

    const uint64_t stride = (uint64_t)gridDim.x * W;
    uint64_t u = p.u_begin + (uint64_t)blockIdx.x * W + wave;
    const uint64_t last_u = p.u_end - 1;
    const bool active = u < p.u_end;

    // prologue: the first segment's entries and loads are in flight while the
    // workgroup stages the tables
    const Meta m_first = load_meta_scalar(p, min_u64(u, last_u));
    constexpr uint32_t kFull = kTabVec / kThreads;
    constexpr uint32_t kTail = kTabVec - kFull * kThreads;
    const u32x4* const tsrc = reinterpret_cast<const u32x4*>(p.tables);
    u32x4* const tdst = reinterpret_cast<u32x4*>(s_tab);
    u32x4 stage[kFull > 0 ? kFull : 1];
#pragma unroll
    for (uint32_t k = 0; k < kFull; ++k) stage[k] = tsrc[tid + k * kThreads];
    u32x4 stage_tail = {0, 0, 0, 0};
    if (kTail && tid < kTail) stage_tail = tsrc[kFull * kThreads + tid];
    Meta cur_m = m_first;
    LaneRaw cur_r = load_lane_raw(p, cur_m, min_u64(u, last_u), lane);
    Meta m_next = load_meta_scalar(p, min_u64(u + stride, last_u));
    // multi-codeword entries gain 8 * (symbol count) in their top byte (the
    // table's own top byte is 0; the rest of the tables are copied as they are)
    auto put = [&](uint32_t i, u32x4 v) {
        if (i < kDecVec) {
            v.x |= (v.x & 0xFF00u) << 19;
            v.z |= (v.z & 0xFF00u) << 19;
        }
        tdst[i] = v;
    };
#pragma unroll
    for (uint32_t k = 0; k < kFull; ++k) put(tid + k * kThreads, stage[k]);
    if (kTail && tid < kTail) put(kFull * kThreads + tid, stage_tail);
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
    uint32_t dot_mat = 0;   // matrix of the wave's current segment

    for (;;) {
        const uint64_t un = u + stride;
        const bool more = un < p.u_end;
        reinterpret_cast<uint4*>(sbuf)[lane] = bswap4(cur_r.q0);
        reinterpret_cast<uint4*>(sbuf)[lane + kWaveLanes] = bswap4(cur_r.q1);
        const uint32_t off = cur_r.off;

        // the next segment's stream and lane offset, this segment's first
        // phase of sign and mantissa bytes and x entries, the table entries
        // of the segment after next
        const LaneRaw nxt = load_lane_raw(p, m_next, min_u64(un, last_u), lane);
        const uint64_t A = cur_m.e0;
        // the planner bounds every segment by the element cap (at most 4096)
        const uint32_t n = min((uint32_t)cur_m.e1 - (uint32_t)cur_m.e0, kGroupMaxElems);
        const uint32_t last_blk = (n - 1) / kMergeElems;
        uint2 smv[kDotSteps];
        auto load_sm = [&](uint32_t k0) {
#pragma unroll
            for (uint32_t i = 0; i < kDotSteps; ++i)
                smv[i] = load_nt8(p.sm + A + kMergeElems * min(lane + (k0 + i) * kWaveLanes, last_blk));
        };
        load_sm(0);
        const DotRows dr = dot_rows(p.dot, A, n, dot_mat);
        uint4 xv[kDotSteps];
        load_dot_x(dr, n, lane, 0, xv);
        const Meta m_after = load_meta_scalar(p, min_u64(un + stride, last_u));
        wave_lds_order();

        const uint32_t nb8 = (n + kLaneBlock - 1) / kLaneBlock;
        const uint32_t cnt = lane < nb8 ? (nb8 - 1 - lane) / kWaveLanes + 1 : 0u;
        uint32_t nsym = kLaneBlock * cnt;
        if (cnt && lane == (nb8 - 1) % kWaveLanes) nsym -= kLaneBlock * nb8 - n;
        // the window of bit position b is kept as nb = -b: staged words
        // (b - 1) >> 5 = -1 - (nb >> 5) (arithmetic: -1 at position 0, the
        // pad's last word, shifted out) and the next, shifted right by
        // nb mod 32 (one instruction fewer per lookup than keeping b - 1).  A
        // lane's first bit is at most 15,999 (the planner bounds lane offsets
        // by the segment's bits) and it makes at most 64 lookups of at most 24
        // bits, so its last window word is at most 548: inside the wave's
        // staging and slots.
        int32_t nb = -(int32_t)((uint32_t)(cur_m.p0 & 127u) + off);
        // debug plans: this lane's string ends at the next lane's first bit
        // (the last lane's: the segment's end); the bits of its last lookup
        uint32_t lane_end = 0, last_bits = 0;
        if constexpr (kCheck) {
            const uint32_t off_next = (uint32_t)__shfl_down((int)off, 1);
            lane_end = (uint32_t)(cur_m.p0 & 127u) +
                       (lane == kWaveLanes - 1 ? (uint32_t)(cur_m.p1 - cur_m.p0) : off_next);
        }
        // the symbol count is kept as the LDS byte address of the next symbol
        // (a local-address-space offset; slots are 4-byte aligned, so its low
        // two bits are the count's)
        typedef __attribute__((address_space(3))) uint8_t LdsByte;
        typedef __attribute__((address_space(3))) uint32_t LdsWord;
        const uint32_t slot_addr = (uint32_t)(uintptr_t)(LdsByte*)slot;
        const uint32_t sbuf_addr = (uint32_t)(uintptr_t)(LdsByte*)(sbuf - 1);   // word -1: the pad's last
        uint32_t a = slot_addr;
        uint32_t acc = 0;
        uint32_t sh = 0;   // 8 * (a & 3) (the phase change moves a by 32, which keeps it)
        const uint32_t full = n / kMergeElems;
        float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            // symbol c of this phase goes to slot byte c - 32h
            const uint32_t end = slot_addr + min(nsym, kDotHalf * (h + 1)) - kDotHalf * h;
            while (a < end) {
                // word -1 - (nb >> 5) of the staging: one v_mad_i32_i24
                // (the compiler otherwise splits the multiply-add in two)
                uint32_t waddr;
                asm("v_mad_i32_i24 %0, %1, -4, %2" : "=v"(waddr) : "v"(nb >> 5), "s"(sbuf_addr));
                const LdsWord* const wp = (const LdsWord*)(uintptr_t)waddr;
                const uint32_t top = __builtin_amdgcn_alignbit(wp[0], wp[1], (uint32_t)nb);
                uint2 e = s_dec[top >> (32 - KD)];
                if (e.x == 0) {
                    e = long_decode_entry<KD>(top, KD + 1, lt);
                    e.x |= 8u << 24;
                }
                const uint64_t w = (uint64_t)e.y << sh;
                const uint32_t lo = (uint32_t)w | acc;
                *(LdsWord*)(uintptr_t)(a & ~3u) = lo;
                const uint32_t s2 = sh + (e.x >> 24);
                acc = s2 >= 32u ? (uint32_t)(w >> 32) : lo;
                sh = s2 & 24u;
                a += (e.x >> 8) & 0xFFu;
                nb -= (int32_t)((e.x >> 16) & 0xFFu);
                if constexpr (kCheck) last_bits = (e.x >> 16) & 0xFFu;
            }
            a -= kDotHalf * (h == 0);
            wave_lds_order();
            // merge steps 4h .. 4h + 3: slot bytes 8i of block lane + 64(4h + i)
            uint2 e2[kDotSteps];
#pragma unroll
            for (uint32_t i = 0; i < kDotSteps; ++i) e2[i] = load_slot8(slot + kMergeElems * i);
            float d[kDotSteps];
            dot_steps(smv, e2, xv, d);
            add_dot_steps(dr, full, lane, kDotSteps * h, d, acc0, acc1);
            if (h == 0) {   // the second phase's operands, in flight while it decodes
                load_sm(kDotSteps);
                load_dot_x(dr, n, lane, kDotSteps, xv);
            }
            wave_lds_order();   // the second phase rewrites the slot
        }
        finish_dot(p.dot, dr, lane, u - p.u_begin, acc0, acc1);
        if constexpr (kCheck) {
            // the window's bit is -nb: the lane's last lookup must span its
            // string's end (an empty lane's string is empty)
            const uint32_t at = (uint32_t)(-nb), start = (uint32_t)(cur_m.p0 & 127u) + off;
            const bool bad = nsym == 0 ? lane_end != start : !(at - last_bits < lane_end && lane_end <= at);
            if (__ballot(bad) != 0 && lane == 0) atomicOr(p.status, WC_DEBUG_LANE_BITS);
        }

        const LaneRaw next_r = nxt;
        const Meta next_m = m_next;
        m_next = m_after;
        if (!more) break;
        wave_lds_order();   // the staging is rewritten by the next segment
        u = un;
        cur_m = next_m;
        cur_r = next_r;
    }
}

template <int KD, int W>
struct LanesDotVariant {
    static hipError_t launch(const DecodeParams& p, uint32_t grid, uint32_t dyn, hipStream_t stream) {
        if (p.status)   // debug plans: the kernel compiled with the lane-end check
            hipLaunchKernelGGL((decode_lanes_dot_kernel<KD, W, true>), dim3(grid), dim3(kWaveLanes * W), dyn, stream, p);
        else
            hipLaunchKernelGGL((decode_lanes_dot_kernel<KD, W>), dim3(grid), dim3(kWaveLanes * W), dyn, stream, p);
        return hipGetLastError();
    }
    static int blocks_per_cu(uint32_t dyn) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_lanes_dot_kernel<KD, W>, kWaveLanes * W, dyn) !=
            hipSuccess)
            return 0;
        return n;
    }
};

template <typename F>
hipError_t dispatch_lanes_dot(uint32_t decode_bits, uint32_t waves, F&& f) {
    if (decode_bits == 11) return waves == 8 ? f(LanesDotVariant<11, 8>{}) : f(LanesDotVariant<11, 4>{});
    return waves == 8 ? f(LanesDotVariant<10, 8>{}) : f(LanesDotVariant<10, 4>{});
}

template <int KD, int W, bool kRans>
struct LanesVariant {
    static hipError_t launch(const DecodeParams& p, uint32_t grid, uint32_t dyn, LanesOut mode, hipStream_t stream) {
        const dim3 g(grid), b(kWaveLanes * W);
        if (mode == kLanesToDot) {
            if constexpr (kRans) {
                if (p.status)   // debug plans: the kernel compiled with the lane-end check
                    hipLaunchKernelGGL((decode_lanes_kernel<KD, W, kLanesToDot, kRans, true>), g, b, dyn, stream, p);
                else
                    hipLaunchKernelGGL((decode_lanes_kernel<KD, W, kLanesToDot, kRans>), g, b, dyn, stream, p);
            } else
                return hipErrorInvalidValue;   // Huffman lanes: launch_decode_lanes_dot
        } else if (mode == kLanesToU8)
            hipLaunchKernelGGL((decode_lanes_kernel<KD, W, kLanesToU8, kRans>), g, b, dyn, stream, p);
        else if (p.status)   // debug plans: the kernel compiled with the lane-end check
            hipLaunchKernelGGL((decode_lanes_kernel<KD, W, kLanesToBf16, kRans, true>), g, b, dyn, stream, p);
        else
            hipLaunchKernelGGL((decode_lanes_kernel<KD, W, kLanesToBf16, kRans>), g, b, dyn, stream, p);
        return hipGetLastError();
    }
    static int blocks_per_cu(uint32_t dyn) {
        int n[3] = {0, 0, 0};
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[0], decode_lanes_kernel<KD, W, kLanesToBf16, kRans>,
                                                         kWaveLanes * W, dyn) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[2], decode_lanes_kernel<KD, W, kLanesToU8, kRans>,
                                                         kWaveLanes * W, dyn) != hipSuccess)
            return 0;
        n[1] = n[0];
        if constexpr (kRans) {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[1], decode_lanes_kernel<KD, W, kLanesToDot, kRans>,
                                                             kWaveLanes * W, dyn) != hipSuccess)
                return 0;
        }
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

uint32_t decode_lanes_dyn_lds_bytes(uint32_t waves, uint32_t l2_cap, LaneLds layout) {
    return waves * lane_wave_bytes(layout) + (l2_cap << kL2Bits) * 2;
}

uint32_t decode_lanes_lds_bytes(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap, LaneLds layout) {
    return ((2u << decode_bits) + kLongWords) * 4 + decode_lanes_dyn_lds_bytes(waves, l2_cap, layout);
}

int decode_lanes_blocks_per_cu(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap, bool rans, LaneLds layout) {
    if ((decode_bits != 11 && decode_bits != 10) || (rans && decode_bits != 11) || !supported_waves(waves)) return 0;
    const uint32_t dyn = decode_lanes_dyn_lds_bytes(waves, l2_cap, layout);
    int n = 0;
    (void)dispatch_lanes(decode_bits, waves, rans, [&](auto v) {
        n = decltype(v)::blocks_per_cu(dyn);
        return hipSuccess;
    });
    return n;
}

uint32_t decode_lanes_dot_lds_bytes(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap) {
    return ((2u << decode_bits) + kLongWords) * 4 + waves * kDotWaveBytes + (l2_cap << kL2Bits) * 2;
}

int decode_lanes_dot_blocks_per_cu(uint32_t decode_bits, uint32_t waves, uint32_t l2_cap) {
    if ((decode_bits != 11 && decode_bits != 10) || !supported_waves(waves)) return 0;
    const uint32_t dyn = waves * kDotWaveBytes + (l2_cap << kL2Bits) * 2;
    int n = 0;
    (void)dispatch_lanes_dot(decode_bits, waves, [&](auto v) {
        n = decltype(v)::blocks_per_cu(dyn);
        return hipSuccess;
    });
    return n;
}

hipError_t launch_decode_lanes_dot(const DecodeParams& p, uint32_t decode_bits, uint32_t waves, uint32_t grid,
                                   hipStream_t stream) {
    if ((decode_bits != 11 && decode_bits != 10) || !supported_waves(waves) || p.l2_cap > kL2Prefixes)
        return hipErrorInvalidValue;
    const uint32_t dyn = waves * kDotWaveBytes + (p.l2_cap << kL2Bits) * 2;
    return dispatch_lanes_dot(decode_bits, waves, [&](auto v) { return decltype(v)::launch(p, grid, dyn, stream); });
}

hipError_t launch_decode_lanes(const DecodeParams& p, uint32_t decode_bits, uint32_t waves, uint32_t grid,
                               LanesOut mode, bool rans, hipStream_t stream) {
    if ((decode_bits != 11 && decode_bits != 10) || (rans && (decode_bits != 11 || p.l2_cap)) ||
        !supported_waves(waves) || p.l2_cap > kL2Prefixes)
        return hipErrorInvalidValue;
    const LaneLds layout = mode != kLanesToU8 || rans ? kLdsSlots : p.one_code ? kLdsCompact : kLdsWide;
    const uint32_t dyn = decode_lanes_dyn_lds_bytes(waves, p.l2_cap, layout);
    return dispatch_lanes(decode_bits, waves, rans,
                          [&](auto v) { return decltype(v)::launch(p, grid, dyn, mode, stream); });
}

}  // namespace wc
