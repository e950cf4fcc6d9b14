// decode_common.h -- device helpers shared by the gfx950 decode kernels of
// libwc (decode.hip: container v2, per-chunk gaps; decode_lanes.hip:
// container v3, interleaved lanes).  Included by each kernel source; every
// definition has internal linkage.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace wc {
namespace {

constexpr uint32_t kCodeLimit = 24;
// bf16 output is written with non-temporal 16-byte stores: it is not read
// again by this kernel and streams past the caches
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 8-byte non-temporal load (data read once by this kernel)
__device__ __forceinline__ uint2 load_nt8(const uint8_t* q) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(q));
    return make_uint2(v.x, v.y);
}

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

// Order this wave's LDS accesses across the point for the compiler; the LDS
// itself executes one wave's accesses in issue order, so lanes then see each
// other's earlier writes without a workgroup barrier.
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
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

// One group's entry pair in the group table (the same for every lane): its
// first element and first bit, and those of the next group.
struct Meta {
    uint64_t e0, p0, e1, p1;
};

__device__ __forceinline__ Meta load_meta(const DecodeParams& p, uint64_t u) {
    const uint4 x = *reinterpret_cast<const uint4*>(p.groups + 2 * u);
    const uint4 y = *reinterpret_cast<const uint4*>(p.groups + 2 * u + 2);
    Meta m;
    m.e0 = ((uint64_t)x.y << 32) | x.x;
    m.p0 = ((uint64_t)x.w << 32) | x.z;
    m.e1 = ((uint64_t)y.y << 32) | y.x;
    m.p1 = ((uint64_t)y.w << 32) | y.z;
    return m;
}

__device__ __forceinline__ Meta uniform_meta(const Meta& m) {
    Meta r;
    r.e0 = uniform64(m.e0);
    r.p0 = uniform64(m.p0);
    r.e1 = uniform64(m.e1);
    r.p1 = uniform64(m.p1);
    return r;
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

// Entry of the multi-codeword table for a code longer than the index: one symbol.
template <int KD>
__device__ __forceinline__ uint2 long_decode_entry(uint32_t win, uint32_t first_len, const LongTables& lt) {
    const uint32_t c = long_code<KD>(win, first_len, lt);
    const uint32_t L = c >> 8;
    return make_uint2(((32u - L) & 31u) | (1u << 8) | (L << 16), c & 0xFFu);
}

}  // namespace
}  // namespace wc
