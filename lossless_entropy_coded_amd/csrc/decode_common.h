// decode_common.h -- device helpers shared by the gfx950 decode kernels of
// libwc (decode.hip: container v2, per-chunk gaps; decode_lanes.hip:
// container v3, interleaved lanes): the long-code tables, group-table
// entries, the bf16 join, and the pieces of the fused matrix-vector product.
// Included by each kernel source; every definition has internal linkage.
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

// A group's or segment's entry pair read through the scalar data cache (the
// table is read-only while a kernel runs, and the index is uniform): the
// entries land in scalar registers, not in every lane's vector registers.
__device__ __forceinline__ Meta load_meta_scalar(const DecodeParams& p, uint64_t u) {
    typedef __attribute__((address_space(4))) const uint32_t* ConstU32;
    const ConstU32 g = (ConstU32)(uintptr_t)(p.groups + 2 * u);
    Meta m;
    m.e0 = ((uint64_t)g[1] << 32) | g[0];
    m.p0 = ((uint64_t)g[3] << 32) | g[2];
    m.e1 = ((uint64_t)g[5] << 32) | g[4];
    m.p1 = ((uint64_t)g[7] << 32) | g[6];
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

// ---- fused decode -> matrix-vector product ----------------------------------

// Dot product of 8 bf16 weights (four words, element k in bits 16(k & 1)..
// of word k / 2) with 8 bf16 inputs in the same layout, in element-pair
// order with v_dot2_f32_bf16.  The instruction adds two exact products to its
// accumulator after aligning the three addends to the largest and dropping
// the bits below 2^-24 of it, then rounds once, so each step errs by at most
// 3 * 2^-24 times the sum of the addends' magnitudes; subnormals are kept.
__device__ __forceinline__ float dot8_bf16(uint32_t o0, uint32_t o1, uint32_t o2, uint32_t o3, const uint4& xv) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, o0), __builtin_bit_cast(bf16x2, xv.x), 0.0f,
                                              false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, o1), __builtin_bit_cast(bf16x2, xv.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, o2), __builtin_bit_cast(bf16x2, xv.z), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, o3), __builtin_bit_cast(bf16x2, xv.w), d, false);
    return d;
}

// Sum of v over the wave's 64 lanes with DPP, in a fixed order of six levels:
// partners within quads (lane xor 1, xor 2), mirrored halves of each 8 and
// each 16 lanes, then rows of 16 added by the row broadcasts (row 1 += row 0,
// row 3 += row 2, then rows 2 and 3 += row 1).  Lane 63 ends with the total.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}
__device__ __forceinline__ float wave_total(float v) {
    v = dpp_add<0xB1, 0xF>(v);    // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E, 0xF>(v);    // quad_perm [2, 3, 0, 1]
    v = dpp_add<0x141, 0xF>(v);   // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);   // row_mirror
    v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t magic, uint32_t shift) {
    const uint32_t t = __umulhi(n, magic);
    return (t + ((n - t) >> 1)) >> shift;
}

// Where one group's elements fall among the rows of the fused product: the
// two rows it may touch, as element offsets relative to the group's first
// element A.  Every field is wave-uniform.
struct DotRows {
    uint32_t lo_rel, hi_rel;    // elements [A + lo_rel, A + hi_rel) are multiplied
    uint32_t r1_rel;            // first element of the second row (>= hi_rel: none)
    int32_t off0, off1;         // column = relative offset + off0 (first row) or + off1 (second row)
    const uint16_t* x0;
    const uint16_t* x1;
    uint32_t row0;              // global index of the first row
    bool starts_row0;           // the group holds the first element of row0
    bool starts_row1;           // the group holds the first element of row0 + 1
    bool simple;                // every element of the group is multiplied, all in row0
};

// `mat` is the matrix of the wave's previous group (0 at first): a wave's
// groups come in increasing order, so it only moves forward.
__device__ __forceinline__ DotRows dot_rows(const DotParams& q, uint64_t A, uint32_t n, uint32_t& mat) {
    DotRows d;
    const uint64_t lo = A > q.bounds[0] ? A : q.bounds[0];
    uint32_t k = mat;
    while (k + 1 < q.n_mats && q.bounds[k + 1] <= lo) ++k;
    mat = k;
    const uint32_t cols = q.cols[k];
    const uint32_t local = div_magic((uint32_t)(lo - q.bounds[k]), q.magic[k], q.shift[k]);
    const uint64_t r0s = q.bounds[k] + (uint64_t)local * cols, r1s = r0s + cols;
    const uint64_t end = min_u64(q.bounds[q.n_mats], A + n);
    d.lo_rel = (uint32_t)(lo - A);
    d.hi_rel = (uint32_t)(end - A);
    d.r1_rel = (uint32_t)min_u64(r1s - A, 0xFFFFFFFFull);
    d.off0 = (int32_t)((int64_t)A - (int64_t)r0s);
    d.off1 = (int32_t)((int64_t)A - (int64_t)r1s);
    d.x0 = q.x[k];
    d.x1 = (r1s == q.bounds[k + 1] && k + 1 < q.n_mats) ? q.x[k + 1] : q.x[k];
    d.row0 = (uint32_t)q.row_base[k] + local;
    d.starts_row0 = r0s == lo;
    d.starts_row1 = r1s < end;
    d.simple = d.lo_rel == 0 && d.hi_rel == n && d.r1_rel >= n;
    return d;
}

// The x entries that steps k0 .. k0 + kN - 1 of this lane multiply: block
// lane + 64k of a group of n elements whose rows dr describes.  In a group
// that lies in one row (most groups) block b takes x0[off0 + 8b ..] from one
// uniform base, blocks past the group's last block repeating it; otherwise
// each block takes its own row's x, and blocks outside the multiplied range
// load x0[0..7].  Those are never used.
template <uint32_t kN>
__device__ __forceinline__ void load_dot_x(const DotRows& dr, uint32_t n, uint32_t lane, uint32_t k0,
                                           uint4 (&xv)[kN]) {
    const uint32_t nblk = n / kMergeElems;
    if (dr.simple) {   // every element multiplied: n is a positive multiple of 8
        const uint8_t* const base = reinterpret_cast<const uint8_t*>(dr.x0 + dr.off0);
        const uint32_t last = __builtin_amdgcn_readfirstlane(nblk - 1);
#pragma unroll
        for (uint32_t i = 0; i < kN; ++i)
            xv[i] = *reinterpret_cast<const uint4*>(base + 16u * min(lane + (k0 + i) * kWaveLanes, last));
    } else {
        // a real branch: an empty volatile asm keeps the compiler from
        // computing these addresses for every group and selecting
        asm volatile("");
#pragma unroll
        for (uint32_t i = 0; i < kN; ++i) {
            const uint32_t blk = lane + (k0 + i) * kWaveLanes;
            const uint32_t rel = kMergeElems * blk;
            const bool ok = blk < nblk && rel >= dr.lo_rel && rel < dr.hi_rel;
            const bool second = rel >= dr.r1_rel;
            const uint16_t* const xp = second ? dr.x1 : dr.x0;
            const int32_t col = ok ? (int32_t)rel + (second ? dr.off1 : dr.off0) : 0;
            xv[i] = *reinterpret_cast<const uint4*>(xp + col);
        }
    }
}

// Adds the block sums d[i] of steps k0 + i (in step order) to this lane's
// partials of the group's first row (acc0) and the next (acc1).  Blocks past
// the group's whole blocks (`full`) or outside the multiplied range are
// dropped by a select, whatever was computed for them.
template <uint32_t kN>
__device__ __forceinline__ void add_dot_steps(const DotRows& dr, uint32_t full, uint32_t lane, uint32_t k0,
                                              const float (&d)[kN], float& acc0, float& acc1) {
    if (dr.simple && full == kWaveLanes * kMergeSteps) {   // most groups: every block, one row
#pragma unroll
        for (uint32_t i = 0; i < kN; ++i) acc0 += d[i];
    } else if (dr.simple) {
#pragma unroll
        for (uint32_t i = 0; i < kN; ++i) acc0 += lane + (k0 + i) * kWaveLanes < full ? d[i] : 0.0f;
    } else {
        asm volatile("");   // a real branch (see load_dot_x)
#pragma unroll
        for (uint32_t i = 0; i < kN; ++i) {
            const uint32_t blk = lane + (k0 + i) * kWaveLanes;
            const uint32_t rel = kMergeElems * blk;
            const bool ok = blk < full && rel >= dr.lo_rel && rel < dr.hi_rel;
            const bool second = rel >= dr.r1_rel;
            acc0 += ok && !second ? d[i] : 0.0f;
            acc1 += ok && second ? d[i] : 0.0f;
        }
    }
}

// Block sums of steps k0 + i: sign+mantissa bytes sm[i] joined with the
// exponent bytes e[i], times the x entries xv[i], four dot2 steps each.
template <uint32_t kN>
__device__ __forceinline__ void dot_steps(const uint2* sm, const uint2 (&e)[kN], const uint4 (&xv)[kN],
                                          float (&d)[kN]) {
#pragma unroll
    for (uint32_t i = 0; i < kN; ++i) {
        uint32_t o0, o1, o2, o3;
        join4(sm[i].x, e[i].x, o0, o1);
        join4(sm[i].y, e[i].y, o2, o3);
        d[i] = dot8_bf16(o0, o1, o2, o3, xv[i]);
    }
}

// The wave's totals of the two row partials; lane 63 writes them for group g
// (g = group - u_begin) and, for a row that starts in the group, that row's
// first group: the group holding the row's first element, or the next one
// when that group started in the row before.
__device__ __forceinline__ void finish_dot(const DotParams& q, const DotRows& dr, uint32_t lane, uint64_t g,
                                           float acc0, float acc1) {
    acc0 = wave_total(acc0);
    if (!dr.simple) acc1 = wave_total(acc1);
    if (lane == kWaveLanes - 1) {
        *reinterpret_cast<float2*>(q.part + 2 * g) = make_float2(acc0, dr.simple ? 0.0f : acc1);
        if (dr.starts_row0)
            q.row_group[dr.row0] = (uint32_t)g;
        else if (dr.starts_row1)
            q.row_group[dr.row0 + 1] = (uint32_t)(g + 1);
    }
}

// One group's partial dot products, in place of its merge: step k joins the
// sign+mantissa bytes smv[k] with the exponent bytes exp_at(k) of block
// lane + 64k (a block of 8 lies in one row: row starts are multiples of 8),
// sums the block with four dot2 steps and adds it to the partial of its row.
// All eight exponent reads are issued first (exp_at must stay inside the
// wave's own LDS for every k).
template <typename ExpAt>
__device__ __forceinline__ void dot_group(const DotParams& q, const DotRows& dr, uint32_t full, uint32_t lane,
                                          const uint2 (&smv)[kMergeSteps], const uint4 (&xv)[kMergeSteps],
                                          uint64_t g, ExpAt exp_at) {
    uint2 e2[kMergeSteps];
#pragma unroll
    for (uint32_t k = 0; k < kMergeSteps; ++k) e2[k] = exp_at(k);
    float d[kMergeSteps];
    dot_steps(smv, e2, xv, d);
    float acc0 = 0.0f, acc1 = 0.0f;
    add_dot_steps(dr, full, lane, 0, d, acc0, acc1);
    finish_dot(q, dr, lane, g, acc0, acc1);
}

}  // namespace
}  // namespace wc
