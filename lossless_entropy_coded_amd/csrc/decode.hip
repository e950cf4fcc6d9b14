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
//            per table lookup (codeword-start table);
//   scan     wave64 inclusive scan with DPP row shifts and row broadcasts,
//            then across the 4 waves through LDS -> each lane's first output;
//   phase 2  each lane decodes its codewords again, one per lookup, and writes
//            the exponent bytes into an LDS staging buffer at their final
//            group-relative position;
//   merge    the workgroup streams the group's sign+mantissa bytes with 16-byte
//            loads, joins them with the staged exponents in integer registers
//            and writes bf16 with 16-byte stores.
// Workgroups are persistent: each stages the tables once and loops over groups.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace wc {
namespace {

constexpr uint32_t kCodeLimit = 24;

struct LongTables {
    const uint32_t* count;
    const uint32_t* first;
    const uint32_t* base;
    const uint8_t* sorted;
};

// Canonical decode of a codeword longer than the first-level index.  `win`
// holds at least 24 valid stream bits, MSB-aligned.  Returns the length; the
// symbol goes to *sym.  A window that matches no code (only in a corrupted
// stream) decodes as a 24-bit codeword of the first sorted symbol.
__device__ __forceinline__ uint32_t decode_long(uint32_t win, uint32_t first_len, const LongTables& t,
                                                uint32_t* sym) {
    uint32_t L = first_len;
    uint32_t idx = 0;
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

// Two bf16 words from two sign+mantissa bytes and two exponent bytes.
// `sel` picks (sm_i, e_i, sm_j, e_j) into the four bytes: each 16-bit half is
// then v = e << 8 | sm and the bf16 word is (sm & 0x80) << 8 | e << 7 | (sm & 0x7F).
__device__ __forceinline__ uint32_t join_pair(uint32_t sm4, uint32_t e4, uint32_t sel) {
    const uint32_t v = __builtin_amdgcn_perm(e4, sm4, sel);
    return ((v >> 1) & 0x7F807F80u) | ((v << 8) & 0x80008000u) | (v & 0x007F007Fu);
}

template <int K>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeParams p) {
    extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
    constexpr uint32_t kEntries = 1u << K;
    constexpr uint32_t kTableWords = (2u << K) + 160u;
    uint32_t* lut1 = smem;
    uint32_t* lutc = smem + kEntries;
    LongTables lt;
    lt.count = smem + 2 * kEntries;
    lt.first = lt.count + 32;
    lt.base = lt.first + 32;
    lt.sorted = reinterpret_cast<const uint8_t*>(lt.base + 32);
    uint32_t* wave_total = smem + kTableWords;              // 16 words
    uint8_t* ebuf = reinterpret_cast<uint8_t*>(smem + kTableWords + 16);

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;

    // stage the decode tables (built once per container) into LDS
    {
        const uint4* src = reinterpret_cast<const uint4*>(p.tables);
        uint4* dst = reinterpret_cast<uint4*>(smem);
        for (uint32_t i = tid; i < kTableWords / 4; i += kDecodeThreads) dst[i] = src[i];
    }
    __syncthreads();

    for (uint64_t g = blockIdx.x; g < p.n_groups; g += gridDim.x) {
        const uint64_t A = p.group_start[g];
        const uint64_t B = p.group_start[g + 1];
        const uint64_t c = g * kDecodeThreads + tid;

        // this lane's chunk: 96 stream bits MSB-first, start offset and end
        uint32_t w0 = 0, w1 = 0, w2 = 0, start = 0, end = 0;
        if (c < p.n_chunks) {
            const uint2 d01 = *reinterpret_cast<const uint2*>(p.stream + 8 * c);
            const uint32_t d2 = *reinterpret_cast<const uint32_t*>(p.stream + 8 * c + 8);
            w0 = __builtin_bswap32(d01.x);
            w1 = __builtin_bswap32(d01.y);
            w2 = __builtin_bswap32(d2);
            start = p.gap[c];
            const uint64_t left = p.stream_bits - 64 * c;
            end = left < 64 ? (uint32_t)left : 64u;
            // align the register on the first codeword (start < 24)
            const uint64_t h01 = ((uint64_t)w0 << 32 | w1) << start;
            const uint64_t h12 = ((uint64_t)w1 << 32 | w2) << start;
            w0 = (uint32_t)(h01 >> 32);
            w1 = (uint32_t)(h12 >> 32);
            w2 = w2 << start;
        }

        // phase 1: count codewords starting in [start, end)
        uint32_t count = 0;
        {
            uint32_t a0 = w0, a1 = w1, a2 = w2, q = start;
            while (q < end) {
                const uint32_t e = lutc[a0 >> (32 - K)];
                uint32_t adv = (e >> 8) & 31u;
                uint32_t sh;
                if (adv == 0) {
                    uint32_t sym;
                    adv = decode_long(a0, K + 1, lt, &sym);
                    count += 1;
                    sh = 32u - adv;
                } else {
                    const uint32_t rem = end - q;
                    uint32_t m = e >> 16;
                    if (rem < 16) m &= (1u << rem) - 1u;
                    count += __popc(m);
                    sh = e;
                }
                consume(a0, a1, a2, sh);
                q += adv;
            }
        }

        // block-wide exclusive scan of the counts
        const uint32_t incl = wave_inclusive_scan(count);
        if (lane == 63) wave_total[wave] = incl;
        __syncthreads();
        uint32_t before = 0;
        for (uint32_t w = 0; w < wave; ++w) before += wave_total[w];
        const uint32_t pos = before + incl - count;

        // phase 2: decode again and stage exponent bytes at their final place;
        // never write past the group's element range, even for a corrupted stream
        const uint32_t n_group = (uint32_t)(B - A);
        const uint32_t room = pos < n_group ? n_group - pos : 0u;
        const uint32_t todo = count < room ? count : room;
        uint8_t* dst = ebuf + (uint32_t)(A & 15u) + pos;
        for (uint32_t j = 0; j < todo; ++j) {
            const uint32_t e = lut1[w0 >> (32 - K)];
            uint32_t sym, sh;
            if ((int32_t)e < 0) {
                const uint32_t L = decode_long(w0, K + 1, lt, &sym);
                sh = 32u - L;
            } else {
                sym = e >> 16;
                sh = e;
            }
            dst[j] = (uint8_t)sym;
            consume(w0, w1, w2, sh);
        }
        __syncthreads();

        // merge: 16 elements per lane per step, 16-byte loads and stores
        const uint64_t A0 = A & ~15ull;
        const uint32_t nblk = (uint32_t)((B - A0 + 15) >> 4);
        for (uint32_t b = tid; b < nblk; b += kDecodeThreads) {
            const uint64_t base = A0 + 16ull * b;
            const uint4 s4 = *reinterpret_cast<const uint4*>(p.sm + base);
            const uint4 e4 = *reinterpret_cast<const uint4*>(ebuf + 16 * b);
            uint32_t o[8];
            o[0] = join_pair(s4.x, e4.x, 0x05010400u);
            o[1] = join_pair(s4.x, e4.x, 0x07030602u);
            o[2] = join_pair(s4.y, e4.y, 0x05010400u);
            o[3] = join_pair(s4.y, e4.y, 0x07030602u);
            o[4] = join_pair(s4.z, e4.z, 0x05010400u);
            o[5] = join_pair(s4.z, e4.z, 0x07030602u);
            o[6] = join_pair(s4.w, e4.w, 0x05010400u);
            o[7] = join_pair(s4.w, e4.w, 0x07030602u);
            if (base >= A && base + 16 <= B) {
                uint4* dst4 = reinterpret_cast<uint4*>(p.out + base);
                dst4[0] = make_uint4(o[0], o[1], o[2], o[3]);
                dst4[1] = make_uint4(o[4], o[5], o[6], o[7]);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint64_t idx = base + i;
                    if (idx >= A && idx < B) p.out[idx] = (uint16_t)(o[i >> 1] >> (16 * (i & 1)));
                }
            }
        }
        __syncthreads();
    }
}

// Decode tables from the 256 code lengths (one workgroup, at plan time).
template <int K>
__global__ __launch_bounds__(1024) void build_tables_kernel(CodeLens lens, uint32_t* tables) {
    constexpr uint32_t kEntries = 1u << K;
    __shared__ uint32_t count[32], first[32], base[32];
    __shared__ uint8_t sorted[256];
    __shared__ uint32_t lut1[kEntries];
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
    // single-codeword table
    for (uint32_t w = tid; w < kEntries; w += blockDim.x) {
        uint32_t entry = 0x80000000u;
        for (uint32_t L = 1; L <= (uint32_t)K; ++L) {
            const uint32_t code = w >> (K - L);
            const uint32_t off = code - first[L];
            if (off < count[L]) {
                const uint32_t sym = sorted[(base[L] + off) & 255u];
                entry = ((32u - L) & 31u) | (L << 8) | (sym << 16);
                break;
            }
        }
        lut1[w] = entry;
        tables[w] = entry;
    }
    __syncthreads();
    // codeword-start table: greedily decode whole codewords inside the window
    for (uint32_t w = tid; w < kEntries; w += blockDim.x) {
        uint32_t at = 0, mask = 0;
        while (at < (uint32_t)K) {
            const uint32_t sub = (w << at) & (kEntries - 1u);   // remaining bits, MSB-aligned, zero fill
            const uint32_t e = lut1[sub];
            if ((int32_t)e < 0) break;
            const uint32_t L = (e >> 8) & 31u;
            if (at + L > (uint32_t)K) break;
            mask |= 1u << at;
            at += L;
        }
        tables[kEntries + w] = at ? (((32u - at) & 31u) | (at << 8) | (mask << 16)) : 0u;
    }
    uint32_t* tail = tables + 2 * kEntries;
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

template <int K>
hipError_t launch_decode_k(const DecodeParams& p, uint32_t grid, uint32_t lds, hipStream_t stream) {
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<K>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(decode_kernel<K>, dim3(grid), dim3(kDecodeThreads), lds, stream, p);
    return hipGetLastError();
}

template <int K>
int blocks_per_cu_k(uint32_t lds) {
    int n = 0;
    if (lds > 64 * 1024) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<K>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return 0;
    }
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<K>, kDecodeThreads, lds) != hipSuccess)
        return 0;
    return n;
}

}  // namespace

uint32_t decode_lds_bytes(uint32_t lut_bits, uint32_t ebuf_bytes) {
    return (table_words(lut_bits) + 16u) * 4u + ebuf_bytes;
}

int decode_blocks_per_cu(uint32_t lut_bits, uint32_t lds_bytes) {
    switch (lut_bits) {
        case 10: return blocks_per_cu_k<10>(lds_bytes);
        case 11: return blocks_per_cu_k<11>(lds_bytes);
        case 12: return blocks_per_cu_k<12>(lds_bytes);
        default: return 0;
    }
}

hipError_t launch_build_tables(const CodeLens& lens, uint32_t lut_bits, uint32_t* d_tables, hipStream_t stream) {
    switch (lut_bits) {
        case 10: hipLaunchKernelGGL(build_tables_kernel<10>, dim3(1), dim3(1024), 0, stream, lens, d_tables); break;
        case 11: hipLaunchKernelGGL(build_tables_kernel<11>, dim3(1), dim3(1024), 0, stream, lens, d_tables); break;
        case 12: hipLaunchKernelGGL(build_tables_kernel<12>, dim3(1), dim3(1024), 0, stream, lens, d_tables); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, uint32_t lut_bits, uint32_t grid, uint32_t lds_bytes,
                         hipStream_t stream) {
    switch (lut_bits) {
        case 10: return launch_decode_k<10>(p, grid, lds_bytes, stream);
        case 11: return launch_decode_k<11>(p, grid, lds_bytes, stream);
        case 12: return launch_decode_k<12>(p, grid, lds_bytes, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wc
