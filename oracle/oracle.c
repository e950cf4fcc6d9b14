/*
 * oracle.c -- plain serial CPU oracle for the lossless entropy-coded bf16
 * weight container.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke entry point and the
 * benchmark's CPU-baseline leg, never by the product library.  It shares no
 * code, header or table with the HIP path.
 *
 * Sources followed (cited by page title and part of the page):
 *  [DF11]  "70% Size, 100% Accuracy: Lossless LLM Compression for Efficient
 *          GPU Inference via Dynamic-Length Float" (DFloat11), abstract:
 *          the low entropy of the bf16 representation is removed by entropy
 *          coding that gives shorter codes to more frequent values; outputs
 *          are bit-for-bit identical; decoding uses lightweight auxiliary
 *          variables (per-thread bit offsets, per-block output positions).
 *  [L2-7B] "From a Lossless (~1.5:1) Compression Algorithm for Llama2 7B
 *          Weights to Variable Precision, Variable Range, Compressed Numeric
 *          Data Types for CNNs and LLMs", abstract: lossless ~1.5:1 coding
 *          of bf16 weights.
 *  [LW]    LazyWeights review page, analogy and verified facts: Huffman
 *          coding, shorter labels for the common values, decoded bit-exact.
 *  [HUFF]  "Huff-LLM: End-to-End Lossless Compression for Efficient LLM
 *          Inference", abstract: weights stay Huffman-compressed end to end.
 *  Textbook material the pages rely on but do not spell out:
 *    Huffman's construction (D. A. Huffman, 1952); package-merge for an
 *    optimal length-limited code (Larmore & Hirschberg, 1990); canonical
 *    code assignment as in RFC 1951 section 3.2.2.
 *
 * Readings where the pages are silent:
 *  - split: e = bits 14..7 of the bf16 word, sm = bit 15 then bits 6..0;
 *  - codes are canonical, at most max_code_len (<= 24) bits, written
 *    MSB-first into bytes in ascending address order;
 *  - one present symbol gets the 1-bit code "0";
 *  - the stream is cut into 64-bit chunks; gap[c] is the offset of the first
 *    codeword that starts at or after bit 64c (stream end if none); gaps are
 *    stored one byte per chunk, or (header byte 10 = 5) packed in 5 bits,
 *    gap c in bits 5c .. 5c + 4 of the section read as a little-endian bit
 *    string (byte k holds bits 8k .. 8k + 7, lowest first): every gap is
 *    below the longest code, at most 23;
 *  - the per-block output positions of the pages are a group table: the
 *    elements are cut into blocks of A (the last block may be shorter); a
 *    group is a run of whole blocks that is as long as possible while the
 *    codewords of its elements touch at most G chunks and it holds at most
 *    M elements (a group takes at least one block; M is a multiple of A);
 *    each entry holds the group's first element and the
 *    stream bit where that element's codeword starts, and a final entry
 *    holds {n, stream bits}.
 *  - interleaved-lane layout (container version 3): the LazyWeights page,
 *    analogy section, stores the Huffman codes in interleaved lanes; the same
 *    code and planes; the elements are cut into segments (runs of whole
 *    A-element blocks, at most M elements and at most B stream bits); inside
 *    a segment, 8-element lane blocks are dealt to 64 lanes in turn (lane j
 *    takes lane blocks j, j + 64, j + 128, ...), each lane's codewords form
 *    one bit string (its lane blocks in order, elements in order), and the
 *    segment's stream is lane 0's string, then lane 1's, ... up to lane 63's;
 *    per segment the table holds its first element and first stream bit, and
 *    64 u16 offsets give where each lane's string starts inside it;
 *  - symbol planes of 8-bit codes (version 3, element kind u8): for already
 *    quantized weights (the LazyWeights page, analogy: Huffman codes for the
 *    integer codes of a quantized model), every byte is one symbol of the
 *    same canonical code, in the same lane layout, with no raw plane; the
 *    decode gives back the bytes;
 *  - rANS in the lane layout (version 3, coder 1): the Llama2-7B page names
 *    ANS as the hardware coder; the LazyWeights page compares a Huffman and
 *    an rANS decoder.  Here each lane is one rANS stream: symbol frequencies
 *    quantized to sum to 2^12 replace the code lengths, a segment is cut by
 *    an upper bound of its encoded size (each symbol grows the state by at
 *    most 12 - log2 f + log2(1 + 2^-4) bits, so ceil(8 (12 - log2 f)) + 1
 *    eighths of a bit bound it; each lane adds 32 bits for its final state).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Container v2 layout, as restated for the oracle (little-endian fields).  */
/* ------------------------------------------------------------------------ */
#define HDR_BYTES       256u
#define ALIGN           256u
#define MAX_LEN_LIMIT   24u
#define CHUNK_BITS      64u

#define F_MAGIC          0   /* "WCBF"                                      */
#define F_VERSION        4   /* u16, 2                                      */
#define F_FLAGS          6   /* u16, 0                                      */
#define F_MAXLEN         8   /* u8                                          */
#define F_CHUNKBITS      9   /* u8, 64                                      */
#define F_RES0          10   /* u16, 0 (low byte: gap width, see below)     */
#define F_GAPBITS       10   /* u8 (version 2): 0 one byte per gap, 5 packed */
#define F_G             12   /* u32 chunks per group                        */
#define F_NTENS         16   /* u32                                         */
#define F_ALIGN         20   /* u32 elements per block A                    */
#define F_N             24   /* u64 elements                                */
#define F_SBITS         32   /* u64 stream bits                             */
#define F_NCHUNKS       40   /* u64                                         */
#define F_NGROUPS       48   /* u64                                         */
#define F_OFF_LEN       56   /* u64: u8 code_len[256]                       */
#define F_OFF_TENS      64   /* u64: {u64 offset, u64 numel}[n_tensors]     */
#define F_OFF_GS        72   /* u64: {u64 elem, u64 bit}[n_groups + 1]      */
#define F_OFF_GAP       80   /* u64: u8 gap[n_chunks]                       */
#define F_OFF_STREAM    88   /* u64: stream bytes                           */
#define F_STREAM_BYTES  96   /* u64: 8 * n_chunks + 16 (zero padded)        */
#define F_OFF_SM       104   /* u64: u8 sm[n]                               */
#define F_TOTAL        112   /* u64: whole container size                   */
#define F_MAXG         120   /* u32 elements per group at most M            */
#define F_KIND         124   /* u8 element kind (version 3): 0 bf16, 1 u8   */
#define F_CODER        125   /* u8 coder (version 3): 0 Huffman, 1 rANS     */
#define F_TAIL         126   /* zero from here to the end of the header     */
#define CODER_HUFFMAN    0
#define CODER_RANS       1
/* rANS [L2-7B abstract: ANS]: 12-bit frequencies, a 32-bit state kept in
 * [2^16, 2^32), 16-bit renormalisation words; a lane's string is its final
 * state (two words, high first) and then the words its decoder reads, each
 * big-endian; a lane with no symbols has an empty string. */
#define RANS_P          12u
#define RANS_L     65536ull
#define RANS_FLUSH      32u
#define KIND_BF16        0   /* exponent coded, sign+mantissa plane raw     */
#define KIND_U8          1   /* the whole byte coded, no raw plane          */

static uint64_t rd(const uint8_t* p, int nbytes) {
    uint64_t v = 0;
    for (int i = nbytes - 1; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}
static void wr(uint8_t* p, uint64_t v, int nbytes) {
    for (int i = 0; i < nbytes; ++i) { p[i] = (uint8_t)(v & 0xFF); v >>= 8; }
}
static uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
static uint64_t ceil_div(uint64_t x, uint64_t a) { return (x + a - 1) / a; }

/* ------------------------------------------------------------------------ */
/* Group table [DF11 abstract (ii): per-block output positions].            */
/* block_bit[k] is the stream bit where block k's first codeword starts,    */
/* k < nb, and block_bit[nb] the stream length.  Writes n_groups + 1 pairs  */
/* into elem[] / bit[] (each of capacity nb + 1) and returns n_groups.       */
/* ------------------------------------------------------------------------ */
static uint64_t chunks_touched(uint64_t p, uint64_t q) {   /* chunks holding bits [p, q), q > p */
    return (q - 1) / CHUNK_BITS - p / CHUNK_BITS + 1;
}

static uint64_t orc_groups(const uint64_t* block_bit, uint64_t nb, uint64_t n, uint32_t A, uint32_t G,
                           uint32_t M, uint64_t* elem, uint64_t* bit) {
    uint64_t g = 0, k = 0;
    elem[0] = 0;
    bit[0] = 0;
    while (k < nb) {
        uint64_t first = k;
        ++k;   /* at least one block */
        while (k < nb && (k + 1 - first) * (uint64_t)A <= M &&
               chunks_touched(block_bit[first], block_bit[k + 1]) <= G)
            ++k;
        ++g;
        elem[g] = k * (uint64_t)A < n ? k * (uint64_t)A : n;
        bit[g] = block_bit[k];
    }
    return g;
}

/* ------------------------------------------------------------------------ */
/* Interleaved-lane layout [LW analogy: Huffman codes in interleaved lanes]. */
/* ------------------------------------------------------------------------ */
#define LANES           64u
#define LANE_BLOCK       8u
#define LANES_SLACK     64u   /* zero bytes after the padded stream          */
/* header fields of version 3 that differ from version 2 */
#define F_LANES          9   /* u8, 64 (version 2: chunk bits)              */
#define F_LANE_BLOCK    10   /* u16, 8 (version 2: reserved)                */
#define F_SEGBITS       12   /* u32 stream bits per segment at most B       */
#define F_OFF_LOFF      80   /* u64: u16 lane_off[64 * n_segs]              */

/* Segments: runs of whole A-blocks, as long as possible while they hold at
 * most M elements and their codewords at most B bits (at least one block).
 * block_bit[k] = stream bits before block k (the layout inside a segment
 * does not change how many bits precede it). */
static uint64_t orc_segments(const uint64_t* block_bit, uint64_t nb, uint64_t n, uint32_t A, uint32_t B,
                             uint32_t M, uint64_t* elem, uint64_t* bit) {
    uint64_t g = 0, k = 0;
    elem[0] = 0;
    bit[0] = 0;
    while (k < nb) {
        uint64_t first = k;
        ++k;
        while (k < nb && (k + 1 - first) * (uint64_t)A <= M && block_bit[k + 1] - block_bit[first] <= B)
            ++k;
        ++g;
        elem[g] = k * (uint64_t)A < n ? k * (uint64_t)A : n;
        bit[g] = block_bit[k];
    }
    return g;
}

/* Element index (inside a segment of m elements) of the t-th symbol of lane
 * j, or m if lane j has fewer symbols. */
static uint64_t lane_elem(uint64_t m, uint32_t j, uint64_t t) {
    uint64_t blk = j + (uint64_t)LANES * (t / LANE_BLOCK);
    uint64_t i = blk * LANE_BLOCK + t % LANE_BLOCK;
    return i < m ? i : m;
}

/* ------------------------------------------------------------------------ */
/* Planes [DF11 abstract; L2-7B abstract]                                   */
/* ------------------------------------------------------------------------ */
void orc_split_planes(const uint16_t* w, uint64_t n, uint8_t* exp_out, uint8_t* sm_out) {
    for (uint64_t i = 0; i < n; ++i) {
        uint16_t b = w[i];
        exp_out[i] = (uint8_t)((b >> 7) & 0xFF);
        sm_out[i] = (uint8_t)(((b >> 8) & 0x80) | (b & 0x7F));
    }
}

void orc_join_planes(const uint8_t* exp_in, const uint8_t* sm_in, uint64_t n, uint16_t* w_out) {
    for (uint64_t i = 0; i < n; ++i) {
        uint16_t e = exp_in[i], s = sm_in[i];
        w_out[i] = (uint16_t)(((s & 0x80) << 8) | (e << 7) | (s & 0x7F));
    }
}

/* ------------------------------------------------------------------------ */
/* Huffman's construction, unrestricted depth [LW analogy; DF11 abstract]   */
/* ------------------------------------------------------------------------ */
int orc_heap_huffman(const uint64_t counts[256], uint8_t lens[256]) {
    /* nodes 0..255 are leaves, 256.. are merged trees */
    uint64_t weight[512];
    int minsym[512], parent[512], alive[512];
    int n_nodes = 256, n_alive = 0;
    for (int s = 0; s < 256; ++s) {
        lens[s] = 0;
        weight[s] = counts[s];
        minsym[s] = s;
        parent[s] = -1;
        alive[s] = counts[s] > 0;
        n_alive += alive[s];
    }
    if (n_alive == 0) return ORC_OK;
    if (n_alive == 1) {
        for (int s = 0; s < 256; ++s) if (alive[s]) lens[s] = 1;
        return ORC_OK;
    }
    while (n_alive > 1) {
        /* pick the two lightest live trees; ties go to the smaller symbol */
        int a = -1, b = -1;
        for (int i = 0; i < n_nodes; ++i) {
            if (!alive[i]) continue;
            if (a < 0 || weight[i] < weight[a] || (weight[i] == weight[a] && minsym[i] < minsym[a])) {
                b = a;
                a = i;
            } else if (b < 0 || weight[i] < weight[b] || (weight[i] == weight[b] && minsym[i] < minsym[b])) {
                b = i;
            }
        }
        int p = n_nodes++;
        weight[p] = weight[a] + weight[b];
        minsym[p] = minsym[a] < minsym[b] ? minsym[a] : minsym[b];
        parent[p] = -1;
        alive[p] = 1;
        alive[a] = alive[b] = 0;
        parent[a] = parent[b] = p;
        n_alive -= 1;
    }
    for (int s = 0; s < 256; ++s) {
        if (counts[s] == 0) continue;
        int d = 0;
        for (int v = s; parent[v] >= 0; v = parent[v]) ++d;
        lens[s] = (uint8_t)d;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Package-merge (Larmore & Hirschberg): optimal code with lengths <= L.    */
/* Each item carries how many times every present symbol occurs in it; the  */
/* final length of a symbol is its number of occurrences among the first    */
/* 2m-2 items of the last list.                                             */
/* ------------------------------------------------------------------------ */
typedef struct {
    uint64_t w;
    uint8_t cnt[256];   /* indexed by rank among present symbols */
} pm_item;

int orc_package_merge(const uint64_t counts[256], uint32_t max_len, uint8_t lens[256]) {
    int sym[256], m = 0;
    for (int s = 0; s < 256; ++s) { lens[s] = 0; if (counts[s]) sym[m++] = s; }
    if (max_len < 1 || max_len > 32) return ORC_E_ARG;
    if (m == 0) return ORC_OK;
    if (m == 1) { lens[sym[0]] = 1; return ORC_OK; }
    if (max_len < 31 && ((uint64_t)1 << max_len) < (uint64_t)m) return ORC_E_ARG;

    /* present symbols sorted by (count, symbol): insertion sort, m <= 256 */
    for (int i = 1; i < m; ++i) {
        int s = sym[i], j = i - 1;
        while (j >= 0 && (counts[sym[j]] > counts[s] || (counts[sym[j]] == counts[s] && sym[j] > s))) {
            sym[j + 1] = sym[j];
            --j;
        }
        sym[j + 1] = s;
    }
    pm_item* leaves = (pm_item*)calloc((size_t)m, sizeof(pm_item));
    pm_item* list = (pm_item*)calloc((size_t)2 * m, sizeof(pm_item));
    pm_item* next = (pm_item*)calloc((size_t)2 * m, sizeof(pm_item));
    pm_item* pk = (pm_item*)calloc((size_t)m, sizeof(pm_item));
    if (!leaves || !list || !next || !pk) {
        free(leaves); free(list); free(next); free(pk);
        return ORC_E_NOMEM;
    }
    for (int k = 0; k < m; ++k) { leaves[k].w = counts[sym[k]]; leaves[k].cnt[k] = 1; }
    memcpy(list, leaves, (size_t)m * sizeof(pm_item));
    int size = m;
    /* lists for depths L-1 down to 1: package pairs, then merge with leaves */
    for (uint32_t level = 1; level < max_len; ++level) {
        int np = size / 2;
        for (int j = 0; j < np; ++j) {
            pk[j].w = list[2 * j].w + list[2 * j + 1].w;
            for (int k = 0; k < m; ++k) pk[j].cnt[k] = (uint8_t)(list[2 * j].cnt[k] + list[2 * j + 1].cnt[k]);
        }
        int a = 0, b = 0, o = 0;
        while (a < m || b < np) {
            if (b >= np || (a < m && leaves[a].w <= pk[b].w)) next[o++] = leaves[a++];
            else next[o++] = pk[b++];
        }
        pm_item* t = list; list = next; next = t;
        size = o;
    }
    int take = 2 * m - 2;
    for (int j = 0; j < take; ++j)
        for (int k = 0; k < m; ++k) lens[sym[k]] = (uint8_t)(lens[sym[k]] + list[j].cnt[k]);
    free(leaves); free(list); free(next); free(pk);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Canonical codes (RFC 1951 section 3.2.2 convention)                      */
/* ------------------------------------------------------------------------ */
int orc_canonical_codes(const uint8_t lens[256], uint32_t codes[256]) {
    int order[256], m = 0;
    for (int s = 0; s < 256; ++s) { codes[s] = 0; if (lens[s]) order[m++] = s; }
    /* sort by (length, symbol) */
    for (int i = 1; i < m; ++i) {
        int s = order[i], j = i - 1;
        while (j >= 0 && (lens[order[j]] > lens[s] || (lens[order[j]] == lens[s] && order[j] > s))) {
            order[j + 1] = order[j];
            --j;
        }
        order[j + 1] = s;
    }
    uint64_t code = 0;
    int prev_len = 0;
    for (int i = 0; i < m; ++i) {
        int s = order[i], L = lens[s];
        if (L > 32) return ORC_E_LENGTHS;
        if (i > 0) code = (code + 1) << (L - prev_len);
        else code = 0;
        if (code >> L) return ORC_E_KRAFT;   /* ran out of codes: over-subscribed */
        codes[s] = (uint32_t)code;
        prev_len = L;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Writer (serial).  Container layout as in the header comment.             */
/* ------------------------------------------------------------------------ */
/* Bytes of the gap section: one per chunk, or 5 bits per chunk. */
static uint64_t gap_section_bytes(uint64_t n_chunks, uint32_t gap_bits) {
    return gap_bits == 5 ? ceil_div(5 * n_chunks, 8) : n_chunks;
}

/* Gap of chunk c from a section of the given width. */
static uint32_t gap_at(const uint8_t* g, uint64_t c, uint32_t gap_bits) {
    if (gap_bits != 5) return g[c];
    uint32_t v = 0;
    for (uint32_t j = 0; j < 5; ++j) {
        uint64_t bit = 5 * c + j;
        v |= (uint32_t)((g[bit >> 3] >> (bit & 7)) & 1u) << j;
    }
    return v;
}

int orc_encode(const uint16_t* w, uint64_t n, const uint64_t* numels, uint32_t n_tensors,
               uint32_t max_code_len, uint32_t G, uint32_t A, uint32_t M, uint8_t** blob, uint64_t* blob_bytes) {
    return orc_encode_gaps(w, n, numels, n_tensors, max_code_len, G, A, M, 8, blob, blob_bytes);
}

int orc_encode_gaps(const uint16_t* w, uint64_t n, const uint64_t* numels, uint32_t n_tensors,
                    uint32_t max_code_len, uint32_t G, uint32_t A, uint32_t M, uint32_t gap_bits, uint8_t** blob,
                    uint64_t* blob_bytes) {
    if (!blob || !blob_bytes || (n && !w)) return ORC_E_ARG;
    if (max_code_len < 1 || max_code_len > MAX_LEN_LIMIT || G < 1 || A < 1 || M < A || M % A) return ORC_E_ARG;
    if (gap_bits != 8 && gap_bits != 5) return ORC_E_ARG;
    uint64_t one_numel = n;
    if (!numels) { numels = &one_numel; n_tensors = 1; }
    uint64_t sum = 0;
    for (uint32_t t = 0; t < n_tensors; ++t) sum += numels[t];
    if (sum != n) return ORC_E_ARG;

    uint8_t* e = (uint8_t*)malloc(n ? n : 1);
    uint8_t* sm = (uint8_t*)malloc(n ? n : 1);
    if (!e || !sm) { free(e); free(sm); return ORC_E_NOMEM; }
    orc_split_planes(w, n, e, sm);

    uint64_t hist[256] = {0};
    for (uint64_t i = 0; i < n; ++i) hist[e[i]]++;
    uint8_t lens[256];
    uint32_t codes[256];
    int st = orc_package_merge(hist, max_code_len, lens);
    if (st == ORC_OK) st = orc_canonical_codes(lens, codes);
    if (st != ORC_OK) { free(e); free(sm); return st; }

    uint64_t bits = 0;
    for (int s = 0; s < 256; ++s) bits += hist[s] * lens[s];
    uint64_t n_chunks = ceil_div(bits, CHUNK_BITS);
    uint64_t stream_bytes = 8 * n_chunks + 16;

    /* where every block of A elements starts in the stream, then the groups */
    uint64_t nb = ceil_div(n, A);
    uint64_t* block_bit = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
    uint64_t* g_elem = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
    uint64_t* g_bit = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
    if (!block_bit || !g_elem || !g_bit) {
        free(block_bit); free(g_elem); free(g_bit); free(e); free(sm);
        return ORC_E_NOMEM;
    }
    {
        uint64_t at = 0;
        for (uint64_t i = 0; i < n; ++i) {
            if (i % A == 0) block_bit[i / A] = at;
            at += lens[e[i]];
        }
        block_bit[nb] = at;
    }
    uint64_t n_groups = orc_groups(block_bit, nb, n, A, G, M, g_elem, g_bit);

    uint64_t off_len = HDR_BYTES;
    uint64_t off_tens = round_up(off_len + 256, ALIGN);
    uint64_t off_gs = round_up(off_tens + 16ull * n_tensors, ALIGN);
    uint64_t off_gap = round_up(off_gs + 16 * (n_groups + 1), ALIGN);
    uint64_t off_stream = round_up(off_gap + gap_section_bytes(n_chunks, gap_bits), ALIGN);
    uint64_t off_sm = round_up(off_stream + stream_bytes, ALIGN);
    uint64_t total = round_up(off_sm + n, ALIGN);

    uint8_t* b = (uint8_t*)calloc(total, 1);
    uint8_t* gap = (uint8_t*)calloc(n_chunks ? n_chunks : 1, 1);   /* gap values, one per chunk */
    if (!b || !gap) { free(b); free(gap); free(block_bit); free(g_elem); free(g_bit); free(e); free(sm); return ORC_E_NOMEM; }

    uint8_t* stream = b + off_stream;
    uint8_t* gs = b + off_gs;
    for (uint64_t g = 0; g <= n_groups; ++g) {
        wr(gs + 16 * g, g_elem[g], 8);
        wr(gs + 16 * g + 8, g_bit[g], 8);
    }
    free(block_bit); free(g_elem); free(g_bit);
    uint64_t pos = 0, next_chunk = 0;
    for (uint64_t i = 0; i < n; ++i) {
        /* auxiliary variables [DF11 abstract (ii)] for every chunk whose first
         * codeword start is this one */
        while (next_chunk < n_chunks && CHUNK_BITS * next_chunk <= pos) {
            gap[next_chunk] = (uint8_t)(pos - CHUNK_BITS * next_chunk);
            ++next_chunk;
        }
        int L = lens[e[i]];
        uint32_t c = codes[e[i]];
        for (int k = L - 1; k >= 0; --k) {
            if ((c >> k) & 1u) stream[pos >> 3] |= (uint8_t)(0x80u >> (pos & 7));
            ++pos;
        }
    }
    while (next_chunk < n_chunks) { gap[next_chunk] = (uint8_t)(bits - CHUNK_BITS * next_chunk); ++next_chunk; }
    /* the gap section: one byte per chunk, or 5 bits per chunk, lowest bit first */
    for (uint64_t c = 0; c < n_chunks; ++c) {
        if (gap_bits == 8) {
            b[off_gap + c] = gap[c];
        } else {
            for (uint32_t j = 0; j < 5; ++j) {
                uint64_t bit = 5 * c + j;
                if ((gap[c] >> j) & 1u) b[off_gap + (bit >> 3)] |= (uint8_t)(1u << (bit & 7));
            }
        }
    }
    free(gap);

    memcpy(b + off_len, lens, 256);
    uint64_t acc = 0;
    for (uint32_t t = 0; t < n_tensors; ++t) {
        wr(b + off_tens + 16ull * t, acc, 8);
        wr(b + off_tens + 16ull * t + 8, numels[t], 8);
        acc += numels[t];
    }
    if (n) memcpy(b + off_sm, sm, n);

    memcpy(b + F_MAGIC, "WCBF", 4);
    wr(b + F_VERSION, 2, 2);
    wr(b + F_FLAGS, 0, 2);
    wr(b + F_MAXLEN, max_code_len, 1);
    wr(b + F_CHUNKBITS, CHUNK_BITS, 1);
    wr(b + F_GAPBITS, gap_bits == 5 ? 5 : 0, 1);
    wr(b + F_G, G, 4);
    wr(b + F_NTENS, n_tensors, 4);
    wr(b + F_ALIGN, A, 4);
    wr(b + F_MAXG, M, 4);
    wr(b + F_N, n, 8);
    wr(b + F_SBITS, bits, 8);
    wr(b + F_NCHUNKS, n_chunks, 8);
    wr(b + F_NGROUPS, n_groups, 8);
    wr(b + F_OFF_LEN, off_len, 8);
    wr(b + F_OFF_TENS, off_tens, 8);
    wr(b + F_OFF_GS, off_gs, 8);
    wr(b + F_OFF_GAP, off_gap, 8);
    wr(b + F_OFF_STREAM, off_stream, 8);
    wr(b + F_STREAM_BYTES, stream_bytes, 8);
    wr(b + F_OFF_SM, off_sm, 8);
    wr(b + F_TOTAL, total, 8);

    free(e);
    free(sm);
    *blob = b;
    *blob_bytes = total;
    return ORC_OK;
}

/* Lanes writer over a symbol plane e (and, for bf16, the raw plane sm). */
static int encode_lanes_planes(uint8_t* e, uint8_t* sm, uint32_t kind, uint64_t n, const uint64_t* numels,
                               uint32_t n_tensors, uint32_t max_code_len, uint32_t A, uint32_t M, uint32_t B,
                               uint8_t** blob, uint64_t* blob_bytes) {
    uint64_t hist[256] = {0};
    for (uint64_t i = 0; i < n; ++i) hist[e[i]]++;
    uint8_t lens[256];
    uint32_t codes[256];
    int st = orc_package_merge(hist, max_code_len, lens);
    if (st == ORC_OK) st = orc_canonical_codes(lens, codes);
    if (st != ORC_OK) { free(e); free(sm); return st; }
    uint64_t bits = 0;
    for (int s = 0; s < 256; ++s) bits += hist[s] * lens[s];
    uint64_t stream_bytes = round_up(ceil_div(bits, 8), 8) + LANES_SLACK;

    uint64_t nb = ceil_div(n, A);
    uint64_t* block_bit = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
    uint64_t* s_elem = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
    uint64_t* s_bit = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
    if (!block_bit || !s_elem || !s_bit) {
        free(block_bit); free(s_elem); free(s_bit); free(e); free(sm);
        return ORC_E_NOMEM;
    }
    {
        uint64_t at = 0;
        for (uint64_t i = 0; i < n; ++i) {
            if (i % A == 0) block_bit[i / A] = at;
            at += lens[e[i]];
        }
        block_bit[nb] = at;
    }
    uint64_t n_segs = orc_segments(block_bit, nb, n, A, B, M, s_elem, s_bit);
    free(block_bit);

    uint64_t off_len = HDR_BYTES;
    uint64_t off_tens = round_up(off_len + 256, ALIGN);
    uint64_t off_segs = round_up(off_tens + 16ull * n_tensors, ALIGN);
    uint64_t off_loff = round_up(off_segs + 16 * (n_segs + 1), ALIGN);
    uint64_t off_stream = round_up(off_loff + 2ull * LANES * n_segs, ALIGN);
    uint64_t off_sm = round_up(off_stream + stream_bytes, ALIGN);
    uint64_t sm_bytes = kind == KIND_BF16 ? n : 0;
    uint64_t total = round_up(off_sm + sm_bytes, ALIGN);
    uint8_t* b = (uint8_t*)calloc(total, 1);
    if (!b) { free(s_elem); free(s_bit); free(e); free(sm); return ORC_E_NOMEM; }

    uint8_t* stream = b + off_stream;
    uint64_t pos = 0;
    for (uint64_t g = 0; g < n_segs; ++g) {
        wr(b + off_segs + 16 * g, s_elem[g], 8);
        wr(b + off_segs + 16 * g + 8, s_bit[g], 8);
        uint64_t e0 = s_elem[g], m = s_elem[g + 1] - e0;
        for (uint32_t j = 0; j < LANES; ++j) {
            wr(b + off_loff + 2 * (LANES * g + j), pos - s_bit[g], 2);
            for (uint64_t t = 0;; ++t) {
                uint64_t i = lane_elem(m, j, t);
                if (i >= m) break;
                int L = lens[e[e0 + i]];
                uint32_t c = codes[e[e0 + i]];
                for (int k = L - 1; k >= 0; --k) {
                    if ((c >> k) & 1u) stream[pos >> 3] |= (uint8_t)(0x80u >> (pos & 7));
                    ++pos;
                }
            }
        }
    }
    wr(b + off_segs + 16 * n_segs, n, 8);
    wr(b + off_segs + 16 * n_segs + 8, bits, 8);
    free(s_elem); free(s_bit);

    memcpy(b + off_len, lens, 256);
    uint64_t acc = 0;
    for (uint32_t t = 0; t < n_tensors; ++t) {
        wr(b + off_tens + 16ull * t, acc, 8);
        wr(b + off_tens + 16ull * t + 8, numels[t], 8);
        acc += numels[t];
    }
    if (sm_bytes) memcpy(b + off_sm, sm, sm_bytes);

    memcpy(b + F_MAGIC, "WCBF", 4);
    wr(b + F_VERSION, 3, 2);
    wr(b + F_KIND, kind, 1);
    wr(b + F_FLAGS, 0, 2);
    wr(b + F_MAXLEN, max_code_len, 1);
    wr(b + F_LANES, LANES, 1);
    wr(b + F_LANE_BLOCK, LANE_BLOCK, 2);
    wr(b + F_SEGBITS, B, 4);
    wr(b + F_NTENS, n_tensors, 4);
    wr(b + F_ALIGN, A, 4);
    wr(b + F_MAXG, M, 4);
    wr(b + F_N, n, 8);
    wr(b + F_SBITS, bits, 8);
    wr(b + F_NGROUPS, n_segs, 8);
    wr(b + F_OFF_LEN, off_len, 8);
    wr(b + F_OFF_TENS, off_tens, 8);
    wr(b + F_OFF_GS, off_segs, 8);
    wr(b + F_OFF_LOFF, off_loff, 8);
    wr(b + F_OFF_STREAM, off_stream, 8);
    wr(b + F_STREAM_BYTES, stream_bytes, 8);
    wr(b + F_OFF_SM, off_sm, 8);
    wr(b + F_TOTAL, total, 8);

    free(e);
    free(sm);
    *blob = b;
    *blob_bytes = total;
    return ORC_OK;
}

static int lanes_args(uint64_t n, const void* src, const uint64_t** numels, uint32_t* n_tensors,
                      uint64_t* one_numel, uint32_t max_code_len, uint32_t A, uint32_t M, uint32_t B,
                      uint8_t** blob, uint64_t* blob_bytes) {
    if (!blob || !blob_bytes || (n && !src)) return ORC_E_ARG;
    if (max_code_len < 1 || max_code_len > MAX_LEN_LIMIT || A < 1 || M < A || M % A) return ORC_E_ARG;
    if (M > LANES * LANE_BLOCK * 1024u || B > 65535u || (uint64_t)A * max_code_len > B) return ORC_E_ARG;
    *one_numel = n;
    if (!*numels) { *numels = one_numel; *n_tensors = 1; }
    uint64_t sum = 0;
    for (uint32_t t = 0; t < *n_tensors; ++t) sum += (*numels)[t];
    return sum == n ? ORC_OK : ORC_E_ARG;
}

int orc_encode_lanes(const uint16_t* w, uint64_t n, const uint64_t* numels, uint32_t n_tensors,
                     uint32_t max_code_len, uint32_t A, uint32_t M, uint32_t B, uint8_t** blob,
                     uint64_t* blob_bytes) {
    uint64_t one;
    int st = lanes_args(n, w, &numels, &n_tensors, &one, max_code_len, A, M, B, blob, blob_bytes);
    if (st != ORC_OK) return st;
    uint8_t* e = (uint8_t*)malloc(n ? n : 1);
    uint8_t* sm = (uint8_t*)malloc(n ? n : 1);
    if (!e || !sm) { free(e); free(sm); return ORC_E_NOMEM; }
    orc_split_planes(w, n, e, sm);
    return encode_lanes_planes(e, sm, KIND_BF16, n, numels, n_tensors, max_code_len, A, M, B, blob, blob_bytes);
}

int orc_encode_lanes_u8(const uint8_t* codes, uint64_t n, const uint64_t* numels, uint32_t n_tensors,
                        uint32_t max_code_len, uint32_t A, uint32_t M, uint32_t B, uint8_t** blob,
                        uint64_t* blob_bytes) {
    uint64_t one;
    int st = lanes_args(n, codes, &numels, &n_tensors, &one, max_code_len, A, M, B, blob, blob_bytes);
    if (st != ORC_OK) return st;
    uint8_t* e = (uint8_t*)malloc(n ? n : 1);
    if (!e) return ORC_E_NOMEM;
    if (n) memcpy(e, codes, n);
    return encode_lanes_planes(e, NULL, KIND_U8, n, numels, n_tensors, max_code_len, A, M, B, blob, blob_bytes);
}

/* ------------------------------------------------------------------------ */
/* rANS in the lane layout [L2-7B abstract: ANS; LW: Huffman vs rANS]       */
/* ------------------------------------------------------------------------ */
/* Frequencies summing to 2^P: f = max(1, floor(count * 2^P / n)) for present
 * symbols, then while the sum is too large take 1 from the largest f (> 1;
 * ties: smallest symbol), while too small give 1 to the most frequent symbol
 * (ties: smallest symbol). */
static void rans_freqs(const uint64_t hist[256], uint64_t n, uint32_t f[256]) {
    uint64_t sum = 0;
    int top = -1;
    for (int s = 0; s < 256; ++s) {
        f[s] = 0;
        if (!hist[s]) continue;
        uint64_t v = hist[s] * ((uint64_t)1 << RANS_P) / n;
        f[s] = (uint32_t)(v ? v : 1);
        sum += f[s];
        if (top < 0 || hist[s] > hist[top]) top = s;
    }
    if (top < 0) return;
    while (sum > ((uint64_t)1 << RANS_P)) {
        int b = -1;
        for (int s = 0; s < 256; ++s)
            if (f[s] > 1 && (b < 0 || f[s] > f[b])) b = s;
        f[b]--;
        sum--;
    }
    while (sum < ((uint64_t)1 << RANS_P)) { f[top]++; sum++; }
}

/* Upper bound, in eighths of a bit, of what one symbol of frequency f adds to
 * a lane's string: encoding x < 2^20 f gives x' < (x / f + 1) 2^P, so log2 x
 * grows by less than P - log2 f + log2(1 + f / x) <= P - log2 f + 0.0875
 * (x >= 2^16, f <= 2^12); the bound is ceil(8 (P - log2 f)) + 1, with the
 * ceiling q the least q such that f^8 2^q >= 2^(8P), exact in integers. */
static uint32_t rans_cost8(uint32_t f) {
    unsigned __int128 f8 = 1;
    for (int i = 0; i < 8; ++i) f8 *= f;
    uint32_t q = 0;
    while ((f8 << q) < ((unsigned __int128)1 << (8 * RANS_P))) ++q;
    return q + 1;
}

/* Segments for rANS: runs of whole A-blocks, at most M elements, whose bound
 * 64 * 32 bits + (sum of rans_cost8 over their elements) / 8 is at most B.
 * cost_before[k] = sum of rans_cost8 over the elements before block k. */
static uint64_t rans_segments(const uint64_t* cost_before, uint64_t nb, uint64_t n, uint32_t A, uint32_t B,
                              uint32_t M, uint64_t* elem) {
    uint64_t g = 0, k = 0;
    elem[0] = 0;
    while (k < nb) {
        uint64_t first = k;
        ++k;
        while (k < nb && (k + 1 - first) * (uint64_t)A <= M &&
               8ull * LANES * RANS_FLUSH + cost_before[k + 1] - cost_before[first] <= 8ull * B)
            ++k;
        ++g;
        elem[g] = k * (uint64_t)A < n ? k * (uint64_t)A : n;
    }
    return g;
}

/* Encode one lane's symbols sym[0..k) (k > 0) into big-endian 16-bit words at
 * out (capacity known sufficient); returns the number of words. */
static uint64_t rans_encode_lane(const uint8_t* sym, uint64_t k, const uint32_t f[256], const uint32_t cum[256],
                                 uint16_t* scratch, uint16_t* out) {
    uint64_t x = RANS_L, nw = 0;
    for (uint64_t t = k; t-- > 0;) {          /* last symbol first */
        uint32_t s = sym[t];
        uint64_t xmax = ((RANS_L >> RANS_P) << 16) * f[s];
        while (x >= xmax) { scratch[nw++] = (uint16_t)(x & 0xFFFF); x >>= 16; }
        x = (x / f[s] << RANS_P) + x % f[s] + cum[s];
    }
    out[0] = (uint16_t)(x >> 16);
    out[1] = (uint16_t)(x & 0xFFFF);
    for (uint64_t i = 0; i < nw; ++i) out[2 + i] = scratch[nw - 1 - i];   /* in the order the decoder reads */
    return nw + 2;
}

static int encode_rans_planes(uint8_t* e, uint8_t* sm, uint32_t kind, uint64_t n, const uint64_t* numels,
                              uint32_t n_tensors, uint32_t A, uint32_t M, uint32_t B, uint8_t** blob,
                              uint64_t* blob_bytes) {
    uint64_t hist[256] = {0};
    for (uint64_t i = 0; i < n; ++i) hist[e[i]]++;
    uint32_t f[256], cum[256], acc = 0;
    rans_freqs(hist, n, f);
    for (int s = 0; s < 256; ++s) { cum[s] = acc; acc += f[s]; }
    uint64_t nb = ceil_div(n, A);
    uint64_t* cost_before = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
    uint64_t* s_elem = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
    /* worst case: 2 words per symbol plus 2 per lane */
    uint16_t* scratch = (uint16_t*)malloc((size_t)(2 * M + 8) * sizeof(uint16_t));
    uint16_t* words = (uint16_t*)malloc((size_t)(2 * M + 2 * LANES + 8) * sizeof(uint16_t));
    uint8_t* lane_sym = (uint8_t*)malloc((size_t)M + 8);
    if (!cost_before || !s_elem || !scratch || !words || !lane_sym) {
        free(cost_before); free(s_elem); free(scratch); free(words); free(lane_sym); free(e); free(sm);
        return ORC_E_NOMEM;
    }
    {
        uint64_t at = 0;
        for (uint64_t i = 0; i < n; ++i) {
            if (i % A == 0) cost_before[i / A] = at;
            at += rans_cost8(f[e[i]]);
        }
        cost_before[nb] = at;
    }
    uint64_t n_segs = rans_segments(cost_before, nb, n, A, B, M, s_elem);
    free(cost_before);
    /* the stream is at most the bound of every segment */
    uint64_t cap_bits = (uint64_t)LANES * RANS_FLUSH * n_segs;
    for (uint64_t i = 0; i < n; ++i) cap_bits += rans_cost8(f[e[i]]);   /* eighths: a generous cap */
    uint8_t* tmp = (uint8_t*)calloc(ceil_div(cap_bits, 8) + 8, 1);
    uint16_t* loff = (uint16_t*)malloc((size_t)(LANES * n_segs + 1) * sizeof(uint16_t));
    uint64_t* s_bit = (uint64_t*)malloc((size_t)(n_segs + 1) * sizeof(uint64_t));
    if (!tmp || !loff || !s_bit) {
        free(tmp); free(loff); free(s_bit); free(s_elem); free(scratch); free(words); free(lane_sym); free(e); free(sm);
        return ORC_E_NOMEM;
    }
    uint64_t pos = 0;   /* bits, always a multiple of 16 */
    for (uint64_t g = 0; g < n_segs; ++g) {
        s_bit[g] = pos;
        uint64_t e0 = s_elem[g], m = s_elem[g + 1] - e0;
        for (uint32_t j = 0; j < LANES; ++j) {
            loff[LANES * g + j] = (uint16_t)(pos - s_bit[g]);
            uint64_t k = 0;
            for (uint64_t t = 0;; ++t) {
                uint64_t i = lane_elem(m, j, t);
                if (i >= m) break;
                lane_sym[k++] = e[e0 + i];
            }
            if (!k) continue;
            uint64_t nw = rans_encode_lane(lane_sym, k, f, cum, scratch, words);
            for (uint64_t w = 0; w < nw; ++w) {
                tmp[pos >> 3] = (uint8_t)(words[w] >> 8);
                tmp[(pos >> 3) + 1] = (uint8_t)(words[w] & 0xFF);
                pos += 16;
            }
        }
    }
    s_bit[n_segs] = pos;
    free(scratch); free(words); free(lane_sym);
    uint64_t bits = pos;
    uint64_t stream_bytes = round_up(ceil_div(bits, 8), 8) + LANES_SLACK;
    uint64_t off_len = HDR_BYTES;
    uint64_t off_tens = round_up(off_len + 512, ALIGN);
    uint64_t off_segs = round_up(off_tens + 16ull * n_tensors, ALIGN);
    uint64_t off_loff = round_up(off_segs + 16 * (n_segs + 1), ALIGN);
    uint64_t off_stream = round_up(off_loff + 2ull * LANES * n_segs, ALIGN);
    uint64_t off_sm = round_up(off_stream + stream_bytes, ALIGN);
    uint64_t sm_bytes = kind == KIND_BF16 ? n : 0;
    uint64_t total = round_up(off_sm + sm_bytes, ALIGN);
    uint8_t* b = (uint8_t*)calloc(total, 1);
    if (!b) { free(tmp); free(loff); free(s_bit); free(s_elem); free(e); free(sm); return ORC_E_NOMEM; }
    for (int s2 = 0; s2 < 256; ++s2) wr(b + off_len + 2 * s2, f[s2], 2);
    uint64_t at = 0;
    for (uint32_t t = 0; t < n_tensors; ++t) {
        wr(b + off_tens + 16ull * t, at, 8);
        wr(b + off_tens + 16ull * t + 8, numels[t], 8);
        at += numels[t];
    }
    for (uint64_t g = 0; g <= n_segs; ++g) {
        wr(b + off_segs + 16 * g, s_elem[g], 8);
        wr(b + off_segs + 16 * g + 8, s_bit[g], 8);
    }
    for (uint64_t i = 0; i < LANES * n_segs; ++i) wr(b + off_loff + 2 * i, loff[i], 2);
    memcpy(b + off_stream, tmp, ceil_div(bits, 8));
    if (sm_bytes) memcpy(b + off_sm, sm, sm_bytes);
    free(tmp); free(loff); free(s_bit); free(s_elem);

    memcpy(b + F_MAGIC, "WCBF", 4);
    wr(b + F_VERSION, 3, 2);
    wr(b + F_FLAGS, 0, 2);
    wr(b + F_MAXLEN, RANS_P, 1);
    wr(b + F_LANES, LANES, 1);
    wr(b + F_LANE_BLOCK, LANE_BLOCK, 2);
    wr(b + F_SEGBITS, B, 4);
    wr(b + F_NTENS, n_tensors, 4);
    wr(b + F_ALIGN, A, 4);
    wr(b + F_MAXG, M, 4);
    wr(b + F_N, n, 8);
    wr(b + F_SBITS, bits, 8);
    wr(b + F_NGROUPS, n_segs, 8);
    wr(b + F_OFF_LEN, off_len, 8);
    wr(b + F_OFF_TENS, off_tens, 8);
    wr(b + F_OFF_GS, off_segs, 8);
    wr(b + F_OFF_LOFF, off_loff, 8);
    wr(b + F_OFF_STREAM, off_stream, 8);
    wr(b + F_STREAM_BYTES, stream_bytes, 8);
    wr(b + F_OFF_SM, off_sm, 8);
    wr(b + F_TOTAL, total, 8);
    wr(b + F_KIND, kind, 1);
    wr(b + F_CODER, CODER_RANS, 1);
    free(e);
    free(sm);
    *blob = b;
    *blob_bytes = total;
    return ORC_OK;
}

static int rans_args(uint64_t n, const void* src, const uint64_t** numels, uint32_t* n_tensors, uint64_t* one,
                     uint32_t A, uint32_t M, uint32_t B, uint8_t** blob, uint64_t* blob_bytes) {
    if (!blob || !blob_bytes || (n && !src)) return ORC_E_ARG;
    /* one block always fits: A symbols of frequency 1 cost 97 eighths each */
    if (A < 1 || M < A || M % A || M > LANES * LANE_BLOCK * 1024u || B > 65535u || B < LANES * RANS_FLUSH ||
        97ull * A > 8ull * (B - LANES * RANS_FLUSH))
        return ORC_E_ARG;
    *one = n;
    if (!*numels) { *numels = one; *n_tensors = 1; }
    uint64_t sum = 0;
    for (uint32_t t = 0; t < *n_tensors; ++t) sum += (*numels)[t];
    return sum == n ? ORC_OK : ORC_E_ARG;
}

int orc_encode_lanes_rans(const uint16_t* w, uint64_t n, const uint64_t* numels, uint32_t n_tensors, uint32_t A,
                          uint32_t M, uint32_t B, uint8_t** blob, uint64_t* blob_bytes) {
    uint64_t one;
    int st = rans_args(n, w, &numels, &n_tensors, &one, A, M, B, blob, blob_bytes);
    if (st != ORC_OK) return st;
    uint8_t* e = (uint8_t*)malloc(n ? n : 1);
    uint8_t* sm = (uint8_t*)malloc(n ? n : 1);
    if (!e || !sm) { free(e); free(sm); return ORC_E_NOMEM; }
    orc_split_planes(w, n, e, sm);
    return encode_rans_planes(e, sm, KIND_BF16, n, numels, n_tensors, A, M, B, blob, blob_bytes);
}

int orc_encode_lanes_rans_u8(const uint8_t* codes, uint64_t n, const uint64_t* numels, uint32_t n_tensors,
                             uint32_t A, uint32_t M, uint32_t B, uint8_t** blob, uint64_t* blob_bytes) {
    uint64_t one;
    int st = rans_args(n, codes, &numels, &n_tensors, &one, A, M, B, blob, blob_bytes);
    if (st != ORC_OK) return st;
    uint8_t* e = (uint8_t*)malloc(n ? n : 1);
    if (!e) return ORC_E_NOMEM;
    if (n) memcpy(e, codes, n);
    return encode_rans_planes(e, NULL, KIND_U8, n, numels, n_tensors, A, M, B, blob, blob_bytes);
}

/* ------------------------------------------------------------------------ */
/* Reader                                                                   */
/* ------------------------------------------------------------------------ */
typedef struct {
    uint32_t version;   /* 2: per-chunk gaps; 3: interleaved lanes */
    uint32_t kind;      /* KIND_BF16 or (version 3) KIND_U8 */
    uint32_t coder;     /* CODER_HUFFMAN or (version 3) CODER_RANS */
    uint32_t gap_bits;  /* version 2: 8 (one byte per gap) or 5 (packed) */
    uint32_t max_len, G, A, M, B, n_tensors;
    uint64_t n, stream_bits, n_chunks, n_groups;
    uint64_t off_len, off_tens, off_gs, off_gap, off_stream, stream_bytes, off_sm, total;
} hdr_t;

static int parse_header_lanes(const uint8_t* blob, uint64_t bytes, hdr_t* h);

static int parse_header(const uint8_t* blob, uint64_t bytes, hdr_t* h) {
    if (!blob || bytes < HDR_BYTES) return ORC_E_TRUNC;
    if (memcmp(blob + F_MAGIC, "WCBF", 4) != 0) return ORC_E_MAGIC;
    if (rd(blob + F_VERSION, 2) == 3) return parse_header_lanes(blob, bytes, h);
    h->version = 2;
    h->kind = KIND_BF16;
    h->coder = CODER_HUFFMAN;
    h->B = 0;
    if (blob[F_KIND] || blob[F_CODER]) return ORC_E_MAGIC;
    if (rd(blob + F_VERSION, 2) != 2 || rd(blob + F_FLAGS, 2) != 0) return ORC_E_MAGIC;
    if (rd(blob + F_CHUNKBITS, 1) != CHUNK_BITS) return ORC_E_MAGIC;
    if (rd(blob + F_GAPBITS, 1) != 0 && rd(blob + F_GAPBITS, 1) != 5) return ORC_E_MAGIC;
    if (rd(blob + F_GAPBITS + 1, 1) != 0) return ORC_E_MAGIC;
    h->gap_bits = rd(blob + F_GAPBITS, 1) == 5 ? 5u : 8u;
    for (uint32_t k = F_TAIL; k < HDR_BYTES; ++k) if (blob[k]) return ORC_E_MAGIC;
    h->max_len = (uint32_t)rd(blob + F_MAXLEN, 1);
    h->G = (uint32_t)rd(blob + F_G, 4);
    h->A = (uint32_t)rd(blob + F_ALIGN, 4);
    h->M = (uint32_t)rd(blob + F_MAXG, 4);
    h->n_tensors = (uint32_t)rd(blob + F_NTENS, 4);
    h->n = rd(blob + F_N, 8);
    h->stream_bits = rd(blob + F_SBITS, 8);
    h->n_chunks = rd(blob + F_NCHUNKS, 8);
    h->n_groups = rd(blob + F_NGROUPS, 8);
    h->off_len = rd(blob + F_OFF_LEN, 8);
    h->off_tens = rd(blob + F_OFF_TENS, 8);
    h->off_gs = rd(blob + F_OFF_GS, 8);
    h->off_gap = rd(blob + F_OFF_GAP, 8);
    h->off_stream = rd(blob + F_OFF_STREAM, 8);
    h->stream_bytes = rd(blob + F_STREAM_BYTES, 8);
    h->off_sm = rd(blob + F_OFF_SM, 8);
    h->total = rd(blob + F_TOTAL, 8);
    if (h->max_len < 1 || h->max_len > MAX_LEN_LIMIT || h->G < 1 || h->A < 1 || h->M < h->A || h->M % h->A)
        return ORC_E_MAGIC;
    /* derived sizes (guard the multiplications against absurd values first) */
    if (h->n > ((uint64_t)1 << 48) || h->stream_bits > ((uint64_t)1 << 56)) return ORC_E_SIZES;
    if (h->n_chunks != ceil_div(h->stream_bits, CHUNK_BITS)) return ORC_E_SIZES;
    if (h->n_groups > h->n || (h->n_groups == 0) != (h->n == 0)) return ORC_E_SIZES;
    if (h->stream_bytes != 8 * h->n_chunks + 16) return ORC_E_SIZES;
    if (h->stream_bits > h->n * (uint64_t)h->max_len || h->stream_bits < h->n) return ORC_E_SIZES;
    /* sections: aligned, in order, inside the blob */
    const uint64_t offs[6] = {h->off_len, h->off_tens, h->off_gs, h->off_gap, h->off_stream, h->off_sm};
    const uint64_t lens[6] = {256, 16ull * h->n_tensors, 16 * (h->n_groups + 1),
                              gap_section_bytes(h->n_chunks, h->gap_bits), h->stream_bytes, h->n};
    uint64_t lo = HDR_BYTES;
    for (int k = 0; k < 6; ++k) {
        if (offs[k] % ALIGN || offs[k] < lo) return ORC_E_TRUNC;
        lo = offs[k] + lens[k];
    }
    if (h->total < lo || h->total > bytes) return ORC_E_TRUNC;
    return ORC_OK;
}

static int parse_header_lanes(const uint8_t* blob, uint64_t bytes, hdr_t* h) {
    h->version = 3;
    h->gap_bits = 8;   /* no gap section */
    h->kind = blob[F_KIND];
    h->coder = blob[F_CODER];
    if (h->kind != KIND_BF16 && h->kind != KIND_U8) return ORC_E_MAGIC;
    if (h->coder != CODER_HUFFMAN && h->coder != CODER_RANS) return ORC_E_MAGIC;
    if (rd(blob + F_FLAGS, 2) != 0 || rd(blob + F_LANES, 1) != LANES || rd(blob + F_LANE_BLOCK, 2) != LANE_BLOCK)
        return ORC_E_MAGIC;
    for (uint32_t k = F_TAIL; k < HDR_BYTES; ++k) if (blob[k]) return ORC_E_MAGIC;
    if (rd(blob + F_NCHUNKS, 8) != 0) return ORC_E_MAGIC;
    h->max_len = (uint32_t)rd(blob + F_MAXLEN, 1);
    h->G = 0;
    h->B = (uint32_t)rd(blob + F_SEGBITS, 4);
    h->A = (uint32_t)rd(blob + F_ALIGN, 4);
    h->M = (uint32_t)rd(blob + F_MAXG, 4);
    h->n_tensors = (uint32_t)rd(blob + F_NTENS, 4);
    h->n = rd(blob + F_N, 8);
    h->stream_bits = rd(blob + F_SBITS, 8);
    h->n_chunks = 0;
    h->n_groups = rd(blob + F_NGROUPS, 8);
    h->off_len = rd(blob + F_OFF_LEN, 8);
    h->off_tens = rd(blob + F_OFF_TENS, 8);
    h->off_gs = rd(blob + F_OFF_GS, 8);
    h->off_gap = rd(blob + F_OFF_LOFF, 8);
    h->off_stream = rd(blob + F_OFF_STREAM, 8);
    h->stream_bytes = rd(blob + F_STREAM_BYTES, 8);
    h->off_sm = rd(blob + F_OFF_SM, 8);
    h->total = rd(blob + F_TOTAL, 8);
    if (h->A < 1 || h->M < h->A || h->M % h->A || h->B > 65535u) return ORC_E_MAGIC;
    if (h->coder == CODER_HUFFMAN &&
        (h->max_len < 1 || h->max_len > MAX_LEN_LIMIT || (uint64_t)h->A * h->max_len > h->B))
        return ORC_E_MAGIC;
    if (h->coder == CODER_RANS && (h->max_len != RANS_P || h->B < LANES * RANS_FLUSH ||
                                   97ull * h->A > 8ull * (h->B - LANES * RANS_FLUSH)))
        return ORC_E_MAGIC;
    if (h->n > ((uint64_t)1 << 48) || h->stream_bits > ((uint64_t)1 << 56)) return ORC_E_SIZES;
    if (h->n_groups > h->n || (h->n_groups == 0) != (h->n == 0)) return ORC_E_SIZES;
    if (h->stream_bytes != round_up(ceil_div(h->stream_bits, 8), 8) + LANES_SLACK) return ORC_E_SIZES;
    if (h->coder == CODER_HUFFMAN && (h->stream_bits > h->n * (uint64_t)h->max_len || h->stream_bits < h->n))
        return ORC_E_SIZES;
    if (h->coder == CODER_RANS && (h->stream_bits % 16 || h->stream_bits > h->n * (uint64_t)(RANS_P + 1) +
                                                                           (uint64_t)LANES * RANS_FLUSH * h->n_groups))
        return ORC_E_SIZES;
    const uint64_t offs[6] = {h->off_len, h->off_tens, h->off_gs, h->off_gap, h->off_stream, h->off_sm};
    const uint64_t lens[6] = {h->coder == CODER_RANS ? 512u : 256u, 16ull * h->n_tensors, 16 * (h->n_groups + 1),
                              2ull * LANES * h->n_groups, h->stream_bytes, h->kind == KIND_BF16 ? h->n : 0};
    uint64_t lo = HDR_BYTES;
    for (int k = 0; k < 6; ++k) {
        if (offs[k] % ALIGN || offs[k] < lo) return ORC_E_TRUNC;
        lo = offs[k] + lens[k];
    }
    if (h->total < lo || h->total > bytes) return ORC_E_TRUNC;
    return ORC_OK;
}

int orc_header(const uint8_t* blob, uint64_t blob_bytes, orc_report* rep) {
    hdr_t h;
    int st = parse_header(blob, blob_bytes, &h);
    if (st != ORC_OK) return st;
    if (rep) {
        memset(rep, 0, sizeof(*rep));
        rep->n_elems = h.n;
        rep->stream_bits = h.stream_bits;
        rep->n_chunks = h.n_chunks;
        rep->n_groups = h.n_groups;
        rep->n_tensors = h.n_tensors;
        rep->chunks_per_group = h.G;
        rep->group_align = h.A;
        rep->group_max_elems = h.M;
        rep->max_code_len = h.max_len;
        rep->layout = h.version == 3 ? 1u : 0u;
        rep->seg_max_bits = h.B;
        rep->elem_kind = h.kind;
        rep->coder = h.coder;
        rep->gap_bits = h.gap_bits;
    }
    return ORC_OK;
}

/* explicit binary trie of the canonical code */
typedef struct {
    int child[2];
    int sym;      /* -1 for an inner node */
} trie_node;

/* Version 2: serial bit-by-bit decode in element order; re-derive the
 * per-chunk gaps and the group table from the codeword starts actually
 * observed and compare them with the stored ones. */
static int decode_chunks(const uint8_t* blob, const hdr_t* h, const trie_node* T, uint16_t* out,
                         uint64_t hist[256]) {
    int st = ORC_OK;
    const uint8_t* stream = blob + h->off_stream;
    const uint8_t* gap = blob + h->off_gap;
    const uint8_t* gs = blob + h->off_gs;
    const uint8_t* sm = blob + h->off_sm;
    uint64_t nb = ceil_div(h->n, h->A);
    uint64_t* block_bit = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
    if (!block_bit) return ORC_E_NOMEM;
    uint64_t pos = 0, next_chunk = 0;
    for (uint64_t i = 0; i < h->n && st == ORC_OK; ++i) {
        while (next_chunk < h->n_chunks && CHUNK_BITS * next_chunk <= pos) {
            uint64_t want = pos - CHUNK_BITS * next_chunk;
            if (want >= CHUNK_BITS || gap_at(gap, next_chunk, h->gap_bits) != want) { st = ORC_E_GAP; break; }
            ++next_chunk;
        }
        if (st != ORC_OK) break;
        if (i % h->A == 0) block_bit[i / h->A] = pos;
        int node = 0;
        for (;;) {
            if (pos >= h->stream_bits) { st = ORC_E_STREAM; break; }
            int bit = (stream[pos >> 3] >> (7 - (pos & 7))) & 1;
            ++pos;
            node = T[node].child[bit];
            if (node < 0) { st = ORC_E_STREAM; break; }
            if (T[node].sym >= 0) break;
        }
        if (st != ORC_OK) break;
        uint8_t e = (uint8_t)T[node].sym;
        hist[e]++;
        uint16_t s = sm[i];
        out[i] = (uint16_t)(((s & 0x80) << 8) | ((uint16_t)e << 7) | (s & 0x7F));
    }
    if (st != ORC_OK) { free(block_bit); return st; }
    if (pos != h->stream_bits) { free(block_bit); return ORC_E_STREAM; }
    while (next_chunk < h->n_chunks) {
        uint64_t want = h->stream_bits - CHUNK_BITS * next_chunk;
        if (want >= CHUNK_BITS || gap_at(gap, next_chunk, h->gap_bits) != want) { free(block_bit); return ORC_E_GAP; }
        ++next_chunk;
    }
    /* the group table, re-derived from the observed block starts */
    block_bit[nb] = pos;
    {
        uint64_t* g_elem = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
        uint64_t* g_bit = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
        if (!g_elem || !g_bit) { free(g_elem); free(g_bit); free(block_bit); return ORC_E_NOMEM; }
        uint64_t ng = orc_groups(block_bit, nb, h->n, h->A, h->G, h->M, g_elem, g_bit);
        if (ng != h->n_groups) st = ORC_E_GROUP;
        for (uint64_t g = 0; st == ORC_OK && g <= ng; ++g)
            if (rd(gs + 16 * g, 8) != g_elem[g] || rd(gs + 16 * g + 8, 8) != g_bit[g]) st = ORC_E_GROUP;
        free(g_elem); free(g_bit);
    }
    free(block_bit);
    return st;
}

/* Walk the trie from bit *pos; -1 if the stream ends or leaves the code. */
static int trie_symbol(const trie_node* T, const uint8_t* stream, uint64_t limit, uint64_t* pos) {
    int node = 0;
    for (;;) {
        if (*pos >= limit) return -1;
        int bit = (stream[*pos >> 3] >> (7 - (*pos & 7))) & 1;
        ++*pos;
        node = T[node].child[bit];
        if (node < 0) return -1;
        if (T[node].sym >= 0) return T[node].sym;
    }
}

/* Version 3 (interleaved lanes): for every stored segment, decode lane 0's
 * symbols, then lane 1's, ... bit by bit, checking that each lane starts at
 * its stored offset and that the segment ends where the next begins; then
 * re-derive the segment table from the decoded code lengths. */
static int decode_lanes(const uint8_t* blob, const hdr_t* h, const trie_node* T, const uint8_t* lens,
                        uint16_t* out, uint8_t* out8, uint64_t hist[256]) {
    const uint8_t* stream = blob + h->off_stream;
    const uint8_t* segs = blob + h->off_gs;
    const uint8_t* loff = blob + h->off_gap;
    const uint8_t* sm = blob + h->off_sm;
    uint8_t* e = (uint8_t*)malloc(h->n ? h->n : 1);
    if (!e) return ORC_E_NOMEM;
    int st = ORC_OK;
    uint64_t pos = 0;
    if (rd(segs, 8) != 0 || rd(segs + 8, 8) != 0) st = ORC_E_GROUP;
    for (uint64_t g = 0; g < h->n_groups && st == ORC_OK; ++g) {
        uint64_t e0 = rd(segs + 16 * g, 8), p0 = rd(segs + 16 * g + 8, 8);
        uint64_t e1 = rd(segs + 16 * (g + 1), 8), p1 = rd(segs + 16 * (g + 1) + 8, 8);
        if (e1 <= e0 || e1 > h->n || p0 != pos || p1 < p0 || p1 > h->stream_bits) { st = ORC_E_GROUP; break; }
        uint64_t m = e1 - e0;
        for (uint32_t j = 0; j < LANES && st == ORC_OK; ++j) {
            if (rd(loff + 2 * (LANES * g + j), 2) != pos - p0) { st = ORC_E_GROUP; break; }
            for (uint64_t t = 0;; ++t) {
                uint64_t i = lane_elem(m, j, t);
                if (i >= m) break;
                int sym = trie_symbol(T, stream, p1, &pos);
                if (sym < 0) { st = ORC_E_STREAM; break; }
                e[e0 + i] = (uint8_t)sym;
            }
        }
        if (st == ORC_OK && pos != p1) st = ORC_E_STREAM;
    }
    if (st == ORC_OK && (rd(segs + 16 * h->n_groups, 8) != h->n || rd(segs + 16 * h->n_groups + 8, 8) != h->stream_bits ||
                         pos != h->stream_bits))
        st = ORC_E_STREAM;
    if (st == ORC_OK) {   /* the segment table, re-derived from the decoded code lengths */
        uint64_t nb = ceil_div(h->n, h->A);
        uint64_t* block_bit = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
        uint64_t* s_elem = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
        uint64_t* s_bit = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
        if (!block_bit || !s_elem || !s_bit) st = ORC_E_NOMEM;
        if (st == ORC_OK) {
            uint64_t at = 0;
            for (uint64_t i = 0; i < h->n; ++i) {
                if (i % h->A == 0) block_bit[i / h->A] = at;
                at += lens[e[i]];
            }
            block_bit[nb] = at;
            uint64_t ns = orc_segments(block_bit, nb, h->n, h->A, h->B, h->M, s_elem, s_bit);
            if (ns != h->n_groups) st = ORC_E_GROUP;
            for (uint64_t g = 0; st == ORC_OK && g <= ns; ++g)
                if (rd(segs + 16 * g, 8) != s_elem[g] || rd(segs + 16 * g + 8, 8) != s_bit[g]) st = ORC_E_GROUP;
        }
        free(block_bit); free(s_elem); free(s_bit);
    }
    for (uint64_t i = 0; st == ORC_OK && i < h->n; ++i) {
        hist[e[i]]++;
        if (h->kind == KIND_U8) {
            out8[i] = e[i];
        } else {
            uint16_t s = sm[i];
            out[i] = (uint16_t)(((s & 0x80) << 8) | ((uint16_t)e[i] << 7) | (s & 0x7F));
        }
    }
    free(e);
    return st;
}

/* rANS lanes: for every stored segment and lane, check the lane's stored
 * offset, read its final state (two words) and decode its symbols with the
 * frequency table (slot = x mod 2^P, the symbol whose cumulative range holds
 * it, x = f (x >> P) + slot - cum, one more word when x < 2^16); each lane must
 * end in the encoder's initial state 2^16 exactly where the next lane begins.
 * Then re-derive the segment table from the frequency bound. */
static int decode_lanes_rans(const uint8_t* blob, const hdr_t* h, const uint32_t f[256], uint16_t* out,
                             uint8_t* out8, uint64_t hist[256]) {
    const uint8_t* stream = blob + h->off_stream;
    const uint8_t* segs = blob + h->off_gs;
    const uint8_t* loff = blob + h->off_gap;
    const uint8_t* sm = blob + h->off_sm;
    uint32_t cum[257];
    cum[0] = 0;
    for (int s = 0; s < 256; ++s) cum[s + 1] = cum[s] + f[s];
    uint8_t* e = (uint8_t*)malloc(h->n ? h->n : 1);
    if (!e) return ORC_E_NOMEM;
    int st = ORC_OK;
    uint64_t pos = 0;
    if (rd(segs, 8) != 0 || rd(segs + 8, 8) != 0) st = ORC_E_GROUP;
    for (uint64_t g = 0; g < h->n_groups && st == ORC_OK; ++g) {
        uint64_t e0 = rd(segs + 16 * g, 8), p0 = rd(segs + 16 * g + 8, 8);
        uint64_t e1 = rd(segs + 16 * (g + 1), 8), p1 = rd(segs + 16 * (g + 1) + 8, 8);
        if (e1 <= e0 || e1 > h->n || p0 != pos || p1 < p0 || p1 > h->stream_bits) { st = ORC_E_GROUP; break; }
        uint64_t m = e1 - e0;
        for (uint32_t j = 0; j < LANES && st == ORC_OK; ++j) {
            if (rd(loff + 2 * (LANES * g + j), 2) != pos - p0) { st = ORC_E_GROUP; break; }
            if (lane_elem(m, j, 0) >= m) continue;          /* an empty lane has an empty string */
            if (pos + 32 > p1) { st = ORC_E_STREAM; break; }
            uint64_t x = ((uint64_t)stream[pos >> 3] << 24) | ((uint64_t)stream[(pos >> 3) + 1] << 16) |
                         ((uint64_t)stream[(pos >> 3) + 2] << 8) | stream[(pos >> 3) + 3];
            pos += 32;
            for (uint64_t t = 0;; ++t) {
                uint64_t i = lane_elem(m, j, t);
                if (i >= m) break;
                uint32_t slot = (uint32_t)(x & (((uint64_t)1 << RANS_P) - 1));
                uint32_t s = 0;
                while (cum[s + 1] <= slot) ++s;
                e[e0 + i] = (uint8_t)s;
                x = f[s] * (x >> RANS_P) + slot - cum[s];
                if (x < RANS_L) {
                    if (pos + 16 > p1) { st = ORC_E_STREAM; break; }
                    x = (x << 16) | ((uint64_t)stream[pos >> 3] << 8) | stream[(pos >> 3) + 1];
                    pos += 16;
                }
            }
            if (st == ORC_OK && x != RANS_L) st = ORC_E_STREAM;
        }
        if (st == ORC_OK && pos != p1) st = ORC_E_STREAM;
    }
    if (st == ORC_OK && (rd(segs + 16 * h->n_groups, 8) != h->n ||
                         rd(segs + 16 * h->n_groups + 8, 8) != h->stream_bits || pos != h->stream_bits))
        st = ORC_E_STREAM;
    if (st == ORC_OK) {
        uint64_t nb = ceil_div(h->n, h->A);
        uint64_t* cost_before = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
        uint64_t* s_elem = (uint64_t*)malloc((size_t)(nb + 1) * sizeof(uint64_t));
        if (!cost_before || !s_elem) st = ORC_E_NOMEM;
        if (st == ORC_OK) {
            uint64_t at = 0;
            for (uint64_t i = 0; i < h->n; ++i) {
                if (i % h->A == 0) cost_before[i / h->A] = at;
                at += rans_cost8(f[e[i]]);
            }
            cost_before[nb] = at;
            uint64_t ns = rans_segments(cost_before, nb, h->n, h->A, h->B, h->M, s_elem);
            if (ns != h->n_groups) st = ORC_E_GROUP;
            for (uint64_t g = 0; st == ORC_OK && g <= ns; ++g)
                if (rd(segs + 16 * g, 8) != s_elem[g]) st = ORC_E_GROUP;
        }
        free(cost_before); free(s_elem);
    }
    for (uint64_t i = 0; st == ORC_OK && i < h->n; ++i) {
        hist[e[i]]++;
        if (h->kind == KIND_U8) {
            out8[i] = e[i];
        } else {
            uint16_t s = sm[i];
            out[i] = (uint16_t)(((s & 0x80) << 8) | ((uint16_t)e[i] << 7) | (s & 0x7F));
        }
    }
    free(e);
    return st;
}

static int decode_container(const uint8_t* blob, uint64_t bytes, uint32_t kind, uint16_t* out, uint8_t* out8,
                            uint64_t out_cap, orc_report* rep) {
    hdr_t h;
    int st = parse_header(blob, bytes, &h);
    if (st != ORC_OK) return st;
    if (h.kind != kind) return ORC_E_KIND;
    if (h.n > out_cap || (h.n && !(kind == KIND_U8 ? (void*)out8 : (void*)out))) return ORC_E_OUTSIZE;

    /* tensor table must be a partition of [0, n) in order */
    {
        uint64_t acc = 0;
        for (uint32_t t = 0; t < h.n_tensors; ++t) {
            uint64_t off = rd(blob + h.off_tens + 16ull * t, 8);
            uint64_t num = rd(blob + h.off_tens + 16ull * t + 8, 8);
            if (off != acc || num > h.n - acc) return ORC_E_TENSORS;
            acc += num;
        }
        if (acc != h.n) return ORC_E_TENSORS;
    }

    uint64_t hist[256] = {0};
    uint32_t m = 0, longest = 0;
    uint64_t kraft = 0;
    const uint8_t* lens = blob + h.off_len;
    if (h.coder == CODER_RANS) {
        /* frequencies: at most 2^P each, summing to 2^P (or all 0 for n = 0) */
        uint32_t f[256];
        uint64_t sum = 0;
        for (int s = 0; s < 256; ++s) {
            f[s] = (uint32_t)rd(lens + 2 * s, 2);
            if (f[s] > (1u << RANS_P)) return ORC_E_LENGTHS;
            sum += f[s];
            m += f[s] != 0;
        }
        if (h.n ? sum != (1u << RANS_P) : sum != 0) return ORC_E_KRAFT;
        st = decode_lanes_rans(blob, &h, f, out, out8, hist);
        if (st != ORC_OK) return st;
        goto padding;
    }
    /* code lengths and Kraft's sum, exactly, in units of 2^-24 */
    for (int s = 0; s < 256; ++s) {
        if (!lens[s]) continue;
        if (lens[s] > h.max_len) return ORC_E_LENGTHS;
        kraft += (uint64_t)1 << (MAX_LEN_LIMIT - lens[s]);
        ++m;
        if (lens[s] > longest) longest = lens[s];
    }
    if (m >= 2 && kraft != ((uint64_t)1 << MAX_LEN_LIMIT)) return ORC_E_KRAFT;
    if (m == 1 && longest != 1) return ORC_E_KRAFT;
    if (m == 0 && h.n != 0) return ORC_E_KRAFT;

    uint32_t codes[256];
    st = orc_canonical_codes(lens, codes);
    if (st != ORC_OK) return st;

    /* build the trie one code bit at a time, rejecting prefix conflicts */
    int cap_nodes = 256 * (MAX_LEN_LIMIT + 1) + 1;
    trie_node* T = (trie_node*)malloc((size_t)cap_nodes * sizeof(trie_node));
    if (!T) return ORC_E_NOMEM;
    int n_nodes = 1;
    T[0].child[0] = T[0].child[1] = -1;
    T[0].sym = -1;
    for (int s = 0; s < 256 && st == ORC_OK; ++s) {
        int L = lens[s];
        if (!L) continue;
        int node = 0;
        for (int k = L - 1; k >= 0; --k) {
            if (T[node].sym >= 0) { st = ORC_E_PREFIX; break; }
            int bit = (int)((codes[s] >> k) & 1u);
            int nxt = T[node].child[bit];
            if (k == 0) {
                if (nxt >= 0) { st = ORC_E_PREFIX; break; }
                nxt = n_nodes++;
                T[nxt].child[0] = T[nxt].child[1] = -1;
                T[nxt].sym = s;
                T[node].child[bit] = nxt;
            } else {
                if (nxt < 0) {
                    nxt = n_nodes++;
                    T[nxt].child[0] = T[nxt].child[1] = -1;
                    T[nxt].sym = -1;
                    T[node].child[bit] = nxt;
                }
                node = nxt;
            }
        }
    }
    if (st != ORC_OK) { free(T); return st; }
    if (h.version == 3)
        st = decode_lanes(blob, &h, T, lens, out, out8, hist);
    else
        st = decode_chunks(blob, &h, T, out, hist);
    free(T);
    if (st != ORC_OK) return st;

padding:;
    /* every bit after stream_bits, up to the end of the section, is zero */
    const uint8_t* stream = blob + h.off_stream;
    for (uint64_t p = h.stream_bits; p < 8 * h.stream_bytes; ++p) {
        if ((p & 7) == 0 && p + 8 <= 8 * h.stream_bytes) {
            if (stream[p >> 3]) return ORC_E_PADDING;
            p += 7;
            continue;
        }
        if ((stream[p >> 3] >> (7 - (p & 7))) & 1) return ORC_E_PADDING;
    }

    if (rep) {
        memset(rep, 0, sizeof(*rep));
        rep->n_elems = h.n;
        rep->stream_bits = h.stream_bits;
        rep->n_chunks = h.n_chunks;
        rep->n_groups = h.n_groups;
        rep->n_tensors = h.n_tensors;
        rep->chunks_per_group = h.G;
        rep->group_align = h.A;
        rep->group_max_elems = h.M;
        rep->max_code_len = h.max_len;
        rep->layout = h.version == 3 ? 1u : 0u;
        rep->seg_max_bits = h.B;
        rep->elem_kind = h.kind;
        rep->coder = h.coder;
        rep->gap_bits = h.gap_bits;
        rep->n_symbols = m;
        rep->longest_code = longest;
        rep->kraft_num = kraft;
        double H = 0.0, Lsum = 0.0;
        for (int s = 0; s < 256; ++s) {
            rep->hist[s] = hist[s];
            if (!hist[s]) continue;
            double p = (double)hist[s] / (double)h.n;
            H -= p * log2(p);
            if (h.coder == CODER_HUFFMAN) Lsum += (double)hist[s] * (double)lens[s];
        }
        if (h.coder == CODER_RANS) Lsum = (double)h.stream_bits;   /* every stored bit, final states included */
        rep->entropy_bits = H;
        rep->mean_code_bits = h.n ? Lsum / (double)h.n : 0.0;
    }
    return ORC_OK;
}

int orc_decode(const uint8_t* blob, uint64_t bytes, uint16_t* out, uint64_t out_cap, orc_report* rep) {
    return decode_container(blob, bytes, KIND_BF16, out, NULL, out_cap, rep);
}

int orc_decode_u8(const uint8_t* blob, uint64_t bytes, uint8_t* out, uint64_t out_cap, orc_report* rep) {
    return decode_container(blob, bytes, KIND_U8, NULL, out, out_cap, rep);
}

/* ------------------------------------------------------------------------ */
/* Batch-1 matrix-vector product over bf16 operands, exact in double:       */
/* the consumer of decoded weights [DF11 abstract: inference kernels read   */
/* the decompressed weights; LW "Truck packing": unpacked right before use].*/
/* A bf16 bit pattern b is the float32 whose bits are b << 16.  Products    */
/* and sums are taken in double, serially, column by column.                */
/* ------------------------------------------------------------------------ */
static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int orc_gemv_bf16(const uint16_t* W, uint64_t rows, uint64_t cols, const uint16_t* x, double* y) {
    if ((rows && cols && (!W || !x)) || (rows && !y)) return ORC_E_ARG;
    for (uint64_t r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (uint64_t c = 0; c < cols; ++c) acc += bf16_value(W[r * cols + c]) * bf16_value(x[c]);
        y[r] = acc;
    }
    return ORC_OK;
}

void orc_free(void* p) { free(p); }
