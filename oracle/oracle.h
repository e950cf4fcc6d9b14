/*
 * oracle.h -- plain serial CPU oracle for the lossless entropy-coded bf16
 * weight container.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this code, and this code includes nothing from the product.  Only
 * the tests, the smoke entry point and the benchmark's CPU-baseline leg may
 * use it.  It shares no header, helper, table or constant with the HIP path:
 * the container layout below is re-stated here from the format description,
 * independently of the product's own definitions.
 *
 * What it computes (pages: "70% Size, 100% Accuracy: Lossless LLM Compression
 * for Efficient GPU Inference via Dynamic-Length Float", abstract -- entropy
 * coding of the bf16 representation by symbol frequency, outputs bit-for-bit
 * identical; "From a Lossless (~1.5:1) Compression Algorithm for Llama2 7B
 * Weights ...", abstract -- lossless ~1.5:1 coding of bf16 weights;
 * "Huff-LLM: End-to-End Lossless Compression for Efficient LLM Inference",
 * abstract -- Huffman-coded weights kept compressed end to end):
 *
 *   every bf16 word b is split into an 8-bit exponent e = (b >> 7) & 0xFF,
 *   which is Huffman-coded, and a raw byte sm = ((b >> 8) & 0x80) | (b & 0x7F)
 *   holding sign and mantissa.  Decoding must give back b exactly.
 *
 * Every function returns 0 on success or a negative ORC_E_* code.
 */
#ifndef WC_ORACLE_H
#define WC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes (oracle-private numbering) */
#define ORC_OK             0
#define ORC_E_ARG         -1   /* bad argument                               */
#define ORC_E_MAGIC       -2   /* wrong magic / version / fixed field        */
#define ORC_E_TRUNC       -3   /* blob shorter than a section it declares    */
#define ORC_E_LENGTHS     -4   /* code length outside 1..max_code_len        */
#define ORC_E_KRAFT       -5   /* code lengths do not form a complete code   */
#define ORC_E_PREFIX      -6   /* prefix conflict while building the trie    */
#define ORC_E_STREAM      -7   /* bit stream does not decode to n symbols    */
#define ORC_E_PADDING     -8   /* non-zero padding bits after stream end     */
#define ORC_E_GAP         -9   /* stored per-chunk gap disagrees             */
#define ORC_E_GROUP      -10   /* stored group table disagrees               */
#define ORC_E_TENSORS    -11   /* tensor table is not a partition of [0, n)  */
#define ORC_E_SIZES      -12   /* n_chunks / n_groups / stream_bytes wrong   */
#define ORC_E_NOMEM      -13
#define ORC_E_OUTSIZE    -14   /* output buffer too small                    */
#define ORC_E_KIND       -15   /* container holds another element kind       */

/* What the decoder observed, for statistics-based pins. */
typedef struct {
    uint64_t n_elems;
    uint64_t stream_bits;
    uint64_t n_chunks;
    uint64_t n_groups;
    uint32_t n_tensors;
    uint32_t chunks_per_group;
    uint32_t max_code_len;     /* header field                               */
    uint32_t n_symbols;        /* symbols with a non-zero code length        */
    uint32_t longest_code;     /* max code length actually assigned          */
    uint32_t group_align;      /* elements per block of the group table      */
    uint32_t group_max_elems;  /* elements per group at most                 */
    uint32_t reserved;
    uint64_t kraft_num;        /* sum over symbols of 2^(24 - len)           */
    double   entropy_bits;     /* H of the exponent histogram, bits/symbol   */
    double   mean_code_bits;   /* sum(count * len) / n                       */
    uint64_t hist[256];        /* exponent histogram of the decoded data     */
    uint32_t layout;           /* 0: per-chunk gaps (version 2); 1: lanes (3) */
    uint32_t seg_max_bits;     /* lanes layout: stream bits per segment max  */
    uint32_t elem_kind;        /* 0: bf16 (exponent coded); 1: u8 symbols    */
    uint32_t coder;            /* 0: canonical Huffman; 1: rANS              */
    uint32_t gap_bits;         /* version 2: 8 or 5 bits per stored gap      */
} orc_report;

/* Split bf16 words into exponent and sign+mantissa planes (definition). */
void orc_split_planes(const uint16_t* w, uint64_t n, uint8_t* exp_out, uint8_t* sm_out);

/* Put the two planes back together (definition). */
void orc_join_planes(const uint8_t* exp_in, const uint8_t* sm_in, uint64_t n, uint16_t* w_out);

/* Textbook Huffman (repeated merge of the two lightest trees), no length
 * limit.  lens[s] = depth of symbol s, 0 for absent symbols.  One present
 * symbol gets length 1. */
int orc_heap_huffman(const uint64_t counts[256], uint8_t lens[256]);

/* Optimal length-limited prefix code by package-merge.  Fails with
 * ORC_E_ARG if 2^max_len is smaller than the number of present symbols. */
int orc_package_merge(const uint64_t counts[256], uint32_t max_len, uint8_t lens[256]);

/* Canonical codes from lengths (shorter codes numerically smaller, equal
 * lengths in symbol order).  codes[s] holds the lens[s] low bits. */
int orc_canonical_codes(const uint8_t lens[256], uint32_t codes[256]);

/* Independent container writer (serial, one bit at a time).
 * w: n bf16 words; numels: n_tensors sizes summing to n (NULL -> one tensor);
 * chunks_per_group G, group_align A and group_max_elems M set the group table.
 * On success *blob is malloc'ed (free with orc_free). */
int orc_encode(const uint16_t* w, uint64_t n, const uint64_t* numels, uint32_t n_tensors,
               uint32_t max_code_len, uint32_t chunks_per_group, uint32_t group_align,
               uint32_t group_max_elems, uint8_t** blob, uint64_t* blob_bytes);

/* The same with the gap width chosen: gap_bits 8 (one byte per chunk, as
 * orc_encode) or 5 (gap c in bits 5c .. 5c + 4 of the section, lowest bit
 * first; header byte 10 = 5). */
int orc_encode_gaps(const uint16_t* w, uint64_t n, const uint64_t* numels, uint32_t n_tensors,
                    uint32_t max_code_len, uint32_t chunks_per_group, uint32_t group_align,
                    uint32_t group_max_elems, uint32_t gap_bits, uint8_t** blob, uint64_t* blob_bytes);

/* Independent writer of the interleaved-lane layout (container version 3):
 * segments of whole group_align-element blocks, at most group_max_elems
 * elements and at most seg_max_bits (< 65536, >= group_align * max_code_len)
 * stream bits; 64 lanes per segment, lane j taking 8-element lane blocks
 * j, j + 64, ...; each lane's codewords contiguous, lanes in order. */
int orc_encode_lanes(const uint16_t* w, uint64_t n, const uint64_t* numels, uint32_t n_tensors,
                     uint32_t max_code_len, uint32_t group_align, uint32_t group_max_elems,
                     uint32_t seg_max_bits, uint8_t** blob, uint64_t* blob_bytes);

/* The same layout over a plane of 8-bit codes (element kind u8): every byte
 * is one symbol, there is no raw plane (the LazyWeights page's setting:
 * Huffman codes for the integer codes of an already quantized model). */
int orc_encode_lanes_u8(const uint8_t* codes, uint64_t n, const uint64_t* numels, uint32_t n_tensors,
                        uint32_t max_code_len, uint32_t group_align, uint32_t group_max_elems,
                        uint32_t seg_max_bits, uint8_t** blob, uint64_t* blob_bytes);

/* rANS in the same lane layout (coder 1): frequencies quantized to sum to
 * 2^12 replace the code lengths (u16[256] in their section); each lane is one
 * rANS stream (32-bit state in [2^16, 2^32), 16-bit renormalisation words);
 * segments are cut by an upper bound of their encoded size; seg_max_bits must
 * leave room for 64 final states and one block.  The _u8 form codes bytes. */
int orc_encode_lanes_rans(const uint16_t* w, uint64_t n, const uint64_t* numels, uint32_t n_tensors,
                          uint32_t group_align, uint32_t group_max_elems, uint32_t seg_max_bits, uint8_t** blob,
                          uint64_t* blob_bytes);
int orc_encode_lanes_rans_u8(const uint8_t* codes, uint64_t n, const uint64_t* numels, uint32_t n_tensors,
                             uint32_t group_align, uint32_t group_max_elems, uint32_t seg_max_bits,
                             uint8_t** blob, uint64_t* blob_bytes);

/* Serial decoder of a u8-kind container into n bytes (out_cap >= n). */
int orc_decode_u8(const uint8_t* blob, uint64_t blob_bytes, uint8_t* out, uint64_t out_cap, orc_report* rep);

/* Serial bit-by-bit decoder with full container checks (either layout,
 * bf16 kind; ORC_E_KIND for a u8 container).
 * out must hold out_cap >= n_elems words.  rep may be NULL. */
int orc_decode(const uint8_t* blob, uint64_t blob_bytes, uint16_t* out, uint64_t out_cap,
               orc_report* rep);

/* Parse only the header: n_elems etc. (rep fields other than the header
 * ones are zeroed). */
int orc_header(const uint8_t* blob, uint64_t blob_bytes, orc_report* rep);

/* y[r] = sum over c of W[r][c] * x[c] for row-major bf16 W (rows x cols) and
 * bf16 x, in double (each bf16 value is exact in double; the sum is serial in
 * column order).  The consumer of decoded weights, for GEMV checks. */
int orc_gemv_bf16(const uint16_t* W, uint64_t rows, uint64_t cols, const uint16_t* x, double* y);

void orc_free(void* p);

#ifdef __cplusplus
}
#endif
#endif /* WC_ORACLE_H */
