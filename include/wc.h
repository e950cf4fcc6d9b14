/*
 * wc.h -- C ABI of libwc: lossless entropy-coded bf16 weights, decoded on
 * demand on an MI355X (gfx950).
 *
 * The method (pages: "70% Size, 100% Accuracy: Lossless LLM Compression for
 * Efficient GPU Inference via Dynamic-Length Float" (DFloat11), abstract;
 * "From a Lossless (~1.5:1) Compression Algorithm for Llama2 7B Weights ...",
 * abstract; "Huff-LLM: End-to-End Lossless Compression for Efficient LLM
 * Inference", abstract):
 *   each bf16 weight is split into its 8-bit exponent, which is Huffman-coded
 *   from the exponent histogram, and a raw byte holding sign and mantissa.
 *   Weights are prepared once on the host, stay compressed in memory, and are
 *   decoded on demand to bit-identical bf16 before compute kernels read them.
 *   One decode call handles a whole transformer block (DFloat11 abstract,
 *   design point (iii)); the kernel uses compact decode tables in on-chip
 *   memory (point (i)) and a two-phase count / scan / decode scheme driven by
 *   small per-chunk and per-group auxiliary variables (point (ii)).
 *
 * Container v2 (all fields little-endian; every section 256-byte aligned):
 *   header (256 B): "WCBF", u16 version=2, u16 flags=0, u8 max_code_len,
 *     u8 chunk_bits=64, u8 gap_bits (0 or 5), u8 0, u32 chunks_per_group G, u32 n_tensors,
 *     u32 group_align A, u64 n_elems, u64 stream_bits, u64 n_chunks,
 *     u64 n_groups, u64 offsets of code_len / tensors / groups / gap / stream,
 *     u64 stream_bytes, u64 offset of sm, u64 total_bytes, u32 group_max_elems M;
 *     rest zero.
 *   code_len    u8[256]   canonical Huffman code length per exponent value
 *                         (0 = absent), at most max_code_len (<= 24);
 *   tensors     {u64 elem_offset, u64 numel}[n_tensors], a partition of
 *                         [0, n_elems) in order;
 *   groups      {u64 first_elem, u64 first_bit}[n_groups+1]: the elements are
 *                         cut into blocks of A (the last may be shorter); a
 *                         group is a run of whole blocks, as long as possible
 *                         while its codewords touch at most G 64-bit chunks
 *                         and it holds at most M elements (and at least one
 *                         block); first_bit is the stream
 *                         bit where the codeword of first_elem starts; the
 *                         last entry is {n_elems, stream_bits};
 *   gap         u8[n_chunks]: bit offset, inside 64-bit chunk c, of the first
 *                         codeword starting at or after bit 64c (or of the
 *                         stream end); every gap is below max_code_len.  With
 *                         header byte 10 = 5 (it is 0 otherwise) the gaps are
 *                         packed in 5 bits, ceil(5 n_chunks / 8) bytes: gap c
 *                         in bits 5c .. 5c + 4 of the section read as a
 *                         little-endian bit string (byte k holds bits 8k ..
 *                         8k + 7, lowest first);
 *   stream      exponent codes, MSB-first, n_chunks*8 + 16 bytes, zero padded;
 *   sm          u8[n_elems]: sign bit << 7 | 7 mantissa bits.
 * Each group is one independent unit of GPU work: its output starts at a
 * multiple of A elements, so with A = 128 every 128-byte line of the bf16
 * output and of the sm plane belongs to one group.
 *
 * Container v3, the interleaved-lane layout (the LazyWeights page, analogy
 * section: Huffman codes stored in interleaved lanes and decoded on demand):
 * the same header positions, code and planes, except
 *   header: u16 version=3; u8 lanes=64 at 9; u16 lane_block=8 at 10;
 *     u32 seg_max_bits B at 12 (in place of G); n_chunks = 0;
 *   groups      the segment table: segments are runs of whole A-element
 *               blocks, as long as possible while they hold at most M
 *               elements and their codewords at most B bits;
 *   lane_off    u16[64 * n_segs] at the gap section's place: inside a
 *               segment, 8-element lane blocks are dealt to 64 lanes (lane j
 *               takes lane blocks j, j + 64, ...); lane j's codewords (its
 *               lane blocks in order) are contiguous and start at bit
 *               first_bit + lane_off[64 g + j]; lanes follow each other;
 *   stream      ceil(stream_bits / 8) rounded up to 8, plus 64 zero bytes.
 * A lane decodes a known number of symbols from its own bit string, so the
 * decoder needs no per-chunk gaps, no counting pass and no scan.
 *
 * Element kind (v3, u8 at header byte 124): 0 = bf16 words as above; 1 = a
 * plane of 8-bit codes (for instance the integer codes of a quantized model,
 * the LazyWeights page's setting), where every byte is one symbol of the
 * canonical code and there is no sm section (its length is 0).  Version 2
 * containers hold bf16 only (byte 124 is 0).
 *
 * Coder (v3, u8 at header byte 125; version 2: 0): 0 = the canonical Huffman
 * code above; 1 = rANS (pages: "From a Lossless (~1.5:1) Compression
 * Algorithm for Llama2 7B Weights ...", abstract, names ANS; the LazyWeights
 * review compares a Huffman and an rANS decoder).  An rANS container differs
 * from a Huffman one in:
 *   max_code_len = 12 (the frequency precision P);
 *   code_len    replaced by u16 freq[256] (512 bytes): quantized symbol
 *               frequencies summing to 2^12 (all 0 when n_elems = 0);
 *               cum[s] = sum of freq[t] for t < s;
 *   lanes       each non-empty lane is one rANS stream over its symbols in
 *               lane order: its string is the 32-bit final state (high
 *               16 bits first) then the 16-bit renormalisation words in the
 *               order the decoder reads them, all big-endian.  Decoding a
 *               symbol from state x: slot = x mod 2^12, s the symbol with
 *               cum[s] <= slot < cum[s] + freq[s],
 *               x = freq[s] * (x >> 12) + slot - cum[s], and while x < 2^16
 *               x = (x << 16) | next word; the encoder starts (and so the
 *               decoder ends) every lane at x = 2^16.  A lane with no symbols
 *               has an empty string; every lane length, lane offset and
 *               segment bit is a multiple of 16;
 *   segments    as long as possible while they hold at most M elements and
 *               64 * 32 + (sum over their elements of c(freq[s])) / 8 <= B,
 *               with c(f) = ceil(8 (12 - log2 f)) + 1 (an upper bound, in
 *               eighths of a bit, of what one symbol adds to a lane);
 *               B >= 2048 and 97 A <= 8 (B - 2048), so one block always fits.
 *
 * Status codes: 0 on success, a negative WC_ERR_* value otherwise.  No C++
 * exception ever crosses this interface.
 */
#ifndef WC_H
#define WC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define WC_OK                    0
#define WC_ERR_INVALID_ARG      -1   /* NULL pointer, misaligned pointer, bad option          */
#define WC_ERR_NOMEM            -2   /* host or device allocation failed                      */
#define WC_ERR_HIP              -3   /* a HIP runtime call or kernel launch failed             */
#define WC_ERR_UNSUPPORTED      -4   /* valid container the GPU decoder cannot decode (A, M, B) */
#define WC_ERR_SCRATCH          -5   /* work larger than WC_NOALLOC_SCRATCH_BYTES              */
#define WC_ERR_BAD_MAGIC        -10  /* magic, version, flags or a fixed field is wrong       */
#define WC_ERR_TRUNCATED        -11  /* blob shorter than the header or total_bytes           */
#define WC_ERR_SECTION_BOUNDS   -12  /* a section is misaligned, out of order or outside blob */
#define WC_ERR_CODE_LENGTHS     -13  /* a code length > max_code_len, or no symbols for n > 0 */
                                     /* (rANS: a frequency above 2^12)                        */
#define WC_ERR_KRAFT            -14  /* code lengths do not form a complete prefix code       */
                                     /* (rANS: frequencies do not sum to 2^12)                */
#define WC_ERR_GAP              -15  /* a per-chunk gap or a lane offset is out of range       */
#define WC_ERR_GROUP_START      -16  /* group table not increasing, misaligned, too wide, or  */
                                     /* not ending at {n_elems, stream_bits}                  */
#define WC_ERR_STREAM_BITS      -17  /* stream_bits / n_chunks / n_groups / stream_bytes wrong */
#define WC_ERR_TENSOR_TABLE     -18  /* tensor table is not an in-order partition of [0, n)   */

/* ---- host encoder ------------------------------------------------------ */
typedef struct {
    uint32_t max_code_len;      /* 1..24; 0 selects the default: 24 for bf16 weights,   */
                                /* 11 for code planes (wc_encode_u8_host)               */
    uint32_t chunk_bytes;       /* must be 8 (or 0 for the default)                     */
    uint32_t chunks_per_group;  /* G >= 1; 0 selects the default 128.  Any G decodes:   */
                                /* a group wider than 128 chunks takes several passes.  */
    uint32_t n_threads;         /* host threads for encoding; 0 = all hardware threads  */
    uint32_t group_align;       /* A, elements per block: a positive multiple of 8; 0   */
                                /* selects the default 128.  Chunks layout:             */
                                /* A * max_code_len + 63 must not exceed 64 * G.        */
    uint32_t group_max_elems;   /* M, a multiple of A: elements per group at most,      */
                                /* <= 4096; 0 selects the default 4096.                 */
    uint32_t layout;            /* WC_LAYOUT_LANES (0, the default: container v3) or    */
                                /* WC_LAYOUT_CHUNKS (1, container v2)                   */
    uint32_t seg_max_bits;      /* v3: stream bits per segment at most, >= A *          */
                                /* max_code_len and <= 15872 (0: that default).         */
    uint32_t coder;             /* WC_CODER_HUFFMAN (0, the default) or WC_CODER_RANS   */
                                /* (1: lanes layout only; max_code_len is ignored and   */
                                /* 97 A <= 8 (seg_max_bits - 2048) is required)         */
    uint32_t gap_bits;          /* v2: bits per stored gap, 8 (or 0: the default) or 5  */
                                /* (packed; chunks layout only)                         */
} wc_encode_opts;

#define WC_LAYOUT_LANES  0u
#define WC_LAYOUT_CHUNKS 1u
#define WC_CODER_HUFFMAN 0u
#define WC_CODER_RANS    1u

/*
 * wc_encode_host -- offline preparation of one container from n_tensors bf16
 * tensors (the weight-preparation step of the pages: the LazyWeights review,
 * practical implications, needs nothing beyond preparing the weights; Huff-LLM
 * abstract keeps them compressed everywhere).
 *   tensors[k]  host pointer to numels[k] bf16 bit patterns (uint16), k < n_tensors;
 *               may be NULL only when numels[k] == 0.
 *   opts        NULL for defaults.
 *   *blob       receives a library-allocated host buffer of *blob_bytes bytes,
 *               256-byte aligned; release it with wc_free_host.
 * All tensors share one codebook (block-level decode).  The sum of numels
 * must be below 2^40.  Returns WC_ERR_INVALID_ARG for bad arguments,
 * WC_ERR_NOMEM if the buffer cannot be allocated.
 */
int wc_encode_host(const uint16_t* const* tensors, const uint64_t* numels, uint32_t n_tensors,
                   const wc_encode_opts* opts, uint8_t** blob, uint64_t* blob_bytes);

/*
 * wc_encode_u8_host -- the same preparation for planes of 8-bit codes
 * (element kind u8): each byte is a symbol of one shared canonical code; the
 * container is the interleaved-lane layout (opts->layout must be
 * WC_LAYOUT_LANES) with no raw plane.  tensors[k] points to numels[k] bytes.
 * Codes are limited to 11 bits unless opts->max_code_len says otherwise: the
 * GPU decoder's table width, so that no code needs its slower long-code path.
 * Decode with wc_decode_u8_async.
 */
int wc_encode_u8_host(const uint8_t* const* tensors, const uint64_t* numels, uint32_t n_tensors,
                      const wc_encode_opts* opts, uint8_t** blob, uint64_t* blob_bytes);

/* Release a buffer returned by wc_encode_host or wc_encode_u8_host (NULL is ignored). */
void wc_free_host(uint8_t* blob);

/* ---- planning ------------------------------------------------------------ */
typedef struct wc_plan_s wc_plan_t;   /* opaque, immutable after creation */

/*
 * wc_plan -- validate a container held in host memory and prepare decoding on
 * HIP device hip_device (DFloat11 page, abstract, design point (ii): the
 * kernel places every thread's reads and writes through small auxiliary
 * variables, so those variables -- per-chunk gaps or lane offsets, the group
 * table -- are checked here, once, before any kernel trusts them; point (i):
 * the compact decode tables that fit in on-chip memory are built here).
 * Parses and checks every section (each failure has its own WC_ERR_* code:
 * a wrong magic or fixed field, a truncated blob, a section out of bounds, a
 * code length above the limit, an incomplete prefix code, a gap or lane
 * offset out of range, a group table that is not increasing or not closed by
 * {n, stream_bits}, inconsistent stream sizes, a tensor table that is not a
 * partition; WC_ERR_UNSUPPORTED for a valid container the GPU decoder cannot
 * decode), builds the decode tables for the container's codebook on that
 * device (a small plan-owned device buffer, freed by wc_plan_destroy) and
 * chooses the launch configuration.  The host blob is read only during this
 * call; nothing is kept from it.  The device copy of the same bytes that is
 * later passed to wc_decode_async is owned by the caller.  Returns
 * WC_ERR_HIP if the device cannot be used, WC_ERR_NOMEM if the table buffer
 * cannot be allocated; *plan is NULL on any failure.
 */
int wc_plan(const uint8_t* blob_host, uint64_t blob_bytes, int hip_device, wc_plan_t** plan);

/*
 * wc_plan_info -- element count, tensor count and, if the arrays are not
 * NULL, each tensor's element offset and size (arrays of n_tensors entries;
 * call once with NULL arrays to learn n_tensors).  Any output may be NULL.
 */
int wc_plan_info(const wc_plan_t* plan, uint64_t* n_elems, uint32_t* n_tensors,
                 uint64_t* tensor_offsets, uint64_t* tensor_numels);

/*
 * wc_plan_stats -- container statistics and launch configuration: total
 * container bytes, stream bits, number of groups, the index widths of the
 * kernel's two LDS tables (codeword-start table, multi-codeword table), the
 * launch grid (workgroups) and the LDS bytes per workgroup of the container's
 * decode entry point (wc_decode_async for bf16, wc_decode_u8_async for code
 * planes; the fused product launches 8-wave workgroups of its own).  Any
 * output may be NULL.
 */
int wc_plan_stats(const wc_plan_t* plan, uint64_t* container_bytes, uint64_t* stream_bits,
                  uint64_t* n_groups, uint32_t* count_bits, uint32_t* decode_bits, uint32_t* grid,
                  uint32_t* lds_bytes);

/*
 * wc_plan_decode_shape -- how the container's decode entry point
 * (wc_decode_async for bf16, wc_decode_u8_async for code planes) launches:
 * the wavefronts per workgroup, the persistent grid (workgroups) and the
 * kernel launches one call makes.  One call decodes the whole container (the
 * DFloat11 page, abstract, design point (iii)); the plain bf16 decode of a
 * container of more than 40 rounds of its grid (WC_LAUNCH_ROUNDS in the
 * environment of wc_plan overrides the bound; 0: no bound) runs as that many
 * consecutive launches on the same stream, each a span of whole rounds, and
 * code planes always take one.  0 launches for an empty container.  Any
 * output may be NULL; WC_ERR_INVALID_ARG for a NULL plan.
 */
int wc_plan_decode_shape(const wc_plan_t* plan, uint32_t* waves_per_group, uint32_t* grid, uint32_t* launches);

/*
 * wc_plan_format -- the container's version (2: chunks, 3: lanes), element
 * kind (0: bf16, 1: u8) and coder (0: Huffman, 1: rANS).  Any output may be
 * NULL.
 */
int wc_plan_format(const wc_plan_t* plan, uint32_t* version, uint32_t* elem_kind, uint32_t* coder);

/*
 * wc_decode_async -- decode every tensor of the container with one kernel
 * launch on `stream` (a hipStream_t; NULL = the device's null stream):
 * DFloat11 page, abstract, design point (iii), decompresses a whole
 * transformer block at once to cut latency; the output is bit-for-bit the
 * original bf16 words (the same abstract; the Llama2-7B page's abstract:
 * lossless).  A container of more than 40 rounds of the persistent grid's
 * segments (on MI355X about 5 x 10^8 elements; an 8B-shape block is 17
 * rounds) is decoded by consecutive launches of at most 40 rounds each on
 * the same stream (a 70B-shape block: two).
 *   blob_dev  device pointer to the same bytes given to wc_plan, 256-byte aligned;
 *   out_dev   device pointer to n_elems bf16 words (caller-owned), 16-byte
 *             aligned; tensor k is out_dev[tensor_offsets[k] ...].
 * The call returns after the launch; completion is observed by synchronising
 * the stream.  Only launch errors are reported (WC_ERR_HIP); the kernel never
 * writes outside out_dev[0, n_elems), even for a corrupted bit stream.
 * n_elems == 0 is a no-op.  A plan may be used on several streams at once.
 * The current device must be the plan's device.
 */
int wc_decode_async(const wc_plan_t* plan, const void* blob_dev, uint16_t* out_dev, void* stream);

/*
 * wc_decode_u8_async -- the same for a u8-kind container: ONE launch decoding
 * every byte into out_dev (n_elems bytes, 16-byte aligned, caller-owned).
 * WC_ERR_INVALID_ARG for a bf16 container (and wc_decode_async rejects u8
 * containers the same way).
 */
int wc_decode_u8_async(const wc_plan_t* plan, const void* blob_dev, uint8_t* out_dev, void* stream);

/* ---- consumer of decoded weights ------------------------------------------ */
/*
 * wc_gemv_bf16_async -- y = W x for a batch-1 input: the compute kernel that
 * reads decoded weights (the pages decode weights on demand before the
 * inference kernels use them: DFloat11 abstract; LazyWeights review, "Truck
 * packing").  One launch on `stream`.
 *   W     device pointer, rows x cols bf16 bit patterns, row-major, 16-byte
 *         aligned (a tensor view of wc_decode_async's output qualifies when
 *         its element offset is a multiple of 8);
 *   x     device pointer, cols bf16, 16-byte aligned;
 *   y     device pointer, rows float32, written (caller-owned).
 * cols must be a positive multiple of 8.  Accumulation is fp32 with fused
 * multiply-adds in a fixed order, so y is a deterministic function of the
 * bits of W and x.  rows == 0 is a no-op.  Returns WC_ERR_INVALID_ARG for bad
 * sizes or alignment, WC_ERR_HIP if the launch fails.
 */
int wc_gemv_bf16_async(const uint16_t* W, uint32_t rows, uint32_t cols, const uint16_t* x, float* y,
                       void* stream);

/* ---- debug status ---------------------------------------------------------- */
/*
 * wc_plan_debug_status -- a plan made with WC_DEBUG=1 in the environment
 * carries a device status word: the chunks-layout decode kernels (the plain
 * decode and the fused product) check that the codewords starting in each
 * group's bits number exactly its elements (phase 1's count; DFloat11 page,
 * abstract, design point (ii): the auxiliary variables that place each
 * block's output) and OR WC_DEBUG_GROUP_COUNT into the word when they do
 * not: a corrupted stream or group bit offset, which wc_plan's host checks
 * cannot see.  The lanes layout's plain bf16 decode (wc_decode_async) and
 * fused product (wc_decode_gemv_async and its no-allocation variant) check
 * that every lane's decode ends its string where the next lane's begins (the
 * lane offsets are its auxiliary variables; the last lane's string ends with
 * the segment's bits) and ORs WC_DEBUG_LANE_BITS into the word when one does
 * not: with Huffman codes the lane's last table lookup must contain that
 * point (its further symbols belong to the next lane), with rANS the lane
 * must be back in the encoder's initial state 2^16 exactly there.  Code
 * planes leave the word alone.  Plans
 * made without WC_DEBUG launch kernels compiled without the checks.
 *   plan    a plan made with WC_DEBUG=1;
 *   status  receives the word (host pointer);
 *   reset   nonzero: the word is cleared after it is read.
 * Synchronises the plan's device first (every launch that uses the plan has
 * finished).  Returns WC_ERR_INVALID_ARG for a NULL argument or a plan made
 * without WC_DEBUG, WC_ERR_HIP if a HIP call fails.
 */
#define WC_DEBUG_GROUP_COUNT 1u
#define WC_DEBUG_LANE_BITS 2u
int wc_plan_debug_status(const wc_plan_t* plan, uint32_t* status, int reset);

/* ---- measurement ----------------------------------------------------------- */
/*
 * wc_stream_reference_async -- the streaming yardstick for the decode kernels'
 * bandwidth (not a step of the method): reads src_bytes from src once and
 * writes dst_bytes to dst, as a decode of a container of src_bytes into
 * dst_bytes of weights does, with the simplest kernel that does so (one
 * workgroup per 4 KiB of output in index order, one non-temporal 16-byte load
 * and store per lane).  With ns = src_bytes / 16 and nd = dst_bytes / 16,
 * 16-byte output item j is the bitwise NOT of input item
 * min(floor(j * r / 2^32), ns - 1), r = ceil(ns * 2^32 / nd); every input item
 * is read.  One launch on `stream`.
 *   src, dst   device pointers, 16-byte aligned; the caller owns both;
 *   src_bytes  a positive multiple of 16, at most dst_bytes;
 *   dst_bytes  a multiple of 16, below 2^43.
 * Both sizes 0 is a no-op.  Returns WC_ERR_INVALID_ARG for bad sizes or
 * alignment, WC_ERR_HIP if the launch fails.
 */
int wc_stream_reference_async(const void* src, uint64_t src_bytes, void* dst, uint64_t dst_bytes, void* stream);

/*
 * Fused decode -> matrix-vector products: y_k = W_k x_k for consecutive
 * tensors W_k of the container, each seen as a row-major matrix, without
 * writing the decoded weights to memory (the decoded block goes straight to
 * its consumer: Huff-LLM abstract keeps weights compressed up to the compute
 * units; the DFloat11 abstract decodes right before the matrix-vector
 * products of batch-1 inference, one transformer block at a time).
 */
typedef struct {
    uint32_t tensor;     /* tensor index; operand i must be tensor ops[0].tensor + i     */
    uint32_t cols;       /* row length: a multiple of 8, below 2^31, dividing the        */
                         /* tensor's numel (which must be below 2^32) and at least the   */
                         /* container's largest group (group_max_elems always suffices)  */
    const uint16_t* x;   /* device, cols bf16, 16-byte aligned                           */
    float* y;            /* device, numel / cols float32 (written), 4-byte aligned       */
} wc_gemv_operand;

/*
 * wc_decode_gemv_work_bytes -- size of the device work buffer that
 * wc_decode_gemv_async needs for these operands (0 when every tensor is
 * empty).  Validates the operands as wc_decode_gemv_async does, except the
 * device pointers of empty tensors, which are never used.
 */
int wc_decode_gemv_work_bytes(const wc_plan_t* plan, const wc_gemv_operand* ops, uint32_t n_ops,
                              uint64_t* work_bytes);

/*
 * wc_decode_gemv_async -- two launches on `stream`: one decode kernel over
 * the groups covering the n_ops tensors (1..16 consecutive tensors of the
 * container, the first at an element offset that is a multiple of 8), each
 * wave leaving its group's fp32 partial dot products with x (for the first
 * row the group touches and the next) in work_dev, then one kernel adding
 * each row's partials in group order into its y.
 *   blob_dev    as for wc_decode_async;
 *   work_dev    device scratch of at least work_bytes = wc_decode_gemv_work_bytes(...)
 *               bytes, 256-byte aligned, caller-owned, overwritten.
 * Each 8-element block's products are summed in element-pair order by the
 * hardware bf16 dot instruction (each step within 3 * 2^-24 of the sum of
 * its addends' magnitudes), blocks are added to the lane's fp32 partial in
 * order, a fixed butterfly adds the wave's 64 lanes and the rows add group
 * partials in group order: y is a deterministic function of the bits of W
 * and x.  Empty tensors are skipped (their y is not touched).  Returns
 * WC_ERR_INVALID_ARG for bad operands, sizes or alignment, WC_ERR_HIP if a
 * launch fails.
 */
int wc_decode_gemv_async(const wc_plan_t* plan, const void* blob_dev, const wc_gemv_operand* ops, uint32_t n_ops,
                         void* work_dev, uint64_t work_bytes, void* stream);

/*
 * wc_decode_gemv_noalloc_async -- wc_decode_gemv_async for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same launches and results,
 * with the work buffer taken from the library's own static device array of
 * WC_NOALLOC_SCRATCH_BYTES (8 MiB: 8 bytes per group plus 4 per row, enough
 * for a transformer block of about 2.5 G weights, e.g. the 70B shape's
 * 855.6 M in 2 MB).  The caller still owns blob_dev, every x and y.
 * The array lives on every GPU the library runs on until the process ends;
 * its address is looked up on the first call on each device.  The call
 * allocates nothing.  Calls on one GPU share the array: calls that overlap
 * on one GPU (e.g. on two streams) race, so the caller must order them.
 * Returns WC_ERR_SCRATCH when wc_decode_gemv_work_bytes for these operands
 * exceeds WC_NOALLOC_SCRATCH_BYTES, otherwise as wc_decode_gemv_async.
 */
#define WC_NOALLOC_SCRATCH_BYTES (8ull << 20)
int wc_decode_gemv_noalloc_async(const wc_plan_t* plan, const void* blob_dev, const wc_gemv_operand* ops,
                                 uint32_t n_ops, void* stream);

/* Destroy a plan and its device tables (NULL is ignored).  Pending decodes
 * that use the plan must have completed. */
void wc_plan_destroy(wc_plan_t* plan);

/* Static, human-readable text for a status code. */
const char* wc_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* WC_H */
