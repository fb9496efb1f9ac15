/*
 * df11.h -- C ABI of libdf11, an MI355X (gfx950) implementation of the
 * DFloat11 (DF11) weight format: BF16 weights whose 8-bit exponents are
 * Huffman coded while each sign|mantissa byte is stored raw.
 *
 * Source: page "DFloat11: lossless BFloat16 compression" (ai-infrastructure.net).
 *   - "What it is": field split, ~2.6-bit exponent entropy, 10.8-11.1 bits/weight.
 *   - "Architecture": hierarchical 8-bit lookup tables; the two-phase kernel
 *     (phase 1 counts, a block prefix sum gives output offsets, phase 2
 *     decodes again and writes); Gaps (per 8-byte slice, bit offset of the
 *     first code starting in it, 5 bits) and BlockOutputPos (one 32-bit
 *     output index per block); one launch per transformer block.
 *   - "How it works: the core algorithm": Huffman lengths, canonical codes,
 *     codes emitted most significant bit first.
 *   - "References", arXiv v1 note: longest code forced to 32 bits by rebuilding
 *     the tree.
 *
 * Conventions for every call:
 *   - Returns DF11_OK (0) or a negative DF11_ERR_* code; never aborts, never
 *     throws, keeps no global state except a per-device cache of the launch
 *     shape (filled on the first df11_decode on that device).
 *   - The caller allocates and frees every buffer.  Host buffers are plain
 *     memory; device buffers are HIP device pointers.  The library never
 *     allocates device memory.
 *
 * Encoded format (all little-endian; each item is defined bit-exactly so an
 * independent implementation can reproduce it):
 *   stream     Huffman codes back to back from bit 0, each most significant
 *              code bit first.  Stream bit k is bit (k % 8) of byte k / 8.
 *              Zero padded to n_blocks * 512 bytes plus DF11_STREAM_GUARD.
 *   slice      64 stream bits (8 bytes); slice g covers bits [64g, 64g+64).
 *   block      64 slices (512 bytes, 4096 bits) -- one wavefront's work.
 *              n_blocks = ceil(total_bits / 4096).
 *   gaps       for g in [0, 64*n_blocks]: (first code start >= 64g) - 64g,
 *              or 0 when no code starts at or after 64g; always in [0, 31]
 *              because codes are at most 32 bits.  Packed as 5-bit fields,
 *              least significant bit first: field g is bits [5g, 5g+5) of
 *              the gaps buffer (same bit order as the stream).
 *   block_pos  n_blocks + 1 uint32: block_pos[b] = number of codes that start
 *              before bit 4096b; block_pos[n_blocks] = n.
 *   signmant   one byte per weight: (sign << 7) | mantissa.
 *   last_start first bit of the final code (total_bits - its length).
 *   luts       device lookup-table image built from code_len[] alone by
 *              df11_build_luts; its layout is private to this library.
 */
#ifndef DF11_H
#define DF11_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DF11_MAX_CODE_LEN 32
#define DF11_SLICE_BITS 64
#define DF11_BLOCK_SLICES 64
#define DF11_BLOCK_BYTES 512
#define DF11_STREAM_GUARD 16
#define DF11_MAX_TABLES 64
/* Largest n: 2^32 - 64.  block_pos is uint32, and the kernels form output
 * positions up to a block's end plus one 8-word group in 32 bits. */
#define DF11_MAX_N 0xFFFFFFC0ull

enum {
    DF11_OK = 0,
    DF11_ERR_ARG = -1,      /* null pointer, n == 0 or n > DF11_MAX_N, bad limit, misaligned pointer */
    DF11_ERR_BUFSIZE = -2,  /* a caller buffer is smaller than the size df11_encoded_sizes gives */
    DF11_ERR_CODELEN = -3,  /* max_code_len below what the alphabet needs, or above 32 */
    DF11_ERR_TABLES = -4,   /* code tree needs more than DF11_MAX_TABLES 8-bit tables */
    DF11_ERR_FORMAT = -5,   /* descriptor fields inconsistent with each other */
    DF11_ERR_HIP = -6       /* the HIP runtime reported an error at launch */
};

/* Human-readable name of a status code (static string). */
const char *df11_status_string(int status);

/* Exponent histogram of n BF16 words (bit patterns), ADDED to hist[256].
 * Section "How it works", exponent histogram.  n_threads = 0 picks the
 * number of hardware threads.  Errors: ARG. */
int df11_histogram(const uint16_t *bf16, uint64_t n, uint64_t hist[256], uint32_t n_threads);

/* Code book: canonical Huffman code defined by code_len[] alone. */
typedef struct df11_codebook {
    uint8_t code_len[256];   /* 0 = symbol absent, else 1..max_code_len */
    uint32_t code[256];      /* canonical value, most significant bit first */
    uint32_t max_len;        /* longest code */
    uint32_t n_symbols;      /* symbols with a code */
    uint32_t n_tables;       /* 256-entry tables in the 8-bit hierarchy */
    uint32_t lut_bytes;      /* size of the device table image */
    uint32_t limit_rounds;   /* times the length limit rebuilt the tree */
    uint32_t reserved;
} df11_codebook;

/* Huffman lengths from hist (ties broken by count, then by creation order,
 * live symbols numbered in increasing symbol order; one live symbol gets a
 * 1-bit code), limited to max_code_len by repeatedly replacing each nonzero
 * count c with (c + 1) / 2 and rebuilding; canonical values in (length,
 * symbol) order.  Sections "How it works" and "References" (v1 note).
 * Errors: ARG (null, empty histogram), CODELEN, TABLES. */
int df11_build_codebook(const uint64_t hist[256], uint32_t max_code_len, df11_codebook *cb);

/* Device table image (cb->lut_bytes bytes) into lut: the hierarchical 8-bit
 * lookup tables of section "Architecture", then a multi-code decode table
 * derived from them, which the kernel copies to LDS as it is (both follow
 * from code_len[] alone).  Errors: ARG, BUFSIZE. */
int df11_build_luts(const df11_codebook *cb, void *lut, uint64_t lut_cap);

/* Sizes of every encoded array for n weights with histogram hist. */
typedef struct df11_sizes {
    uint64_t n;
    uint64_t total_bits;
    uint64_t last_start;       /* first bit of the final code (df11_encode
                                  fills it; df11_encoded_sizes cannot and
                                  leaves 0) */
    uint64_t stream_bytes;     /* n_blocks * 512 + DF11_STREAM_GUARD */
    uint64_t gaps_bytes;       /* 40 * n_blocks + 8 (5-bit fields, dword padded) */
    uint64_t block_pos_count;  /* n_blocks + 1 */
    uint64_t signmant_bytes;   /* n rounded up to a multiple of 16 */
    uint64_t lut_bytes;
    uint32_t n_blocks;
    uint32_t reserved;
} df11_sizes;

/* Sizes of the encoded arrays (section "Architecture": the code stream cut
 * into 8-byte per-thread slices, one Gaps field per slice and one
 * BlockOutputPos entry per block; section "How it works": the stream holds
 * sum over symbols of count x code length bits), from the histogram alone.
 * last_start depends on the order of the weights and is left 0: take it,
 * with the rest of the sizes, from df11_encode's output.
 * Errors: ARG, FORMAT (hist does not sum to n or holds a symbol without a
 * code). */
int df11_encoded_sizes(const uint64_t hist[256], uint64_t n, const df11_codebook *cb,
                       df11_sizes *out);

/* Encode n BF16 words (host memory).  Section "How it works": each weight is
 * split into its exponent byte and its sign|mantissa byte; the exponent's
 * canonical code is appended to the stream most significant code bit first;
 * the sign|mantissa byte is stored raw.  Section "Architecture": while the
 * codes are emitted, each slice's Gaps field (offset of the first code that
 * starts in it) and each block's BlockOutputPos (index of its first code) are
 * recorded.  Writes stream, packed gaps, block_pos, signmant (padding bytes
 * zeroed) and fills *out.  n_threads = 0 picks the number of hardware
 * threads; the output does not depend on it.
 * Errors: ARG, BUFSIZE, FORMAT (a weight's exponent has no code). */
int df11_encode(const uint16_t *bf16, uint64_t n, const df11_codebook *cb,
                uint8_t *stream, uint64_t stream_cap,
                uint8_t *gaps, uint64_t gaps_cap,
                uint32_t *block_pos, uint64_t block_pos_cap,
                uint8_t *signmant, uint64_t signmant_cap,
                df11_sizes *out, uint32_t n_threads);

/* One encoded tensor resident in device memory.  The *_bytes fields state
 * the sizes of the caller's device buffers; df11_decode checks them against
 * the minimum the format needs. */
typedef struct df11_device_stream {
    const uint8_t *stream;
    const uint8_t *gaps;
    const uint32_t *block_pos;
    const uint8_t *signmant;
    const void *luts;
    uint64_t stream_bytes, gaps_bytes, block_pos_count, signmant_bytes, lut_bytes;
    uint64_t n, total_bits, last_start;
    uint32_t n_blocks, n_tables;
    uint32_t max_len;  /* longest code of the code book (1..32) */
    uint32_t max_groups; /* 0: launch as many workgroups as fit on the GPU at
                            once; otherwise at most this many (rounded down to
                            a multiple of 8, at least 8), leaving compute units
                            to kernels that run alongside on other streams */
    uint32_t *status;  /* optional device word; each block whose decoded
                          count differs from its block_pos range, or whose
                          block_pos range is malformed, adds 1 (the block's
                          output is then left unwritten or wrong) */
} df11_device_stream;

/* Decode on the GPU: out[0..n) = the original BF16 words, bit for bit.
 * The two-phase kernel of section "Architecture", one wavefront per 512-byte
 * block: each lane starts at its slice's Gaps offset and decodes the codes
 * that start in its slice once, into a private LDS staging slot (the number
 * decoded is its count); a wave prefix sum of the counts, offset by the
 * block's BlockOutputPos, gives every lane its output position; the staged
 * exponents move to an LDS tile at those positions (blocks whose lanes hold
 * more than 32 or, short of the block's end, fewer than 3 codes instead
 * decode their slices a second time straight into the tile, the page's own
 * route; a stream whose codes average under 2.51 bits runs with slots of 56
 * codes instead of 32); each exponent is joined with its sign|mantissa byte and the
 * words are written with coalesced 16-byte stores.  Enqueued on hip_stream
 * (a hipStream_t; NULL = the null stream) and returns without waiting.  out
 * must be 16-byte aligned; stream, signmant 8-byte; gaps, block_pos 4-byte.
 * Errors: ARG, BUFSIZE, FORMAT, TABLES, HIP.  A corrupt stream is not
 * detected in general (a flipped bit silently desynchronises the decoder);
 * it never makes the kernel read or write outside the stated buffers. */
int df11_decode(const df11_device_stream *s, uint16_t *out, void *hip_stream);

/* ------------------------------------------------------------------ GEMV */

/* One row-major [rows, cols] matrix of a decoded stream, for the fused GEMV. */
typedef struct df11_gemv_matrix {
    uint64_t offset;   /* index of its first weight in the decoded output */
    uint32_t rows, cols;
    uint32_t x_offset; /* its input is x[x_offset .. x_offset + cols); multiple of 8 */
    uint32_t y_offset; /* its result goes to y[y_offset .. y_offset + rows) */
} df11_gemv_matrix;

#define DF11_GEMV_MAX_MATRICES 16
#define DF11_GEMV_MIN_COLS 2048

/* Bytes of device workspace df11_decode_gemv needs for s: 16 per block (its
 * partial row sums), then 4 per possible row and 4 more (each row's first
 * block; rows hold at least DF11_GEMV_MIN_COLS weights, so there are at most
 * n / DF11_GEMV_MIN_COLS of them). */
uint64_t df11_gemv_workspace_bytes(const df11_device_stream *s);

/* Fused decode and matrix-vector product: for each matrix m,
 * y[y_offset_m + r] = sum_c W_m[r][c] * x[x_offset_m + c] (products of the
 * decoded BF16 weights with the BF16 inputs, exact in fp32, summed in fp32),
 * without writing the BF16 weights anywhere.  This is the decompress-then-matmul step of DF11
 * inference (section "Architecture") at batch 1, with the decompressed block
 * kept on chip.  The n_mats (1..16) matrices must lie end to end in output
 * order from offset 0 and cover all n weights; cols must be a multiple of 8
 * and at least 2048.  x is a device array of BF16 words (16-byte aligned), y
 * a device fp32 array (4-byte aligned); workspace is caller-owned device memory of at least
 * df11_gemv_workspace_bytes(s), 16-byte aligned, overwritten.  Each row's sum
 * is formed in a fixed order (per block, then blocks in stream order), so the
 * result is the same on every run.  Two kernels are enqueued on hip_stream.
 * It is df11_decode_gemm with batch 1.
 * Errors: those of df11_decode, ARG for a matrix list that breaks the rules,
 * BUFSIZE for a short workspace. */
int df11_decode_gemv(const df11_device_stream *s, const df11_gemv_matrix *mats, uint32_t n_mats,
                     const uint16_t *x, float *y, void *workspace, uint64_t workspace_bytes,
                     void *hip_stream);

#define DF11_GEMM_MAX_BATCH 8

/* Bytes of device workspace df11_decode_gemm needs for s at this batch
 * (1..8; 0 for any other batch or a null s): the partial sums of each block
 * for the batch's capacity (1, 2, 4 or 8 vectors: 16, 32, 64 or 112 bytes),
 * then the row table of df11_gemv_workspace_bytes. */
uint64_t df11_gemm_workspace_bytes(const df11_device_stream *s, uint32_t batch);

/* Fused decode and product with `batch` input vectors (1..8): for each vector
 * b < batch and matrix m,
 * y[b * y_stride + y_offset_m + r] = sum_c W_m[r][c] * x[b * x_stride + x_offset_m + c],
 * with the decoded weights used for all vectors while they are on chip (the
 * same decompress-then-matmul step as df11_decode_gemv, at small batch).
 * Strides count elements: x_stride a multiple of 8, below 2^32 and at least
 * the end of every matrix's inputs (max x_offset_m + cols_m); y_stride below
 * 2^32 and at least max y_offset_m + rows_m (both ignored for batch 1).  The
 * matrix rules, alignments, ownership, ordering and errors are those of
 * df11_decode_gemv; the workspace must hold df11_gemm_workspace_bytes(s,
 * batch).  Batches of 1 and 2 run at the decode's occupancy; 3 to 8 at two
 * thirds of it. */
int df11_decode_gemm(const df11_device_stream *s, const df11_gemv_matrix *mats, uint32_t n_mats,
                     const uint16_t *x, uint32_t batch, uint64_t x_stride, float *y,
                     uint64_t y_stride, void *workspace, uint64_t workspace_bytes,
                     void *hip_stream);

/* ------------------------------------------------------------ tiled product
 *
 * The decompress-then-matmul step of DF11 inference (section "Architecture":
 * a transformer block's weights are decompressed just before its matrix
 * products) for 1 to 64 input vectors, on the matrix cores, without writing
 * the BF16 weights anywhere.  The block's matrices are encoded in operand-tile
 * order: each matrix (rows a multiple of 16, cols of 32) is cut into row tiles
 * of 16 rows, each row tile into k-steps of 32 columns, and each k-step's 512
 * weights are stored as 64 groups of 8, group L holding
 * W[16 rt + L % 16][32 ks + 8 (L / 16) + 0..7] (the first operand of a
 * 16x16x32 bf16 matrix instruction, lane by lane).  The permuted words are
 * then encoded with df11_encode as any BF16 tensor (the histogram, and so the
 * code book, does not depend on the order). */

/* out[] = the n words of w[] (row-major matrices laid end to end as mats
 * lists them) in operand-tile order.  Host memory, w != out.  n_threads = 0
 * picks the number of hardware threads.  Errors: ARG (null, n out of range,
 * matrices not end to end from 0 covering n, rows not a multiple of 16 or
 * cols of 32). */
int df11_tile_order(const uint16_t *w, uint64_t n, const df11_gemv_matrix *mats, uint32_t n_mats,
                    uint16_t *out, uint32_t n_threads);

/* Row tiles (segments) of a matrix list: the sum of rows / 16; 0 for a bad
 * list. */
uint64_t df11_tile_segment_count(const df11_gemv_matrix *mats, uint32_t n_mats);

/* Segment table of a tile-order stream (host memory): seg_blk[s] = the block
 * holding the first weight of segment s (segments in matrix order, row
 * tiles in order), and seg_blk[S] = the block holding the last weight,
 * where a block holds the weights [block_pos[b], block_pos[b + 1]).  The
 * product decodes blocks seg_blk[s] .. seg_blk[s + 1] for segment s.
 * seg_cap must be at least df11_tile_segment_count + 1.
 * Errors: ARG, FORMAT (block_pos[0] != 0), BUFSIZE. */
int df11_tile_segments(const uint32_t *block_pos, uint32_t n_blocks, const df11_gemv_matrix *mats,
                       uint32_t n_mats, uint32_t *seg_blk, uint64_t seg_cap);

#define DF11_TILED_MAX_BATCH 64

/* Bytes of device workspace df11_decode_gemm_tiled needs for this matrix list
 * and batch: 0 below 12 vectors; from 12 on, room for the inputs rewritten
 * k-step-major (2 bytes x 16 vectors per group of 16 in the batch x the
 * columns of the distinct input ranges (x_offset, cols)).  0 also for a bad
 * list or batch. */
uint64_t df11_tiled_workspace_bytes(const df11_gemv_matrix *mats, uint32_t n_mats, uint32_t batch);

/* Tiled fused product: for each vector b < batch (1..64) and matrix m,
 * y[b * y_stride + y_offset_m + r] = sum_c W_m[r][c] * x[b * x_stride + x_offset_m + c]
 * from a stream s of the block in operand-tile order, with seg_blk its
 * segment table in device memory (4-byte aligned).  One workgroup per row
 * tile decodes that tile's blocks and multiplies each 512-word operand tile
 * with the matching inputs of 16 vectors at a time (v_mfma_f32_16x16x32_bf16:
 * BF16 products exact in fp32, summed in fp32), its waves' sums added in a
 * fixed order, so the result is the same on every run.  Matrices: 1..16, end
 * to end from offset 0 covering all n weights, rows a multiple of 16, cols of
 * 32, x_offset of 8.  x: BF16 device array, 16-byte aligned; y: fp32 device
 * array, 4-byte aligned; strides in elements as for df11_decode_gemm (a
 * multiple of 8 for x, below 2^32, at least every matrix's end; ignored for
 * batch 1).  workspace: caller-owned device memory of at least
 * df11_tiled_workspace_bytes (16-byte aligned; may be null when that is 0),
 * overwritten: from 12 vectors on, a first kernel copies the inputs there
 * k-step-major ([k-step][vector][32 columns]), so that each wave's loads of
 * one k-step read one contiguous kilobyte.  One or two kernels enqueued on
 * hip_stream.  A block whose decoded count disagrees with block_pos is
 * counted in s->status and left out of the sums.  Errors: those of
 * df11_decode, ARG for a matrix list, batch, stride or workspace pointer that
 * breaks the rules, BUFSIZE for a short workspace. */
int df11_decode_gemm_tiled(const df11_device_stream *s, const df11_gemv_matrix *mats,
                           uint32_t n_mats, const uint32_t *seg_blk, const uint16_t *x,
                           uint32_t batch, uint64_t x_stride, float *y, uint64_t y_stride,
                           void *workspace, uint64_t workspace_bytes, void *hip_stream);

/* Decode of a stream in operand-tile order back to the row-major BF16 words
 * the tile order was taken from (what df11_tile_order was given), for callers
 * that keep only the tile-order encoding and need the weights themselves
 * (more than 64 input vectors, other uses).  The decode is the one of
 * df11_decode (page "DFloat11: lossless BFloat16 compression", sections
 * "Architecture" and "How it works: the core algorithm"); each group of 8
 * decoded words is 8 consecutive columns of one row and goes there with one
 * 16-byte store.  mats, n_mats: as for df11_decode_gemm_tiled (1..16
 * matrices, end to end from 0 over all n words, rows a multiple of 16, cols
 * of 32; x and y offsets ignored).  out: device array of n BF16 words,
 * 16-byte aligned, overwritten.  Corrupt blocks: as df11_decode.  Enqueued
 * on hip_stream.  Errors: those of df11_decode, ARG for a matrix list that
 * breaks the rules. */
int df11_decode_tiled(const df11_device_stream *s, const df11_gemv_matrix *mats, uint32_t n_mats,
                      uint16_t *out, void *hip_stream);

/* Workspace bytes df11_decode_gemm_noalloc can use (32 MiB): enough for
 * batches 1-8 on the 218 M-weight Llama-3.1-8B-shaped block and batches 1-2 on
 * the 856 M-weight Llama-3.3-70B-shaped block. */
#define DF11_NOALLOC_SCRATCH_BYTES (32u << 20)

/* df11_decode_gemm for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as df11_decode_gemm, without the
 * workspace: the library's own static device array of
 * DF11_NOALLOC_SCRATCH_BYTES serves instead (each GPU the library runs on
 * holds one until the process ends; its address is looked up on the first
 * call on each device).  It allocates nothing and frees nothing.  A stream
 * and batch whose workspace (df11_gemm_workspace_bytes) exceeds that size is
 * refused with BUFSIZE before any device call.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  Nothing in the array
 * needs to start at zero: each call writes every entry it reads for intact
 * blocks. */
int df11_decode_gemm_noalloc(const df11_device_stream *s, const df11_gemv_matrix *mats,
                             uint32_t n_mats, const uint16_t *x, uint32_t batch,
                             uint64_t x_stride, float *y, uint64_t y_stride, void *hip_stream);

/* ------------------------------------------------------- measurement aid */

/* Streaming ceiling: a kernel that moves the bytes of one df11_decode launch
 * and does no decoding, as the floor its time is measured against (not part
 * of the decode path).  Reads a[0..n) with one 8-byte load per 8 words (as
 * the decode reads sign|mantissa bytes) and b[0..b_bytes) with 16-byte loads
 * spread evenly over those groups; writes out[0..n) (n 16-bit words) with one
 * 16-byte store per 8 words, a wave's loads of 128 consecutive groups issued
 * before their stores.  n a multiple of 8; b_bytes a multiple of 16; a
 * 8-byte, b and out 16-byte aligned device pointers.  Grid: 3 workgroups of
 * 512 threads per compute unit (the decode's), at most max_groups if
 * nonzero.  The words written are a function of the bytes
 * read, of no use beyond that.  Enqueued on hip_stream.  Errors: ARG, HIP. */
int df11_stream_ceiling(const uint8_t *a, const uint8_t *b, uint64_t b_bytes, uint16_t *out,
                        uint64_t n, uint32_t max_groups, void *hip_stream);

/* Plain streams (measurement aids, not part of the decode path): the GPU's
 * own read-only, write-only and copy rates, beside which the decode and the
 * ceiling above are read.  bytes: a multiple of 16, above 0; src/dst: 16-byte
 * aligned device pointers; 16-byte accesses, four in flight per thread, grid
 * workgroups of 256 threads (0: 128 per compute unit; never more than the
 * bytes need).  Enqueued on hip_stream.  Errors: ARG, HIP, and BUFSIZE for a
 * short out.
 *   df11_stream_read: reads src[0..bytes); thread t writes to out[t] the XOR
 *     of the 32-bit words it read (so the XOR of all of out is the XOR of all
 *     of src); out: device array of out_count uint32, at least
 *     df11_stream_read_slots(bytes, grid) (0 for bad arguments).
 *   df11_stream_write: fills dst[0..bytes) with 16-byte records {value,
 *     value, value, record index (low 32 bits)}.
 *   df11_stream_copy: dst[0..bytes) = src[0..bytes) (not overlapping). */
uint32_t df11_stream_read_slots(uint64_t bytes, uint32_t grid);
int df11_stream_read(const void *src, uint64_t bytes, uint32_t *out, uint64_t out_count,
                     uint32_t grid, void *hip_stream);
int df11_stream_write(void *dst, uint64_t bytes, uint32_t value, uint32_t grid, void *hip_stream);
int df11_stream_copy(const void *src, void *dst, uint64_t bytes, uint32_t grid, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* DF11_H */
