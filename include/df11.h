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
#define DF11_MAX_N 0xFFFFFFFFull /* n must be below 2^32: block_pos is uint32 */

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
    uint64_t last_start;       /* first bit of the final code */
    uint64_t stream_bytes;     /* n_blocks * 512 + DF11_STREAM_GUARD */
    uint64_t gaps_bytes;       /* 40 * n_blocks + 8 (5-bit fields, dword padded) */
    uint64_t block_pos_count;  /* n_blocks + 1 */
    uint64_t signmant_bytes;   /* n rounded up to a multiple of 16 */
    uint64_t lut_bytes;
    uint32_t n_blocks;
    uint32_t reserved;
} df11_sizes;

/* Errors: ARG, FORMAT (hist does not sum to n or holds a symbol without a
 * code). */
int df11_encoded_sizes(const uint64_t hist[256], uint64_t n, const df11_codebook *cb,
                       df11_sizes *out);

/* Encode n BF16 words (host memory).  Writes stream, packed gaps, block_pos,
 * signmant (padding bytes zeroed) and fills *out.  n_threads = 0 picks the
 * number of hardware threads; the output does not depend on it.
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
 * Two-phase wave-per-block decode (section "Architecture", two-phase kernel):
 * per 64-bit slice, count codes; wave prefix sum of the counts; decode again
 * into an LDS tile; merge each exponent with its sign|mantissa byte; write
 * coalesced 16-byte stores.  Enqueued on hip_stream (a hipStream_t; NULL =
 * the null stream) and returns without waiting.  out must be 16-byte
 * aligned; stream, signmant 8-byte; gaps, block_pos 4-byte.
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

#ifdef __cplusplus
}
#endif

#endif /* DF11_H */
