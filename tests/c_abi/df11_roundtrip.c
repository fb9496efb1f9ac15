/* A C program that uses libdf11 through its C ABI alone (include/df11.h and
 * the HIP runtime's C API; no Python, no torch): it encodes seeded synthetic
 * BF16 weights on the host, copies the arrays to the GPU, decodes them with
 * df11_decode and checks the result against the original words bit for bit.
 * With --host it stops after the host encode (for machines without a GPU).
 *
 *   df11_roundtrip [--host] [n] [seed]
 *
 * Exit status 0 when every check passes.  The input is N(0, 0.02)-like BF16
 * (a sum of four uniforms, rounded to nearest even), with every 997th weight
 * scaled by 2^-20 and every 4093rd one replaced by a special word. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "df11.h"

static uint64_t rng;
static uint32_t next_u32(void) { /* xorshift64* */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (uint32_t)((rng * 0x2545F4914F6CDD1Dull) >> 32);
}
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static uint16_t weight(uint64_t i) {
    static const uint16_t special[4] = {0x0000, 0x8000, 0x7F80, 0x0001};
    if (i % 4093 == 4092) return special[(i / 4093) % 4];
    float s = 0.0f;
    for (int k = 0; k < 4; ++k) s += (float)next_u32() * (1.0f / 4294967296.0f);
    float v = (s - 2.0f) * 0.0346f; /* variance 4/12, scaled to sigma ~0.02 */
    if (i % 997 == 996) v *= 1.0f / 1048576.0f;
    return to_bf16(v);
}

#define CHECK(call)                                                                      \
    do {                                                                                 \
        int st_ = (call);                                                                \
        if (st_ != DF11_OK) {                                                            \
            fprintf(stderr, "%s failed: %s\n", #call, df11_status_string(st_));          \
            return 1;                                                                    \
        }                                                                                \
    } while (0)
#define HIP(call)                                                                        \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));            \
            return 1;                                                                    \
        }                                                                                \
    } while (0)

int main(int argc, char **argv) {
    int host_only = 0, a = 1;
    if (a < argc && strcmp(argv[a], "--host") == 0) host_only = 1, ++a;
    const uint64_t n = a < argc ? strtoull(argv[a++], NULL, 10) : 1000003ull;
    rng = (a < argc ? strtoull(argv[a++], NULL, 10) : 7ull) * 0x9E3779B97F4A7C15ull + 1;
    if (n == 0) return 1;

    uint16_t *w = malloc(n * sizeof *w);
    if (!w) return 1;
    for (uint64_t i = 0; i < n; ++i) w[i] = weight(i);

    /* host: histogram, code book, table image, sizes, encode */
    uint64_t hist[256] = {0}; /* df11_histogram adds to it */
    CHECK(df11_histogram(w, n, hist, 0));
    df11_codebook cb;
    CHECK(df11_build_codebook(hist, DF11_MAX_CODE_LEN, &cb));
    void *luts = malloc(cb.lut_bytes);
    CHECK(df11_build_luts(&cb, luts, cb.lut_bytes));
    df11_sizes sz;
    CHECK(df11_encoded_sizes(hist, n, &cb, &sz));
    uint8_t *stream = malloc(sz.stream_bytes), *gaps = malloc(sz.gaps_bytes);
    uint32_t *block_pos = malloc(sz.block_pos_count * sizeof *block_pos);
    uint8_t *signmant = malloc(sz.signmant_bytes);
    if (!luts || !stream || !gaps || !block_pos || !signmant) return 1;
    df11_sizes got;
    CHECK(df11_encode(w, n, &cb, stream, sz.stream_bytes, gaps, sz.gaps_bytes, block_pos,
                      sz.block_pos_count, signmant, sz.signmant_bytes, &got, 0));
    if (got.total_bits != sz.total_bits || got.n_blocks != sz.n_blocks || block_pos[0] != 0 ||
        block_pos[sz.n_blocks] != n) {
        fprintf(stderr, "encode disagrees with its sizes\n");
        return 1;
    }
    printf("encoded n=%llu: %.4f bits/weight, max code %u bits, %u tables, %u blocks\n",
           (unsigned long long)n, 8.0 + (double)sz.total_bits / (double)n, cb.max_len, cb.n_tables,
           sz.n_blocks);
    if (host_only) {
        printf("df11_roundtrip host ok\n");
        return 0;
    }

    /* device: copy the arrays, decode, compare */
    df11_device_stream ds;
    memset(&ds, 0, sizeof ds);
    void *d_stream, *d_gaps, *d_pos, *d_sm, *d_luts, *d_out, *d_status;
    HIP(hipMalloc(&d_stream, sz.stream_bytes));
    HIP(hipMalloc(&d_gaps, sz.gaps_bytes));
    HIP(hipMalloc(&d_pos, sz.block_pos_count * 4));
    HIP(hipMalloc(&d_sm, sz.signmant_bytes));
    HIP(hipMalloc(&d_luts, cb.lut_bytes));
    HIP(hipMalloc(&d_out, (n + 8) * 2));
    HIP(hipMalloc(&d_status, 4));
    HIP(hipMemcpy(d_stream, stream, sz.stream_bytes, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_gaps, gaps, sz.gaps_bytes, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_pos, block_pos, sz.block_pos_count * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_sm, signmant, sz.signmant_bytes, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_luts, luts, cb.lut_bytes, hipMemcpyHostToDevice));
    HIP(hipMemset(d_out, 0x55, (n + 8) * 2));
    HIP(hipMemset(d_status, 0, 4));
    ds.stream = d_stream;
    ds.gaps = d_gaps;
    ds.block_pos = d_pos;
    ds.signmant = d_sm;
    ds.luts = d_luts;
    ds.stream_bytes = sz.stream_bytes;
    ds.gaps_bytes = sz.gaps_bytes;
    ds.block_pos_count = sz.block_pos_count;
    ds.signmant_bytes = sz.signmant_bytes;
    ds.lut_bytes = cb.lut_bytes;
    ds.n = n;
    ds.total_bits = got.total_bits;
    ds.last_start = got.last_start; /* known only once encoded (the final code's start) */
    ds.n_blocks = got.n_blocks;
    ds.n_tables = cb.n_tables;
    ds.max_len = cb.max_len;
    ds.status = d_status;

    /* a misaligned output is refused before any launch */
    if (df11_decode(&ds, (uint16_t *)((char *)d_out + 2), NULL) != DF11_ERR_ARG) {
        fprintf(stderr, "a misaligned output was not refused\n");
        return 1;
    }
    CHECK(df11_decode(&ds, d_out, NULL));
    HIP(hipDeviceSynchronize());
    uint16_t *back = malloc((n + 8) * 2);
    uint32_t status = 1;
    HIP(hipMemcpy(back, d_out, (n + 8) * 2, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
    uint64_t bad = 0;
    for (uint64_t i = 0; i < n; ++i) bad += back[i] != w[i];
    for (uint64_t i = n; i < n + 8; ++i) bad += back[i] != 0x5555;
    printf("decoded n=%llu: %llu words differ, status %u\n", (unsigned long long)n,
           (unsigned long long)bad, status);
    if (bad || status) return 1;
    printf("df11_roundtrip ok\n");
    return 0;
}
