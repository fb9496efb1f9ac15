/*
 * df11_oracle.c -- a plain, slow CPU model of the DFloat11 (DF11) exponent
 * codec, used to check the product library bit for bit.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or constant generator with the product (libdf11); the
 * two meet only in the byte layout of the encoded arrays, which both sides
 * implement from the same written description.
 *
 * What it follows (page "DFloat11: lossless BFloat16 compression",
 * ai-infrastructure.net):
 *   - "What it is": a BF16 word is 1 sign, 8 exponent and 7 mantissa bits;
 *     the exponent byte is Huffman coded, sign and mantissa are kept as one
 *     raw byte per weight.
 *   - "How it works: the core algorithm": Huffman code lengths from the
 *     exponent histogram with ties broken by (count, creation order), a single
 *     live symbol gets a 1-bit code; canonical code values assigned in
 *     (length, symbol) order; codes written most significant bit first;
 *     decoding from a known start offset gives the same symbols as a serial
 *     decode.
 *   - "Architecture", two-phase kernel paragraph: Gaps = per 8-byte slice,
 *     the bit offset of the first code that starts inside it (0..31, 5 bits);
 *     BlockOutputPos = one 32-bit output index per thread block.
 *   - "References", note on arXiv v1 section 3.3.1: the maximum code length
 *     is forced to 32 by rebuilding the tree.
 *
 * Readings where the page is silent (each is listed in the design notes):
 *   - Length limit: while the longest code exceeds the limit, every nonzero
 *     count c becomes (c + 1) / 2 (integer division) and the tree is rebuilt.
 *     Parity unpinned for the exact lengths when the limit binds: the page
 *     fixes no rule, so only invariants pin them (longest code within the
 *     limit, Kraft equality, cost between the unlimited and the brute-force
 *     limited optimum, plain Huffman when the limit does not bind).
 *   - Packed bit order: stream bit k is bit (k mod 8) of byte k / 8 (least
 *     significant bit first inside a byte; the page keeps an unpacked array).
 *   - A slice is 64 bits; a block is 64 slices (4096 bits, 512 bytes).
 *     gap[g] = (first code start >= 64 g) - 64 g, or 0 when no code starts at
 *     or after bit 64 g.  block_pos[b] = number of codes that start before bit
 *     4096 b (so the last entry, one past the final block, is n).
 *   - Gaps are packed as 5-bit fields, least significant bit first:
 *     field g occupies packed bits 5g .. 5g+4, same bit order as the stream.
 *
 * Every routine below works one symbol or one bit at a time on purpose.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG -1
#define ORC_ERR_BUF -2
#define ORC_ERR_LIMIT -3
#define ORC_ERR_STREAM -4

/* ---------------------------------------------------------------- fields */

/* BF16 word -> (exponent byte, sign|mantissa byte).  "What it is": 1 sign bit
 * (bit 15), 8 exponent bits (14..7), 7 mantissa bits (6..0); the raw byte
 * keeps the sign in its top bit and the mantissa below it. */
int orc_split(const uint16_t *w, uint64_t n, uint8_t *expo, uint8_t *signmant)
{
    if (!w || !expo || !signmant) return ORC_ERR_ARG;
    for (uint64_t i = 0; i < n; i++) {
        unsigned word = w[i];
        unsigned sign = (word >> 15) & 1u;
        unsigned exponent = (word >> 7) & 0xFFu;
        unsigned mantissa = word & 0x7Fu;
        expo[i] = (uint8_t)exponent;
        signmant[i] = (uint8_t)((sign << 7) | mantissa);
    }
    return ORC_OK;
}

/* Inverse of orc_split. */
int orc_join(const uint8_t *expo, const uint8_t *signmant, uint64_t n, uint16_t *w)
{
    if (!w || !expo || !signmant) return ORC_ERR_ARG;
    for (uint64_t i = 0; i < n; i++) {
        unsigned sign = (signmant[i] >> 7) & 1u;
        unsigned mantissa = signmant[i] & 0x7Fu;
        unsigned exponent = expo[i];
        w[i] = (uint16_t)((sign << 15) | (exponent << 7) | mantissa);
    }
    return ORC_OK;
}

int orc_histogram(const uint8_t *expo, uint64_t n, uint64_t hist[256])
{
    if (!expo || !hist) return ORC_ERR_ARG;
    for (int s = 0; s < 256; s++) hist[s] = 0;
    for (uint64_t i = 0; i < n; i++) hist[expo[i]]++;
    return ORC_OK;
}

/* ------------------------------------------------------------- lengths */

/* Huffman's procedure, done naively.  Every live symbol (count > 0) starts
 * as its own group; groups are numbered 0..k-1 in increasing symbol order and
 * merged groups take the next unused number.  Each round finds the two groups
 * that are smallest by (count, number), adds one bit to the code of every
 * symbol in either group, and replaces the pair with one group holding the
 * summed count.  With a single live symbol its code is 1 bit long.
 * Returns the number of live symbols (0 if none). */
int orc_huffman_lengths(const uint64_t hist[256], uint8_t len[256])
{
    uint64_t gcount[512];
    int galive[512];
    int group_of[256];
    int ngroups = 0, live = 0;

    if (!hist || !len) return ORC_ERR_ARG;
    for (int s = 0; s < 256; s++) {
        len[s] = 0;
        group_of[s] = -1;
        if (hist[s] > 0) {
            group_of[s] = ngroups;
            gcount[ngroups] = hist[s];
            galive[ngroups] = 1;
            ngroups++;
            live++;
        }
    }
    if (live == 0) return 0;
    if (live == 1) {
        for (int s = 0; s < 256; s++)
            if (hist[s] > 0) len[s] = 1;
        return 1;
    }
    for (int remaining = live; remaining > 1; remaining--) {
        int a = -1, b = -1;
        /* smallest by (count, number): numbers increase with the index */
        for (int g = 0; g < ngroups; g++) {
            if (!galive[g]) continue;
            if (a < 0 || gcount[g] < gcount[a]) a = g;
        }
        for (int g = 0; g < ngroups; g++) {
            if (!galive[g] || g == a) continue;
            if (b < 0 || gcount[g] < gcount[b]) b = g;
        }
        int merged = ngroups++;
        gcount[merged] = gcount[a] + gcount[b];
        galive[merged] = 1;
        galive[a] = 0;
        galive[b] = 0;
        for (int s = 0; s < 256; s++) {
            if (group_of[s] == a || group_of[s] == b) {
                len[s] = (uint8_t)(len[s] + 1);
                group_of[s] = merged;
            }
        }
    }
    return live;
}

/* Length-limited variant (reading of "forced to 32 by rebuilding the tree"):
 * rebuild with every nonzero count replaced by (count + 1) / 2 until the
 * longest code fits.  *rounds receives the number of rebuilds. */
int orc_limited_lengths(const uint64_t hist[256], uint32_t max_len, uint8_t len[256],
                        uint32_t *rounds)
{
    uint64_t c[256];
    int live = 0;

    if (!hist || !len || max_len < 1) return ORC_ERR_ARG;
    for (int s = 0; s < 256; s++) {
        c[s] = hist[s];
        if (c[s] > 0) live++;
    }
    /* smallest limit that can hold `live` codes in a prefix code */
    uint32_t need = 0;
    while (need < 9 && (1u << need) < (uint32_t)live) need++;
    if (live > 1 && max_len < need) return ORC_ERR_LIMIT;

    for (uint32_t r = 0;; r++) {
        int got = orc_huffman_lengths(c, len);
        if (got < 0) return got;
        uint32_t longest = 0;
        for (int s = 0; s < 256; s++)
            if (len[s] > longest) longest = len[s];
        if (longest <= max_len) {
            if (rounds) *rounds = r;
            return got;
        }
        for (int s = 0; s < 256; s++)
            if (c[s] > 0) c[s] = (c[s] + 1) / 2;
    }
}

/* Canonical code values: visit symbols in (length, symbol) order; before each
 * one, shift the running value left by the growth in length; give it the
 * value; then add one. */
int orc_canonical_codes(const uint8_t len[256], uint32_t code[256])
{
    if (!len || !code) return ORC_ERR_ARG;
    for (int s = 0; s < 256; s++) code[s] = 0;
    uint64_t value = 0;
    uint32_t prev = 0;
    for (uint32_t L = 1; L <= 255; L++) {
        for (int s = 0; s < 256; s++) {
            if (len[s] != L) continue;
            if (L > 32) return ORC_ERR_LIMIT;
            value <<= (L - prev);
            prev = L;
            code[s] = (uint32_t)value;
            value += 1;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------ bit I/O */

static int get_bit(const uint8_t *stream, uint64_t avail_bits, uint64_t k)
{
    if (k >= avail_bits) return 0; /* past the data: zero padding */
    return (stream[k >> 3] >> (k & 7)) & 1;
}

static void put_bit(uint8_t *stream, uint64_t k, int bit)
{
    if (bit) stream[k >> 3] |= (uint8_t)(1u << (k & 7));
}

/* Write every exponent's code, most significant code bit first, back to back
 * from bit 0.  The buffer is cleared first.  Returns the number of bits
 * written, or a negative status. */
int64_t orc_encode(const uint8_t *expo, uint64_t n, const uint8_t len[256],
                   uint8_t *stream, uint64_t stream_cap)
{
    uint32_t code[256];
    if (!expo || !len || !stream) return ORC_ERR_ARG;
    int st = orc_canonical_codes(len, code);
    if (st != ORC_OK) return st;
    uint64_t bits = 0;
    for (uint64_t i = 0; i < n; i++) {
        if (len[expo[i]] == 0) return ORC_ERR_ARG; /* symbol without a code */
        bits += len[expo[i]];
    }
    if ((bits + 7) / 8 > stream_cap) return ORC_ERR_BUF;
    memset(stream, 0, stream_cap);
    uint64_t pos = 0;
    for (uint64_t i = 0; i < n; i++) {
        uint32_t L = len[expo[i]];
        uint32_t c = code[expo[i]];
        for (uint32_t j = 0; j < L; j++) {
            int bit = (int)((c >> (L - 1 - j)) & 1u);
            put_bit(stream, pos++, bit);
        }
    }
    return (int64_t)pos;
}

/* ------------------------------------------------------------- decoding */

/* Binary code tree built from the canonical codes: node 0 is the root;
 * child[node][bit] is a node index or -1; leaf_sym >= 0 marks a leaf. */
typedef struct {
    int child[512][2];
    int leaf_sym[512];
    int nodes;
} orc_tree;

static int build_tree(const uint8_t len[256], orc_tree *t)
{
    uint32_t code[256];
    int st = orc_canonical_codes(len, code);
    if (st != ORC_OK) return st;
    t->nodes = 1;
    t->child[0][0] = t->child[0][1] = -1;
    t->leaf_sym[0] = -1;
    for (int s = 0; s < 256; s++) {
        uint32_t L = len[s];
        if (L == 0) continue;
        int node = 0;
        for (uint32_t j = 0; j < L; j++) {
            int bit = (int)((code[s] >> (L - 1 - j)) & 1u);
            if (t->leaf_sym[node] >= 0) return ORC_ERR_STREAM; /* not prefix free */
            if (t->child[node][bit] < 0) {
                if (t->nodes >= 512) return ORC_ERR_STREAM;
                int fresh = t->nodes++;
                t->child[fresh][0] = t->child[fresh][1] = -1;
                t->leaf_sym[fresh] = -1;
                t->child[node][bit] = fresh;
            }
            node = t->child[node][bit];
        }
        if (t->leaf_sym[node] >= 0 || t->child[node][0] >= 0 || t->child[node][1] >= 0)
            return ORC_ERR_STREAM;
        t->leaf_sym[node] = s;
    }
    return ORC_OK;
}

/* Walk the tree one bit at a time from start_bit for exactly `count`
 * symbols (bits past avail_bits read as zero).  *end_bit receives the bit
 * after the last symbol. */
int orc_decode(const uint8_t *stream, uint64_t avail_bits, uint64_t start_bit, uint64_t count,
               const uint8_t len[256], uint8_t *out, uint64_t *end_bit)
{
    orc_tree *t;
    if (!stream || !len || (!out && count)) return ORC_ERR_ARG;
    t = (orc_tree *)malloc(sizeof(orc_tree));
    if (!t) return ORC_ERR_BUF;
    int st = build_tree(len, t);
    if (st != ORC_OK) { free(t); return st; }
    uint64_t pos = start_bit;
    for (uint64_t i = 0; i < count; i++) {
        int node = 0;
        /* a single-symbol code has only the child reached by bit 0 */
        while (t->leaf_sym[node] < 0) {
            int bit = get_bit(stream, avail_bits, pos++);
            node = t->child[node][bit];
            if (node < 0) { free(t); return ORC_ERR_STREAM; }
        }
        out[i] = (uint8_t)t->leaf_sym[node];
    }
    if (end_bit) *end_bit = pos;
    free(t);
    return ORC_OK;
}

/* Decode every code whose first bit lies in [start_bit, stop_bit), assuming
 * start_bit is a code boundary.  Returns the number of symbols (at most
 * out_cap), or a negative status. */
int64_t orc_decode_range(const uint8_t *stream, uint64_t avail_bits, uint64_t start_bit,
                         uint64_t stop_bit, const uint8_t len[256], uint8_t *out, uint64_t out_cap)
{
    orc_tree *t;
    if (!stream || !len) return ORC_ERR_ARG;
    t = (orc_tree *)malloc(sizeof(orc_tree));
    if (!t) return ORC_ERR_BUF;
    int st = build_tree(len, t);
    if (st != ORC_OK) { free(t); return st; }
    uint64_t pos = start_bit;
    int64_t k = 0;
    while (pos < stop_bit) {
        int node = 0;
        while (t->leaf_sym[node] < 0) {
            int bit = get_bit(stream, avail_bits, pos++);
            node = t->child[node][bit];
            if (node < 0) { free(t); return ORC_ERR_STREAM; }
        }
        if ((uint64_t)k >= out_cap) { free(t); return ORC_ERR_BUF; }
        if (out) out[k] = (uint8_t)t->leaf_sym[node];
        k++;
    }
    free(t);
    return k;
}

/* ------------------------------------------------ auxiliary arrays */

/* Gaps and block output positions by their definitions (see header), from
 * the code start offsets of the exponent sequence.  gaps has n_gaps entries
 * (slice g covers bits 64g..64g+63); block_pos has n_bp entries (block b
 * starts at bit 4096 b). */
int orc_aux(const uint8_t *expo, uint64_t n, const uint8_t len[256],
            uint32_t *gaps, uint64_t n_gaps, uint32_t *block_pos, uint64_t n_bp)
{
    if (!expo || !len || !gaps || !block_pos) return ORC_ERR_ARG;
    uint64_t next_g = 0, next_b = 0;
    uint64_t start = 0;
    for (uint64_t i = 0; i < n; i++) {
        if (len[expo[i]] == 0) return ORC_ERR_ARG;
        /* the first code start at or after 64 g is this one for every slice
           g not yet given a gap with 64 g <= start */
        while (next_g < n_gaps && 64 * next_g <= start) {
            gaps[next_g] = (uint32_t)(start - 64 * next_g);
            next_g++;
        }
        while (next_b < n_bp && 4096 * next_b <= start) {
            block_pos[next_b] = (uint32_t)i; /* codes before this one started earlier */
            next_b++;
        }
        start += len[expo[i]];
    }
    while (next_g < n_gaps) gaps[next_g++] = 0;
    while (next_b < n_bp) block_pos[next_b++] = (uint32_t)n;
    return ORC_OK;
}

/* 5-bit fields, least significant bit first, into a zeroed buffer. */
int orc_pack_gaps(const uint32_t *gaps, uint64_t n_gaps, uint8_t *packed, uint64_t packed_cap)
{
    if (!gaps || !packed) return ORC_ERR_ARG;
    if ((5 * n_gaps + 7) / 8 > packed_cap) return ORC_ERR_BUF;
    memset(packed, 0, packed_cap);
    for (uint64_t g = 0; g < n_gaps; g++) {
        if (gaps[g] > 31) return ORC_ERR_ARG;
        for (int j = 0; j < 5; j++)
            put_bit(packed, 5 * g + (uint64_t)j, (int)((gaps[g] >> j) & 1u));
    }
    return ORC_OK;
}

/* Number of 256-entry tables in the page's 8-bit hierarchy: one root, plus
 * one table per distinct 8-, 16- and 24-bit prefix of codes longer than that
 * prefix ("Architecture", hierarchical lookup tables). */
int orc_count_subtables(const uint8_t len[256], uint32_t chunk)
{
    uint32_t code[256];
    if (!len || chunk < 1 || chunk > 16) return ORC_ERR_ARG;
    if (orc_canonical_codes(len, code) != ORC_OK) return ORC_ERR_LIMIT;
    int tables = 1;
    for (uint32_t depth = chunk; depth < 32; depth += chunk) {
        uint32_t seen[256];
        int nseen = 0;
        for (int s = 0; s < 256; s++) {
            if (len[s] <= depth) continue;
            uint32_t prefix = code[s] >> (len[s] - depth);
            int dup = 0;
            for (int k = 0; k < nseen; k++)
                if (seen[k] == prefix) dup = 1;
            if (!dup) seen[nseen++] = prefix;
        }
        tables += nseen;
    }
    return tables;
}
