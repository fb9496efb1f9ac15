// Host-side driver for sanitizer builds (AddressSanitizer + UndefinedBehavior-
// Sanitizer, and ThreadSanitizer): runs the host half of libdf11 (histogram,
// code book, tables, sizes, the threaded encoder, the tile layout helpers)
// and the CPU oracle over small seeded inputs, checks that the two agree and
// that the encoder's output does not depend on its thread count, and walks
// the documented error paths.  It is built by tests/test_sanitizers.py with
// g++ from the sources (no GPU code).  Exit status 0 means every check held;
// the sanitizers abort on their own findings.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "df11.h"

// the oracle's C entry points (oracle/df11_oracle.c)
extern "C" {
int orc_split(const uint16_t *w, uint64_t n, uint8_t *expo, uint8_t *signmant);
int orc_join(const uint8_t *expo, const uint8_t *signmant, uint64_t n, uint16_t *w);
int orc_histogram(const uint8_t *expo, uint64_t n, uint64_t hist[256]);
int orc_limited_lengths(const uint64_t hist[256], uint32_t max_len, uint8_t len[256],
                        uint32_t *rounds);
int64_t orc_encode(const uint8_t *expo, uint64_t n, const uint8_t len[256], uint8_t *stream,
                   uint64_t stream_cap);
int orc_decode(const uint8_t *stream, uint64_t avail_bits, uint64_t start_bit, uint64_t count,
               const uint8_t len[256], uint8_t *out, uint64_t *end_bit);
int orc_aux(const uint8_t *expo, uint64_t n, const uint8_t len[256], uint32_t *gaps,
            uint64_t n_gaps, uint32_t *block_pos, uint64_t n_bp);
int orc_pack_gaps(const uint32_t *gaps, uint64_t n_gaps, uint8_t *packed, uint64_t packed_cap);
}

static int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

// seeded inputs (xorshift64*): BF16 words of a few kinds
struct Rng {
    uint64_t s;
    uint64_t next() {
        s ^= s >> 12, s ^= s << 25, s ^= s >> 27;
        return s * 0x2545F4914F6CDD1Dull;
    }
};

static std::vector<uint16_t> make_words(uint64_t n, uint64_t seed, int kind) {
    Rng r{seed * 0x9E3779B97F4A7C15ull + 1};
    std::vector<uint16_t> w(n);
    for (uint64_t i = 0; i < n; ++i) {
        const uint64_t v = r.next();
        uint32_t e;
        if (kind == 0) {  // narrow, bell-shaped exponents around 2^-6
            const int tri = (int)(v & 7) + (int)((v >> 3) & 7) + (int)((v >> 6) & 7) - 10;
            e = (uint32_t)(121 + tri);
        } else if (kind == 1) {  // one exponent
            e = 120;
        } else if (kind == 2) {  // any 16-bit word
            w[i] = (uint16_t)(v >> 32);
            continue;
        } else {  // geometric: long codes
            e = 121 - (uint32_t)__builtin_ctzll(v | (1ull << 40)) % 34;
        }
        w[i] = (uint16_t)(((v >> 40) & 0x8000u) | (e << 7) | ((v >> 50) & 0x7Fu));
    }
    return w;
}

// Encodes w with the product (n_threads) and returns the arrays.
struct Enc {
    df11_codebook cb;
    df11_sizes sz;
    std::vector<uint8_t> stream, gaps, signmant, luts;
    std::vector<uint32_t> block_pos;
};

static bool product_encode(const std::vector<uint16_t> &w, uint32_t threads, Enc &e) {
    uint64_t hist[256] = {0};
    if (df11_histogram(w.data(), w.size(), hist, threads) != DF11_OK) return false;
    if (df11_build_codebook(hist, DF11_MAX_CODE_LEN, &e.cb) != DF11_OK) return false;
    if (df11_encoded_sizes(hist, w.size(), &e.cb, &e.sz) != DF11_OK) return false;
    e.stream.assign(e.sz.stream_bytes, 0xEE);
    e.gaps.assign(e.sz.gaps_bytes, 0xEE);
    e.signmant.assign(e.sz.signmant_bytes, 0xEE);
    e.block_pos.assign(e.sz.block_pos_count, 0xEEEEEEEEu);
    e.luts.assign(e.cb.lut_bytes, 0xEE);
    if (df11_build_luts(&e.cb, e.luts.data(), e.luts.size()) != DF11_OK) return false;
    df11_sizes out;
    return df11_encode(w.data(), w.size(), &e.cb, e.stream.data(), e.stream.size(), e.gaps.data(),
                       e.gaps.size(), e.block_pos.data(), e.block_pos.size(), e.signmant.data(),
                       e.signmant.size(), &out, threads) == DF11_OK &&
           out.total_bits == e.sz.total_bits;
}

static void check_tensor(uint64_t n, uint64_t seed, int kind) {
    const std::vector<uint16_t> w = make_words(n, seed, kind);
    Enc one, many;
    CHECK(product_encode(w, 1, one));
    CHECK(product_encode(w, 8, many));
    if (failures) return;
    CHECK(one.stream == many.stream && one.gaps == many.gaps && one.block_pos == many.block_pos &&
          one.signmant == many.signmant && one.luts == many.luts);

    // the oracle's encoding of the same words
    std::vector<uint8_t> ex(n), sm(n);
    CHECK(orc_split(w.data(), n, ex.data(), sm.data()) == 0);
    uint64_t oh[256] = {0};
    CHECK(orc_histogram(ex.data(), n, oh) == 0);
    uint8_t len[256];
    uint32_t rounds = 0;
    CHECK(orc_limited_lengths(oh, DF11_MAX_CODE_LEN, len, &rounds) >= 0);
    CHECK(std::memcmp(len, one.cb.code_len, 256) == 0);
    std::vector<uint8_t> ostream(one.sz.stream_bytes, 0);
    const int64_t bits = orc_encode(ex.data(), n, len, ostream.data(), ostream.size());
    CHECK(bits == (int64_t)one.sz.total_bits);
    CHECK(std::memcmp(ostream.data(), one.stream.data(), (size_t)((bits + 7) / 8)) == 0);
    const uint64_t nb = one.sz.n_blocks;
    std::vector<uint32_t> ogaps(64 * nb + 1), obp(nb + 1);
    CHECK(orc_aux(ex.data(), n, len, ogaps.data(), ogaps.size(), obp.data(), obp.size()) == 0);
    CHECK(std::memcmp(obp.data(), one.block_pos.data(), 4 * obp.size()) == 0);
    std::vector<uint8_t> opacked(one.sz.gaps_bytes, 0);
    CHECK(orc_pack_gaps(ogaps.data(), ogaps.size(), opacked.data(), opacked.size()) == 0);
    CHECK(opacked == one.gaps);
    CHECK(std::memcmp(sm.data(), one.signmant.data(), n) == 0);
    // decode the product's stream with the oracle and join
    std::vector<uint8_t> dec(n);
    uint64_t end = 0;
    CHECK(orc_decode(one.stream.data(), one.sz.total_bits, 0, n, one.cb.code_len, dec.data(),
                     &end) == 0);
    CHECK(end == one.sz.total_bits);
    std::vector<uint16_t> back(n);
    CHECK(orc_join(dec.data(), one.signmant.data(), n, back.data()) == 0);
    CHECK(back == w);
}

static void check_tiles() {
    df11_gemv_matrix mats[3] = {{0, 32, 4096, 0, 0}, {32 * 4096, 16, 2048, 4096, 32},
                                {32 * 4096 + 16 * 2048, 48, 1024, 6144, 48}};
    const uint64_t n = 32 * 4096 + 16 * 2048 + 48 * 1024;
    const std::vector<uint16_t> w = make_words(n, 77, 0);
    std::vector<uint16_t> t1(n), t8(n);
    CHECK(df11_tile_order(w.data(), n, mats, 3, t1.data(), 1) == DF11_OK);
    CHECK(df11_tile_order(w.data(), n, mats, 3, t8.data(), 8) == DF11_OK);
    CHECK(t1 == t8);
    Enc e;
    CHECK(product_encode(t1, 8, e));
    const uint64_t segs = df11_tile_segment_count(mats, 3);
    CHECK(segs == 2 + 1 + 3);
    std::vector<uint32_t> seg(segs + 1);
    CHECK(df11_tile_segments(e.block_pos.data(), e.sz.n_blocks, mats, 3, seg.data(), seg.size()) ==
          DF11_OK);
    CHECK(df11_tile_segments(e.block_pos.data(), e.sz.n_blocks, mats, 3, seg.data(), segs) ==
          DF11_ERR_BUFSIZE);
    df11_gemv_matrix bad = mats[1];
    bad.rows = 24;
    CHECK(df11_tile_order(w.data(), 24 * 2048, &bad, 1, t1.data(), 4) == DF11_ERR_ARG);
}

static void check_errors() {
    uint64_t hist[256] = {0};
    df11_codebook cb;
    CHECK(df11_histogram(nullptr, 4, hist, 1) == DF11_ERR_ARG);
    CHECK(df11_build_codebook(hist, 32, &cb) == DF11_ERR_ARG);  // empty histogram
    hist[120] = 10, hist[121] = 5;
    CHECK(df11_build_codebook(hist, 0, &cb) != DF11_OK);
    CHECK(df11_build_codebook(hist, 33, &cb) != DF11_OK);
    CHECK(df11_build_codebook(hist, 32, &cb) == DF11_OK);
    df11_sizes sz;
    CHECK(df11_encoded_sizes(hist, 14, &cb, &sz) == DF11_ERR_FORMAT);  // does not sum to n
    CHECK(df11_encoded_sizes(hist, 15, &cb, &sz) == DF11_OK);
    std::vector<uint8_t> lut(cb.lut_bytes);
    CHECK(df11_build_luts(&cb, lut.data(), lut.size() - 1) == DF11_ERR_BUFSIZE);
    const std::vector<uint16_t> w = make_words(15, 5, 1);  // exponent 120 only
    std::vector<uint8_t> st(sz.stream_bytes), ga(sz.gaps_bytes), smb(sz.signmant_bytes);
    std::vector<uint32_t> bp(sz.block_pos_count);
    df11_sizes out;
    CHECK(df11_encode(w.data(), 15, &cb, st.data(), st.size() - 1, ga.data(), ga.size(), bp.data(),
                      bp.size(), smb.data(), smb.size(), &out, 2) == DF11_ERR_BUFSIZE);
    CHECK(df11_encode(w.data(), 15, &cb, st.data(), st.size(), ga.data(), ga.size(), bp.data(),
                      bp.size(), smb.data(), smb.size(), &out, 2) == DF11_OK);
    CHECK(std::strlen(df11_status_string(DF11_ERR_FORMAT)) > 0);
    CHECK(std::strlen(df11_status_string(-1000)) > 0);
}

int main() {
    const uint64_t sizes[] = {1, 2, 63, 64, 65, 4097, 100003};
    for (uint64_t n : sizes)
        for (int kind = 0; kind < 4; ++kind) check_tensor(n, n + 17 * kind, kind);
    check_tensor(1 << 20, 3, 0);  // enough for every encoder thread to own a range
    check_tensor(1 << 20, 4, 3);
    check_tiles();
    check_errors();
    std::printf("sanitizer driver: %d failed checks\n", failures);
    return failures ? 1 : 0;
}
