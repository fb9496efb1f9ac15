// Host side of libdf11: histogram, code book, device tables and the encoder.
//
// Page "DFloat11: lossless BFloat16 compression" (ai-infrastructure.net):
//   "How it works: the core algorithm" -- histogram of the exponent byte,
//   Huffman lengths, canonical code values, codes emitted MSB first;
//   "Architecture" -- 8-bit hierarchical lookup tables, Gaps, BlockOutputPos;
//   "References", v1 note -- the longest code is limited to 32 bits by
//   rebuilding the tree.
//
// The encoder runs on many threads: each takes a contiguous range of weights,
// learns its starting bit from a prefix sum of code lengths, and packs 64-bit
// words; only the two words it shares with its neighbours are merged with an
// atomic OR.  The output does not depend on the thread count.
#include "df11.h"
#include "df11_internal.h"

#include <algorithm>
#include <atomic>
#include <cstring>
#include <thread>
#include <vector>

namespace {

unsigned pick_threads(uint32_t requested, uint64_t work, uint64_t min_per_thread) {
    unsigned hw = std::max(1u, std::thread::hardware_concurrency());
    unsigned t = requested ? requested : hw;
    uint64_t cap = std::max<uint64_t>(1, work / std::max<uint64_t>(1, min_per_thread));
    return (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(t, cap));
}

template <class F>
void parallel_for(unsigned threads, F &&fn) {
    if (threads <= 1) {
        fn(0u);
        return;
    }
    std::vector<std::thread> pool;
    pool.reserve(threads - 1);
    for (unsigned t = 1; t < threads; ++t) pool.emplace_back(fn, t);
    fn(0u);
    for (auto &th : pool) th.join();
}

// Huffman code lengths with the (count, creation number) order.  Leaves are
// numbered 0..k-1 in increasing symbol order and internal nodes k, k+1, ...
// as they are made.  Two sorted queues give the same pops as a priority
// queue keyed by (count, number): leaves are sorted by (count, symbol),
// internal nodes come out in non-decreasing count with increasing numbers,
// and a leaf beats an internal node of equal count because its number is
// smaller.
void huffman_lengths(const uint64_t *count, uint8_t *len) {
    struct Leaf { uint64_t c; int sym; };
    std::vector<Leaf> leaves;
    for (int s = 0; s < 256; ++s) {
        len[s] = 0;
        if (count[s]) leaves.push_back({count[s], s});
    }
    const int k = (int)leaves.size();
    if (k == 0) return;
    if (k == 1) {
        len[leaves[0].sym] = 1;
        return;
    }
    std::stable_sort(leaves.begin(), leaves.end(),
                     [](const Leaf &a, const Leaf &b) { return a.c < b.c; });
    // node ids: 0..k-1 leaves (in sorted-queue order), k.. internal
    std::vector<uint64_t> ncount(2 * k);
    std::vector<int> parent(2 * k, -1);
    std::vector<int> leaf_node(k);
    for (int i = 0; i < k; ++i) leaf_node[i] = i, ncount[i] = leaves[i].c;
    int li = 0, ni = k, nend = k;
    auto pop = [&]() -> int {
        // leaf wins ties: its creation number is always lower
        if (li < k && (ni >= nend || ncount[li] <= ncount[ni])) return li++;
        return ni++;
    };
    for (int m = 0; m < k - 1; ++m) {
        int a = pop(), b = pop();
        int node = nend++;
        ncount[node] = ncount[a] + ncount[b];
        parent[a] = node;
        parent[b] = node;
    }
    std::vector<int> depth(2 * k, 0);
    for (int node = nend - 2; node >= 0; --node) depth[node] = depth[parent[node]] + 1;
    for (int i = 0; i < k; ++i) {
        int d = depth[leaf_node[i]];
        len[leaves[i].sym] = (uint8_t)std::min(d, 255);
    }
}

uint32_t reverse_bits(uint32_t v, unsigned n) {
    uint32_t r = 0;
    for (unsigned i = 0; i < n; ++i) r |= ((v >> i) & 1u) << (n - 1 - i);
    return r;
}

}  // namespace

extern "C" const char *df11_status_string(int status) {
    switch (status) {
        case DF11_OK: return "ok";
        case DF11_ERR_ARG: return "invalid argument";
        case DF11_ERR_BUFSIZE: return "buffer too small";
        case DF11_ERR_CODELEN: return "code length limit cannot be met";
        case DF11_ERR_TABLES: return "code tree needs too many lookup tables";
        case DF11_ERR_FORMAT: return "inconsistent encoded format";
        case DF11_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" int df11_histogram(const uint16_t *bf16, uint64_t n, uint64_t hist[256],
                              uint32_t n_threads) {
    if (!bf16 || !hist) return DF11_ERR_ARG;
    unsigned T = pick_threads(n_threads, n, 1u << 20);
    std::vector<uint64_t> part((size_t)T * 256, 0);
    parallel_for(T, [&](unsigned t) {
        uint64_t lo = n * t / T, hi = n * (t + 1) / T;
        uint64_t *h = &part[(size_t)t * 256];
        for (uint64_t i = lo; i < hi; ++i) h[(bf16[i] >> 7) & 0xFF]++;
    });
    for (unsigned t = 0; t < T; ++t)
        for (int s = 0; s < 256; ++s) hist[s] += part[(size_t)t * 256 + s];
    return DF11_OK;
}

extern "C" int df11_build_codebook(const uint64_t hist[256], uint32_t max_code_len,
                                   df11_codebook *cb) {
    if (!hist || !cb) return DF11_ERR_ARG;
    if (max_code_len < 1 || max_code_len > DF11_MAX_CODE_LEN) return DF11_ERR_CODELEN;
    std::memset(cb, 0, sizeof(*cb));
    uint64_t c[256];
    unsigned live = 0;
    for (int s = 0; s < 256; ++s) {
        c[s] = hist[s];
        live += hist[s] != 0;
    }
    if (live == 0) return DF11_ERR_ARG;
    unsigned need = 0;
    while ((1u << need) < live) ++need;
    if (live > 1 && max_code_len < need) return DF11_ERR_CODELEN;

    uint32_t rounds = 0;
    for (;;) {
        huffman_lengths(c, cb->code_len);
        unsigned longest = *std::max_element(cb->code_len, cb->code_len + 256);
        if (longest <= max_code_len) break;
        for (int s = 0; s < 256; ++s)
            if (c[s]) c[s] = (c[s] + 1) / 2;  // flatten and rebuild
        ++rounds;
    }
    // canonical values: per length, consecutive in symbol order
    uint32_t count_of_len[DF11_MAX_CODE_LEN + 2] = {0};
    for (int s = 0; s < 256; ++s) count_of_len[cb->code_len[s]]++;
    // first value of each length: first[1] = 0, first[L] = (first[L-1] + count[L-1]) << 1
    uint32_t next[DF11_MAX_CODE_LEN + 2] = {0};
    uint64_t first = 0;
    for (unsigned L = 1; L <= DF11_MAX_CODE_LEN; ++L) {
        if (L > 1) first = (first + count_of_len[L - 1]) << 1;
        next[L] = (uint32_t)first;
    }
    for (int s = 0; s < 256; ++s) {
        unsigned L = cb->code_len[s];
        if (L) cb->code[s] = next[L]++;
    }
    cb->max_len = *std::max_element(cb->code_len, cb->code_len + 256);
    cb->n_symbols = live;
    cb->limit_rounds = rounds;
    int tables = df11_internal::count_tables(cb->code_len, cb->code);
    if (tables > DF11_MAX_TABLES) return DF11_ERR_TABLES;
    cb->n_tables = (uint32_t)tables;
    cb->lut_bytes = (uint32_t)df11_internal::lut_image_bytes((uint32_t)tables);
    return DF11_OK;
}

namespace df11_internal {

// Distinct 8-, 16- and 24-bit stream prefixes of codes longer than the
// prefix, plus the root: one 256-entry table each.
int count_tables(const uint8_t *len, const uint32_t *code) {
    int tables = 1;
    for (unsigned depth = 8; depth < 32; depth += 8) {
        std::vector<uint32_t> prefixes;
        for (int s = 0; s < 256; ++s)
            if (len[s] > depth) prefixes.push_back(code[s] >> (len[s] - depth));
        std::sort(prefixes.begin(), prefixes.end());
        tables += (int)(std::unique(prefixes.begin(), prefixes.end()) - prefixes.begin());
    }
    return tables;
}

uint64_t lut_image_bytes(uint32_t n_tables) {
    return (uint64_t)n_tables * 256 * 2 + kDecodeTableBytes;
}

}  // namespace df11_internal

namespace {

using df11_internal::kDecodeTableBits;
using df11_internal::kDecodeTableEntries;

// The leaf the 8-bit tables give for stream window w (first bit in bit 0),
// following at most three pointers; a pointer to a table past n_tables goes
// to table 0, and a pointer left after the last hop reads as a leaf.
uint32_t table_leaf(const uint16_t *lut, uint32_t w, uint32_t n_tables) {
    uint32_t e = lut[w & 0xFFu];
    for (int lvl = 1; lvl < 4 && (e & 0x8000u); ++lvl) {
        const uint32_t t = (e & 63u) < n_tables ? (e & 63u) : 0u;
        e = lut[t * 256u + ((w >> (8 * lvl)) & 0xFFu)];
    }
    return e;
}

// The multi-code decode table for the kernel.  Entry i covers the codes at
// the start of window i that end within its first width = min(max_len - 1,
// kDecodeTableBits) bits, at most four.  It stores their total length |
// their number << 16, then their symbols one per byte, each rotated right
// by one bit (unused bytes 0).
// All ones is a prefix of the longest code, so a window of ones never
// completes one here.  A code longer than the window leaves the entry empty,
// and the kernel resolves it through the 8-bit tables.  The next code of
// window i is the first code of window i >> length.
void build_decode_table(const uint16_t *lut, uint32_t n_tables, uint32_t max_len, uint32_t *out) {
    const uint32_t width = max_len - 1 < kDecodeTableBits ? max_len - 1 : kDecodeTableBits;
    std::vector<uint32_t> first(kDecodeTableEntries);
    for (uint32_t i = 0; i < kDecodeTableEntries; ++i) first[i] = table_leaf(lut, i, n_tables);
    for (uint32_t i = 0; i < kDecodeTableEntries; ++i) {
        uint32_t pos = 0, cnt = 0, syms = 0;
        for (uint32_t k = 0; k < 4; ++k) {
            const uint32_t e = first[i >> pos];
            const uint32_t len = ((e >> 8) & 31u) + 1;
            if (pos + len > width) break;
            // the symbol (an exponent byte) rotated right by one bit, the form
            // the kernel joins with the sign|mantissa byte
            const uint32_t sym = e & 0xFFu;
            syms |= (((sym >> 1) | (sym << 7)) & 0xFFu) << (8 * k);
            pos += len;
            ++cnt;
        }
        out[2 * i] = pos | (cnt << 16);
        out[2 * i + 1] = syms;
    }
}

}  // namespace

// Device table image: n_tables tables of 256 uint16 entries, indexed by the
// next 8 stream bits with the first stream bit in bit 0 of the index,
//   leaf    : bits 0-7 symbol, bits 8-12 (total code length - 1), bit 15 = 0
//   pointer : bit 15 = 1, bits 0-5 child table (the next 8 bits index it),
// then the multi-code decode table (build_decode_table above).
// Unreachable entries (only the one-symbol code has any) are leaves of
// symbol 0, length 1, so a decoder always advances.
extern "C" int df11_build_luts(const df11_codebook *cb, void *lut, uint64_t lut_cap) {
    if (!cb || !lut || cb->n_tables < 1 || cb->n_tables > DF11_MAX_TABLES) return DF11_ERR_ARG;
    const uint64_t bytes = df11_internal::lut_image_bytes(cb->n_tables);
    if (lut_cap < bytes) return DF11_ERR_BUFSIZE;
    uint16_t *t = static_cast<uint16_t *>(lut);
    std::fill(t, t + cb->n_tables * 256, (uint16_t)0);
    // child table of (parent table, index), in creation order
    std::vector<int> child((size_t)cb->n_tables * 256, -1);
    int made = 1;
    // visit in canonical order so table numbering is deterministic
    std::vector<int> order;
    for (int s = 0; s < 256; ++s)
        if (cb->code_len[s]) order.push_back(s);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
        return cb->code_len[a] < cb->code_len[b];
    });
    for (int s : order) {
        const unsigned L = cb->code_len[s];
        const uint32_t r = reverse_bits(cb->code[s], L);  // stream order, first bit in bit 0
        int tab = 0;
        unsigned used = 0;
        while (L - used > 8) {
            unsigned idx = (r >> used) & 0xFF;
            int &c = child[(size_t)tab * 256 + idx];
            if (c < 0) {
                if (made >= (int)cb->n_tables) return DF11_ERR_TABLES;
                c = made++;
            }
            t[tab * 256 + idx] = (uint16_t)(0x8000u | (unsigned)c);
            tab = c;
            used += 8;
        }
        const unsigned rest = L - used;  // 1..8 bits resolved in this table
        const uint32_t low = (r >> used) & ((1u << rest) - 1);
        const uint16_t leaf = (uint16_t)((unsigned)s | ((L - 1) << 8));
        for (uint32_t hi = 0; hi < (1u << (8 - rest)); ++hi) t[tab * 256 + (low | (hi << rest))] = leaf;
    }
    // the decode table follows the 8-bit tables (16-byte aligned: n_tables x 512 bytes)
    build_decode_table(t, cb->n_tables, cb->max_len,
                       reinterpret_cast<uint32_t *>(t + cb->n_tables * 256));
    return DF11_OK;
}

extern "C" int df11_encoded_sizes(const uint64_t hist[256], uint64_t n, const df11_codebook *cb,
                                  df11_sizes *out) {
    if (!hist || !cb || !out || n == 0 || n > DF11_MAX_N) return DF11_ERR_ARG;
    uint64_t total = 0, sum = 0;
    for (int s = 0; s < 256; ++s) {
        if (hist[s] && !cb->code_len[s]) return DF11_ERR_FORMAT;
        total += hist[s] * cb->code_len[s];
        sum += hist[s];
    }
    if (sum != n) return DF11_ERR_FORMAT;
    std::memset(out, 0, sizeof(*out));
    const uint64_t nb = (total + 4095) / 4096;
    out->n = n;
    out->total_bits = total;
    out->last_start = 0;  // known only after encoding
    out->n_blocks = (uint32_t)nb;
    out->stream_bytes = nb * DF11_BLOCK_BYTES + DF11_STREAM_GUARD;
    out->gaps_bytes = 40 * nb + 8;
    out->block_pos_count = nb + 1;
    out->signmant_bytes = (n + 15) & ~uint64_t(15);
    out->lut_bytes = df11_internal::lut_image_bytes(cb->n_tables);
    return DF11_OK;
}

extern "C" int df11_encode(const uint16_t *bf16, uint64_t n, const df11_codebook *cb,
                           uint8_t *stream, uint64_t stream_cap, uint8_t *gaps, uint64_t gaps_cap,
                           uint32_t *block_pos, uint64_t block_pos_cap, uint8_t *signmant,
                           uint64_t signmant_cap, df11_sizes *out, uint32_t n_threads) {
    if (!bf16 || !cb || !stream || !gaps || !block_pos || !signmant || !out) return DF11_ERR_ARG;
    if (n == 0 || n > DF11_MAX_N) return DF11_ERR_ARG;
    if (reinterpret_cast<uintptr_t>(stream) % 8) return DF11_ERR_ARG;

    // code in stream order (first bit in bit 0) and its length, per exponent
    uint32_t rcode[256];
    uint8_t len[256];
    for (int s = 0; s < 256; ++s) {
        len[s] = cb->code_len[s];
        rcode[s] = len[s] ? reverse_bits(cb->code[s], len[s]) : 0;
    }

    const unsigned T = pick_threads(n_threads, n, 1u << 18);
    std::vector<uint64_t> bits_of(T, 0);
    std::vector<int> bad(T, 0);
    parallel_for(T, [&](unsigned t) {
        uint64_t lo = n * t / T, hi = n * (t + 1) / T, b = 0;
        int missing = 0;
        for (uint64_t i = lo; i < hi; ++i) {
            unsigned L = len[(bf16[i] >> 7) & 0xFF];
            missing |= (L == 0);
            b += L;
        }
        bits_of[t] = b;
        bad[t] = missing;
    });
    for (unsigned t = 0; t < T; ++t)
        if (bad[t]) return DF11_ERR_FORMAT;
    std::vector<uint64_t> start_bit(T + 1, 0);
    for (unsigned t = 0; t < T; ++t) start_bit[t + 1] = start_bit[t] + bits_of[t];
    const uint64_t total = start_bit[T];
    const uint64_t nb = (total + 4095) / 4096;
    const uint64_t n_slices = nb * DF11_BLOCK_SLICES;
    const uint64_t need_stream = nb * DF11_BLOCK_BYTES + DF11_STREAM_GUARD;
    const uint64_t need_gaps = 40 * nb + 8;
    const uint64_t need_sm = (n + 15) & ~uint64_t(15);
    if (stream_cap < need_stream || gaps_cap < need_gaps || block_pos_cap < nb + 1 ||
        signmant_cap < need_sm)
        return DF11_ERR_BUFSIZE;

    // slice gaps, unpacked, one byte each (slices without a code start stay 0)
    std::vector<uint8_t> gap_u8(n_slices + 1, 0);
    uint64_t *words = reinterpret_cast<uint64_t *>(stream);
    const uint64_t n_words = need_stream / 8;
    {
        const unsigned Z = pick_threads(n_threads, n_words, 1u << 16);
        parallel_for(Z, [&](unsigned z) {
            uint64_t lo = n_words * z / Z, hi = n_words * (z + 1) / Z;
            std::memset(words + lo, 0, (hi - lo) * 8);
        });
    }

    parallel_for(T, [&](unsigned t) {
        const uint64_t lo = n * t / T, hi = n * (t + 1) / T;
        if (lo >= hi) return;
        uint64_t p = start_bit[t];
        // slice and block of the previous code start (from the neighbour's last weight)
        int64_t prev_slice = -1, prev_block = -1;
        if (lo > 0) {
            uint64_t prev_start = p - len[(bf16[lo - 1] >> 7) & 0xFF];
            prev_slice = (int64_t)(prev_start >> 6);
            prev_block = (int64_t)(prev_start >> 12);
        }
        uint64_t word_idx = p >> 6;
        const uint64_t first_word = word_idx;
        unsigned nb_acc = (unsigned)(p & 63);
        uint64_t acc = 0;
        auto emit = [&](uint64_t w) {
            if (word_idx == first_word && (start_bit[t] & 63))
                __atomic_fetch_or(&words[word_idx], w, __ATOMIC_RELAXED);
            else
                words[word_idx] = w;
            ++word_idx;
        };
        for (uint64_t i = lo; i < hi; ++i) {
            const uint16_t w = bf16[i];
            const unsigned e = (w >> 7) & 0xFF;
            signmant[i] = (uint8_t)(((w >> 8) & 0x80) | (w & 0x7F));
            const int64_t sl = (int64_t)(p >> 6);
            if (sl != prev_slice) {
                gap_u8[sl] = (uint8_t)(p & 63);
                prev_slice = sl;
            }
            const int64_t bl = (int64_t)(p >> 12);
            while (prev_block < bl) block_pos[++prev_block] = (uint32_t)i;
            const unsigned L = len[e];
            const uint64_t r = rcode[e];
            acc |= r << nb_acc;
            if (nb_acc + L >= 64) {
                emit(acc);
                acc = (nb_acc + L > 64) ? (r >> (64 - nb_acc)) : 0;
                nb_acc = nb_acc + L - 64;
            } else {
                nb_acc += L;
            }
            p += L;
        }
        if (nb_acc) __atomic_fetch_or(&words[word_idx], acc, __ATOMIC_RELAXED);
    });
    // blocks with no code start (only a trailing one can lack one) and the end mark
    {
        // highest block index that received a position
        uint64_t last_start = total - len[(bf16[n - 1] >> 7) & 0xFF];
        for (uint64_t b = (last_start >> 12) + 1; b <= nb; ++b) block_pos[b] = (uint32_t)n;
        out->last_start = last_start;
    }
    for (uint64_t i = n; i < need_sm; ++i) signmant[i] = 0;

    // pack gaps: 8 slices = 40 bits = 5 bytes, so groups of 8 are independent
    std::memset(gaps, 0, need_gaps);
    const uint64_t n_fields = n_slices + 1;
    const uint64_t groups = (n_fields + 7) / 8;
    const unsigned G = pick_threads(n_threads, groups, 1u << 14);
    parallel_for(G, [&](unsigned t) {
        uint64_t lo = groups * t / G, hi = groups * (t + 1) / G;
        for (uint64_t gi = lo; gi < hi; ++gi) {
            uint64_t v = 0;
            for (unsigned j = 0; j < 8; ++j) {
                uint64_t f = gi * 8 + j;
                if (f < n_fields) v |= (uint64_t)(gap_u8[f] & 31) << (5 * j);
            }
            for (unsigned j = 0; j < 5; ++j) gaps[gi * 5 + j] = (uint8_t)(v >> (8 * j));
        }
    });

    out->n = n;
    out->total_bits = total;
    out->n_blocks = (uint32_t)nb;
    out->stream_bytes = need_stream;
    out->gaps_bytes = need_gaps;
    out->block_pos_count = nb + 1;
    out->signmant_bytes = need_sm;
    out->lut_bytes = df11_internal::lut_image_bytes(cb->n_tables);
    return DF11_OK;
}

// ------------------------------------------------ layout for the tiled product
//
// The tiled fused product multiplies 16-row tiles of a matrix with up to 64
// input vectors on the matrix cores.  Its weights are stored in the order in
// which a 16x16x32 bf16 matrix instruction takes its first operand, so that
// the decoded words come out of a block already in operand order: per matrix,
// row tiles rt (16 rows), then k-steps ks (32 columns) of the row tile, then
// for the 64 lanes L of the instruction the 8 consecutive weights
// W[16 rt + L % 16][32 ks + 8 (L / 16) + j], j = 0..7.

namespace {

// Matrices end to end from 0 that cover n, rows multiples of 16, cols of 32.
bool tiled_matrices_ok(const df11_gemv_matrix *mats, uint32_t n_mats, uint64_t n) {
    if (!mats || n_mats < 1 || n_mats > DF11_GEMV_MAX_MATRICES) return false;
    uint64_t off = 0;
    for (uint32_t m = 0; m < n_mats; ++m) {
        const df11_gemv_matrix &mm = mats[m];
        if (mm.offset != off || mm.rows == 0 || mm.rows % 16 != 0 || mm.cols == 0 ||
            mm.cols % 32 != 0)
            return false;
        off += (uint64_t)mm.rows * mm.cols;
    }
    return off == n;
}

}  // namespace

extern "C" int df11_tile_order(const uint16_t *w, uint64_t n, const df11_gemv_matrix *mats,
                               uint32_t n_mats, uint16_t *out, uint32_t n_threads) {
    if (!w || !out || w == out || n == 0 || n > DF11_MAX_N) return DF11_ERR_ARG;
    if (!tiled_matrices_ok(mats, n_mats, n)) return DF11_ERR_ARG;
    // one task per row tile of any matrix
    std::vector<std::pair<uint32_t, uint32_t>> tasks;  // (matrix, row tile)
    for (uint32_t m = 0; m < n_mats; ++m)
        for (uint32_t rt = 0; rt < mats[m].rows / 16; ++rt) tasks.emplace_back(m, rt);
    const unsigned threads = pick_threads(n_threads, n, 1u << 20);
    std::atomic<size_t> next{0};
    parallel_for(threads, [&](unsigned) {
        for (size_t t; (t = next.fetch_add(1)) < tasks.size();) {
            const df11_gemv_matrix &mm = mats[tasks[t].first];
            const uint64_t c = mm.cols, rt = tasks[t].second;
            const uint16_t *src = w + mm.offset + rt * 16 * c;
            uint16_t *dst = out + mm.offset + rt * 16 * c;
            for (uint64_t ks = 0; ks < c / 32; ++ks)
                for (uint32_t lane = 0; lane < 64; ++lane) {
                    const uint16_t *row = src + (lane % 16) * c + 32 * ks + 8 * (lane / 16);
                    std::memcpy(dst + (ks * 64 + lane) * 8, row, 16);
                }
        }
    });
    return DF11_OK;
}

extern "C" uint64_t df11_tile_segment_count(const df11_gemv_matrix *mats, uint32_t n_mats) {
    if (!mats || n_mats < 1 || n_mats > DF11_GEMV_MAX_MATRICES) return 0;
    uint64_t s = 0;
    for (uint32_t m = 0; m < n_mats; ++m) s += mats[m].rows / 16;
    return s;
}

extern "C" int df11_tile_segments(const uint32_t *block_pos, uint32_t n_blocks,
                                  const df11_gemv_matrix *mats, uint32_t n_mats,
                                  uint32_t *seg_blk, uint64_t seg_cap) {
    if (!block_pos || !seg_blk || n_blocks == 0) return DF11_ERR_ARG;
    if (block_pos[0] != 0) return DF11_ERR_FORMAT;
    const uint64_t n = block_pos[n_blocks];
    if (n == 0 || !tiled_matrices_ok(mats, n_mats, n)) return DF11_ERR_ARG;
    const uint64_t segs = df11_tile_segment_count(mats, n_mats);
    if (seg_cap < segs + 1) return DF11_ERR_BUFSIZE;
    // the block holding weight q: the last block whose first code index is <= q
    auto holder = [&](uint64_t q) {
        const uint32_t *it = std::upper_bound(block_pos, block_pos + n_blocks, (uint32_t)q);
        return (uint32_t)(it - block_pos) - 1;
    };
    uint64_t s = 0;
    for (uint32_t m = 0; m < n_mats; ++m)
        for (uint64_t rt = 0; rt < mats[m].rows / 16; ++rt)
            seg_blk[s++] = holder(mats[m].offset + rt * 16 * (uint64_t)mats[m].cols);
    seg_blk[segs] = holder(n - 1);
    return DF11_OK;
}
