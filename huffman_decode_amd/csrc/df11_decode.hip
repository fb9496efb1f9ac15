// df11_decode: gfx950 (CDNA4) kernel that turns a DF11-encoded tensor back
// into its BF16 words, and its C-ABI launcher.
//
// Page "DFloat11: lossless BFloat16 compression" (ai-infrastructure.net),
// section "Architecture": each thread owns 8 bytes of the code stream and
// starts at its Gaps offset; phase 1 only counts codes; a block prefix sum
// turns counts into output offsets (the block's first index is its
// BlockOutputPos); phase 2 decodes again and writes; exponents are joined
// with their sign|mantissa bytes and written with coalesced stores.  The
// page's hierarchical 8-bit tables are what the host ships and what every
// workgroup stages in LDS.
//
// Mapping onto CDNA4 (the decoder is integer VALU + LDS work; no MFMA):
//  * a format block (64 slices, 512 stream bytes) is one wave64, so the prefix
//    sum is a wave-level scan and no workgroup barrier sits in the block loop;
//  * workgroups are persistent; each stages the 8-bit tables and expands them
//    in LDS into two multi-code tables indexed by the next W stream bits:
//      count table  : bits taken by all codes that end inside the W bits, and
//                     their number (phase 1 counts ~4 codes per lookup);
//      decode table : the first (up to 4) of those symbols, bits and count
//                     (phase 2 emits up to 4 exponents per lookup);
//    codes longer than W fall back to the 8-bit tables;
//  * a lane's 96 relevant stream bits live in three VGPRs; windows come from
//    one funnel shift (v_alignbit) of a dword pair, with the data pre-shifted
//    so that the window's low bits are already the table's byte offset;
//  * bits after the lane's last code are forced to 1 for phase 1: the all-ones
//    prefix is the longest code's prefix, which never completes inside the
//    count window (its width is kept below the longest code), so a lookup
//    never counts the next lane's codes; phase 2 reads the real bits, so any
//    symbol it decodes past the lane's end is the true next symbol;
//  * phase 2 writes exponent bytes into a per-wave LDS tile aligned to 8
//    outputs; the merge joins 8 exponents with 8 prefetched sign|mantissa
//    bytes per lane and writes one 16-byte store;
//  * blocks are split into 8 contiguous ranges, one per XCD (workgroups are
//    dispatched round-robin over the XCDs), so neighbouring blocks, which
//    share cache lines at their edges, meet in the same L2.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "df11.h"
#include "df11_internal.h"

namespace {

constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kGroupThreads = kWave * kWavesPerGroup;
constexpr int kMaxBlockCodes = DF11_BLOCK_SLICES * DF11_SLICE_BITS;  // all 1-bit codes
constexpr int kTileBytes = kMaxBlockCodes + 16;
constexpr int kTableBytes = 256 * 2;
constexpr int kXcds = 8;

// multi-code tables (LDS): window widths
constexpr int kCountBits = 11;
constexpr int kDecodeBits = 11;
constexpr int kCountBytes = (1 << kCountBits) * 4;
constexpr int kDecodeBytes = (1 << kDecodeBits) * 8;
constexpr int kMaxSymbolsPerStep = 4;
constexpr int kPrefetchGroups = 4;  // sign|mantissa groups of 8 per lane loaded up front

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    // low 32 bits of a flat address inside the LDS aperture are the LDS offset
    return (uint32_t)(uintptr_t)p;
}

struct DecodeArgs {
    const uint32_t *stream;  // as dwords
    const uint32_t *gaps;    // packed 5-bit fields, as dwords
    const uint32_t *block_pos;
    const uint8_t *signmant;
    const uint4 *luts;
    uint16_t *out;
    uint32_t *status;
    uint64_t n;
    uint64_t total_bits;
    uint64_t stop_bit;       // codes start strictly before this bit
    uint32_t n_blocks;
    uint32_t n_tables;
    uint32_t max_len;
    uint32_t blocks_per_xcd;  // contiguous block range of one XCD
};

// 8-bit table entry: leaf = symbol | (length - 1) << 8; pointer = 0x8000 |
// child.  Resolve window w (stream order, first bit in bit 0) to a leaf.
__device__ __forceinline__ uint32_t lookup8(const uint16_t *lut, uint32_t w, uint32_t n_tables) {
    uint32_t e = lut[w & 0xFFu];
#pragma unroll
    for (int lvl = 1; lvl < 4; ++lvl) {
        if (!(e & 0x8000u)) break;
        uint32_t t = e & 63u;
        t = t < n_tables ? t : 0u;
        e = lut[t * 256u + ((w >> (8 * lvl)) & 0xFFu)];
    }
    return e;  // a pointer entry left here reads as a 1-bit leaf
}

__device__ __forceinline__ uint32_t leaf_len(uint32_t e) { return ((e >> 8) & 31u) + 1u; }

// Expand the 8-bit tables into the count and decode tables (whole workgroup).
__device__ void build_fast_tables(const uint16_t *lut, uint32_t *count_t, uint2 *dec_t,
                                  uint32_t n_tables, uint32_t max_len) {
    // the count window must stay shorter than the longest code (see header)
    const uint32_t count_w = max_len - 1 < (uint32_t)kCountBits ? max_len - 1 : kCountBits;
    constexpr int kEntries = (1 << kCountBits) > (1 << kDecodeBits) ? (1 << kCountBits)
                                                                     : (1 << kDecodeBits);
    constexpr uint32_t kSpan = kCountBits > kDecodeBits ? kCountBits : kDecodeBits;
    for (int i = threadIdx.x; i < kEntries; i += kGroupThreads) {
        // codes of the bit pattern i (first stream bit in bit 0; zeros past
        // the table width never complete a code that is counted)
        uint32_t pos = 0, k = 0, cpos = 0, ck = 0, dpos = 0, dk = 0;
        uint32_t s01 = 0, s23 = 0;
        for (uint32_t step = 0; step < kSpan; ++step) {
            const uint32_t e = lookup8(lut, (uint32_t)i >> pos, n_tables);
            const uint32_t len = leaf_len(e);
            if (pos + len > kSpan) break;
            if (pos + len <= count_w) cpos = pos + len, ck = k + 1;
            if (pos + len <= (uint32_t)kDecodeBits && k < (uint32_t)kMaxSymbolsPerStep) {
                const uint32_t sym = e & 0xFFu;
                if (k == 0) s01 |= sym;
                if (k == 1) s01 |= sym << 16;
                if (k == 2) s23 |= sym;
                if (k == 3) s23 |= sym << 16;
                dpos = pos + len;
                dk = k + 1;
            }
            pos += len;
            ++k;
        }
        if (i < (1 << kCountBits)) count_t[i] = cpos | (ck << 16);
        if (i < (1 << kDecodeBits))
            dec_t[i] = make_uint2(s01 | (dpos << 8) | (dk << 24), s23);
    }
}

__device__ __forceinline__ uint32_t join2(uint32_t e4, uint32_t s4, uint32_t sel_s, uint32_t sel_e) {
    // two BF16 words from two exponent bytes and two sign|mantissa bytes:
    // x = [s0 s0 s1 s1] supplies mantissa (bits 6:0, 22:16) and sign (15, 31);
    // y = [.. e0 .. e1] >> 1 supplies the exponents at bits 14:7 and 30:23.
    const uint32_t x = __builtin_amdgcn_perm(s4, s4, sel_s);
    const uint32_t y = __builtin_amdgcn_perm(e4, e4, sel_e) >> 1;
    return (x & 0x807F807Fu) | (y & ~0x807F807Fu);
}

__device__ __forceinline__ uint4 join8(uint2 e, uint2 s) {
    uint4 o;
    o.x = join2(e.x, s.x, 0x01010000u, 0x010C000Cu);
    o.y = join2(e.x, s.x, 0x03030202u, 0x030C020Cu);
    o.z = join2(e.y, s.y, 0x01010000u, 0x010C000Cu);
    o.w = join2(e.y, s.y, 0x03030202u, 0x030C020Cu);
    return o;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bits at and after `end` (lane-relative, 0..95) forced to 1.
__device__ __forceinline__ uint32_t pad_ones(uint32_t d, int end, int base) {
    const int keep = end - base;  // bits of this dword to keep
    if (keep >= 32) return d;
    if (keep <= 0) return 0xFFFFFFFFu;
    return d | (0xFFFFFFFFu << keep);
}

__global__ __launch_bounds__(kGroupThreads) void df11_decode_kernel(DecodeArgs a) {
    // LDS: count table | decode table (fixed offsets, folded into the
    // ds_read immediates) | 8-bit tables | per-wave exponent tiles
    __shared__ uint32_t count_t[1 << kCountBits];
    __shared__ uint2 dec_t[1 << kDecodeBits];
    extern __shared__ uint4 smem_u4[];
    uint8_t *smem = reinterpret_cast<uint8_t *>(smem_u4);
    uint16_t *lut = reinterpret_cast<uint16_t *>(smem);
    const uint32_t hier_bytes = a.n_tables * kTableBytes;
    uint8_t *tiles = smem + hier_bytes;

    uint4 *lut_u4 = reinterpret_cast<uint4 *>(lut);
    for (uint32_t i = threadIdx.x; i < hier_bytes / 16; i += kGroupThreads) lut_u4[i] = a.luts[i];
    __syncthreads();
    build_fast_tables(lut, count_t, dec_t, a.n_tables, a.max_len);
    __syncthreads();

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = (int)(threadIdx.x % kWave);
    uint8_t *tile = tiles + wave * kTileBytes;
    const uint32_t tile_addr = lds_offset(tile);

    // XCD-contiguous assignment: group g runs on XCD g % 8 and takes the
    // blocks of that XCD's range with a stride of (groups per XCD * waves)
    const uint32_t xcd = blockIdx.x % kXcds;
    const uint32_t slot = blockIdx.x / kXcds;
    const uint32_t groups_per_xcd = gridDim.x / kXcds;
    const uint32_t range_lo = xcd * a.blocks_per_xcd;
    uint32_t range_hi = range_lo + a.blocks_per_xcd;
    range_hi = range_hi < a.n_blocks ? range_hi : a.n_blocks;
    const uint32_t stride = groups_per_xcd * kWavesPerGroup;

    const uint8_t *lds_count = reinterpret_cast<const uint8_t *>(count_t);
    const uint8_t *lds_dec = reinterpret_cast<const uint8_t *>(dec_t);

    for (uint32_t b = range_lo + slot * kWavesPerGroup + wave; b < range_hi; b += stride) {
        const uint64_t g = (uint64_t)b * DF11_BLOCK_SLICES + (uint32_t)lane;
        const uint32_t p0 = a.block_pos[b], p1 = a.block_pos[b + 1];
        const bool sane = p1 >= p0 && p1 <= a.n && p1 - p0 <= (uint32_t)kMaxBlockCodes;

        // sign|mantissa for this lane's first output groups, loaded up front
        const uint32_t base = p0 & ~7u;
        const uint32_t groups = sane ? (p1 - base + 7) >> 3 : 0u;
        uint2 smv[kPrefetchGroups];
#pragma unroll
        for (int i = 0; i < kPrefetchGroups; ++i) {
            const uint32_t j = (uint32_t)lane + kWave * i;
            smv[i] = j < groups ? *reinterpret_cast<const uint2 *>(a.signmant + base + 8 * j)
                                : make_uint2(0, 0);
        }

        const uint32_t *sp = a.stream + 2 * g;
        const uint32_t d0 = sp[0], d1 = sp[1], d2 = sp[2];
        const uint64_t q = 5 * g;  // bit offset of this slice's gap field
        const uint32_t *gp = a.gaps + (q >> 5);
        const uint32_t gw = __builtin_amdgcn_alignbit(gp[1], gp[0], (uint32_t)(q & 31));
        const int gap = (int)(gw & 31u), gap_next = (int)((gw >> 5) & 31u);
        const int64_t rel = (int64_t)a.stop_bit - (int64_t)(g * DF11_SLICE_BITS);
        const int lim = rel <= 0 ? 0 : (rel >= 64 ? 64 : (int)rel);
        // end of this lane's last code: the next slice's first code start, or
        // the end of the stream for the lane holding the final code
        const int end = rel > 0 && rel <= 64
                            ? (int)((int64_t)a.total_bits - (int64_t)(g * DF11_SLICE_BITS))
                            : 64 + gap_next;

        // ---- phase 1: count
        uint32_t cnt;
        {
            const uint32_t f0 = pad_ones(d0, end, 0), f1 = pad_ones(d1, end, 32),
                           f2 = pad_ones(d2, end, 64);
            // pre-shift by 2: window bits [2, 2+W) are the entry's byte offset / 4 * 4
            const uint32_t c0 = f0 << 2, c1 = __builtin_amdgcn_alignbit(f1, f0, 30),
                           c2 = __builtin_amdgcn_alignbit(f2, f1, 30);
            constexpr uint32_t kMask = ((1u << kCountBits) - 1) << 2;
            uint32_t acc = lim > 0 ? (uint32_t)gap : 0u;  // pos | count << 16
            const uint32_t stop1 = lim > 0 ? (uint32_t)end : 0u;
            const uint32_t stop0 = stop1 < 32u ? stop1 : 32u;
            while ((acc & 0xFFFFu) < stop0) {
                const uint32_t w = __builtin_amdgcn_alignbit(c1, c0, acc);
                uint32_t x = *reinterpret_cast<const uint32_t *>(lds_count + (w & kMask));
                if (x < 0x10000u) {
                    const uint32_t e = lookup8(lut, __builtin_amdgcn_alignbit(d1, d0, acc), a.n_tables);
                    x = leaf_len(e) | 0x10000u;
                }
                acc += x;
            }
            while ((acc & 0xFFFFu) < stop1) {
                const uint32_t w = __builtin_amdgcn_alignbit(c2, c1, acc);
                uint32_t x = *reinterpret_cast<const uint32_t *>(lds_count + (w & kMask));
                if (x < 0x10000u) {
                    const uint32_t e = lookup8(lut, __builtin_amdgcn_alignbit(d2, d1, acc), a.n_tables);
                    x = leaf_len(e) | 0x10000u;
                }
                acc += x;
            }
            cnt = acc >> 16;
        }

        // wave-wide inclusive scan of the counts
        uint32_t incl = cnt;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t y = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += y;
        }
        const uint32_t excl = incl - cnt;
        const uint32_t total = __shfl(incl, kWave - 1, kWave);
        if ((!sane || total != p1 - p0) && lane == 0 && a.status) atomicAdd(a.status, 1u);
        if (!sane) continue;

        // ---- phase 2: decode into the tile
        {
            const uint32_t r0 = d0 << 3, r1 = __builtin_amdgcn_alignbit(d1, d0, 29),
                           r2 = __builtin_amdgcn_alignbit(d2, d1, 29);
            constexpr uint32_t kMask = ((1u << kDecodeBits) - 1) << 3;
            // pos | (LDS address of the next exponent byte) << 16
            uint32_t acc = (lim > 0 ? (uint32_t)gap : 0u) |
                           ((tile_addr + (p0 - base) + excl) << 16);
            const uint32_t stop1 = (uint32_t)lim;
            const uint32_t stop0 = stop1 < 32u ? stop1 : 32u;
#define DF11_DECODE_STEP(HI, LO, DHI, DLO)                                                      \
    {                                                                                            \
        const uint32_t w = __builtin_amdgcn_alignbit(HI, LO, acc);                               \
        const uint2 dv = *reinterpret_cast<const uint2 *>(lds_dec + (w & kMask));                \
        lds_u8 *o = (lds_u8 *)(uintptr_t)(acc >> 16);                                            \
        if (dv.x < 0x1000000u) {                                                                 \
            const uint32_t e = lookup8(lut, __builtin_amdgcn_alignbit(DHI, DLO, acc), a.n_tables);\
            o[0] = (uint8_t)e;                                                                   \
            acc += leaf_len(e) | 0x10000u;                                                       \
        } else {                                                                                 \
            o[0] = (uint8_t)dv.x;                                                                \
            if (dv.x >= 0x2000000u) o[1] = (uint8_t)(dv.x >> 16);                                \
            if (dv.x >= 0x3000000u) o[2] = (uint8_t)dv.y;                                        \
            if (dv.x >= 0x4000000u) o[3] = (uint8_t)(dv.y >> 16);                                \
            acc += __builtin_amdgcn_perm(dv.x, dv.x, 0x0C030C01u);                               \
        }                                                                                        \
    }
            while ((acc & 0xFFFFu) < stop0) DF11_DECODE_STEP(r1, r0, d1, d0)
            while ((acc & 0xFFFFu) < stop1) DF11_DECODE_STEP(r2, r1, d2, d1)
#undef DF11_DECODE_STEP
        }
        wave_lds_sync();

        // ---- merge with sign|mantissa, 8 BF16 per lane per 16-byte store
#pragma unroll
        for (int i = 0; i < kPrefetchGroups; ++i) {
            const uint32_t j = (uint32_t)lane + kWave * i;
            if (j < groups) {
                const uint32_t i0 = base + 8 * j;
                const uint4 o = join8(*reinterpret_cast<const uint2 *>(tile + 8 * j), smv[i]);
                if (i0 >= p0 && i0 + 8 <= p1) {
                    *reinterpret_cast<uint4 *>(a.out + i0) = o;
                } else {
                    const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
                    for (uint32_t k = 0; k < 8; ++k)
                        if (i0 + k >= p0 && i0 + k < p1)
                            a.out[i0 + k] = (uint16_t)(ow[k >> 1] >> (16 * (k & 1)));
                }
            }
        }
        for (uint32_t j = (uint32_t)lane + kWave * kPrefetchGroups; j < groups; j += kWave) {
            const uint32_t i0 = base + 8 * j;
            const uint2 s = *reinterpret_cast<const uint2 *>(a.signmant + i0);
            const uint4 o = join8(*reinterpret_cast<const uint2 *>(tile + 8 * j), s);
            if (i0 + 8 <= p1) {
                *reinterpret_cast<uint4 *>(a.out + i0) = o;
            } else {
                const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
                for (uint32_t k = 0; k < 8; ++k)
                    if (i0 + k < p1) a.out[i0 + k] = (uint16_t)(ow[k >> 1] >> (16 * (k & 1)));
            }
        }
        wave_lds_sync();
    }
}

// Launch shape per device: compute units and resident workgroups per CU for
// each table count (the LDS footprint depends on it).
constexpr int kMaxDevices = 16;
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_occ[kMaxDevices][DF11_MAX_TABLES + 1];

// dynamic LDS per workgroup (the two multi-code tables are static)
size_t lds_bytes(uint32_t n_tables) {
    return (size_t)n_tables * kTableBytes + (size_t)kWavesPerGroup * kTileBytes;
}

int launch_groups(int dev, uint32_t n_tables, uint32_t n_blocks, int *groups) {
    if (dev < 0 || dev >= kMaxDevices) return DF11_ERR_HIP;
    int cus = g_cus[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return DF11_ERR_HIP;
        g_cus[dev].store(cus, std::memory_order_relaxed);
    }
    int occ = g_occ[dev][n_tables].load(std::memory_order_relaxed);
    if (occ <= 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, df11_decode_kernel, kGroupThreads,
                                                         lds_bytes(n_tables)) != hipSuccess)
            return DF11_ERR_HIP;
        if (occ <= 0) occ = 1;
        g_occ[dev][n_tables].store(occ, std::memory_order_relaxed);
    }
    // a multiple of the XCD count, no more than there are blocks to share
    const uint64_t want = ((uint64_t)n_blocks + kWavesPerGroup - 1) / kWavesPerGroup;
    uint64_t cap = (uint64_t)cus * (uint64_t)occ;
    uint64_t g = want < cap ? want : cap;
    g = (g + kXcds - 1) / kXcds * kXcds;
    *groups = (int)g;
    return DF11_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" int df11_decode(const df11_device_stream *s, uint16_t *out, void *hip_stream) {
    if (!s || !out || !s->stream || !s->gaps || !s->block_pos || !s->signmant || !s->luts)
        return DF11_ERR_ARG;
    if (s->n == 0 || s->n > DF11_MAX_N) return DF11_ERR_ARG;
    if (!aligned(out, 16) || !aligned(s->stream, 8) || !aligned(s->signmant, 8) ||
        !aligned(s->gaps, 4) || !aligned(s->block_pos, 4) || !aligned(s->luts, 16))
        return DF11_ERR_ARG;
    if (s->n_tables < 1 || s->n_tables > DF11_MAX_TABLES) return DF11_ERR_TABLES;
    const uint64_t nb = s->n_blocks;
    if (s->total_bits < s->n || s->total_bits > (uint64_t)DF11_MAX_CODE_LEN * s->n ||
        nb != (s->total_bits + 4095) / 4096 || s->last_start >= s->total_bits ||
        s->last_start + DF11_MAX_CODE_LEN < s->total_bits)
        return DF11_ERR_FORMAT;
    if (s->max_len < 1 || s->max_len > DF11_MAX_CODE_LEN) return DF11_ERR_FORMAT;
    if (s->stream_bytes < nb * DF11_BLOCK_BYTES + DF11_STREAM_GUARD ||
        s->gaps_bytes < 40 * nb + 8 || s->block_pos_count < nb + 1 ||
        s->signmant_bytes < ((s->n + 7) & ~uint64_t(7)) ||
        s->lut_bytes < df11_internal::lut_image_bytes(s->n_tables))
        return DF11_ERR_BUFSIZE;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DF11_ERR_HIP;
    int groups = 0;
    int st = launch_groups(dev, s->n_tables, s->n_blocks, &groups);
    if (st != DF11_OK) return st;

    DecodeArgs a;
    a.stream = reinterpret_cast<const uint32_t *>(s->stream);
    a.gaps = reinterpret_cast<const uint32_t *>(s->gaps);
    a.block_pos = s->block_pos;
    a.signmant = s->signmant;
    a.luts = reinterpret_cast<const uint4 *>(s->luts);
    a.out = out;
    a.status = s->status;
    a.n = s->n;
    a.total_bits = s->total_bits;
    a.stop_bit = s->last_start + 1;
    a.n_blocks = s->n_blocks;
    a.n_tables = s->n_tables;
    a.max_len = s->max_len;
    a.blocks_per_xcd = (s->n_blocks + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(df11_decode_kernel, dim3(groups), dim3(kGroupThreads),
                       lds_bytes(s->n_tables), static_cast<hipStream_t>(hip_stream), a);
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_ERR_HIP;
}
