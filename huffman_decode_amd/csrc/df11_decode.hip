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
//    in LDS into a multi-code decode table indexed by the next 11 stream bits:
//    each entry holds the first (up to 4) codes that end inside a window
//    narrower than the longest code -- their symbols packed in one dword,
//    their total length and their number -- so one lookup yields up to 4
//    exponents, stored with one 4-byte LDS store (ROCm runs gfx9 LDS in
//    unaligned mode); codes longer than the window fall back to the 8-bit
//    tables;
//  * a lane's 96 relevant stream bits live in three VGPRs; windows come from
//    one funnel shift (v_alignbit) of a dword pair, with the data pre-shifted
//    so that the window's low bits are already the table's byte offset;
//  * the phases are merged: phase 1 decodes each lane's codes once, into a
//    private 40-byte staging slot in LDS, and its step count is the lane's
//    code count.  The count is exact because the bits after the lane's last
//    code are forced to 1 for these lookups: all ones is a prefix of the
//    longest code, which never completes inside the window.  After the scan
//    each lane copies its staged exponents to its output position in the
//    wave's tile.  Lanes with more codes than a slot holds (only near-flat
//    streams of 1- and 2-bit codes) send their wave down the page's own
//    route: decode the real bits again, straight into the tile;
//  * the merge joins 8 exponents with 8 prefetched sign|mantissa bytes per
//    lane and writes one 16-byte store;
//  * blocks are split into 8 contiguous ranges, one per XCD (workgroups are
//    dispatched round-robin over the XCDs), so neighbouring blocks, which
//    share cache lines at their edges, meet in the same L2.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "df11.h"
#include "df11_internal.h"

namespace {

#ifndef DF11_WAVES_PER_GROUP
#define DF11_WAVES_PER_GROUP 8
#endif
#ifndef DF11_DECODE_BITS
#define DF11_DECODE_BITS 11
#endif

constexpr int kWave = 64;
constexpr int kWavesPerGroup = DF11_WAVES_PER_GROUP;
constexpr int kGroupThreads = kWave * kWavesPerGroup;
constexpr int kMaxBlockCodes = DF11_BLOCK_SLICES * DF11_SLICE_BITS;  // all 1-bit codes
// staging: lane t's phase-1 exponents at byte 4 + 40 t of its wave's LDS
// region (the 4 bytes in front let every lane read the dword before its slot);
// a lane with more than 32 codes, or with fewer than 3 before the block's last
// code, sends the wave to the re-decode route
constexpr int kStageBase = 4;
constexpr int kStageStride = 40;
constexpr int kStageCodes = 32;
constexpr int kStageMinCodes = 3;
// exponent bytes one tile holds (the tile reuses the wave's staging region);
// blocks with more symbols take several passes
constexpr int kTileCap = 2560;
// a lane's stores reach at most 3 bytes past its last code; a lane holds at
// most 64 codes, so 4 + 63 * 40 + 67 bytes bound the staging stores of valid data
constexpr int kTileBytes = kTileCap + 32;
static_assert(kTileCap % 8 == 0, "tile windows must stay 8-aligned");
static_assert(kTileBytes >= kStageBase + 63 * kStageStride + 64 + 3, "staging must fit");
static_assert(kStageStride % 4 == 0 && kStageBase % 4 == 0 && kTileBytes % 8 == 0,
              "staging dwords are aligned");
static_assert(kStageStride >= kStageCodes + 4, "a full slot takes 4 stray bytes");
constexpr int kTableBytes = 256 * 2;
constexpr int kXcds = 8;
// multi-code decode table (LDS): index width
constexpr int kDecodeBits = DF11_DECODE_BITS;
constexpr int kDecodeBytes = (1 << kDecodeBits) * 8;
constexpr int kMaxSymbolsPerStep = 4;
constexpr int kTilesBytes = kWavesPerGroup * kTileBytes;
constexpr int kStaticLds = kTilesBytes + kDecodeBytes;
static_assert(kTilesBytes < 0x10000, "tile addresses must fit 16 bits");
#ifndef DF11_PREFETCH_GROUPS
#define DF11_PREFETCH_GROUPS 2
#endif
// sign|mantissa groups of 8 per lane loaded up front
constexpr int kPrefetchGroups = DF11_PREFETCH_GROUPS;

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) uint64_t lds_u64;

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

// Expand the 8-bit tables into the decode table (whole workgroup).  An entry
// covers the codes that end within the first `width` bits of its index, at
// most four: their length in bits | their number << 16, then the symbols one
// per byte (unused bytes 0).  width = min(longest code - 1, 11): all ones is a
// prefix of the longest code, so a run of ones never completes a code here.
__device__ void build_decode_table(const uint16_t *lut, uint2 *dec_t, uint32_t n_tables,
                                   uint32_t max_len) {
    const uint32_t width = max_len - 1 < (uint32_t)kDecodeBits ? max_len - 1 : kDecodeBits;
    for (int i = threadIdx.x; i < (1 << kDecodeBits); i += kGroupThreads) {
        uint32_t pos = 0, k = 0, syms = 0;
        while (k < (uint32_t)kMaxSymbolsPerStep) {
            const uint32_t e = lookup8(lut, (uint32_t)i >> pos, n_tables);
            const uint32_t len = leaf_len(e);
            if (pos + len > width) break;
            syms |= (e & 0xFFu) << (8 * k);
            pos += len;
            ++k;
        }
        dec_t[i] = make_uint2(pos | (k << 16), syms);
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

// Inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (no LDS round trip): rows of 16 first, then row 0's total into
// row 1 and row 2's into row 3, then lane 31's total into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
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

// Phase 1 for one lane: decode the codes starting in [pos, stop) of its slice
// into its staging slot at LDS address `slot` (4-aligned) and return their
// number.  f* are the slice's dwords with the bits after its last code set to
// 1 (so a step never runs past that code and the count is exact), d* the plain
// dwords (for codes longer than the table window).
//
// Stores are aligned: `cur` holds the slot's partly filled dword, and each
// step ORs its symbols (unused table bytes are 0) in at the next byte and
// stores the two dwords they can touch.  Stores are clamped to `clamp` so
// that corrupt input cannot reach past the wave's region; valid data never
// gets there.
__device__ __forceinline__ uint32_t stage_codes(const uint8_t *lds_dec, const uint16_t *lut,
                                                uint32_t n_tables, uint32_t d0, uint32_t d1,
                                                uint32_t d2, uint32_t f0, uint32_t f1, uint32_t f2,
                                                uint32_t pos, uint32_t stop, uint32_t slot,
                                                uint32_t clamp) {
    // pre-shift by 3: window bits [3, 3+W) are the entry's byte offset
    const uint32_t e0 = f0 << 3, e1 = __builtin_amdgcn_alignbit(f1, f0, 29),
                   e2 = __builtin_amdgcn_alignbit(f2, f1, 29);
    constexpr uint32_t kMask = ((1u << kDecodeBits) - 1) << 3;
    uint32_t acc = pos | (slot << 16);  // pos | (LDS address of the next byte) << 16
    uint32_t cur = 0;                   // the dword holding that byte, bytes before it
    auto step = [&](uint32_t hi, uint32_t lo, uint32_t dhi, uint32_t dlo) {
        const uint32_t w = __builtin_amdgcn_alignbit(hi, lo, acc);
        const uint2 dv = *reinterpret_cast<const uint2 *>(lds_dec + (w & kMask));
        uint32_t inc = dv.x, syms = dv.y;
        if (dv.x < 0x10000u) {  // longer than the window: 8-bit tables, real bits
            const uint32_t e = lookup8(lut, __builtin_amdgcn_alignbit(dhi, dlo, acc), n_tables);
            syms = e & 0xFFu;
            inc = leaf_len(e) | 0x10000u;
        }
        uint32_t at = acc >> 16;
        at = at < clamp ? at : clamp;
        // bits 13..17 of acc: pos >> 13 (always 0) | (byte address & 3) << 3
        const uint64_t t = (uint64_t)syms << __builtin_amdgcn_ubfe(acc, 13, 5);
        const uint32_t w0 = cur | (uint32_t)t, w1 = (uint32_t)(t >> 32);
        lds_u32 *p = (lds_u32 *)(uintptr_t)(at & ~3u);
        p[0] = w0;
        p[1] = w1;
        acc += inc;
        cur = ((acc >> 16) ^ at) & ~3u ? w1 : w0;
    };
    // every step moves at least one bit on (table entries and 8-bit leaves
    // have lengths >= 1), so a lane takes at most 64 steps, whatever the data
    const uint32_t stop0 = stop < 32u ? stop : 32u;
    while ((acc & 0xFFFFu) < stop0) step(e1, e0, d1, d0);
    while ((acc & 0xFFFFu) < stop) step(e2, e1, d2, d1);
    return (acc >> 16) - slot;
}

// After the scan: move the lane's `cnt` staged exponents (at most 32) from its
// slot to tile address `dst` with aligned dword stores only.  The lane writes
// every aligned dword that ends inside its own output bytes; the first of
// them starts with the previous lane's last bytes (`prev`, taken from that
// lane's slot), and the lane holding the block's last code (`last_lane`) also
// writes its final, partial dword.  Every tile dword is thus written exactly
// once, provided each lane before the last one holds at least 3 codes.
__device__ __forceinline__ void place_staged(uint32_t slot, uint32_t dst, uint32_t cnt,
                                             uint32_t prev, bool last_lane) {
    uint32_t v[9];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *(const lds_u32 *)(uintptr_t)(slot + 4 * i);
    v[8] = 0;
    const uint32_t s = dst & 3u, a0 = dst & ~3u;
    // byte t of output dword j is byte 4 j + t - s of the lane's sequence;
    // v_perm picks it from {v[j], v[j - 1]} (bytes 4..7 and 0..3)
    const uint32_t sel = 0x07060504u - s * 0x01010101u;
    const int last = cnt == 0 ? -1
                     : last_lane ? (int)((s + cnt - 1) >> 2)
                                 : (int)((s + cnt) >> 2) - 1;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
        const uint32_t val = __builtin_amdgcn_perm(v[j], j ? v[j - 1] : prev, sel);
        if (j <= last) *(lds_u32 *)(uintptr_t)(a0 + 4 * j) = val;
    }
}

// The 4 bytes of a lane's slot that end at its last code (the first byte is
// junk when it holds 3 codes).
__device__ __forceinline__ uint32_t staged_tail(uint32_t slot, uint32_t cnt) {
    const int b = (int)cnt - 4;  // >= -4: the slot is preceded by 4 bytes
    const uint32_t at = (uint32_t)((int)slot + (b & ~3));
    const uint32_t lo = *(const lds_u32 *)(uintptr_t)at;
    const uint32_t hi = *(const lds_u32 *)(uintptr_t)(at + 4);
    return __builtin_amdgcn_alignbit(hi, lo, 8u * (uint32_t)(b & 3));
}

// Phase 2 for one lane: decode the codes starting in [pos, stop) and store
// their exponent bytes from tile position `at` on (a tile position is the
// output index minus the block's 8-aligned base).
//
// Unranged (the block fits one tile): every lookup stores all four slots of
// its decode entry.  A slot past the entry's complete codes holds a stray
// byte, but the lane's next step starts storing exactly there; only the
// lane's last step can leave stray bytes behind, and at most 3 of them, all
// on the following lanes' first 3 positions.  Symbols decoded past the
// lane's own codes are the true next symbols (the bits are real), so they
// are harmless.  rewrite_head() then restores every lane's first symbols.
// With kRanged only positions in [r0, r0 + kTileCap) are stored, at
// tile[position - r0], one checked slot at a time.
template <bool kRanged>
__device__ __forceinline__ void decode_codes(const uint8_t *lds_dec, const uint16_t *lut,
                                             uint32_t n_tables, uint32_t d0, uint32_t d1,
                                             uint32_t d2, uint32_t pos, uint32_t stop,
                                             uint32_t tile_addr, uint32_t at, uint32_t r0) {
    const uint32_t e0 = d0 << 3, e1 = __builtin_amdgcn_alignbit(d1, d0, 29),
                   e2 = __builtin_amdgcn_alignbit(d2, d1, 29);
    constexpr uint32_t kMask = ((1u << kDecodeBits) - 1) << 3;
    // pos | (LDS address of the next exponent byte) << 16; ranged: position << 16
    uint32_t acc = pos | ((kRanged ? at : tile_addr + at) << 16);
    const uint32_t stop0 = stop < 32u ? stop : 32u;
    auto step = [&](uint32_t hi, uint32_t lo, uint32_t dhi, uint32_t dlo) {
        const uint32_t w = __builtin_amdgcn_alignbit(hi, lo, acc);
        const uint2 dv = *reinterpret_cast<const uint2 *>(lds_dec + (w & kMask));
        if (!kRanged) {
            // all four symbol bytes in one (possibly unaligned) LDS store; a
            // code longer than the table's window then overwrites byte 0
            const uint32_t at_lds = acc >> 16;
            *(lds_u32 *)(uintptr_t)at_lds = dv.y;
            uint32_t inc = dv.x;
            if (dv.x < 0x10000u) {
                const uint32_t e = lookup8(lut, __builtin_amdgcn_alignbit(dhi, dlo, acc), n_tables);
                *(lds_u8 *)(uintptr_t)at_lds = (uint8_t)e;
                inc = leaf_len(e) | 0x10000u;
            }
            acc += inc;
        } else {
            uint32_t syms, k;
            if (dv.x < 0x10000u) {
                const uint32_t e = lookup8(lut, __builtin_amdgcn_alignbit(dhi, dlo, acc), n_tables);
                syms = e & 0xFFu;
                k = 1;
                acc += leaf_len(e) | 0x10000u;
            } else {
                syms = dv.y;
                k = dv.x >> 16;
                acc += dv.x;
            }
            const uint32_t p = (acc >> 16) - k;  // position of the first symbol
            for (uint32_t j = 0; j < 4; ++j) {
                const uint32_t rel = p + j - r0;
                if (j < k && rel < (uint32_t)kTileCap)
                    *((lds_u8 *)(uintptr_t)(tile_addr + rel)) = (uint8_t)(syms >> (8 * j));
            }
        }
    };
    while ((acc & 0xFFFFu) < stop0) step(e1, e0, d1, d0);  // at most 64 steps, as above
    while ((acc & 0xFFFFu) < stop) step(e2, e1, d2, d1);
}

// After every lane's unranged decode: store this lane's first min(3, cnt)
// symbols again (the previous lanes' last steps may have overwritten them).
// Runs after the loops of all lanes, so these stores land last.
__device__ __forceinline__ void rewrite_head(const uint8_t *lds_dec, const uint16_t *lut,
                                             uint32_t n_tables, uint32_t d0, uint32_t d1,
                                             uint32_t d2, uint32_t pos, uint32_t cnt,
                                             uint32_t addr) {
    constexpr uint32_t kMask = ((1u << kDecodeBits) - 1) << 3;
    const uint32_t need = cnt < 3u ? cnt : 3u;
    uint32_t done = 0;
    for (int it = 0; it < 3 && done < need; ++it) {
        const bool second = pos >= 32;  // codes start below bit 64 of the slice
        const uint32_t lo = second ? d1 : d0, hi = second ? d2 : d1;
        const uint32_t wd = __builtin_amdgcn_alignbit(hi, lo, pos);  // plain window
        const uint2 dv = *reinterpret_cast<const uint2 *>(lds_dec + ((wd << 3) & kMask));
        lds_u8 *o = (lds_u8 *)(uintptr_t)(addr + done);
        uint32_t k, b, syms;
        if (dv.x < 0x10000u) {
            const uint32_t e = lookup8(lut, wd, n_tables);
            syms = e & 0xFFu;
            k = 1;
            b = leaf_len(e);
        } else {
            syms = dv.y;
            k = dv.x >> 16;
            b = dv.x & 0xFFFFu;
        }
        for (uint32_t j = 0; j < 3; ++j)
            if (j < k && done + j < need) o[j] = (uint8_t)(syms >> (8 * j));
        done += k;
        pos += b;
    }
}

// One BF16 word from an exponent byte and a sign|mantissa byte.
__device__ __forceinline__ uint32_t join1(uint32_t e, uint32_t sm) {
    return ((sm & 0x80u) << 8) | ((e & 0xFFu) << 7) | (sm & 0x7Fu);
}

// at least 6 waves per SIMD: keeps the register budget at 80 VGPRs, the
// most that still lets 3 workgroups of 8 waves share a CU
#ifndef DF11_WAVES_PER_EU
#define DF11_WAVES_PER_EU 6
#endif
#define DF11_OCCUPANCY_HINT __attribute__((amdgpu_waves_per_eu(DF11_WAVES_PER_EU)))
__global__ __launch_bounds__(kGroupThreads) DF11_OCCUPANCY_HINT void df11_decode_kernel(DecodeArgs a) {
    // LDS: per-wave regions (staging slots, then the exponent tile) | decode
    // table in one static array (fixed offsets fold into the ds_read/ds_write
    // immediates, and the regions sit at the lowest addresses so that their
    // addresses fit the 16-bit field of the phase accumulators), then the 8-bit
    // tables in dynamic LDS.
    __shared__ __attribute__((aligned(16))) uint8_t lds_static[kStaticLds];
    __shared__ uint32_t wg_next;  // next block index of this workgroup's share
    if (threadIdx.x == 0) wg_next = 0;
    uint8_t *tiles = lds_static;
    uint2 *dec_t = reinterpret_cast<uint2 *>(lds_static + kTilesBytes);
    extern __shared__ uint4 smem_u4[];
    uint16_t *lut = reinterpret_cast<uint16_t *>(smem_u4);
    const uint32_t hier_bytes = a.n_tables * kTableBytes;
    if (lds_offset(tiles) + kTilesBytes > 0x10000u) {
        // tile addresses would not fit the accumulator: decode nothing
        if (threadIdx.x == 0 && a.status) atomicAdd(a.status, 1u);
        return;
    }

    uint4 *lut_u4 = reinterpret_cast<uint4 *>(lut);
    for (uint32_t i = threadIdx.x; i < hier_bytes / 16; i += kGroupThreads) lut_u4[i] = a.luts[i];
    __syncthreads();
    build_decode_table(lut, dec_t, a.n_tables, a.max_len);
    __syncthreads();

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    uint8_t *tile = tiles + wave * kTileBytes;
    const uint32_t tile_addr = lds_offset(tile);
    const uint8_t *lds_dec = reinterpret_cast<const uint8_t *>(dec_t);

    // XCD-contiguous assignment: group g runs on XCD g % 8 (workgroups are
    // dispatched round-robin over the XCDs) and owns the blocks
    // range_lo + 8 slot + {0..7} + i * stride of that XCD's range.
    const uint32_t xcd = blockIdx.x % kXcds;
    const uint32_t slot = blockIdx.x / kXcds;
    const uint32_t groups_per_xcd = gridDim.x / kXcds;
    const uint32_t range_lo = xcd * a.blocks_per_xcd;
    uint32_t range_hi = range_lo + a.blocks_per_xcd;
    range_hi = range_hi < a.n_blocks ? range_hi : a.n_blocks;
    const uint32_t stride = groups_per_xcd * kWavesPerGroup;

    // slice g = 64 b + lane: its stream dwords are 2g..2g+2 and its 5-bit
    // gap field sits at bit 5 * lane of the block's 320 gap bits (dword 10 b)
    auto stream_at = [&](uint32_t blk) { return a.stream + 2 * (blk * DF11_BLOCK_SLICES + lane); };
    auto gaps_at = [&](uint32_t blk) { return a.gaps + 10 * blk + ((5 * lane) >> 5); };
    const uint32_t gap_shift = (5 * lane) & 31;

    // The workgroup's blocks go to its waves one at a time through an LDS
    // counter, claimed a block ahead, so a wave that the SIMD serves less
    // often simply takes fewer blocks.  (Workgroups keep fixed shares: global
    // atomics would queue every wave of an XCD on one address.)
    auto wg_block = [&](uint32_t i) {
        const uint32_t blk = range_lo + slot * kWavesPerGroup + (i % kWavesPerGroup) +
                             (i / kWavesPerGroup) * stride;
        return blk < range_hi ? blk : 0xFFFFFFFFu;
    };
    auto claim = [&]() {
        uint32_t v = 0;
        if (lane == 0) v = atomicAdd(&wg_next, 1u);
        return v;
    };
    uint32_t b = wg_block(__builtin_amdgcn_readfirstlane(claim()));
    uint32_t nb = b != 0xFFFFFFFFu ? wg_block(__builtin_amdgcn_readfirstlane(claim())) : 0xFFFFFFFFu;
    uint32_t nd0 = 0, nd1 = 0, nd2 = 0, ng0 = 0, ng1 = 0, npos = 0;
    if (b != 0xFFFFFFFFu) {
        const uint32_t *sp = stream_at(b);
        nd0 = sp[0], nd1 = sp[1], nd2 = sp[2];
        const uint32_t *gp = gaps_at(b);
        ng0 = gp[0], ng1 = gp[1];
        npos = a.block_pos[b + (lane & 1)];
    }
    asm volatile("" ::"v"(nd0), "v"(nd1), "v"(nd2), "v"(ng0), "v"(ng1), "v"(npos));
    uint32_t k = 0;
    while (b != 0xFFFFFFFFu) {
        // Rotate the wave's issue priority from block to block.  At equal
        // priority a SIMD issues the oldest wave first, so with fixed shares of
        // blocks the youngest workgroups of a CU would finish far behind the
        // oldest; rotating priorities spreads that preference over all waves.
        switch ((k + wave + slot) & 3u) {
        case 0: __builtin_amdgcn_s_setprio(0); break;
        case 1: __builtin_amdgcn_s_setprio(1); break;
        case 2: __builtin_amdgcn_s_setprio(2); break;
        default: __builtin_amdgcn_s_setprio(3); break;
        }
        const uint32_t p0 = __builtin_amdgcn_readlane(npos, 0);
        const uint32_t p1 = __builtin_amdgcn_readlane(npos, 1);
        const uint32_t d0 = nd0, d1 = nd1, d2 = nd2, gw0 = ng0, gw1 = ng1;
        uint32_t pend = 0;
        if (nb != 0xFFFFFFFFu) {
            const uint32_t *sp = stream_at(nb);
            nd0 = sp[0], nd1 = sp[1], nd2 = sp[2];
            const uint32_t *gp = gaps_at(nb);
            ng0 = gp[0], ng1 = gp[1];
            npos = a.block_pos[nb + (lane & 1)];
            pend = claim();
        }
        const bool sane = p1 >= p0 && p1 <= a.n && p1 - p0 <= (uint32_t)kMaxBlockCodes;
        const uint32_t base = p0 & ~7u;
        const uint32_t groups = sane ? (p1 - base + 7) >> 3 : 0u;
        const bool one_pass = groups * 8 + 4 <= (uint32_t)kTileCap;
        // groups [full_lo, full_hi) lie inside [p0, p1) and get 16-byte stores;
        // the partial head group (p0 unaligned) and tail group (p1 unaligned)
        // are stored one element per lane: lanes 0-7 the head, 8-15 the tail
        const uint32_t full_lo = p0 != base ? 1u : 0u;
        const uint32_t full_hi = sane ? (p1 - base) >> 3 : 0u;
        const uint32_t head_end = p0 != base ? (p1 < base + 8 ? p1 : base + 8) : p0;
        const uint32_t tail_lo = base + 8 * full_hi > head_end ? base + 8 * full_hi : head_end;
        const uint32_t edge_i = lane < 8 ? base + lane : base + 8 * full_hi + (lane - 8);
        const bool edge = sane && lane < 16 &&
                          (lane < 8 ? (edge_i >= p0 && edge_i < head_end)
                                    : (edge_i >= tail_lo && edge_i < p1));
        const uint32_t edge_sm = edge ? a.signmant[edge_i] : 0u;

        // sign|mantissa of this lane's first output groups, loaded up front
        uint2 smv[kPrefetchGroups];
#pragma unroll
        for (int i = 0; i < kPrefetchGroups; ++i) {
            const uint32_t j = lane + kWave * i;
            smv[i] = one_pass && j < groups
                         ? *reinterpret_cast<const uint2 *>(a.signmant + base + 8 * j)
                         : make_uint2(0, 0);
        }

        const uint32_t gw = __builtin_amdgcn_alignbit(gw1, gw0, gap_shift);
        const uint32_t gap = gw & 31u, gap_next = (gw >> 5) & 31u;
        // the stop bit and the stream end relative to this lane's slice, in
        // 32 bits: wave-uniform 64-bit differences to the block start,
        // clamped far outside the block's 4096 bits, minus the lane's offset
        const uint64_t blk_bit = (uint64_t)b * (DF11_BLOCK_SLICES * DF11_SLICE_BITS);
        auto near = [](int64_t v) {
            return (int32_t)(v < -(1 << 30) ? -(1 << 30) : (v > (1 << 30) ? (1 << 30) : v));
        };
        const int32_t lane_bit = (int32_t)(lane * DF11_SLICE_BITS);
        const int32_t rel = near((int64_t)a.stop_bit - (int64_t)blk_bit) - lane_bit;
        // codes of this lane start in [gap, lim); the last one ends at `end`:
        // the next slice's first code start, or the stream's end for the lane
        // holding the final code
        const uint32_t lim = rel <= 0 ? 0u : (rel >= 64 ? 64u : (uint32_t)rel);
        const uint32_t end = rel > 0 && rel <= 64
                                 ? (uint32_t)(near((int64_t)a.total_bits - (int64_t)blk_bit) - lane_bit)
                                 : 64u + gap_next;

        // ---- phase 1: decode into the lane's staging slot, counting
        const uint32_t slot = tile_addr + kStageBase + lane * kStageStride;
        const uint32_t cnt =
            lim ? stage_codes(lds_dec, lut, a.n_tables, d0, d1, d2, pad_ones(d0, (int)end, 0),
                              pad_ones(d1, (int)end, 32), pad_ones(d2, (int)end, 64), gap, lim,
                              slot, tile_addr + kTileBytes - 8)
                : 0u;

        // wave-wide prefix sum of the counts
        const uint32_t incl = wave_inclusive_sum(cnt);
        const uint32_t excl = incl - cnt;
        const uint32_t total = __builtin_amdgcn_readlane(incl, kWave - 1);
        // vmcnt is an in-order counter that also counts stores: take the wait
        // for the next block's prefetched inputs here, on every path and before
        // this block's stores are issued, so that no later wait (the loop
        // header's in particular) has to cover those stores
        asm volatile("" ::"v"(nd0), "v"(nd1), "v"(nd2), "v"(ng0), "v"(ng1), "v"(npos));
        {
            const uint32_t nnb = nb != 0xFFFFFFFFu ? wg_block(__builtin_amdgcn_readfirstlane(pend))
                                                   : 0xFFFFFFFFu;
            b = nb;  // the rest of this iteration only uses p0, p1 and the lanes' data
            nb = nnb;
            ++k;
        }
        // a count that disagrees with block_pos means a corrupt block: report
        // it and leave its output unwritten
        if (!sane || total != p1 - p0) {
            if (lane == 0 && a.status) atomicAdd(a.status, 1u);
            continue;
        }
        const uint32_t at = (p0 - base) + excl;  // tile position of this lane's first symbol
        const uint32_t stop = lim ? lim : 0u;
        const uint32_t start = lim ? gap : 0u;
        // every lane's codes fit its slot (then the block fits one tile, too)
        // and every lane before the last code holds enough for its neighbour
        const bool last_lane = incl == total;
        const bool odd = cnt > (uint32_t)kStageCodes || (cnt < (uint32_t)kStageMinCodes && !last_lane);
        const bool staged = one_pass && __builtin_amdgcn_ballot_w64(odd) == 0;

        wave_lds_sync();
        if (staged) {
            // ---- move the staged exponents to their tile positions
            const uint32_t tail = staged_tail(slot, cnt);
            const uint32_t prev = (uint32_t)__builtin_amdgcn_ds_bpermute(
                (int)(((lane + kWave - 1) % kWave) * 4), (int)tail);
            place_staged(slot, tile_addr + at, cnt, prev, last_lane);
            wave_lds_sync();
        } else if (one_pass) {
            // ---- phase 2: decode the real bits again into the tile, then
            // restore each lane's head
            decode_codes<false>(lds_dec, lut, a.n_tables, d0, d1, d2, start, stop, tile_addr, at, 0);
            wave_lds_sync();
            rewrite_head(lds_dec, lut, a.n_tables, d0, d1, d2, start, cnt, tile_addr + at);
            wave_lds_sync();
        }
        if (one_pass) {
            // ---- merge with sign|mantissa, 8 BF16 per lane per 16-byte store
#pragma unroll
            for (int i = 0; i < kPrefetchGroups; ++i) {
                const uint32_t j = lane + kWave * i;
                if (j >= full_lo && j < full_hi)
                    *reinterpret_cast<uint4 *>(a.out + base + 8 * j) =
                        join8(*reinterpret_cast<const uint2 *>(tile + 8 * j), smv[i]);
            }
            for (uint32_t j = lane + kWave * kPrefetchGroups; j < full_hi; j += kWave) {
                const uint2 sm = *reinterpret_cast<const uint2 *>(a.signmant + base + 8 * j);
                *reinterpret_cast<uint4 *>(a.out + base + 8 * j) =
                    join8(*reinterpret_cast<const uint2 *>(tile + 8 * j), sm);
            }
            if (edge) a.out[edge_i] = (uint16_t)join1(tile[edge_i - base], edge_sm);
            wave_lds_sync();
        } else {
            // more symbols than one tile holds: decode again per tile-sized window
            for (uint32_t r0 = 0; r0 < groups * 8; r0 += kTileCap) {
                decode_codes<true>(lds_dec, lut, a.n_tables, d0, d1, d2, start, stop, tile_addr,
                                   at, r0);
                wave_lds_sync();
                const uint32_t j_hi = (r0 + kTileCap) / 8 < groups ? (r0 + kTileCap) / 8 : groups;
                for (uint32_t j = r0 / 8 + lane; j < j_hi; j += kWave) {
                    if (j < full_lo || j >= full_hi) continue;  // edge groups: below
                    const uint2 sm = *reinterpret_cast<const uint2 *>(a.signmant + base + 8 * j);
                    *reinterpret_cast<uint4 *>(a.out + base + 8 * j) =
                        join8(*reinterpret_cast<const uint2 *>(tile + 8 * j - r0), sm);
                }
                const uint32_t er = edge_i - base - r0;
                if (edge && er < (uint32_t)kTileCap)
                    a.out[edge_i] = (uint16_t)join1(tile[er], edge_sm);
                wave_lds_sync();
            }
        }
    }
}

// Launch shape per device: compute units and resident workgroups per CU for
// each table count (the LDS footprint depends on it).
constexpr int kMaxDevices = 16;
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_occ[kMaxDevices][DF11_MAX_TABLES + 1];

// dynamic LDS per workgroup: the 8-bit tables (tiles and fast tables are static)
size_t lds_bytes(uint32_t n_tables) { return (size_t)n_tables * kTableBytes; }

int launch_groups(int dev, uint32_t n_tables, uint32_t n_blocks, uint32_t max_groups,
                  int *groups) {
    if (dev < 0 || dev >= kMaxDevices) return DF11_ERR_HIP;
    int cus = g_cus[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return DF11_ERR_HIP;
        g_cus[dev].store(cus, std::memory_order_relaxed);
    }
    int occ = g_occ[dev][n_tables].load(std::memory_order_relaxed);
    if (occ <= 0) {
        // a workgroup whose LDS exceeds what one CU can give it would never be
        // dispatched: refuse the launch instead
        int max_lds = 0;
        hipFuncAttributes attr;
        if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess ||
            hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(df11_decode_kernel)) !=
                hipSuccess)
            return DF11_ERR_HIP;
        if (attr.sharedSizeBytes + lds_bytes(n_tables) > (size_t)max_lds) return DF11_ERR_TABLES;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, df11_decode_kernel, kGroupThreads,
                                                         lds_bytes(n_tables)) != hipSuccess)
            return DF11_ERR_HIP;
        if (occ <= 0) return DF11_ERR_TABLES;
#ifdef DF11_MAX_OCCUPANCY
        occ = occ < DF11_MAX_OCCUPANCY ? occ : DF11_MAX_OCCUPANCY;
#endif
        g_occ[dev][n_tables].store(occ, std::memory_order_relaxed);
    }
    // a multiple of the XCD count, no more than there are blocks to share
    const uint64_t want = ((uint64_t)n_blocks + kWavesPerGroup - 1) / kWavesPerGroup;
    uint64_t cap = (uint64_t)cus * (uint64_t)occ;
    if (max_groups) {
        const uint64_t lim = max_groups < (uint32_t)kXcds ? kXcds : max_groups / kXcds * kXcds;
        cap = cap < lim ? cap : lim;
    }
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
    int st = launch_groups(dev, s->n_tables, s->n_blocks, s->max_groups, &groups);
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
