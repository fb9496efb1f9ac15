// df11_decode: gfx950 (CDNA4) kernel that turns a DF11-encoded tensor back
// into its BF16 words, the fused variant that multiplies the decoded weights
// with 1-8 input vectors instead of storing them, and their C-ABI launchers.
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
//  * workgroups are persistent; each stages in LDS the 8-bit tables and the
//    multi-code decode table that the host library appends to them (built
//    once per codebook), indexed by the next 11 stream bits:
//    each entry holds the first (up to 4) codes that end inside a window
//    narrower than the longest code -- their symbols packed in one dword,
//    their total length and their number -- so one lookup yields up to 4
//    exponents; codes longer than the window fall back to the 8-bit tables;
//  * a lane's 96 relevant stream bits live in three VGPRs; windows come from
//    one funnel shift (v_alignbit) of a dword pair, with the data pre-shifted
//    so that the window's low bits are already the table's byte offset;
//  * the phases are merged: phase 1 decodes each lane's codes once, into a
//    private 40-byte staging slot in LDS (each step ORs its symbols into the
//    slot's partly filled dword and writes the next dword, so every LDS store
//    is aligned), and its step count is the lane's code count.  The count
//    is exact because the bits after the lane's last code are forced to 1
//    for these lookups: all ones is a prefix of the longest code, which
//    never completes inside the window.  After the scan each lane copies
//    its staged exponents to its output position in the wave's tile.  Lanes
//    with more codes than a slot holds (only near-flat streams of 1- and
//    2-bit codes) send their wave down the page's own route: decode the real
//    bits again, straight into the tile;
//  * exponent bytes are kept rotated right by one bit from the decode table
//    to the merge, so that joining them with sign|mantissa bytes takes only
//    bit-field inserts and byte permutes (no shifts);
//  * the merge joins 8 exponents with 8 prefetched sign|mantissa bytes per
//    lane and writes one 16-byte store (the fused variant instead takes the
//    dot products of the 8 words with each input vector, with a copy of the
//    loop without row selects for blocks that lie in one row);
//  * workgroups take blocks in runs of 8 from one window that moves through
//    the whole stream, so all XCDs read and write near each other: one
//    contiguous range per XCD put eight write fronts in step and was slower.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <type_traits>

#include "df11.h"
#include "df11_internal.h"

namespace {

constexpr int kWave = 64;
constexpr int kWavesPerGroup = 8;
constexpr int kGroupThreads = kWave * kWavesPerGroup;
constexpr int kMaxBlockCodes = DF11_BLOCK_SLICES * DF11_SLICE_BITS;  // all 1-bit codes
// Staging: lane t's phase-1 exponents at byte 4 + t * stride of its wave's
// LDS region (the 4 bytes in front let every lane read the dword before its
// slot); a lane with more than kCodes codes, or with fewer than 3 before the
// block's last code, sends the wave to the re-decode route.  The tile that
// phase 2 fills reuses the region.  32 codes per lane (40-byte slots) serve
// every stream of ordinary weights (about 24 codes of 2.6 bits per 64-bit
// slice); streams of much shorter codes get 56 codes per lane in 60-byte
// slots, in a larger region (both run 3 workgroups per CU).  (The odd stride
// of 15 dwords starts consecutive lanes' slots on distinct LDS banks; with
// 64-byte slots they start on a few banks, and their conflicts cost the wide
// kernel a quarter of its speed.)
constexpr int kStageBase = 4;
constexpr int kStageMinCodes = 3;
// phase 1 writes at most 71 bytes from a slot's start, whatever the data: a
// step begins below bit 64 and every code takes at least one bit, so the
// last step begins after at most 63 codes and stores two aligned dwords
constexpr int kStageReach = 63 + 8;
template <int kCodes, int kStride> struct StageGeo {
    static constexpr int kStageCodes = kCodes;
    static constexpr int kStageStride = kStride;
    // the wave's region: all 64 slots, 8-aligned
    static constexpr int kTileBytes = (kStageBase + 63 * kStageStride + kStageReach + 7) / 8 * 8;
    // exponent bytes one tile holds; blocks with more symbols take several passes
    static constexpr int kTileCap = kTileBytes - 40;
    static constexpr int kTilesBytes = 8 * kTileBytes;
    static_assert(kTileCap % 8 == 0, "tile windows must stay 8-aligned");
    static_assert(kStageStride % 4 == 0 && kTileBytes % 8 == 0, "staging dwords are aligned");
    static_assert(kStageStride >= kStageCodes + 4, "a full slot takes 4 stray bytes");
    static_assert(kCodes % 4 == 0, "slots move in whole dwords");
    static_assert(kTilesBytes < 0x10000, "tile addresses must fit 16 bits");
};
using NarrowGeo = StageGeo<32, 40>;
using WideGeo = StageGeo<56, 60>;
template <int kCodes>
using GeoFor = typename std::conditional<kCodes == NarrowGeo::kStageCodes, NarrowGeo, WideGeo>::type;
constexpr int kStageStride = NarrowGeo::kStageStride;
constexpr int kStageCodes = NarrowGeo::kStageCodes;
constexpr int kTileCap = NarrowGeo::kTileCap;
constexpr int kTileBytes = NarrowGeo::kTileBytes;
static_assert(kTileCap == 2560 && kTileBytes == 2600, "the narrow geometry");
constexpr int kTableBytes = 256 * 2;
constexpr int kXcds = 8;
// multi-code decode table (built by the host after the 8-bit tables of the
// table image, copied to LDS by each workgroup): index width
constexpr int kDecodeBits = (int)df11_internal::kDecodeTableBits;
constexpr int kDecodeBytes = (int)df11_internal::kDecodeTableBytes;
static_assert(kWavesPerGroup == 8, "one region per wave of a workgroup");
constexpr int kTilesBytes = NarrowGeo::kTilesBytes;
constexpr int kStaticLds = kTilesBytes + kDecodeBytes;
// sign|mantissa groups of 8 per lane loaded up front
constexpr int kPrefetchGroups = 2;
static_assert(kPrefetchGroups >= 1, "at least one group is prefetched");

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) uint64_t lds_u64;
// global-memory views: pointers that reach device code inside a struct would
// otherwise be accessed with FLAT instructions, which also count against the
// LDS wait counter
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const uint16_t g_cu16;
typedef __attribute__((address_space(1))) const u32x4 g_cu32x4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) float g_f32;
typedef __attribute__((address_space(1))) const u32x2 g_cu32x2;
typedef __attribute__((address_space(1))) f32x4 g_f32x4;
typedef __attribute__((address_space(1))) uint32_t g_u32;

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
    // codes start strictly before bit 4096 stop_blk + stop_rem; the stream
    // ends at bit 4096 end_blk + end_rem (block index and offset in it)
    uint32_t stop_blk, stop_rem, end_blk, end_rem;
    uint32_t n_blocks;
    uint32_t n_tables;
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

// Workgroup barrier that orders LDS accesses only: global loads in flight
// stay in flight across it (__syncthreads would wait for them).
__device__ __forceinline__ void group_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exponent bytes travel through LDS rotated right by one bit (bit 0 in bit
// 7): the decode table holds them so, and a symbol taken from the 8-bit
// tables is rotated with rotr8.  Then a BF16 word's high byte is
// (e' & 0x7F) | (sm & 0x80) and its low byte (e' & 0x80) | (sm & 0x7F): one
// v_bfi_b32 each per 4 words, and a v_perm_b32 interleaves them.
__device__ __forceinline__ uint32_t rotr8(uint32_t e) {  // e: an 8-bit table entry or a byte
    const uint32_t b = e & 0xFFu;
    return ((b >> 1) | (b << 7)) & 0xFFu;
}

__device__ __forceinline__ uint4 join8(uint2 e, uint2 s) {
    const uint32_t hx = (e.x & 0x7F7F7F7Fu) | (s.x & 0x80808080u);
    const uint32_t lx = (e.x & 0x80808080u) | (s.x & 0x7F7F7F7Fu);
    const uint32_t hy = (e.y & 0x7F7F7F7Fu) | (s.y & 0x80808080u);
    const uint32_t ly = (e.y & 0x80808080u) | (s.y & 0x7F7F7F7Fu);
    uint4 o;  // words 2i, 2i+1: [low 2i, high 2i, low 2i+1, high 2i+1]
    o.x = __builtin_amdgcn_perm(hx, lx, 0x05010400u);
    o.y = __builtin_amdgcn_perm(hx, lx, 0x07030602u);
    o.z = __builtin_amdgcn_perm(hy, ly, 0x05010400u);
    o.w = __builtin_amdgcn_perm(hy, ly, 0x07030602u);
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
// Stores are aligned: each step ORs its symbols (unused table bytes are 0)
// into the slot's partly filled dword with an LDS atomic and writes the dword
// after it; the two dwords stay inside the wave's region for any data
// (kStageReach).  The OR in LDS replaces a register copy of the partly filled
// dword, which took four more VALU instructions per step.
__device__ __forceinline__ uint32_t stage_codes(const uint8_t *lds_dec, const uint16_t *lut,
                                                uint32_t n_tables, uint32_t d0, uint32_t d1,
                                                uint32_t d2, uint32_t f0, uint32_t f1, uint32_t f2,
                                                uint32_t pos, uint32_t stop, uint32_t slot) {
    // pre-shift by 3: window bits [3, 3+W) are the entry's byte offset
    const uint32_t e0 = f0 << 3, e1 = __builtin_amdgcn_alignbit(f1, f0, 29),
                   e2 = __builtin_amdgcn_alignbit(f2, f1, 29);
    constexpr uint32_t kMask = ((1u << kDecodeBits) - 1) << 3;
    uint32_t acc = pos | (slot << 16);  // pos | (LDS address of the next byte) << 16
    // Each step ORs its symbols into the dword holding the next byte, whose
    // bytes from that one on are 0, and writes the dword after it whole.  The
    // symbol bytes an entry does not use are 0, so both dwords end with zeros
    // past the last symbol: the invariant holds for the next step, and the
    // first dword only needs clearing here.
    *(lds_u32 *)(uintptr_t)slot = 0;
    auto step = [&](uint32_t hi, uint32_t lo, uint32_t dhi, uint32_t dlo) {
        const uint32_t w = __builtin_amdgcn_alignbit(hi, lo, acc);
        const uint2 dv = *reinterpret_cast<const uint2 *>(lds_dec + (w & kMask));
        uint32_t inc = dv.x, syms = dv.y;
        if (dv.x < 0x10000u) {  // longer than the window: 8-bit tables, real bits
            const uint32_t e = lookup8(lut, __builtin_amdgcn_alignbit(dhi, dlo, acc), n_tables);
            syms = rotr8(e);
            inc = leaf_len(e) | 0x10000u;
        }
        const uint32_t at = acc >> 16;
        // bits 13..17 of acc: pos >> 13 (always 0) | (byte address & 3) << 3
        const uint64_t t = (uint64_t)syms << __builtin_amdgcn_ubfe(acc, 13, 5);
        lds_u32 *p = (lds_u32 *)(uintptr_t)(at & ~3u);
        __atomic_fetch_or(p, (uint32_t)t, __ATOMIC_RELAXED);  // ds_or_b32, no return
        p[1] = (uint32_t)(t >> 32);
        acc += inc;
    };
    // every step moves at least one bit on (table entries and 8-bit leaves
    // have lengths >= 1), so a lane takes at most 64 steps, whatever the data
    const uint32_t stop0 = stop < 32u ? stop : 32u;
    while ((acc & 0xFFFFu) < stop0) step(e1, e0, d1, d0);
    while ((acc & 0xFFFFu) < stop) step(e2, e1, d2, d1);
    return (acc >> 16) - slot;
}

// After the scan: move the lane's `cnt` staged exponents (at most kStageCodes) from its
// slot to tile address `dst` with aligned dword stores only.  The lane writes
// every aligned dword that ends inside its own output bytes; the first of
// them starts with the previous lane's last bytes (`prev`, taken from that
// lane's slot), and the lane holding the block's last code (`last_lane`) also
// writes its final, partial dword.  Every tile dword is thus written exactly
// once, provided each lane before the last one holds at least 3 codes.
template <class G = NarrowGeo>
__device__ __forceinline__ void place_staged(uint32_t slot, uint32_t dst, uint32_t cnt,
                                             uint32_t prev, bool last_lane) {
    constexpr int kN = G::kStageCodes / 4;
    uint32_t v[kN + 1];
#pragma unroll
    for (int i = 0; i < kN; ++i) v[i] = *(const lds_u32 *)(uintptr_t)(slot + 4 * i);
    v[kN] = 0;
    const uint32_t s = dst & 3u, a0 = dst & ~3u;
    // byte t of output dword j is byte 4 j + t - s of the lane's sequence;
    // v_perm picks it from {v[j], v[j - 1]} (bytes 4..7 and 0..3)
    const uint32_t sel = 0x07060504u - s * 0x01010101u;
    const int last = cnt == 0 ? -1
                     : last_lane ? (int)((s + cnt - 1) >> 2)
                                 : (int)((s + cnt) >> 2) - 1;
#pragma unroll
    for (int j = 0; j <= kN; ++j) {
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
template <bool kRanged, class G = NarrowGeo>
__device__ __forceinline__ void decode_codes(const uint8_t *lds_dec, const uint16_t *lut,
                                             uint32_t n_tables, uint32_t d0, uint32_t d1,
                                             uint32_t d2, uint32_t pos, uint32_t stop,
                                             uint32_t tile_addr, uint32_t at, uint32_t r0) {
    const uint32_t e0 = d0 << 3, e1 = __builtin_amdgcn_alignbit(d1, d0, 29),
                   e2 = __builtin_amdgcn_alignbit(d2, d1, 29);
    constexpr uint32_t kMask = ((1u << kDecodeBits) - 1) << 3;
    // pos | (LDS address of the next exponent byte) << 16; ranged: position << 16
    uint32_t acc = pos | ((kRanged ? at : tile_addr + at) << 16);
    const uint32_t tile_end = tile_addr + G::kTileBytes - 4;  // last 4-byte store address
    const uint32_t stop0 = stop < 32u ? stop : 32u;
    auto step = [&](uint32_t hi, uint32_t lo, uint32_t dhi, uint32_t dlo) {
        const uint32_t w = __builtin_amdgcn_alignbit(hi, lo, acc);
        const uint2 dv = *reinterpret_cast<const uint2 *>(lds_dec + (w & kMask));
        if (!kRanged) {
            // all four symbol bytes in one (possibly unaligned) LDS store; a
            // code longer than the table's window then overwrites byte 0.
            // Valid data stays inside the block's symbols; a corrupt stream
            // that decodes more codes here than phase 1 counted is held to
            // the wave's region
            const uint32_t at_lds = (acc >> 16) < tile_end ? (acc >> 16) : tile_end;
            *(lds_u32 *)(uintptr_t)at_lds = dv.y;
            uint32_t inc = dv.x;
            if (dv.x < 0x10000u) {
                const uint32_t e = lookup8(lut, __builtin_amdgcn_alignbit(dhi, dlo, acc), n_tables);
                *(lds_u8 *)(uintptr_t)at_lds = (uint8_t)rotr8(e);
                inc = leaf_len(e) | 0x10000u;
            }
            acc += inc;
        } else {
            uint32_t syms, k;
            if (dv.x < 0x10000u) {
                const uint32_t e = lookup8(lut, __builtin_amdgcn_alignbit(dhi, dlo, acc), n_tables);
                syms = rotr8(e);
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
                if (j < k && rel < (uint32_t)G::kTileCap)
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
            syms = rotr8(e);
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
// one BF16 word from a rotated exponent byte and its sign|mantissa byte
__device__ __forceinline__ uint32_t join1(uint32_t e, uint32_t sm) {
    return ((((e & 0x7Fu) | (sm & 0x80u)) << 8) | (e & 0x80u) | (sm & 0x7Fu)) & 0xFFFFu;
}

// What a decoded block's BF16 words go to.  The kernel body calls
// begin(p0, p1, base, j_lo, j_hi) once a block's output range [p0, p1) is
// known (its full 8-word groups are j in [j_lo, j_hi), group j at output
// index base + 8 j;
// this lane handles j = lane + 64 i); for each full group starting at output
// index pos, f = fetch(pos) (issued early: the sink's own loads for that
// group) and later group(pos, e8, sm8, f); one() for the single head/tail
// words; and end(block) after the block.
struct StoreSink {  // plain decode: BF16 words to out[]
    uint16_t *out;
    struct Fetched {};
    static constexpr int kEarlyFetch = 0;
    static constexpr bool kRowPaths = false;
    __device__ __forceinline__ bool one_row() const { return false; }
    __device__ __forceinline__ void begin(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t) {}
    template <bool = false>
    __device__ __forceinline__ Fetched fetch(uint32_t) const { return {}; }
    template <bool = false>
    __device__ __forceinline__ void group(uint32_t pos, uint2 e8, uint2 sm8, Fetched) {
        *reinterpret_cast<uint4 *>(out + pos) = join8(e8, sm8);
    }
    template <bool = false>
    __device__ __forceinline__ void one(uint32_t pos, uint32_t e, uint32_t sm) {
        out[pos] = (uint16_t)join1(e, sm);
    }
    __device__ __forceinline__ void end(uint32_t, uint32_t) {}
};

// Decode of a stream stored in operand-tile order back to the row-major
// words.  The group of 8 words at tile-order position pos (tile t = pos >>
// 9, lane group g = (pos >> 3) & 63) holds row 16 r + g % 16, columns 32 k +
// 8 (g / 16) .. + 7 of its matrix, where r = u / ks and k = u % ks for u the
// tile's index within the matrix (ks = cols / 32): 8 consecutive words of one
// row, one 16-byte store.
constexpr int kTileMapMats = 16;
struct TileMap {
    uint32_t n_mats;
    uint32_t tile0[kTileMapMats + 1];  // each matrix's first tile; then the total
    uint32_t ks[kTileMapMats];         // k-steps (cols / 32)
    uint32_t cols[kTileMapMats];
    uint64_t off[kTileMapMats];        // each matrix's first word
};

// The map in LDS, one 32-bit word per field: tile0[17], ks[16], cols[16],
// off_lo[16], off_hi[16].
constexpr int kTileMapWords = (kTileMapMats + 1) + 4 * kTileMapMats;

struct TileStoreSink {
    uint16_t *out;
    const uint32_t *lmap;  // in LDS
    uint32_t n_mats, lane;
    struct Fetched {};
    static constexpr int kEarlyFetch = 0;
    static constexpr bool kRowPaths = false;
    __device__ __forceinline__ bool one_row() const { return false; }
    // the block's matrix when all its tiles are in one (the usual case)
    bool single;
    uint32_t m_tile0, m_ks, m_cols;
    uint64_t m_off;
    float m_inv;
    __device__ __forceinline__ uint32_t tile0(uint32_t i) const { return lmap[i]; }
    __device__ __forceinline__ uint32_t ks(uint32_t i) const { return lmap[kTileMapMats + 1 + i]; }
    __device__ __forceinline__ uint32_t cols(uint32_t i) const {
        return lmap[2 * kTileMapMats + 1 + i];
    }
    __device__ __forceinline__ uint64_t off(uint32_t i) const {
        return lmap[3 * kTileMapMats + 1 + i] | ((uint64_t)lmap[4 * kTileMapMats + 1 + i] << 32);
    }
    // the matrix of tile t: the matrices 1.. starting at or before it (a
    // search through the map in LDS, the same for every lane when t is)
    __device__ __forceinline__ uint32_t matrix(uint32_t t) const {
        uint32_t m = 0;
        for (uint32_t i = 1; i < n_mats; ++i) m += t >= tile0(i) ? 1u : 0u;
        return m;
    }
    __device__ __forceinline__ void begin(uint32_t p0, uint32_t p1, uint32_t, uint32_t, uint32_t) {
        const uint32_t t0 = p0 >> 9, t1 = p1 > p0 ? (p1 - 1) >> 9 : t0;
        const uint32_t m = __builtin_amdgcn_readfirstlane(matrix(t0));
        m_tile0 = tile0(m), m_ks = ks(m), m_cols = cols(m), m_off = off(m);
        single = t1 < tile0(m + 1);
        m_inv = 1.0f / (float)m_ks;
    }
    // row-major index of the group at tile-order position pos (8-aligned)
    __device__ __forceinline__ uint64_t where(uint32_t pos) const {
        uint32_t t0 = m_tile0, k_steps = m_ks, c = m_cols;
        uint64_t o = m_off;
        float inv = m_inv;
        const uint32_t t = pos >> 9, g = (pos >> 3) & 63u;
        if (!single) {  // a block across matrices (small ones): each group looks its own up
            const uint32_t m = matrix(t);
            t0 = tile0(m), k_steps = ks(m), c = cols(m), o = off(m);
            inv = 1.0f / (float)k_steps;
        }
        // u / k_steps through the reciprocal: u < 2^23, so the float quotient
        // is off by at most one, and one step fixes it
        const uint32_t u = t - t0;
        uint32_t r = (uint32_t)((float)u * inv);
        if ((uint64_t)r * k_steps > u) --r;
        else if (u - r * k_steps >= k_steps) ++r;
        const uint32_t k = u - r * k_steps;
        return o + (uint64_t)(16 * r + (g & 15u)) * c + 32 * k + 8 * (g >> 4);
    }
    template <bool = false>
    __device__ __forceinline__ Fetched fetch(uint32_t) const { return {}; }
    template <bool = false>
    __device__ __forceinline__ void group(uint32_t pos, uint2 e8, uint2 sm8, Fetched) {
        *reinterpret_cast<uint4 *>(out + where(pos)) = join8(e8, sm8);
    }
    template <bool = false>
    __device__ __forceinline__ void one(uint32_t pos, uint32_t e, uint32_t sm) {
        out[where(pos & ~7u) + (pos & 7u)] = (uint16_t)join1(e, sm);
    }
    __device__ __forceinline__ void end(uint32_t, uint32_t) {}
};

// Fused product: y_b = W x_b for row-major matrices laid end to end in the
// decoded output, for up to 8 input vectors x_b at once.  Every matrix row
// holds at least 2048 words, so one block's output (at most 4096 words)
// touches at most three rows; a wave sums its products per row and input
// vector and stores those sums and the first row's index per block.
// df11_gemm_reduce_kernel then adds them per row in block order, so the
// result does not depend on scheduling.
constexpr int kGemvMaxMats = 16;
constexpr uint32_t kGemvMinCols = 2048;
constexpr int kGemmMaxBatch = 8;
// floats of partial sums per block for a batch capacity of kB vectors: three
// rows x kB sums, then the first row's index, rounded up to whole float4s
constexpr int partial_floats(int kB) { return (3 * kB + 1 + 3) / 4 * 4; }
struct GemvArgs {
    const uint16_t *x;      // all matrices' BF16 x vectors, matrix m's at x + xoff[m];
                            // vector b at x + b * x_stride
    float *y;               // all matrices' results, matrix m's at y + yoff[m];
                            // vector b's at y + b * y_stride
    float *partials;        // per block: partial_floats(capacity) floats
    uint32_t *row_blk;      // per row and one more: 2 b + (row starts after block b's start)
    uint64_t x_stride, y_stride;
    uint32_t batch;         // vectors in use, 1..capacity
    uint32_t n_mats;
    uint32_t off[kGemvMaxMats + 1];   // first output index of each matrix; off[n_mats] = n
    uint32_t cols[kGemvMaxMats];
    uint32_t row0[kGemvMaxMats + 1];  // running row count before each matrix
    uint32_t xoff[kGemvMaxMats];
    uint32_t yoff[kGemvMaxMats];
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }

// a.lo * b.lo + a.hi * b.hi + c for two BF16 pairs (v_dot2c_f32_bf16)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// 8 sign|mantissa bytes (8-byte aligned).  (Non-temporal loads here were
// slower for the decode and no faster for the fused product.)
__device__ __forceinline__ uint2 load_sm8(const uint8_t *p) {
    const u32x2 v = *(g_cu32x2 *)p;
    return make_uint2(v.x, v.y);
}

// x moved across lanes by one DPP control (lanes without a source read 0)
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xF, false));
}

// Sum over the 64 lanes (every lane gets it) with the DPP row shifts and
// broadcasts of wave_inclusive_sum, in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0x111, 0xF>(v);  // row_shr:1
    v += dpp_f<0x112, 0xF>(v);  // row_shr:2
    v += dpp_f<0x114, 0xF>(v);  // row_shr:4
    v += dpp_f<0x118, 0xF>(v);  // row_shr:8
    v += dpp_f<0x142, 0xA>(v);  // row_bcast:15
    v += dpp_f<0x143, 0xC>(v);  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// The matrix table in LDS (copied from the kernel argument once per workgroup).
struct GemvTable {
    uint32_t off[kGemvMaxMats + 1];
    uint32_t cols[kGemvMaxMats];
    float inv_cols[kGemvMaxMats];  // 1 / cols, for the row of an output index
    uint32_t row0[kGemvMaxMats + 1];
    uint32_t xoff[kGemvMaxMats];
};

template <int kB>
struct DotSink {
    // inputs of a lane's first groups are fetched at the block's top, before
    // phase 1, only while they fit the register budget (one vector: 79 VGPRs)
    static constexpr int kEarlyFetch = kB == 1;
    // blocks inside one row (most of them: rows are longer than blocks)
    // take a copy of the merge loop without the row selects
    static constexpr bool kRowPaths = true;
    __device__ __forceinline__ bool one_row() const { return !row1; }
    const GemvTable *tab;  // in LDS
    const g_cu16 *x;       // BF16
    g_f32x4 *partials;
    g_u32 *row_blk;
    uint64_t x_stride;
    uint32_t batch, n_mats, lane;
    uint32_t n, total_rows;
    bool first_here;     // the block's first row starts at the block's first weight
    bool last_words;     // the block holds the last weight
    uint32_t s1, s2;     // first output index of the block's second and third row
    // x index - output index: d0 in the first row, + dd1 from the second,
    // + dd2 from the third (selecting among three fields would become an
    // indexed load and keep this object in scratch memory)
    uint32_t d0, dd1, dd2;
    uint32_t grow;       // global index of the block's first row
    bool row1, row2;     // the block reaches its second / third row
    float acc0[kB], acc1[kB], acc2[kB];
    __device__ __forceinline__ void begin(uint32_t p0, uint32_t p1, uint32_t, uint32_t, uint32_t) {
        // lane l reads table entry l once (all entries in one LDS round
        // trip); the block's matrix m = the entries 1..n_mats-1 starting at
        // or before p0, counted by ballot, and its fields come back by readlane
        const uint32_t l = lane <= (uint32_t)kGemvMaxMats ? lane : (uint32_t)kGemvMaxMats;
        const uint32_t lc = l < (uint32_t)kGemvMaxMats ? l : (uint32_t)kGemvMaxMats - 1;
        const uint32_t off_l = tab->off[l], row0_l = tab->row0[l];
        const uint32_t cols_l = tab->cols[lc], xoff_l = tab->xoff[lc];
        const float inv_l = tab->inv_cols[lc];
        const uint32_t m = (uint32_t)__builtin_popcountll(
            __builtin_amdgcn_ballot_w64(lane >= 1 && lane < n_mats && off_l <= p0));
        auto at = [](uint32_t v, uint32_t i) { return (uint32_t)__builtin_amdgcn_readlane((int)v, (int)i); };
        const uint32_t c0 = at(cols_l, m), off_m = at(off_l, m);
        // row = q / c0 through the reciprocal: q < 2^32 and c0 >= 2048, so
        // the float quotient is off by at most one, and one step fixes it
        const uint32_t q = p0 - off_m;
        uint32_t r = (uint32_t)((float)q * __int_as_float((int)at(__float_as_uint(inv_l), m)));
        if ((uint64_t)r * c0 > q) --r;
        else if (q - r * c0 >= c0) ++r;
        const uint32_t s0 = off_m + r * c0;
        grow = at(row0_l, m) + r;
        first_here = s0 == p0;
        last_words = p1 == n && p0 < n;
        d0 = at(xoff_l, m) - s0;
        s1 = s0 + c0;
        const uint32_t m1 = (m + 1 < n_mats && s1 >= at(off_l, m + 1)) ? m + 1 : m;
        const uint32_t d1 = at(xoff_l, m1) - s1;
        s2 = s1 + at(cols_l, m1);
        const uint32_t m2 = (m1 + 1 < n_mats && s2 >= at(off_l, m1 + 1)) ? m1 + 1 : m1;
        const uint32_t d2 = at(xoff_l, m2) - s2;
        dd1 = d1 - d0;
        dd2 = d2 - d1;
        row1 = s1 < p1;
        row2 = s2 < p1;
#pragma unroll
        for (int b = 0; b < kB; ++b) acc0[b] = acc1[b] = acc2[b] = 0.0f;
    }
    template <bool kOne>
    __device__ __forceinline__ void add(uint32_t pos, int b, float v) {
        if constexpr (kOne) {
            acc0[b] += v;
        } else {
            acc0[b] += pos < s1 ? v : 0.0f;
            acc1[b] += pos >= s1 && pos < s2 ? v : 0.0f;
            acc2[b] += pos >= s2 ? v : 0.0f;
        }
    }
    // x index of output index pos; modular 32-bit arithmetic keeps it exact
    template <bool kOne>
    __device__ __forceinline__ uint32_t xi(uint32_t pos) const {
        if constexpr (kOne) return pos + d0;
        return pos + d0 + (pos >= s1 ? dd1 : 0u) + (pos >= s2 ? dd2 : 0u);
    }
    struct Fetched {
        u32x4 v[kB];  // the group's 8 BF16 inputs of each vector
    };
    template <bool kOne = false>
    __device__ __forceinline__ Fetched fetch(uint32_t pos) const {
        Fetched f;
        const g_cu16 *p = x + xi<kOne>(pos);
#pragma unroll
        for (int b = 0; b < kB; ++b)
            f.v[b] = b == 0 || (uint32_t)b < batch ? *(const g_cu32x4 *)(p + b * x_stride)
                                                  : u32x4{0, 0, 0, 0};
        return f;
    }
    template <bool kOne = false>
    __device__ __forceinline__ void group(uint32_t pos, uint2 e8, uint2 sm8, const Fetched &f) {
        const uint4 w = join8(e8, sm8);
        // BF16 x BF16 products are exact in fp32; pairs of them are added to
        // the running fp32 sum by the packed dot instruction
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            float v = dot2_bf16(w.x, f.v[b].x, 0.0f);
            v = dot2_bf16(w.y, f.v[b].y, v);
            v = dot2_bf16(w.z, f.v[b].z, v);
            v = dot2_bf16(w.w, f.v[b].w, v);
            add<kOne>(pos, b, v);
        }
    }
    template <bool kOne = false>
    __device__ __forceinline__ void one(uint32_t pos, uint32_t e, uint32_t sm) {
        const float w = bf16_lo(join1(e, sm));
        const g_cu16 *p = x + xi<kOne>(pos);
#pragma unroll
        for (int b = 0; b < kB; ++b)
            if (b == 0 || (uint32_t)b < batch) add<kOne>(pos, b, w * bf16_lo(p[b * x_stride]));
    }
    __device__ __forceinline__ void end(uint32_t blk, uint32_t) {
        // the block of each row that starts here (the reduce's row ranges),
        // and after the last row the block past the last weight
        if (lane == 0) {
            if (first_here) row_blk[grow] = 2 * blk;
            if (row1) row_blk[grow + 1] = 2 * blk + 1;
            if (row2) row_blk[grow + 2] = 2 * blk + 1;
            if (last_words) row_blk[total_rows] = 2 * (blk + 1);
        }
        // sums only for the rows the block reaches: the reduce reads a
        // block's slot for a row only if the block holds words of that row
        if constexpr (kB == 1) {
            const float t0 = wave_sum(acc0[0]);
            const float t1 = row1 ? wave_sum(acc1[0]) : 0.0f;
            const float t2 = row2 ? wave_sum(acc2[0]) : 0.0f;
            if (lane == 0) partials[blk] = f32x4{t0, t1, t2, __uint_as_float(grow)};
        } else {
            // one sum at a time, stored by lane 0 as soon as it is formed
            g_f32 *dst = (g_f32 *)partials + (uint64_t)blk * partial_floats(kB);
            if (lane == 0) dst[3 * kB] = __uint_as_float(grow);
#pragma unroll
            for (int b = 0; b < kB; ++b) {
                const float t = wave_sum(acc0[b]);
                if (lane == 0) dst[b] = t;
            }
            if (row1) {
#pragma unroll
                for (int b = 0; b < kB; ++b) {
                    const float t = wave_sum(acc1[b]);
                    if (lane == 0) dst[kB + b] = t;
                }
            }
            if (row2) {
#pragma unroll
                for (int b = 0; b < kB; ++b) {
                    const float t = wave_sum(acc2[b]);
                    if (lane == 0) dst[2 * kB + b] = t;
                }
            }
        }
    }
};

// at least 6 waves per SIMD: keeps the register budget at 80 VGPRs, the
// most that still lets 3 workgroups of 8 waves share a CU
constexpr int kWavesPerEu = 6;
#define DF11_OCCUPANCY_HINT __attribute__((amdgpu_waves_per_eu(kWavesPerEu)))
template <class G, class Sink>
__device__ __forceinline__ void decode_blocks(const DecodeArgs &a, Sink &sink) {
    // LDS: per-wave regions (staging slots, then the exponent tile) | decode
    // table in one static array (fixed offsets fold into the ds_read/ds_write
    // immediates, and the regions sit at the lowest addresses so that their
    // addresses fit the 16-bit field of the phase accumulators), then the 8-bit
    // tables in dynamic LDS.
    __shared__ __attribute__((aligned(16))) uint8_t lds_static[G::kTilesBytes + kDecodeBytes];
    __shared__ uint32_t wg_next;  // next block index of this workgroup's share
    if (threadIdx.x == 0) wg_next = kWavesPerGroup;  // claims 0..7: one per wave, below
    uint8_t *tiles = lds_static;
    uint2 *dec_t = reinterpret_cast<uint2 *>(lds_static + G::kTilesBytes);
    extern __shared__ uint4 smem_u4[];
    uint16_t *lut = reinterpret_cast<uint16_t *>(smem_u4);
    const uint32_t hier_bytes = a.n_tables * kTableBytes;
    if (lds_offset(tiles) + G::kTilesBytes > 0x10000u) {
        // tile addresses would not fit the accumulator: decode nothing
        if (threadIdx.x == 0 && a.status) atomicAdd(a.status, 1u);
        return;
    }

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    uint8_t *tile = tiles + wave * G::kTileBytes;
    const uint32_t tile_addr = lds_offset(tile);
    const uint8_t *lds_dec = reinterpret_cast<const uint8_t *>(dec_t);

    // One window over the whole stream: group g owns the blocks
    // 8 g + {0..7} + i * 8 * groups, so at any moment all XCDs work on one
    // contiguous run of blocks.  (Splitting the blocks into one contiguous
    // range per XCD was slower: eight write fronts moving in step through
    // memory.)  `slot` tells apart the groups that share an XCD.
    const uint32_t slot = blockIdx.x / kXcds;
    const uint32_t stride = gridDim.x * kWavesPerGroup;

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
        const uint32_t blk = blockIdx.x * kWavesPerGroup + (i % kWavesPerGroup) +
                             (i / kWavesPerGroup) * stride;
        return blk < a.n_blocks ? blk : 0xFFFFFFFFu;
    };
    auto claim = [&]() {
        uint32_t v = 0;
        if (lane == 0) v = atomicAdd(&wg_next, 1u);
        return v;
    };
    // The tables' loads go first (the 8-bit tables, up to 16 of them in one
    // 16-B load per thread, more below; then the decode table), then each
    // wave's first block: wave w takes the workgroup's claim w without the
    // counter, so that its loads are in flight while the tables are staged.
    const uint32_t lut_u4_count = hier_bytes / 16;
    const bool lut_one_load = lut_u4_count <= kGroupThreads;
    uint4 lv = {0, 0, 0, 0};
    if (lut_one_load && threadIdx.x < lut_u4_count) lv = a.luts[threadIdx.x];
    // the decode table follows the 8-bit tables in the image: two 16-byte
    // loads per thread
    static_assert(kDecodeBytes == 2 * 16 * kGroupThreads, "two uint4 per thread");
    const uint4 *dec_src = a.luts + lut_u4_count;
    const uint4 dv0 = dec_src[threadIdx.x], dv1 = dec_src[threadIdx.x + kGroupThreads];
    uint32_t b = wg_block(wave);
    uint32_t nd0, nd1, nd2, ng0, ng1, npos;
    {
        // (a wave without blocks loads block 0's inputs and ignores them:
        // unconditional loads let the staging below wait for the table load
        // alone)
        const uint32_t b0 = b != 0xFFFFFFFFu ? b : 0;
        const uint32_t *sp = stream_at(b0);
        nd0 = sp[0], nd1 = sp[1], nd2 = sp[2];
        const uint32_t *gp = gaps_at(b0);
        ng0 = gp[0], ng1 = gp[1];
        npos = a.block_pos[b0 + (lane & 1)];
    }

    uint4 *lut_u4 = reinterpret_cast<uint4 *>(lut);
    if (lut_one_load) {
        if (threadIdx.x < lut_u4_count) lut_u4[threadIdx.x] = lv;
    } else {
        for (uint32_t i = threadIdx.x; i < lut_u4_count; i += kGroupThreads) lut_u4[i] = a.luts[i];
    }
    reinterpret_cast<uint4 *>(dec_t)[threadIdx.x] = dv0;
    reinterpret_cast<uint4 *>(dec_t)[threadIdx.x + kGroupThreads] = dv1;
    group_lds_sync();

    uint32_t nb = b != 0xFFFFFFFFu ? wg_block(__builtin_amdgcn_readfirstlane(claim())) : 0xFFFFFFFFu;
    asm volatile("" ::"v"(nd0), "v"(nd1), "v"(nd2), "v"(ng0), "v"(ng1), "v"(npos));
    uint32_t k = 0, cur_blk = 0;
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
        const bool one_pass = groups * 8 + 4 <= (uint32_t)G::kTileCap;
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
                         ? load_sm8(a.signmant + base + 8 * j)
                         : make_uint2(0, 0);
        }

        // a sink that fetches inputs: its block set-up and the inputs of the
        // lane's first groups go out here, so that their latency passes
        // during phase 1 (a lane without a group there fetches for full_lo)
        typename Sink::Fetched fx0[kPrefetchGroups];
        if constexpr (Sink::kEarlyFetch != 0) {
            if (sane) {
                sink.begin(p0, p1, base, 0, 0);
                if (one_pass && full_lo < full_hi) {
#pragma unroll
                    for (int i = 0; i < kPrefetchGroups; ++i) {
                        const uint32_t j = lane + kWave * i;
                        const uint32_t jf = j >= full_lo && j < full_hi ? j : full_lo;
                        fx0[i] = sink.fetch(base + 8 * jf);
                    }
                }
            }
        }
        const uint32_t gw = __builtin_amdgcn_alignbit(gw1, gw0, gap_shift);
        const uint32_t gap = gw & 31u, gap_next = (gw >> 5) & 31u;
        // the stop bit and the stream end relative to this lane's slice:
        // wave-uniform offsets from the block start, exact within a block of
        // it and clamped far outside farther away, minus the lane's offset
        auto from_block = [&](uint32_t blk, uint32_t rem) {
            const int32_t d = (int32_t)(blk - b);  // block indices are below 2^27
            return d > 1 ? (1 << 30) : (d < -1 ? -(1 << 30) : d * 4096 + (int32_t)rem);
        };
        // codes of a lane start in [gap, lim); the last one ends at `end`: the
        // next slice's first code start, or the stream's end for the lane
        // holding the final code.  f* are the slice's dwords with the bits from
        // `end` on set to 1.  A block whose every slice lies before the stop
        // bit (all but the stream's last block or two) has lim = 64 and end =
        // 64 + gap_next in every lane, which leaves only the third dword to pad
        // (wave-uniform branch)
        const int32_t stop_at = from_block(a.stop_blk, a.stop_rem);
        uint32_t lim, f0, f1, f2;
        if (stop_at > kWave * DF11_SLICE_BITS) {
            lim = 64u;
            f0 = d0;
            f1 = d1;
            f2 = d2 | (0xFFFFFFFFu << gap_next);
        } else {
            const int32_t lane_bit = (int32_t)(lane * DF11_SLICE_BITS);
            const int32_t rel = stop_at - lane_bit;
            lim = rel <= 0 ? 0u : (rel >= 64 ? 64u : (uint32_t)rel);
            const uint32_t end = rel > 0 && rel <= 64
                                     ? (uint32_t)(from_block(a.end_blk, a.end_rem) - lane_bit)
                                     : 64u + gap_next;
            f0 = pad_ones(d0, (int)end, 0);
            f1 = pad_ones(d1, (int)end, 32);
            f2 = pad_ones(d2, (int)end, 64);
        }

        // ---- phase 1: decode into the lane's staging slot, counting
        const uint32_t slot = tile_addr + kStageBase + lane * G::kStageStride;
        const uint32_t cnt =
            lim ? stage_codes(lds_dec, lut, a.n_tables, d0, d1, d2, f0, f1, f2, gap, lim, slot)
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
            cur_blk = b;
            b = nb;  // the rest of this iteration only uses p0, p1 and the lanes' data
            nb = nnb;
            ++k;
        }
        // a count that disagrees with block_pos means a corrupt block: report
        // it and leave its output unwritten
        if (!sane || total != p1 - p0) {
            if (lane == 0 && a.status) atomicAdd(a.status, 1u);
            if (sane) {  // leave a defined (empty) result for the block
                if constexpr (Sink::kEarlyFetch == 0) sink.begin(p0, p1, base, 0, 0);
                sink.end(cur_blk, lane);
            }
            continue;
        }
        if constexpr (Sink::kEarlyFetch == 0)  // (a fetching sink began at the block's top)
            sink.begin(p0, p1, base, one_pass ? full_lo : 0u, one_pass ? full_hi : 0u);
        const uint32_t at = (p0 - base) + excl;  // tile position of this lane's first symbol
        const uint32_t stop = lim ? lim : 0u;
        const uint32_t start = lim ? gap : 0u;
        // every lane's codes fit its slot (then the block fits one tile, too)
        // and every lane before the last code holds enough for its neighbour
        const bool last_lane = incl == total;
        const bool odd = cnt > (uint32_t)G::kStageCodes || (cnt < (uint32_t)kStageMinCodes && !last_lane);
        const bool staged = one_pass && __builtin_amdgcn_ballot_w64(odd) == 0;

        wave_lds_sync();
        if (staged) {
            // ---- move the staged exponents to their tile positions
            const uint32_t tail = staged_tail(slot, cnt);
            const uint32_t prev = (uint32_t)__builtin_amdgcn_ds_bpermute(
                (int)(((lane + kWave - 1) % kWave) * 4), (int)tail);
            place_staged<G>(slot, tile_addr + at, cnt, prev, last_lane);
            wave_lds_sync();
        } else if (one_pass) {
            // ---- phase 2: decode the real bits again into the tile, then
            // restore each lane's head
            decode_codes<false, G>(lds_dec, lut, a.n_tables, d0, d1, d2, start, stop, tile_addr, at, 0);
            wave_lds_sync();
            rewrite_head(lds_dec, lut, a.n_tables, d0, d1, d2, start, cnt, tile_addr + at);
            wave_lds_sync();
        }
        if (one_pass && Sink::kRowPaths) {
            // a sink with row paths gets the block's one-row case as its own
            // copy of the loop: the branch is taken once per block.  (The
            // plain decode keeps the single loop below: the same code shape
            // for it measured 26% slower, from scheduling alone.)
            if constexpr (Sink::kRowPaths) {
            auto tile_e8 = [&](uint32_t j) { return *reinterpret_cast<const uint2 *>(tile + 8 * j); };
            auto merge = [&](auto one_row) {
                constexpr bool kOne = decltype(one_row)::value;
                // ---- merge with sign|mantissa, 8 BF16 per lane per group; where
                // the sink allows, its loads for the first rounds are issued
                // together first (a lane without a group there fetches for group
                // full_lo)
                if constexpr (Sink::kEarlyFetch != 0) {
                    const typename Sink::Fetched *fx = fx0;  // fetched at the block's top
#pragma unroll
                    for (int i = 0; i < kPrefetchGroups; ++i) {
                        const uint32_t j = lane + kWave * i;
                        if (j >= full_lo && j < full_hi)
                            sink.template group<kOne>(base + 8 * j, tile_e8(j), smv[i], fx[i]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < kPrefetchGroups; ++i) {
                        const uint32_t j = lane + kWave * i;
                        if (j >= full_lo && j < full_hi)
                            sink.template group<kOne>(base + 8 * j, tile_e8(j), smv[i],
                                                      sink.template fetch<kOne>(base + 8 * j));
                    }
                }
                for (uint32_t j = lane + kWave * kPrefetchGroups; j < full_hi; j += kWave) {
                    const uint2 sm = load_sm8(a.signmant + base + 8 * j);
                    sink.template group<kOne>(base + 8 * j, tile_e8(j), sm,
                                              sink.template fetch<kOne>(base + 8 * j));
                }
                if (edge) sink.template one<kOne>(edge_i, tile[edge_i - base], edge_sm);
            };
            if (sink.one_row()) merge(std::integral_constant<bool, true>{});
            else merge(std::integral_constant<bool, false>{});
            wave_lds_sync();
            }
        } else if (one_pass) {
            // ---- merge with sign|mantissa, 8 BF16 per lane per group (a sink
            // without row paths fetches nothing ahead)
            static_assert(Sink::kRowPaths || Sink::kEarlyFetch == 0, "early fetches need the row-path loop");
#pragma unroll
            for (int i = 0; i < kPrefetchGroups; ++i) {
                const uint32_t j = lane + kWave * i;
                if (j >= full_lo && j < full_hi)
                    sink.group(base + 8 * j, *reinterpret_cast<const uint2 *>(tile + 8 * j),
                               smv[i], sink.fetch(base + 8 * j));
            }
            for (uint32_t j = lane + kWave * kPrefetchGroups; j < full_hi; j += kWave) {
                const uint2 sm = load_sm8(a.signmant + base + 8 * j);
                sink.group(base + 8 * j, *reinterpret_cast<const uint2 *>(tile + 8 * j), sm,
                           sink.fetch(base + 8 * j));
            }
            if (edge) sink.one(edge_i, tile[edge_i - base], edge_sm);
            wave_lds_sync();
        } else {
            // more symbols than one tile holds: decode again per tile-sized window
            for (uint32_t r0 = 0; r0 < groups * 8; r0 += G::kTileCap) {
                decode_codes<true, G>(lds_dec, lut, a.n_tables, d0, d1, d2, start, stop, tile_addr,
                                   at, r0);
                wave_lds_sync();
                const uint32_t j_hi = (r0 + G::kTileCap) / 8 < groups ? (r0 + G::kTileCap) / 8 : groups;
                for (uint32_t j = r0 / 8 + lane; j < j_hi; j += kWave) {
                    if (j < full_lo || j >= full_hi) continue;  // edge groups: below
                    const uint2 sm = load_sm8(a.signmant + base + 8 * j);
                    sink.group(base + 8 * j, *reinterpret_cast<const uint2 *>(tile + 8 * j - r0), sm,
                               sink.fetch(base + 8 * j));
                }
                const uint32_t er = edge_i - base - r0;
                if (edge && er < (uint32_t)G::kTileCap) sink.one(edge_i, tile[er], edge_sm);
                wave_lds_sync();
            }
        }
        sink.end(cur_blk, lane);
    }
}

template <int kCodes>
__global__ __launch_bounds__(kGroupThreads) DF11_OCCUPANCY_HINT void df11_decode_kernel(DecodeArgs a) {
    StoreSink sink{a.out};
    decode_blocks<GeoFor<kCodes>>(a, sink);
}

// The decode of a tile-order stream into row-major words.  Thread 0 copies
// the map to LDS (constant indices into the kernel argument); the decode's
// first workgroup barrier, after its table staging, orders the copy before
// any block's use of it.
__global__ __launch_bounds__(kGroupThreads) DF11_OCCUPANCY_HINT void df11_decode_tiled_kernel(
    DecodeArgs a, TileMap m) {
    __shared__ uint32_t lmap[kTileMapWords];
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i <= kTileMapMats; ++i) lmap[i] = m.tile0[i];
#pragma unroll
        for (int i = 0; i < kTileMapMats; ++i) {
            lmap[kTileMapMats + 1 + i] = m.ks[i];
            lmap[2 * kTileMapMats + 1 + i] = m.cols[i];
            lmap[3 * kTileMapMats + 1 + i] = (uint32_t)m.off[i];
            lmap[4 * kTileMapMats + 1 + i] = (uint32_t)(m.off[i] >> 32);
        }
    }
    TileStoreSink sink;
    sink.out = a.out;
    sink.lmap = lmap;
    sink.n_mats = m.n_mats;
    sink.lane = threadIdx.x % kWave;
    decode_blocks<NarrowGeo>(a, sink);
}

// Occupancy of the fused product kernel for capacity kB.  Up to 2 vectors
// it keeps the decode's budget of 80 VGPRs (3 workgroups per CU); 4 and 8
// vectors need more registers and run 2 workgroups per CU.
template <int kB> struct GemmOccupancy {
    static constexpr int kValue = kB <= 2 ? kWavesPerEu : 4;
};

template <int kB>
__global__ __launch_bounds__(kGroupThreads)
__attribute__((amdgpu_waves_per_eu(GemmOccupancy<kB>::kValue)))
void df11_gemm_kernel(DecodeArgs a, GemvArgs g) {
    // the matrix table goes to LDS with constant indices (indexing the kernel
    // argument at run time would make the compiler copy it to scratch); the
    // first barrier in decode_blocks publishes it
    __shared__ GemvTable tab;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i <= kGemvMaxMats; ++i) {
            tab.off[i] = g.off[i];
            tab.row0[i] = g.row0[i];
        }
#pragma unroll
        for (int i = 0; i < kGemvMaxMats; ++i) {
            tab.cols[i] = g.cols[i];
            tab.inv_cols[i] = g.cols[i] ? 1.0f / (float)g.cols[i] : 0.0f;
            tab.xoff[i] = g.xoff[i];
        }
    }
    DotSink<kB> sink;
    sink.tab = &tab;
    sink.x = (const g_cu16 *)g.x;
    sink.partials = (g_f32x4 *)g.partials;
    sink.row_blk = (g_u32 *)g.row_blk;
    sink.n = a.n;
    sink.total_rows = g.row0[g.n_mats];
    sink.x_stride = g.x_stride;
    sink.batch = g.batch;
    sink.n_mats = g.n_mats;
    sink.lane = threadIdx.x % kWave;
    decode_blocks<NarrowGeo>(a, sink);
}

// y of every row and vector: the sums its blocks stored, in block order.
template <int kB>
__global__ __launch_bounds__(256) void df11_gemm_reduce_kernel(GemvArgs g, uint32_t n_blocks) {
    const uint32_t row = blockIdx.x * 256 + threadIdx.x;
    if (row >= g.row0[g.n_mats]) return;
    // the row's matrix and its fields, with constant indices into the
    // kernel argument (all entries load at once; a loop would wait for each)
    uint32_t m = 0;
#pragma unroll
    for (int i = 1; i < kGemvMaxMats; ++i) m += (uint32_t)i < g.n_mats && row >= g.row0[i] ? 1u : 0u;
    uint32_t row0_m = 0, yoff_m = 0;
#pragma unroll
    for (int i = 0; i < kGemvMaxMats; ++i)
        if ((uint32_t)i == m) row0_m = g.row0[i], yoff_m = g.yoff[i];
    const uint32_t r = row - row0_m;
    // the row's blocks: from the one holding its first word to the one
    // holding its last, which is the next row's first block, or the block
    // before when the next row starts a block; each of them holds words of
    // the row, so its slot for the row was written.  (The entries of rows
    // that start in a corrupt block's place are left over from earlier
    // calls: the range is only kept inside the workspace.)
    const uint32_t e0 = g.row_blk[row], e1 = g.row_blk[row + 1];
    const uint32_t lo0 = e0 >> 1, hi0 = (e1 >> 1) + (e1 & 1u);
    const uint32_t lo = lo0 < n_blocks ? lo0 : n_blocks;
    const uint32_t hi = hi0 < n_blocks ? hi0 : n_blocks;
    constexpr int kP = partial_floats(kB);
    float sum[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) sum[b] = 0.0f;
    if constexpr (kB == 1) {
        // one vector load per record, four blocks at a time; the records stay
        // in named registers (an array here was copied through LDS to index it)
        auto take = [&](const f32x4 &rec, bool use) {
            const uint32_t seg = row - __float_as_uint(rec.w);  // 0, 1 or 2
            if (use && seg < 3) sum[0] += seg == 0 ? rec.x : seg == 1 ? rec.y : rec.z;
        };
        const g_f32x4 *q = (const g_f32x4 *)g.partials;
        for (uint32_t blk = lo; blk < hi; blk += 4) {
            const f32x4 ra = q[blk];
            const f32x4 rb = q[blk + 1 < hi ? blk + 1 : blk];
            const f32x4 rc = q[blk + 2 < hi ? blk + 2 : blk];
            const f32x4 rd = q[blk + 3 < hi ? blk + 3 : blk];
            take(ra, true);
            take(rb, blk + 1 < hi);
            take(rc, blk + 2 < hi);
            take(rd, blk + 3 < hi);
        }
    } else if constexpr (kB <= 4) {
        // whole records (16-byte loads), two blocks at a time; each loaded
        // word is pinned to a register so that the segment select stays a
        // select between registers (for 8 vectors the records are too large
        // for this to pay: measured slower)
        constexpr int kV = kP / 4;
        const g_f32x4 *q = (const g_f32x4 *)g.partials;
        for (uint32_t blk = lo; blk < hi; blk += 2) {
            const uint32_t bb = blk + 1 < hi ? blk + 1 : blk;
            f32x4 ra[kV], rb[kV];
#pragma unroll
            for (int v = 0; v < kV; ++v) {
                ra[v] = q[(uint64_t)blk * kV + v];
                rb[v] = q[(uint64_t)bb * kV + v];
            }
#pragma unroll
            for (int v = 0; v < kV; ++v) asm volatile("" : "+v"(ra[v]), "+v"(rb[v]));
            auto take = [&](const f32x4 (&r)[kV], bool use) {
                const uint32_t seg = row - __float_as_uint(r[(3 * kB) / 4][(3 * kB) % 4]);
                if (use && seg < 3) {
#pragma unroll
                    for (int b = 0; b < kB; ++b) {
                        const float v0 = r[b / 4][b % 4];
                        const float v1 = r[(kB + b) / 4][(kB + b) % 4];
                        const float v2 = r[(2 * kB + b) / 4][(2 * kB + b) % 4];
                        sum[b] += seg == 0 ? v0 : seg == 1 ? v1 : v2;
                    }
                }
            };
            take(ra, true);
            take(rb, blk + 1 < hi);
        }
    } else {
        for (uint32_t blk = lo; blk < hi; ++blk) {
            const float *p = g.partials + (uint64_t)blk * kP;
            const uint32_t seg = row - __float_as_uint(p[3 * kB]);  // 0, 1 or 2
            if (seg < 3) {
#pragma unroll
                for (int b = 0; b < kB; ++b) sum[b] += p[seg * kB + b];
            }
        }
    }
#pragma unroll
    for (int b = 0; b < kB; ++b)
        if ((uint32_t)b < g.batch) g.y[b * g.y_stride + yoff_m + r] = sum[b];
}

// ------------------------------------------------------------ tiled product
//
// y_b = W x_b for 1-64 vectors on the matrix cores, from a stream whose
// weights are in operand-tile order (df11_tile_order): per matrix, row tiles
// of 16 rows, then k-steps of 32 columns, then for each lane L of a
// v_mfma_f32_16x16x32_bf16 the 8 weights W[16 rt + L % 16][32 ks + 8 (L / 16)
// + 0..7].  So 512 consecutive decoded words are one operand tile A, and the
// lane that takes group L of a tile from the LDS exponent tile holds exactly
// its part of A.  (Row tiles of 32 rows, whose two halves share each k-step's
// inputs, halve the bytes of x read but were slower overall: half as many
// workgroups left more of them to a last, partly filled round.)
//
// One workgroup per segment (the 16 rows of one row tile); its waves take the
// segment's blocks in turn (blk_lo + wave + 8 i: a fixed assignment, so sums
// are formed in the same order on every run), decode each block into the
// wave's LDS tile as the plain decode does, and multiply every operand tile
// the block holds with the 32 x 16 slabs of x for each group of 16 vectors,
// accumulating in registers (words outside the block or the segment are zero
// in A).  At the end the waves' sums are added in LDS in wave order and the
// workgroup writes its 16 results per vector.  Segments of the widest
// matrices are launched first, so that the longest workgroups start early.
constexpr int kTiledMaxBatch = 64;

struct TiledArgs {
    const uint16_t *x;        // matrix m's inputs at x + xoff; vector b at + b * x_stride
    // or, when xt is set, the inputs rewritten k-step-major by
    // df11_tile_inputs_kernel: element (k-step ks, vector b, column c) of the
    // range at column offset xoff (xoff then counts columns of xt) at
    // xt[16 NT (xoff + 32 ks) + 32 b + c]
    const uint16_t *xt;
    float *y;                 // matrix m's results at y + yoff; vector b at + b * y_stride
    const uint32_t *seg_blk;  // per segment (matrix order) its first block; then the last block
    uint64_t x_stride, y_stride;
    uint32_t batch, n_mats;
    // per launch-order entry e (matrices by decreasing cols): its first
    // segment in launch order (first[n_mats] = number of segments), the
    // matrix's first operand tile (offset / 512), k-steps (cols / 32),
    // the matrix-order index of its first segment, and its x and y offsets
    uint32_t first[kGemvMaxMats + 1];
    uint32_t tile0[kGemvMaxMats];
    uint32_t ksteps[kGemvMaxMats];
    uint32_t seg0[kGemvMaxMats];
    uint32_t xoff[kGemvMaxMats];
    uint32_t yoff[kGemvMaxMats];
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// One lane's inputs for one block: its stream dwords, its gap dwords and
// (even lanes) block_pos[blk] or (odd lanes) block_pos[blk + 1].
struct BlockIn {
    uint32_t d0, d1, d2, g0, g1, pos;
};

__device__ __forceinline__ BlockIn load_block(const DecodeArgs &a, uint32_t blk, uint32_t lane) {
    BlockIn r;
    const uint32_t *sp = a.stream + 2 * (blk * DF11_BLOCK_SLICES + lane);
    r.d0 = sp[0], r.d1 = sp[1], r.d2 = sp[2];
    const uint32_t *gp = a.gaps + 10 * blk + ((5 * lane) >> 5);
    r.g0 = gp[0], r.g1 = gp[1];
    r.pos = a.block_pos[blk + (lane & 1)];
    return r;
}

// Where the lane's B operands come from: vector 16 nt + lane % 16 of the
// batch, inputs xl + 16 nt x_stride + 32 ks + 0..7 for k-step ks (xl already
// holds the lane's vector, the matrix's x offset and the lane's 8 columns).
// (One vector: xl is the matrix's inputs, and the inputs of k-steps [ks0,
// ks0 + 4) are held across the wave, two per lane (lane l: columns 32 ks0 +
// 2 l and + 1), in xw.)
struct XSrc {
    const g_cu16 *xl;       // the lane's 8 inputs of group 0, k-step 0
    uint64_t group_stride;  // from one group of 16 vectors to the next
    uint64_t ks_stride;     // from one k-step to the next
    uint32_t live;          // vectors of the lane's column below the batch: bit nt
    uint32_t ks0, xw, cols;
};

// The lane's B operands of k-step ks: 8 inputs of vector 16 nt + lane % 16.
// kX1 (one vector): gathered from the four k-steps held in xw (every lane
// gets vector 0's inputs of its column group: the extra columns of the
// product are never written out); a k-step outside them loads the next four.
template <int NT, bool kX1>
__device__ __forceinline__ void tile_x(u32x4 (&bv)[NT], XSrc &xs, uint32_t ks) {
    if constexpr (kX1) {
        if (ks - xs.ks0 >= 4u) {  // rare: a block reaching past its window's first 4 k-steps
            xs.ks0 = ks;
            uint32_t col = 32 * ks + 2 * (threadIdx.x % 64);
            col = col < xs.cols - 2 ? col : xs.cols - 2;
            xs.xw = *(const __attribute__((address_space(1))) uint32_t *)(xs.xl + col);
            // wait here, so that the common path, where this branch joins it,
            // carries no load in flight into its next wait
            __builtin_amdgcn_s_waitcnt(0);
        }
        const int at = (int)(64 * (ks - xs.ks0) + 16 * ((threadIdx.x % 64) / 16));
        bv[0] = u32x4{(uint32_t)__builtin_amdgcn_ds_bpermute(at, (int)xs.xw),
                      (uint32_t)__builtin_amdgcn_ds_bpermute(at + 4, (int)xs.xw),
                      (uint32_t)__builtin_amdgcn_ds_bpermute(at + 8, (int)xs.xw),
                      (uint32_t)__builtin_amdgcn_ds_bpermute(at + 12, (int)xs.xw)};
    } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            bv[nt] = (xs.live >> nt) & 1u
                         ? *(const g_cu32x4 *)(xs.xl + nt * xs.group_stride + ks * xs.ks_stride)
                         : u32x4{0, 0, 0, 0};
    }
}

// The lane's 8 exponent bytes of the group at word q (rotated, as in LDS):
// words at or after `split` from the LDS tile (the word at q at byte q -
// t_base), those before it from `carry` (what the wave's previous blocks
// decoded of the same operand tile).  The tile is read only for a group that
// holds words of [split, hi): q >= t_base then holds, since t_base is split
// rounded down to 8, and q - t_base stays inside the block's decoded range.
__device__ __forceinline__ uint2 tile_exps(const uint8_t *tile, uint32_t t_base, uint32_t q,
                                           uint32_t split, uint32_t hi, uint2 carry) {
    if (q + 8 <= split || q >= hi) return carry;
    const uint2 t = *reinterpret_cast<const uint2 *>(tile + (q - t_base));
    if (q >= split) return t;
    // bytes [0, k) from carry, [k, 8) from the tile (0 < k < 8)
    const uint64_t keep = (1ull << (8 * (split - q))) - 1;
    const uint64_t c64 = ((uint64_t)carry.y << 32) | carry.x, t64 = ((uint64_t)t.y << 32) | t.x;
    const uint64_t m = (c64 & keep) | (t64 & ~keep);
    return make_uint2((uint32_t)m, (uint32_t)(m >> 32));
}

// The lane's A operand of the group at word q: its 8 words joined from
// exponent bytes e and sign|mantissa bytes sm, those outside [w_lo, w_hi)
// zero.
__device__ __forceinline__ u32x4 tile_a(uint2 e, uint2 sm, uint32_t q, uint32_t w_lo, uint32_t w_hi) {
    const uint32_t lo = q > w_lo ? q : w_lo, hi = q + 8 < w_hi ? q + 8 : w_hi;
    u32x4 av = {0, 0, 0, 0};
    if (lo < hi) {
        const uint4 w = join8(e, sm);
        av = u32x4{w.x, w.y, w.z, w.w};
        if (hi - lo < 8) {
            const uint32_t a0 = lo - q, a1 = hi - q;  // words [a0, a1) are kept
            auto keep = [&](uint32_t j) { return j >= a0 && j < a1; };
            av.x &= (keep(0) ? 0xFFFFu : 0u) | (keep(1) ? 0xFFFF0000u : 0u);
            av.y &= (keep(2) ? 0xFFFFu : 0u) | (keep(3) ? 0xFFFF0000u : 0u);
            av.z &= (keep(4) ? 0xFFFFu : 0u) | (keep(5) ? 0xFFFF0000u : 0u);
            av.w &= (keep(6) ? 0xFFFFu : 0u) | (keep(7) ? 0xFFFF0000u : 0u);
        }
    }
    return av;
}

template <int NT>
__device__ __forceinline__ void tile_mfma(f32x4 (&acc)[NT], u32x4 av, const u32x4 (&bv)[NT]) {
    const bf16x8_t a8 = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, __builtin_bit_cast(bf16x8_t, bv[nt]),
                                                          acc[nt], 0, 0, 0);
}

// One operand tile tt into acc: words [w_lo, w_hi) of it, exponent bytes as
// tile_exps gives them.
// (kMerge false: no word of the tile lies before split.)
// With `pre` the tile's sign|mantissa bytes are sm_pre (loaded earlier for
// the whole tile).
template <int NT, bool kX1, bool kMerge>
__device__ __forceinline__ void tile_step(uint32_t tt, uint32_t w_lo, uint32_t w_hi, uint32_t split,
                                          uint32_t t_base, const uint8_t *tile,
                                          const uint8_t *signmant, XSrc &xs, uint32_t seg_tile,
                                          uint32_t lane, uint2 carry, bool pre, uint2 sm_pre,
                                          f32x4 (&acc)[NT]) {
    u32x4 bv[NT];
    tile_x<NT, kX1>(bv, xs, tt - seg_tile);
    const uint32_t q = (tt << 9) + 8 * lane;
    const uint2 sm = pre ? sm_pre
                         : (q + 8 > w_lo && q < w_hi ? load_sm8(signmant + q) : make_uint2(0, 0));
    uint2 e;
    if (kMerge)
        e = tile_exps(tile, t_base, q, split, w_hi, carry);
    else
        e = q < w_hi ? *reinterpret_cast<const uint2 *>(tile + (q - t_base)) : make_uint2(0, 0);
    tile_mfma<NT>(acc, tile_a(e, sm, q, w_lo, w_hi), bv);
}

// An operand tile wholly inside the block's decoded words: no masks.
template <int NT, bool kX1>
__device__ __forceinline__ void tile_whole(uint32_t tt, uint32_t t_base, const uint8_t *tile,
                                           const uint8_t *signmant, XSrc &xs, uint32_t seg_tile,
                                           uint32_t lane, bool pre, uint2 sm_pre, f32x4 (&acc)[NT]) {
    u32x4 bv[NT];
    tile_x<NT, kX1>(bv, xs, tt - seg_tile);
    const uint32_t q = (tt << 9) + 8 * lane;
    const uint4 w = join8(*reinterpret_cast<const uint2 *>(tile + (q - t_base)),
                          pre ? sm_pre : load_sm8(signmant + q));
    tile_mfma<NT>(acc, u32x4{w.x, w.y, w.z, w.w}, bv);
}

// Sign|mantissa bytes of a window's first operand tiles, loaded at the top
// of the block so that they arrive while it decodes.
// (Two with one vector: a third takes that kernel past its 64 VGPRs.)
template <bool kX1> constexpr int kSmAhead = kX1 ? 2 : 3;

// Multiply the operand tiles that words [w_lo, w_hi) reach into acc.  Words
// [w_lo, split) were decoded by the wave's earlier blocks and sit in carry
// (they share the first tile); words [split, w_hi) are this block's, in the
// LDS tile (word q at byte q - t_base).  With `defer` the last tile, which
// the wave's next block completes, is not multiplied: its exponent bytes go
// to carry instead.
// With `pre`, smp[k] holds the sign|mantissa bytes of tile (w_lo >> 9) + k.
template <int NT, bool kX1>
__device__ __forceinline__ void mfma_window(uint32_t w_lo, uint32_t split, uint32_t w_hi,
                                            bool defer, uint32_t t_base, const uint8_t *tile,
                                            const uint8_t *signmant, XSrc &xs,
                                            uint32_t seg_tile, uint32_t lane, uint2 &carry,
                                            bool pre, const uint2 (&smp)[kSmAhead<kX1>],
                                            f32x4 (&acc)[NT]) {
    uint32_t tt = w_lo >> 9;
    const uint32_t t_end = defer ? w_hi >> 9 : (w_hi + 511) >> 9;
    const uint32_t t_whole = w_hi >> 9;  // tiles below it end inside the window
    if (tt < t_end) {  // the first tile: carried words merged
        tile_step<NT, kX1, true>(tt, w_lo, w_hi, split, t_base, tile, signmant, xs, seg_tile, lane, carry,
                            pre, smp[0], acc);
        ++tt;
        // the block's later tiles (split lies below them): whole ones, then a
        // last partial one; the first of them with the bytes loaded ahead
#pragma unroll
        for (int k = 1; k < kSmAhead<kX1>; ++k) {
            if (tt >= t_end) break;
            if (tt < t_whole)
                tile_whole<NT, kX1>(tt, t_base, tile, signmant, xs, seg_tile, lane, pre, smp[k], acc);
            else
                tile_step<NT, kX1, false>(tt, w_lo, w_hi, split, t_base, tile, signmant, xs, seg_tile,
                                     lane, carry, pre, smp[k], acc);
            ++tt;
        }
        for (; tt < t_whole; ++tt)
            tile_whole<NT, kX1>(tt, t_base, tile, signmant, xs, seg_tile, lane, false, smp[0], acc);
        if (tt < t_end) {
            tile_step<NT, kX1, false>(tt, w_lo, w_hi, split, t_base, tile, signmant, xs, seg_tile, lane,
                                 carry, false, smp[0], acc);
            ++tt;
        }
    }
    if (defer) carry = tile_exps(tile, t_base, (tt << 9) + 8 * lane, split, w_hi, carry);
}

// The carried words [c_lo, c_hi) alone (the wave's next block does not go on
// with them).
template <int NT, bool kX1>
__device__ __forceinline__ void flush_carry(uint32_t c_lo, uint32_t c_hi, const uint8_t *signmant,
                                            XSrc &xs, uint32_t seg_tile, uint32_t lane,
                                            uint2 carry, f32x4 (&acc)[NT]) {
    // split past the window: every exponent byte from carry, no LDS read
    tile_step<NT, kX1, true>(c_lo >> 9, c_lo, c_hi, 0xFFFFFFFFu, 0u, nullptr, signmant, xs, seg_tile,
                        lane, carry, false, carry, acc);
}

// Input ranges for df11_tile_inputs_kernel: range r is x[b * x_stride +
// xoff[r] + c], c < cols[r], rewritten from column offset txoff[r] of xt.
struct TileInputs {
    const uint16_t *x;
    uint16_t *xt;
    uint64_t x_stride;
    uint32_t batch, rows;  // vectors in use; vectors per k-step slab of xt (16 NT)
    uint32_t n_ranges;
    uint32_t first[kGemvMaxMats + 1];  // first 16-byte chunk of each range; then the total
    uint32_t xoff[kGemvMaxMats];
    uint32_t cols[kGemvMaxMats];
    uint32_t txoff[kGemvMaxMats];
};

// x (row-major, one row per vector) -> xt (per range, per 32-column k-step,
// a slab of `rows` vectors x 32 columns), one 16-byte chunk per thread:
// consecutive threads read consecutive chunks of one row of x.  Slab rows of
// vectors at or past the batch are not written (the product never reads them).
__global__ __launch_bounds__(256) void df11_tile_inputs_kernel(TileInputs t) {
    const uint32_t id = blockIdx.x * 256 + threadIdx.x;
    if (id >= t.first[t.n_ranges]) return;
    uint32_t r = 0;
#pragma unroll
    for (int i = 1; i < kGemvMaxMats; ++i) r += ((uint32_t)i < t.n_ranges && id >= t.first[i]) ? 1u : 0u;
    uint32_t first_r = 0, xoff_r = 0, cols_r = 0, txoff_r = 0;
#pragma unroll
    for (int i = 0; i < kGemvMaxMats; ++i)
        if ((uint32_t)i == r) first_r = t.first[i], xoff_r = t.xoff[i], cols_r = t.cols[i], txoff_r = t.txoff[i];
    const uint32_t k = id - first_r, per_row = cols_r / 8;
    const uint32_t b = k / per_row, c8 = k % per_row;  // vector, chunk of 8 columns
    const u32x4 v = *(const g_cu32x4 *)((const g_cu16 *)t.x + (uint64_t)b * t.x_stride + xoff_r + 8 * c8);
    const uint64_t at = (uint64_t)t.rows * (txoff_r + 32 * (c8 / 4)) + 32 * b + 8 * (c8 % 4);
    *(__attribute__((address_space(1))) u32x4 *)((__attribute__((address_space(1))) uint16_t *)t.xt + at) = v;
}

// Occupancy: up to 16 vectors 8 waves per SIMD (64 VGPRs, ~80 SGPRs: 4
// workgroups per CU); up to 32 the decode's 80-VGPR budget (3 per CU); 64
// vectors 128 VGPRs (2 per CU).
template <int NT> struct TiledOccupancy {
    static constexpr int kValue = NT == 1 ? 8 : NT == 2 ? kWavesPerEu : 4;
};

// kX1: one vector (NT 1, row-major x).
template <int NT, bool kX1>
__global__ __launch_bounds__(kGroupThreads)
__attribute__((amdgpu_waves_per_eu(TiledOccupancy<NT>::kValue)))
void df11_tiled_kernel(DecodeArgs a, TiledArgs t) {
    static_assert(!kX1 || NT == 1, "the one-vector inputs are for one group of vectors");
    __shared__ __attribute__((aligned(16))) uint8_t lds_static[kStaticLds];
    static_assert(8 * 4 * 256 * 4 <= kStaticLds, "the final sums of 8 waves fit the static LDS");
    extern __shared__ uint4 smem_u4[];
    uint16_t *lut = reinterpret_cast<uint16_t *>(smem_u4);
    uint8_t *tiles = lds_static;
    const uint8_t *lds_dec = lds_static + kTilesBytes;
    if (lds_offset(tiles) + kTilesBytes > 0x10000u) {
        if (threadIdx.x == 0 && a.status) atomicAdd(a.status, 1u);
        return;
    }
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    uint8_t *tile = tiles + wave * kTileBytes;
    const uint32_t tile_addr = lds_offset(tile);

    // this workgroup's segment: row tile rt of launch-order entry e (fields
    // taken with constant indices: a run-time index into the kernel argument
    // would copy it to scratch memory)
    const uint32_t k = blockIdx.x;
    uint32_t e = 0;
#pragma unroll
    for (int i = 1; i < kGemvMaxMats; ++i) e += ((uint32_t)i < t.n_mats && k >= t.first[i]) ? 1u : 0u;
    uint32_t first_e = 0, tile0_e = 0, ks_e = 0, seg0_e = 0, xoff_e = 0, yoff_e = 0;
#pragma unroll
    for (int i = 0; i < kGemvMaxMats; ++i)
        if ((uint32_t)i == e) {
            first_e = t.first[i], tile0_e = t.tile0[i], ks_e = t.ksteps[i];
            seg0_e = t.seg0[i], xoff_e = t.xoff[i], yoff_e = t.yoff[i];
        }
    const uint32_t rt = k - first_e;
    const uint32_t seg_tile = tile0_e + rt * ks_e;  // the segment's first operand tile
    const uint32_t seg_lo = seg_tile << 9, seg_hi = seg_lo + (ks_e << 9);
    const uint32_t seg = seg0_e + rt;
    const uint32_t blk_lo = t.seg_blk[seg];
    uint32_t blk_hi = t.seg_blk[seg + 1];
    blk_hi = blk_hi < a.n_blocks ? blk_hi : a.n_blocks - 1;

    // the lane's B operand: vector 16 nt + lane % 16, columns 8 (lane / 16)
    // + 0..7 of each 32-column slab
    XSrc xs;
    if (t.xt) {  // inputs rewritten k-step-major: [k-step][16 NT vectors][32 columns]
        xs.xl = (const g_cu16 *)t.xt + (uint64_t)xoff_e * (16 * NT) + (lane % 16) * 32 + 8 * (lane / 16);
        xs.group_stride = 16 * 32;
        xs.ks_stride = 32 * 16 * NT;
    } else {  // row-major x
        xs.xl = (const g_cu16 *)t.x + (uint64_t)(lane % 16) * t.x_stride + xoff_e + 8 * (lane / 16);
        xs.group_stride = 16 * t.x_stride;
        xs.ks_stride = 32;
    }
    xs.live = 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) xs.live |= (16 * nt + lane % 16 < t.batch ? 1u : 0u) << nt;
    xs.ks0 = 0xFFFFFFF0u;  // none held
    xs.xw = 0;
    xs.cols = 32 * ks_e;
    if (kX1) xs.xl = (const g_cu16 *)t.x + xoff_e;  // vector 0's inputs of the matrix

    // tables into LDS while the wave's first block loads
    const uint32_t hier_bytes = a.n_tables * kTableBytes;
    const uint32_t lut_u4_count = hier_bytes / 16;
    const bool lut_one_load = lut_u4_count <= kGroupThreads;
    uint4 lv = {0, 0, 0, 0};
    if (lut_one_load && threadIdx.x < lut_u4_count) lv = a.luts[threadIdx.x];
    const uint4 *dec_src = a.luts + lut_u4_count;
    const uint4 dv0 = dec_src[threadIdx.x], dv1 = dec_src[threadIdx.x + kGroupThreads];
    // the wave's run of consecutive blocks [b, r_hi): an operand tile that a
    // block leaves unfinished is completed by the next block of the run
    const uint32_t nb = blk_hi + 1 - blk_lo;
    uint32_t b = blk_lo + wave * nb / kWavesPerGroup;
    const uint32_t r_hi = blk_lo + (wave + 1) * nb / kWavesPerGroup;
    BlockIn nxt = load_block(a, b, lane);
    uint4 *lut_u4 = reinterpret_cast<uint4 *>(lut);
    if (lut_one_load) {
        if (threadIdx.x < lut_u4_count) lut_u4[threadIdx.x] = lv;
    } else {
        for (uint32_t i = threadIdx.x; i < lut_u4_count; i += kGroupThreads) lut_u4[i] = a.luts[i];
    }
    reinterpret_cast<uint4 *>(lds_static + kTilesBytes)[threadIdx.x] = dv0;
    reinterpret_cast<uint4 *>(lds_static + kTilesBytes)[threadIdx.x + kGroupThreads] = dv1;
    group_lds_sync();

    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t gap_shift = (5 * lane) & 31;
    // carried words [c_lo, c_hi) of one operand tile (c_hi == c_lo: none)
    uint2 carry = make_uint2(0, 0);
    uint32_t c_lo = 0, c_hi = 0;
    for (; b < r_hi; ++b) {
        // Every load of the last block is done by now (this block's inputs were
        // issued a block ago).  Saying so here leaves the compiler no load in
        // flight to guard across the loop: otherwise a register reused in
        // phase 1 can draw a wait for everything, this block's prefetches
        // included.
        __builtin_amdgcn_s_waitcnt(0);
        const BlockIn cur = nxt;
        const uint32_t p0 = __builtin_amdgcn_readlane(cur.pos, 0);
        const uint32_t p1 = __builtin_amdgcn_readlane(cur.pos, 1);
        const bool sane = p1 >= p0 && p1 <= a.n && p1 - p0 <= (uint32_t)kMaxBlockCodes;
        const uint32_t base = p0 & ~7u;
        const uint32_t groups = sane ? (p1 - base + 7) >> 3 : 0u;
        const bool one_pass = groups * 8 + 4 <= (uint32_t)kTileCap;
        // the block's words in this segment
        const uint32_t w_lo = p0 > seg_lo ? p0 : seg_lo, w_hi = p1 < seg_hi ? p1 : seg_hi;
        // the carried words go on at w_lo (a run's blocks are consecutive)
        const bool go_on = c_lo < c_hi && c_hi == w_lo && w_lo < w_hi;
        // Loads for this block and the next, oldest first: loads complete in
        // order, so the tiles' first wait (for the inputs) must not sit behind
        // the next block's stream words.  One vector: the inputs of the
        // window's first 4 k-steps (a column past the matrix repeats its last
        // pair).  Then the next block, then the sign|mantissa bytes of the
        // window's first tiles (a tile past the window's last one repeats
        // that one).
        const bool pre = one_pass && w_lo < w_hi;
        if (kX1 && pre) {
            xs.ks0 = ((go_on ? c_lo : w_lo) >> 9) - seg_tile;
            uint32_t col = 32 * xs.ks0 + 2 * lane;
            col = col < xs.cols - 2 ? col : xs.cols - 2;
            xs.xw = *(const __attribute__((address_space(1))) uint32_t *)(xs.xl + col);
        }
        if (b + 1 < r_hi) nxt = load_block(a, b + 1, lane);
        uint2 smp[kSmAhead<kX1>];
        {
            const uint32_t t0 = (go_on ? c_lo : w_lo) >> 9, t_last = pre ? (w_hi - 1) >> 9 : t0;
#pragma unroll
            for (int k = 0; k < kSmAhead<kX1>; ++k) {
                const uint32_t t = t0 + k < t_last ? t0 + k : t_last;
                smp[k] = pre ? load_sm8(a.signmant + (t << 9) + 8 * lane) : make_uint2(0, 0);
            }
        }
        const uint32_t gw = __builtin_amdgcn_alignbit(cur.g1, cur.g0, gap_shift);
        const uint32_t gap = gw & 31u, gap_next = (gw >> 5) & 31u;
        // stop bit and stream end relative to this lane's slice (as in the decode)
        auto from_block = [&](uint32_t blk, uint32_t rem) {
            const int32_t d = (int32_t)(blk - b);
            return d > 1 ? (1 << 30) : (d < -1 ? -(1 << 30) : d * 4096 + (int32_t)rem);
        };
        const int32_t stop_at = from_block(a.stop_blk, a.stop_rem);
        uint32_t lim, f0, f1, f2;
        if (stop_at > kWave * DF11_SLICE_BITS) {
            lim = 64u;
            f0 = cur.d0;
            f1 = cur.d1;
            f2 = cur.d2 | (0xFFFFFFFFu << gap_next);
        } else {
            const int32_t lane_bit = (int32_t)(lane * DF11_SLICE_BITS);
            const int32_t rel = stop_at - lane_bit;
            lim = rel <= 0 ? 0u : (rel >= 64 ? 64u : (uint32_t)rel);
            const uint32_t end = rel > 0 && rel <= 64
                                     ? (uint32_t)(from_block(a.end_blk, a.end_rem) - lane_bit)
                                     : 64u + gap_next;
            f0 = pad_ones(cur.d0, (int)end, 0);
            f1 = pad_ones(cur.d1, (int)end, 32);
            f2 = pad_ones(cur.d2, (int)end, 64);
        }
        // phase 1, scan
        const uint32_t slot = tile_addr + kStageBase + lane * kStageStride;
        const uint32_t cnt = lim ? stage_codes(lds_dec, lut, a.n_tables, cur.d0, cur.d1, cur.d2, f0,
                                               f1, f2, gap, lim, slot)
                                 : 0u;
        const uint32_t incl = wave_inclusive_sum(cnt);
        const uint32_t excl = incl - cnt;
        const uint32_t total = __builtin_amdgcn_readlane(incl, kWave - 1);
        if (!sane || total != p1 - p0) {  // a corrupt block: reported, its words left out
            if (lane == 0 && a.status) atomicAdd(a.status, 1u);
            if (c_lo < c_hi) flush_carry<NT, kX1>(c_lo, c_hi, a.signmant, xs, seg_tile, lane, carry, acc);
            c_hi = c_lo;
            wave_lds_sync();
            continue;
        }
        const uint32_t at = (p0 - base) + excl;
        const uint32_t start = lim ? gap : 0u;
        const bool last_lane = incl == total;
        const bool odd = cnt > (uint32_t)kStageCodes || (cnt < (uint32_t)kStageMinCodes && !last_lane);
        const bool staged = one_pass && __builtin_amdgcn_ballot_w64(odd) == 0;
        wave_lds_sync();
        if (staged) {
            const uint32_t tail = staged_tail(slot, cnt);
            const uint32_t prev = (uint32_t)__builtin_amdgcn_ds_bpermute(
                (int)(((lane + kWave - 1) % kWave) * 4), (int)tail);
            place_staged(slot, tile_addr + at, cnt, prev, last_lane);
            wave_lds_sync();
        } else if (one_pass) {
            decode_codes<false>(lds_dec, lut, a.n_tables, cur.d0, cur.d1, cur.d2, start, lim,
                                tile_addr, at, 0);
            wave_lds_sync();
            rewrite_head(lds_dec, lut, a.n_tables, cur.d0, cur.d1, cur.d2, start, cnt,
                         tile_addr + at);
            wave_lds_sync();
        }
        if (c_lo < c_hi && !(go_on && one_pass))
            flush_carry<NT, kX1>(c_lo, c_hi, a.signmant, xs, seg_tile, lane, carry, acc);
        if (one_pass) {
            if (w_lo < w_hi) {
                // leave the last tile to the next block if that block completes it
                const bool defer = b + 1 < r_hi && (w_hi & 511u) != 0;
                const uint32_t lo = go_on ? c_lo : w_lo;
                mfma_window<NT, kX1>(lo, w_lo, w_hi, defer, base, tile, a.signmant, xs, seg_tile, lane,
                                carry, pre, smp, acc);
                c_lo = defer ? (lo > ((w_hi - 1) & ~511u) ? lo : (w_hi - 1) & ~511u) : 0u;
                c_hi = defer ? w_hi : 0u;
            } else {
                c_lo = c_hi = 0;
            }
            wave_lds_sync();
        } else {
            c_lo = c_hi = 0;
            // more symbols than one tile holds: decode again per tile-sized window
            for (uint32_t r0 = 0; r0 < groups * 8; r0 += kTileCap) {
                decode_codes<true>(lds_dec, lut, a.n_tables, cur.d0, cur.d1, cur.d2, start, lim,
                                   tile_addr, at, r0);
                wave_lds_sync();
                // (the window's end clamped to the block's, so that it cannot
                // pass 2^32 at the end of the largest stream)
                const uint32_t r_lo = base + r0, room = p1 > r_lo ? p1 - r_lo : 0u;
                const uint32_t r_hi = r_lo + (room < (uint32_t)kTileCap ? room : (uint32_t)kTileCap);
                const uint32_t v_lo = w_lo > r_lo ? w_lo : r_lo, v_hi = w_hi < r_hi ? w_hi : r_hi;
                if (v_lo < v_hi)
                    mfma_window<NT, kX1>(v_lo, v_lo, v_hi, false, r_lo, tile, a.signmant, xs, seg_tile,
                                    lane, carry, false, smp, acc);
                wave_lds_sync();
            }
        }
    }

    // every wave's blocks are done and the LDS is free: sum the waves' 16 x 16
    // results per group of vectors in wave order and write them
    group_lds_sync();
    float *red = reinterpret_cast<float *>(lds_static);  // [wave][nt][lane][4]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<f32x4 *>(red + ((wave * NT + nt) * kWave + lane) * 4) = acc[nt];
    group_lds_sync();
    for (uint32_t o = threadIdx.x; o < (uint32_t)NT * 256; o += kGroupThreads) {
        const uint32_t nt = o / 256, j = (o % 256) / 16, i = o % 16;  // vector 16 nt + j, row i
        const uint32_t src = (j + 16 * (i / 4)) * 4 + i % 4;           // D[i][j]: lane, register
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWavesPerGroup; ++w) sum += red[(w * NT + nt) * 256 + src];
        const uint32_t vb = 16 * nt + j;
        if (vb < t.batch) t.y[(uint64_t)vb * t.y_stride + yoff_e + 16 * rt + i] = sum;
    }
}

// Launch shape per device: compute units and, per kernel, resident
// workgroups per CU for each table count (the LDS footprint depends on it).
constexpr int kMaxDevices = 16;
// 0: decode, 1..4: fused product for 1, 2, 4, 8 vectors, 5: decode of a tile-order stream,
// 6: decode with 56-code staging slots
constexpr int kKernels = 7;
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_occ[kKernels][kMaxDevices][DF11_MAX_TABLES + 1];

// dynamic LDS per workgroup: the 8-bit tables (tiles and fast tables are static)
size_t lds_bytes(uint32_t n_tables) { return (size_t)n_tables * kTableBytes; }

template <class K>
int launch_groups(K kernel, int which, int dev, uint32_t n_tables, uint32_t n_blocks,
                  uint32_t max_groups, int *groups) {
    if (dev < 0 || dev >= kMaxDevices) return DF11_ERR_HIP;
    int cus = g_cus[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return DF11_ERR_HIP;
        g_cus[dev].store(cus, std::memory_order_relaxed);
    }
    int occ = g_occ[which][dev][n_tables].load(std::memory_order_relaxed);
    if (occ <= 0) {
        // a workgroup whose LDS exceeds what one CU can give it would never be
        // dispatched: refuse the launch instead
        int max_lds = 0;
        hipFuncAttributes attr;
        if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess ||
            hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(kernel)) != hipSuccess)
            return DF11_ERR_HIP;
        if (attr.sharedSizeBytes + lds_bytes(n_tables) > (size_t)max_lds) return DF11_ERR_TABLES;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kGroupThreads,
                                                         lds_bytes(n_tables)) != hipSuccess)
            return DF11_ERR_HIP;
        if (occ <= 0) return DF11_ERR_TABLES;
        g_occ[which][dev][n_tables].store(occ, std::memory_order_relaxed);
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

// The plain decode stages up to 56 codes per lane (instead of 32) for a
// stream whose codes average under 64 / 25.5 = 2.51 bits: about 26 or more
// codes start in a 64-bit slice, and most blocks hold a lane with more than
// 32, which would send them to the re-decode route (ordinary BF16 weights
// average 2.6-2.8 bits, 23-25 codes per slice, decode as fast with either,
// and keep the 32-code slots, whose LDS leaves more room for the tables).
// Either kernel decodes every stream; the choice only decides which blocks
// take the re-decode route.
bool uses_wide_slots(const df11_device_stream *s) {
    return 128 * (unsigned __int128)s->n > 51 * (unsigned __int128)s->total_bits;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks a descriptor and fills the kernel arguments (out may be null).
int prepare(const df11_device_stream *s, uint16_t *out, DecodeArgs *a) {
    if (!s || !s->stream || !s->gaps || !s->block_pos || !s->signmant || !s->luts)
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
    a->stream = reinterpret_cast<const uint32_t *>(s->stream);
    a->gaps = reinterpret_cast<const uint32_t *>(s->gaps);
    a->block_pos = s->block_pos;
    a->signmant = s->signmant;
    a->luts = reinterpret_cast<const uint4 *>(s->luts);
    a->out = out;
    a->status = s->status;
    a->n = s->n;
    static_assert(DF11_BLOCK_SLICES * DF11_SLICE_BITS == 4096, "4096-bit blocks");
    a->stop_blk = (uint32_t)((s->last_start + 1) >> 12);
    a->stop_rem = (uint32_t)((s->last_start + 1) & 4095);
    a->end_blk = (uint32_t)(s->total_bits >> 12);
    a->end_rem = (uint32_t)(s->total_bits & 4095);
    a->n_blocks = s->n_blocks;
    a->n_tables = s->n_tables;
    return DF11_OK;
}

}  // namespace

extern "C" int df11_decode(const df11_device_stream *s, uint16_t *out, void *hip_stream) {
    if (!out) return DF11_ERR_ARG;
    DecodeArgs a;
    int st = prepare(s, out, &a);
    if (st != DF11_OK) return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DF11_ERR_HIP;
    int groups = 0;
    // (the wide kernel's LDS is 10 KB larger: with a table hierarchy that
    // leaves it no room, the narrow one decodes the stream)
    st = uses_wide_slots(s) ? launch_groups(df11_decode_kernel<WideGeo::kStageCodes>, 6, dev,
                                            s->n_tables, s->n_blocks, s->max_groups, &groups)
                            : DF11_ERR_TABLES;
    if (st == DF11_OK) {
        hipLaunchKernelGGL(df11_decode_kernel<WideGeo::kStageCodes>, dim3(groups),
                           dim3(kGroupThreads), lds_bytes(s->n_tables),
                           static_cast<hipStream_t>(hip_stream), a);
    } else {
        if (st != DF11_ERR_TABLES) return st;
        st = launch_groups(df11_decode_kernel<NarrowGeo::kStageCodes>, 0, dev, s->n_tables,
                           s->n_blocks, s->max_groups, &groups);
        if (st != DF11_OK) return st;
        hipLaunchKernelGGL(df11_decode_kernel<NarrowGeo::kStageCodes>, dim3(groups),
                           dim3(kGroupThreads), lds_bytes(s->n_tables),
                           static_cast<hipStream_t>(hip_stream), a);
    }
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_ERR_HIP;
}

extern "C" int df11_decode_tiled(const df11_device_stream *s, const df11_gemv_matrix *mats,
                                 uint32_t n_mats, uint16_t *out, void *hip_stream) {
    if (!out || !mats || n_mats < 1 || n_mats > (uint32_t)kTileMapMats) return DF11_ERR_ARG;
    DecodeArgs a;
    int st = prepare(s, out, &a);
    if (st != DF11_OK) return st;
    // the matrices in the tile layout: end to end from 0 over all n words,
    // rows a multiple of 16, cols of 32
    TileMap m = {};
    m.n_mats = n_mats;
    uint64_t off = 0;
    for (uint32_t i = 0; i < n_mats; ++i) {
        const df11_gemv_matrix &mm = mats[i];
        if (mm.offset != off || mm.rows == 0 || mm.rows % 16 != 0 || mm.cols == 0 ||
            mm.cols % 32 != 0)
            return DF11_ERR_ARG;
        m.tile0[i] = (uint32_t)(off / 512);
        m.ks[i] = mm.cols / 32;
        m.cols[i] = mm.cols;
        m.off[i] = off;
        off += (uint64_t)mm.rows * mm.cols;
        if (off > s->n) return DF11_ERR_ARG;
    }
    if (off != s->n) return DF11_ERR_ARG;
    for (uint32_t i = n_mats; i <= (uint32_t)kTileMapMats; ++i) m.tile0[i] = (uint32_t)(off / 512);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DF11_ERR_HIP;
    int groups = 0;
    st = launch_groups(df11_decode_tiled_kernel, 5, dev, s->n_tables, s->n_blocks, s->max_groups,
                       &groups);
    if (st != DF11_OK) return st;
    hipLaunchKernelGGL(df11_decode_tiled_kernel, dim3(groups), dim3(kGroupThreads),
                       lds_bytes(s->n_tables), static_cast<hipStream_t>(hip_stream), a, m);
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_ERR_HIP;
}

// batch capacity (1, 2, 4 or 8) used for a batch of 1..8 vectors
static int gemm_capacity(uint32_t batch) { return batch <= 1 ? 1 : batch <= 2 ? 2 : batch <= 4 ? 4 : 8; }

// Workspace: partial_floats(capacity) floats per block, then the row table:
// one word per row and one more (rows have at least kGemvMinCols weights).
static uint64_t partials_bytes(const df11_device_stream *s, uint32_t batch) {
    return 4ull * partial_floats(gemm_capacity(batch)) * s->n_blocks;
}
extern "C" uint64_t df11_gemm_workspace_bytes(const df11_device_stream *s, uint32_t batch) {
    if (!s || batch < 1 || batch > (uint32_t)kGemmMaxBatch) return 0;
    return partials_bytes(s, batch) + 4ull * (s->n / kGemvMinCols + 1);
}

extern "C" uint64_t df11_gemv_workspace_bytes(const df11_device_stream *s) {
    return df11_gemm_workspace_bytes(s, 1);
}

template <int kB>
static int launch_gemm(const df11_device_stream *s, const DecodeArgs &a, const GemvArgs &g,
                       uint64_t rows, hipStream_t hs) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DF11_ERR_HIP;
    int groups = 0;
    const int which = kB == 1 ? 1 : kB == 2 ? 2 : kB == 4 ? 3 : 4;
    int st = launch_groups(df11_gemm_kernel<kB>, which, dev, s->n_tables, s->n_blocks, s->max_groups,
                           &groups);
    if (st != DF11_OK) return st;
    hipLaunchKernelGGL(df11_gemm_kernel<kB>, dim3(groups), dim3(kGroupThreads),
                       lds_bytes(s->n_tables), hs, a, g);
    hipLaunchKernelGGL(df11_gemm_reduce_kernel<kB>, dim3((uint32_t)((rows + 255) / 256)), dim3(256),
                       0, hs, g, a.n_blocks);
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_ERR_HIP;
}

// The fused product with its workspace given as a device address.
static int decode_gemm(const df11_device_stream *s, const df11_gemv_matrix *mats, uint32_t n_mats,
                       const uint16_t *x, uint32_t batch, uint64_t x_stride, float *y,
                       uint64_t y_stride, void *workspace, uint64_t workspace_bytes,
                       void *hip_stream) {
    if (!mats || !x || !y || !workspace) return DF11_ERR_ARG;
    DecodeArgs a;
    int st = prepare(s, nullptr, &a);
    if (st != DF11_OK) return st;
    if (n_mats < 1 || n_mats > (uint32_t)kGemvMaxMats || batch < 1 ||
        batch > (uint32_t)kGemmMaxBatch || !aligned(x, 16) || !aligned(y, 4) ||
        !aligned(workspace, 16))
        return DF11_ERR_ARG;
    // vector b's inputs start 16-byte aligned; offsets stay 32-bit
    if (batch > 1 && (x_stride % 8 != 0 || x_stride >= (1ull << 32) || y_stride >= (1ull << 32)))
        return DF11_ERR_ARG;
    if (workspace_bytes < df11_gemm_workspace_bytes(s, batch)) return DF11_ERR_BUFSIZE;
    GemvArgs g;
    g.x = x;
    g.y = y;
    g.partials = static_cast<float *>(workspace);
    g.row_blk = reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(workspace) + partials_bytes(s, batch));
    g.x_stride = batch > 1 ? x_stride : 0;
    g.y_stride = batch > 1 ? y_stride : 0;
    g.batch = batch;
    g.n_mats = n_mats;
    uint64_t off = 0, rows = 0, x_end = 0, y_end = 0;
    for (uint32_t m = 0; m < n_mats; ++m) {
        const df11_gemv_matrix &mm = mats[m];
        // matrices end to end in output order; rows long enough that a block
        // touches at most three of them; 8-aligned groups never straddle rows
        if (mm.offset != off || mm.rows == 0 || mm.cols < kGemvMinCols || mm.cols % 8 != 0 ||
            mm.x_offset % 8 != 0)
            return DF11_ERR_ARG;
        g.off[m] = (uint32_t)off;
        g.cols[m] = mm.cols;
        g.row0[m] = (uint32_t)rows;
        g.xoff[m] = mm.x_offset;
        g.yoff[m] = mm.y_offset;
        off += (uint64_t)mm.rows * mm.cols;
        rows += mm.rows;
        const uint64_t xe = (uint64_t)mm.x_offset + mm.cols, ye = (uint64_t)mm.y_offset + mm.rows;
        x_end = xe > x_end ? xe : x_end;
        y_end = ye > y_end ? ye : y_end;
        if (off > s->n || rows >= 0x80000000ull) return DF11_ERR_ARG;
    }
    if (off != s->n) return DF11_ERR_ARG;
    // each vector's inputs and results end before the next vector's begin
    if (batch > 1 && (x_stride < x_end || y_stride < y_end)) return DF11_ERR_ARG;
    g.off[n_mats] = (uint32_t)off;
    g.row0[n_mats] = (uint32_t)rows;
    const hipStream_t hs = static_cast<hipStream_t>(hip_stream);
    switch (gemm_capacity(batch)) {
    case 1: return launch_gemm<1>(s, a, g, rows, hs);
    case 2: return launch_gemm<2>(s, a, g, rows, hs);
    case 4: return launch_gemm<4>(s, a, g, rows, hs);
    default: return launch_gemm<8>(s, a, g, rows, hs);
    }
}

extern "C" int df11_decode_gemm(const df11_device_stream *s, const df11_gemv_matrix *mats,
                                uint32_t n_mats, const uint16_t *x, uint32_t batch,
                                uint64_t x_stride, float *y, uint64_t y_stride, void *workspace,
                                uint64_t workspace_bytes, void *hip_stream) {
    return decode_gemm(s, mats, n_mats, x, batch, x_stride, y, y_stride, workspace,
                       workspace_bytes, hip_stream);
}

extern "C" int df11_decode_gemv(const df11_device_stream *s, const df11_gemv_matrix *mats,
                                uint32_t n_mats, const uint16_t *x, float *y, void *workspace,
                                uint64_t workspace_bytes, void *hip_stream) {
    return decode_gemm(s, mats, n_mats, x, 1, 0, y, 0, workspace, workspace_bytes, hip_stream);
}

// ------------------------------------------------ the product without allocation
//
// The workspace of df11_decode_gemm_noalloc: one static device array, which
// every GPU the library runs on holds (at its own address) until the process
// ends.  Host code never names it directly (the name is a host-side stand-in):
// its device address is taken once per device with hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[DF11_NOALLOC_SCRATCH_BYTES];
static std::atomic<void *> g_scratch[kMaxDevices];

// scratch's address on the current device (`dev`), looked up on the first call
// there; null if the runtime refuses
static void *scratch_on(int dev) {
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
    return p;
}

extern "C" int df11_decode_gemm_noalloc(const df11_device_stream *s, const df11_gemv_matrix *mats,
                                        uint32_t n_mats, const uint16_t *x, uint32_t batch,
                                        uint64_t x_stride, float *y, uint64_t y_stride,
                                        void *hip_stream) {
    if (!s || batch < 1 || batch > (uint32_t)kGemmMaxBatch) return DF11_ERR_ARG;
    const uint64_t need = df11_gemm_workspace_bytes(s, batch);
    if (need > (uint64_t)DF11_NOALLOC_SCRATCH_BYTES) return DF11_ERR_BUFSIZE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DF11_ERR_HIP;
    void *ws = scratch_on(dev);
    if (!ws) return DF11_ERR_HIP;
    return decode_gemm(s, mats, n_mats, x, batch, x_stride, y, y_stride, ws,
                       (uint64_t)DF11_NOALLOC_SCRATCH_BYTES, hip_stream);
}


// ------------------------------------------------------------ tiled product launch

// Batches from this size on read their inputs rewritten k-step-major: a wave's
// 16 B loads of one k-step then cover 1 KB in one piece instead of 64 bytes
// of each of 16 rows, which the memory pipeline serves far faster (batch 64:
// 0.34 -> 0.23 ms on the 8B-shaped block), at the cost of a ~5 us kernel.
// Smaller batches read x directly: at 8 vectors that is 2% faster, at 12 the
// two tie, at 16 the rewrite is 4% faster.
constexpr uint32_t kTiledRewriteBatch = 12;

static uint32_t tiled_groups(uint32_t batch) { return batch <= 16 ? 1u : batch <= 32 ? 2u : 4u; }

// The distinct input ranges (x_offset, cols) of a matrix list, in order of
// first use; range_of[m] is matrix m's.
static uint32_t input_ranges(const df11_gemv_matrix *mats, uint32_t n_mats, uint32_t *xoff,
                             uint32_t *cols, uint32_t *range_of) {
    uint32_t n = 0;
    for (uint32_t m = 0; m < n_mats; ++m) {
        uint32_t r = 0;
        while (r < n && !(xoff[r] == mats[m].x_offset && cols[r] == mats[m].cols)) ++r;
        if (r == n) xoff[n] = mats[m].x_offset, cols[n] = mats[m].cols, ++n;
        range_of[m] = r;
    }
    return n;
}

extern "C" uint64_t df11_tiled_workspace_bytes(const df11_gemv_matrix *mats, uint32_t n_mats,
                                               uint32_t batch) {
    if (!mats || n_mats < 1 || n_mats > (uint32_t)kGemvMaxMats || batch < 1 ||
        batch > (uint32_t)kTiledMaxBatch)
        return 0;
    if (batch < kTiledRewriteBatch) return 0;
    uint32_t xoff[kGemvMaxMats], cols[kGemvMaxMats], range_of[kGemvMaxMats];
    const uint32_t nr = input_ranges(mats, n_mats, xoff, cols, range_of);
    uint64_t total = 0;
    for (uint32_t r = 0; r < nr; ++r) total += cols[r];
    return 2ull * 16 * tiled_groups(batch) * total;
}

extern "C" int df11_decode_gemm_tiled(const df11_device_stream *s, const df11_gemv_matrix *mats,
                                      uint32_t n_mats, const uint32_t *seg_blk, const uint16_t *x,
                                      uint32_t batch, uint64_t x_stride, float *y,
                                      uint64_t y_stride, void *workspace, uint64_t workspace_bytes,
                                      void *hip_stream) {
    if (!mats || !seg_blk || !x || !y) return DF11_ERR_ARG;
    DecodeArgs a;
    int st = prepare(s, nullptr, &a);
    if (st != DF11_OK) return st;
    if (n_mats < 1 || n_mats > (uint32_t)kGemvMaxMats || batch < 1 ||
        batch > (uint32_t)kTiledMaxBatch || !aligned(x, 16) || !aligned(y, 4) || !aligned(seg_blk, 4))
        return DF11_ERR_ARG;
    if (batch > 1 && (x_stride % 8 != 0 || x_stride >= (1ull << 32) || y_stride >= (1ull << 32)))
        return DF11_ERR_ARG;
    uint64_t off = 0, segs = 0, x_end = 0, y_end = 0;
    uint32_t seg0[kGemvMaxMats];
    for (uint32_t m = 0; m < n_mats; ++m) {
        const df11_gemv_matrix &mm = mats[m];
        if (mm.offset != off || mm.rows == 0 || mm.rows % 16 != 0 || mm.cols == 0 ||
            mm.cols % 32 != 0 || mm.x_offset % 8 != 0)
            return DF11_ERR_ARG;
        seg0[m] = (uint32_t)segs;
        off += (uint64_t)mm.rows * mm.cols;
        segs += mm.rows / 16;
        const uint64_t xe = (uint64_t)mm.x_offset + mm.cols, ye = (uint64_t)mm.y_offset + mm.rows;
        x_end = xe > x_end ? xe : x_end;
        y_end = ye > y_end ? ye : y_end;
        if (off > s->n || ye >= (1ull << 32)) return DF11_ERR_ARG;
    }
    if (off != s->n) return DF11_ERR_ARG;
    if (batch > 1 && (x_stride < x_end || y_stride < y_end)) return DF11_ERR_ARG;
    const bool rewrite = batch >= kTiledRewriteBatch;
    const uint64_t need = df11_tiled_workspace_bytes(mats, n_mats, batch);
    if (rewrite && (!workspace || !aligned(workspace, 16))) return DF11_ERR_ARG;
    if (workspace_bytes < need) return DF11_ERR_BUFSIZE;
    const uint32_t groups = tiled_groups(batch);
    const hipStream_t hs = static_cast<hipStream_t>(hip_stream);

    // the inputs, rewritten k-step-major into the workspace
    uint32_t rxoff[kGemvMaxMats], rcols[kGemvMaxMats], range_of[kGemvMaxMats], rtx[kGemvMaxMats];
    const uint32_t nr = input_ranges(mats, n_mats, rxoff, rcols, range_of);
    if (rewrite) {
        TileInputs ti;
        std::memset(&ti, 0, sizeof(ti));
        ti.x = x;
        ti.xt = static_cast<uint16_t *>(workspace);
        ti.x_stride = batch > 1 ? x_stride : 0;
        ti.batch = batch;
        ti.rows = 16 * groups;
        ti.n_ranges = nr;
        uint64_t chunks = 0, tx = 0;
        for (uint32_t r = 0; r < nr; ++r) {
            ti.first[r] = (uint32_t)chunks;
            ti.xoff[r] = rxoff[r];
            ti.cols[r] = rcols[r];
            ti.txoff[r] = rtx[r] = (uint32_t)tx;
            chunks += (uint64_t)batch * (rcols[r] / 8);
            tx += rcols[r];
        }
        if (chunks >= (1ull << 31)) return DF11_ERR_ARG;
        ti.first[nr] = (uint32_t)chunks;
        hipLaunchKernelGGL(df11_tile_inputs_kernel, dim3((uint32_t)((chunks + 255) / 256)), dim3(256),
                           0, hs, ti);
    }

    // launch order: matrices by decreasing cols (their segments take longest)
    uint32_t order[kGemvMaxMats];
    for (uint32_t m = 0; m < n_mats; ++m) order[m] = m;
    std::stable_sort(order, order + n_mats,
                     [&](uint32_t p, uint32_t q) { return mats[p].cols > mats[q].cols; });
    TiledArgs t;
    std::memset(&t, 0, sizeof(t));
    t.x = x;
    t.xt = rewrite ? static_cast<const uint16_t *>(workspace) : nullptr;
    t.y = y;
    t.seg_blk = seg_blk;
    t.x_stride = batch > 1 ? x_stride : 0;
    t.y_stride = batch > 1 ? y_stride : 0;
    t.batch = batch;
    t.n_mats = n_mats;
    uint32_t run = 0;
    for (uint32_t e = 0; e < n_mats; ++e) {
        const df11_gemv_matrix &mm = mats[order[e]];
        t.first[e] = run;
        t.tile0[e] = (uint32_t)(mm.offset / 512);
        t.ksteps[e] = mm.cols / 32;
        t.seg0[e] = seg0[order[e]];
        t.xoff[e] = rewrite ? rtx[range_of[order[e]]] : mm.x_offset;
        t.yoff[e] = mm.y_offset;
        run += mm.rows / 16;
    }
    t.first[n_mats] = run;
    const dim3 grid(run), block(kGroupThreads);
    const size_t lds = lds_bytes(s->n_tables);
    if (groups == 1 && batch == 1 && !t.xt)
        hipLaunchKernelGGL((df11_tiled_kernel<1, true>), grid, block, lds, hs, a, t);
    else if (groups == 1) hipLaunchKernelGGL((df11_tiled_kernel<1, false>), grid, block, lds, hs, a, t);
    else if (groups == 2) hipLaunchKernelGGL((df11_tiled_kernel<2, false>), grid, block, lds, hs, a, t);
    else hipLaunchKernelGGL((df11_tiled_kernel<4, false>), grid, block, lds, hs, a, t);
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_ERR_HIP;
}
