// df11_decode: gfx950 (CDNA4) kernel that turns a DF11-encoded tensor back
// into its BF16 words, and its C-ABI launcher.
//
// Page "DFloat11: lossless BFloat16 compression" (ai-infrastructure.net),
// section "Architecture": each thread owns 8 bytes of the code stream and
// starts at its Gaps offset; phase 1 only counts codes; a block prefix sum
// turns counts into output offsets (the block's first index is its
// BlockOutputPos); phase 2 decodes again and writes; exponents are joined
// with their sign|mantissa bytes and written with coalesced stores.
//
// Mapping onto CDNA4:
//  * a format block (64 slices, 512 stream bytes) is one wave64, so the prefix
//    sum is a wave-level scan and no workgroup barrier sits in the loop;
//  * workgroups are persistent (a few per CU) and stage the lookup tables in
//    LDS once; waves then stride over blocks;
//  * a lane's 96 relevant stream bits live in three VGPRs; codes that start in
//    the first or second dword are read with one funnel shift (v_alignbit)
//    from a dword pair, so no per-code register shuffling is needed;
//  * phase 2 writes exponent bytes into a per-wave LDS tile aligned to 8
//    output elements; the merge reads 8 exponents and 8 sign|mantissa bytes
//    per lane and writes 8 BF16 words with one 16-byte store.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "df11.h"
#include "df11_internal.h"

namespace {

constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kGroupThreads = kWave * kWavesPerGroup;
constexpr int kMaxBlockCodes = DF11_BLOCK_SLICES * DF11_SLICE_BITS;  // 1-bit codes
constexpr int kTileBytes = kMaxBlockCodes + 16;
constexpr int kTableBytes = 256 * 2;

struct DecodeArgs {
    const uint32_t *stream;     // as dwords
    const uint32_t *gaps;       // packed 5-bit fields, as dwords
    const uint32_t *block_pos;
    const uint8_t *signmant;
    const uint4 *luts;
    uint16_t *out;
    uint32_t *status;
    uint64_t n;
    uint64_t stop_bit;          // codes start strictly before this bit
    uint32_t n_blocks;
    uint32_t n_tables;
};

// Leaf entry: symbol in bits 0-7, (code length - 1) in bits 8-12.
// Pointer entry: bit 15 set, child table in bits 0-5; the next 8 bits of the
// window index the child.  A code of at most 32 bits needs at most 3 descents.
__device__ __forceinline__ uint32_t descend(const uint16_t *lut, uint32_t e, uint32_t w,
                                            uint32_t n_tables) {
#pragma unroll
    for (int lvl = 1; lvl < 4; ++lvl) {
        if (!(e & 0x8000u)) break;
        uint32_t t = e & 63u;
        t = t < n_tables ? t : 0u;
        e = lut[t * 256u + ((w >> (8 * lvl)) & 0xFFu)];
    }
    return e;
}

// Decode the codes that start in [pos, lim) of one lane's slice.  Bits are
// the slice's two dwords d0, d1 and the next slice's first dword d2 (a code
// starting at bit 63 ends by bit 94).  Returns the number of codes; with
// kWrite, symbol k is stored at tp[k].
template <bool kWrite>
__device__ __forceinline__ int walk_slice(const uint16_t *lut, uint32_t n_tables, uint32_t d0,
                                          uint32_t d1, uint32_t d2, int pos, int lim,
                                          uint8_t *tp) {
    int cnt = 0;
    uint32_t lo = d0, hi = d1;
    int chunk_lim = lim < 32 ? lim : 32;
    for (int half = 0; half < 2; ++half) {
        while (pos < chunk_lim) {
            const uint32_t w = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)pos);
            uint32_t e = lut[w & 0xFFu];
            if (e & 0x8000u) e = descend(lut, e, w, n_tables);
            if (kWrite) tp[cnt] = (uint8_t)e;
            pos += (int)((e >> 8) & 31u) + 1;
            ++cnt;
        }
        pos -= 32;
        chunk_lim = lim - 32;
        lo = hi;
        hi = d2;
    }
    return cnt;
}

__device__ __forceinline__ uint32_t join2(uint32_t e2, uint32_t sm2) {
    // two weights: exponents in bytes 0/1 of e2, sign|mantissa in bytes 0/1 of sm2
    const uint32_t e0 = e2 & 0xFFu, e1 = (e2 >> 8) & 0xFFu;
    const uint32_t s0 = sm2 & 0xFFu, s1 = (sm2 >> 8) & 0xFFu;
    const uint32_t w0 = ((s0 & 0x80u) << 8) | (e0 << 7) | (s0 & 0x7Fu);
    const uint32_t w1 = ((s1 & 0x80u) << 8) | (e1 << 7) | (s1 & 0x7Fu);
    return w0 | (w1 << 16);
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kGroupThreads) void df11_decode_kernel(DecodeArgs a) {
    extern __shared__ uint4 smem_u4[];
    uint8_t *smem = reinterpret_cast<uint8_t *>(smem_u4);
    const uint16_t *lut = reinterpret_cast<const uint16_t *>(smem);

    const uint32_t lut_u4 = a.n_tables * (kTableBytes / 16);
    for (uint32_t i = threadIdx.x; i < lut_u4; i += kGroupThreads) smem_u4[i] = a.luts[i];
    __syncthreads();

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = (int)(threadIdx.x % kWave);
    uint8_t *tile = smem + a.n_tables * kTableBytes + wave * kTileBytes;
    const uint32_t stride = gridDim.x * kWavesPerGroup;

    for (uint32_t b = blockIdx.x * kWavesPerGroup + wave; b < a.n_blocks; b += stride) {
        const uint64_t g = (uint64_t)b * DF11_BLOCK_SLICES + (uint32_t)lane;
        const uint32_t *sp = a.stream + 2 * g;
        const uint32_t d0 = sp[0], d1 = sp[1], d2 = sp[2];
        const uint64_t q = 5 * g;  // bit offset of this slice's gap field
        const uint32_t *gp = a.gaps + (q >> 5);
        const int gap = (int)(__builtin_amdgcn_alignbit(gp[1], gp[0], (uint32_t)(q & 31)) & 31u);
        const int64_t rem = (int64_t)a.stop_bit - (int64_t)(g * DF11_SLICE_BITS);
        const int lim = rem <= 0 ? 0 : (rem >= 64 ? 64 : (int)rem);

        // phase 1: count
        const int cnt = walk_slice<false>(lut, a.n_tables, d0, d1, d2, gap, lim, nullptr);

        // wave-wide inclusive scan of the counts
        int incl = cnt;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += y;
        }
        const int excl = incl - cnt;
        const uint32_t total = (uint32_t)__shfl(incl, kWave - 1, kWave);

        const uint32_t p0 = a.block_pos[b], p1 = a.block_pos[b + 1];
        const bool sane = p1 >= p0 && p1 <= a.n && p1 - p0 <= (uint32_t)kMaxBlockCodes;
        if ((!sane || total != p1 - p0) && lane == 0 && a.status) atomicAdd(a.status, 1u);
        if (!sane) continue;

        // phase 2: decode again, exponent bytes into the tile
        const uint32_t base = p0 & ~7u;
        walk_slice<true>(lut, a.n_tables, d0, d1, d2, gap, lim, tile + (p0 - base) + excl);
        wave_lds_sync();

        // merge with sign|mantissa and store 8 BF16 per lane
        const uint32_t groups = (p1 - base + 7) >> 3;
        for (uint32_t j = (uint32_t)lane; j < groups; j += kWave) {
            const uint32_t i0 = base + 8 * j;
            if (i0 >= p0 && i0 + 8 <= p1) {
                const uint2 ex = *reinterpret_cast<const uint2 *>(tile + 8 * j);
                const uint2 sm = *reinterpret_cast<const uint2 *>(a.signmant + i0);
                uint4 o;
                o.x = join2(ex.x, sm.x);
                o.y = join2(ex.x >> 16, sm.x >> 16);
                o.z = join2(ex.y, sm.y);
                o.w = join2(ex.y >> 16, sm.y >> 16);
                *reinterpret_cast<uint4 *>(a.out + i0) = o;
            } else {
                for (uint32_t k = 0; k < 8; ++k) {
                    const uint32_t i = i0 + k;
                    if (i >= p0 && i < p1)
                        a.out[i] = (uint16_t)join2(tile[8 * j + k], a.signmant[i]);
                }
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
    const uint64_t want = ((uint64_t)n_blocks + kWavesPerGroup - 1) / kWavesPerGroup;
    const uint64_t cap = (uint64_t)cus * (uint64_t)occ;
    *groups = (int)(want < cap ? want : cap);
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
    a.stop_bit = s->last_start + 1;
    a.n_blocks = s->n_blocks;
    a.n_tables = s->n_tables;
    hipLaunchKernelGGL(df11_decode_kernel, dim3(groups), dim3(kGroupThreads),
                       lds_bytes(s->n_tables), static_cast<hipStream_t>(hip_stream), a);
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_ERR_HIP;
}
