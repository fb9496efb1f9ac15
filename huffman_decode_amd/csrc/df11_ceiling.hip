// df11_stream_ceiling: a traffic-only kernel that moves the same bytes as one
// df11_decode launch, with the same vector widths and the same persistent
// grid, and does no decoding.  Its time is the practical floor for those
// bytes on this GPU (a plain streaming ceiling), which the decode's own time
// is measured against.
//
// Bytes, per 8-word output group g (g in [0, n/8)):
//   * 8 bytes of `a` (the sign|mantissa array: one byte per weight, loaded 8
//     at a time as the decode does);
//   * 16 bytes written to `out` (the 8 BF16 words, one 16-byte store);
//   * `b` (b_bytes, the rest of what the decode reads: code stream, gaps,
//     block positions, tables) in 16-byte loads spread evenly over the tiles
//     of groups below.
// A wave takes tiles of 64 x kUnroll consecutive groups, lane l the groups
// l + 64 u, and issues all of a tile's loads before its stores.  Every
// written word depends on the loaded bytes, so no load can be dropped.  (Of
// 2, 4 and 8 groups per lane and 768 to 6144 workgroups, 2 groups at the
// decode's grid was as fast as any: within 1%.)
#include <hip/hip_runtime.h>

#include "df11.h"

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
// resident workgroups per CU, as for the decode kernel (3 of 8 waves)
constexpr int kGroupsPerCu = 3;
constexpr int kUnroll = 2;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x2 g_cu32x2;
typedef __attribute__((address_space(1))) const u32x4 g_cu32x4;
typedef __attribute__((address_space(1))) u32x4 g_u32x4;

__global__ __launch_bounds__(kThreads) void df11_ceiling_kernel(const uint8_t *a, const uint8_t *b,
                                                                uint64_t b_units, uint16_t *out,
                                                                uint64_t groups) {
    const uint32_t lane = threadIdx.x % 64;
    const uint64_t wave = (uint64_t)blockIdx.x * kWaves + threadIdx.x / 64;
    const uint64_t n_waves = (uint64_t)gridDim.x * kWaves;
    const uint64_t tiles = (groups + 64 * kUnroll - 1) / (64 * kUnroll);
    for (uint64_t t = wave; t < tiles; t += n_waves) {
        const uint64_t g0 = t * 64 * kUnroll;
        u32x2 s[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t g = g0 + 64 * u + lane;
            s[u] = g < groups ? *(g_cu32x2 *)(a + 8 * g) : u32x2{0, 0};
        }
        // this tile's share of b: units [ub0, ub1)
        const uint64_t ub0 = t * b_units / tiles, ub1 = (t + 1) * b_units / tiles;
        u32x4 extra = {0, 0, 0, 0};
        for (uint64_t uu = ub0 + lane; uu < ub1; uu += 64) extra ^= *(g_cu32x4 *)(b + 16 * uu);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t g = g0 + 64 * u + lane;
            u32x4 w;  // the 8 bytes widened to 8 words
            w.x = (s[u].x & 0xFFu) | ((s[u].x & 0xFF00u) << 8);
            w.y = ((s[u].x >> 16) & 0xFFu) | ((s[u].x >> 8) & 0xFF0000u);
            w.z = (s[u].y & 0xFFu) | ((s[u].y & 0xFF00u) << 8);
            w.w = ((s[u].y >> 16) & 0xFFu) | ((s[u].y >> 8) & 0xFF0000u);
            if (g < groups) *(g_u32x4 *)(out + 8 * g) = w ^ extra;
        }
    }
}

}  // namespace

extern "C" int df11_stream_ceiling(const uint8_t *a, const uint8_t *b, uint64_t b_bytes,
                                   uint16_t *out, uint64_t n, uint32_t max_groups,
                                   void *hip_stream) {
    if (!a || !out || n == 0 || n % 8 != 0 || (b_bytes && !b) || b_bytes % 16 != 0)
        return DF11_ERR_ARG;
    if (reinterpret_cast<uintptr_t>(a) % 8 || reinterpret_cast<uintptr_t>(b) % 16 ||
        reinterpret_cast<uintptr_t>(out) % 16)
        return DF11_ERR_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return DF11_ERR_HIP;
    uint64_t grid = (uint64_t)cus * kGroupsPerCu;
    if (max_groups && max_groups < grid) grid = max_groups;
    const uint64_t groups = n / 8;
    const uint64_t want = (groups + (uint64_t)kThreads * kUnroll - 1) / ((uint64_t)kThreads * kUnroll);
    if (want < grid) grid = want;
    hipLaunchKernelGGL(df11_ceiling_kernel, dim3((uint32_t)grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(hip_stream), a, b, b_bytes / 16, out, groups);
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_ERR_HIP;
}

// ---------------------------------------------------------------- plain streams
//
// Read-only, write-only and copy kernels over `bytes` (a multiple of 16) with
// 16-byte accesses: the GPU's own streaming limits, beside which the decode's
// figure and its same-pattern ceiling above are read.  A thread keeps four
// accesses in flight (at a stride of the workgroup size: each access of a
// wave covers 1 KB in one piece, which was faster than 64 contiguous bytes
// per thread).  The default grid, 128 workgroups of 256 threads per compute
// unit, was the fastest tried for writes and copies (1 or 4 deep, 2048 to
// 32768 workgroups); reads run faster on fewer (2048).

namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamDepth = 4;
constexpr int kStreamGroupsPerCu = 128;

__global__ __launch_bounds__(kStreamThreads) void df11_stream_read_kernel(const u32x4 *src,
                                                                          uint64_t n16,
                                                                          uint32_t *out) {
    const uint64_t t = (uint64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * kStreamThreads * kStreamDepth;
    u32x4 acc = {0, 0, 0, 0};
    for (uint64_t i = (uint64_t)blockIdx.x * kStreamThreads * kStreamDepth + threadIdx.x; i < n16;
         i += stride) {
        u32x4 r[kStreamDepth];
#pragma unroll
        for (int d = 0; d < kStreamDepth; ++d) {
            const uint64_t j = i + (uint64_t)d * kStreamThreads;
            r[d] = j < n16 ? src[j] : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int d = 0; d < kStreamDepth; ++d) acc ^= r[d];
    }
    out[t] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(kStreamThreads) void df11_stream_write_kernel(u32x4 *dst, uint64_t n16,
                                                                           uint32_t value) {
    const uint64_t stride = (uint64_t)gridDim.x * kStreamThreads * kStreamDepth;
    for (uint64_t i = (uint64_t)blockIdx.x * kStreamThreads * kStreamDepth + threadIdx.x; i < n16;
         i += stride) {
#pragma unroll
        for (int d = 0; d < kStreamDepth; ++d) {
            const uint64_t j = i + (uint64_t)d * kStreamThreads;
            if (j < n16) dst[j] = u32x4{value, value, value, (uint32_t)j};
        }
    }
}

__global__ __launch_bounds__(kStreamThreads) void df11_stream_copy_kernel(const u32x4 *src,
                                                                          u32x4 *dst,
                                                                          uint64_t n16) {
    const uint64_t stride = (uint64_t)gridDim.x * kStreamThreads * kStreamDepth;
    for (uint64_t i = (uint64_t)blockIdx.x * kStreamThreads * kStreamDepth + threadIdx.x; i < n16;
         i += stride) {
        u32x4 r[kStreamDepth];
#pragma unroll
        for (int d = 0; d < kStreamDepth; ++d) {
            const uint64_t j = i + (uint64_t)d * kStreamThreads;
            r[d] = j < n16 ? src[j] : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int d = 0; d < kStreamDepth; ++d) {
            const uint64_t j = i + (uint64_t)d * kStreamThreads;
            if (j < n16) dst[j] = r[d];
        }
    }
}

int stream_grid(uint32_t grid, uint64_t n16, uint32_t *out) {
    if (grid == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return DF11_ERR_HIP;
        grid = (uint32_t)cus * kStreamGroupsPerCu;
    }
    const uint64_t want = (n16 + (uint64_t)kStreamThreads * kStreamDepth - 1) /
                          ((uint64_t)kStreamThreads * kStreamDepth);
    *out = (uint32_t)(want < grid ? want : grid);
    return DF11_OK;
}

bool bad16(const void *p) { return !p || reinterpret_cast<uintptr_t>(p) % 16 != 0; }

}  // namespace

extern "C" uint32_t df11_stream_read_slots(uint64_t bytes, uint32_t grid) {
    uint32_t g = 0;
    if (bytes == 0 || bytes % 16 != 0 || stream_grid(grid, bytes / 16, &g) != DF11_OK) return 0;
    return g * kStreamThreads;
}

extern "C" int df11_stream_read(const void *src, uint64_t bytes, uint32_t *out, uint64_t out_count,
                                uint32_t grid, void *hip_stream) {
    if (bad16(src) || !out || bytes == 0 || bytes % 16 != 0) return DF11_ERR_ARG;
    uint32_t g = 0;
    const int st = stream_grid(grid, bytes / 16, &g);
    if (st != DF11_OK) return st;
    if (out_count < (uint64_t)g * kStreamThreads) return DF11_ERR_BUFSIZE;
    hipLaunchKernelGGL(df11_stream_read_kernel, dim3(g), dim3(kStreamThreads), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<const u32x4 *>(src),
                       bytes / 16, out);
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_ERR_HIP;
}

extern "C" int df11_stream_write(void *dst, uint64_t bytes, uint32_t value, uint32_t grid,
                                 void *hip_stream) {
    if (bad16(dst) || bytes == 0 || bytes % 16 != 0) return DF11_ERR_ARG;
    uint32_t g = 0;
    const int st = stream_grid(grid, bytes / 16, &g);
    if (st != DF11_OK) return st;
    hipLaunchKernelGGL(df11_stream_write_kernel, dim3(g), dim3(kStreamThreads), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<u32x4 *>(dst), bytes / 16,
                       value);
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_ERR_HIP;
}

extern "C" int df11_stream_copy(const void *src, void *dst, uint64_t bytes, uint32_t grid,
                                void *hip_stream) {
    if (bad16(src) || bad16(dst) || bytes == 0 || bytes % 16 != 0) return DF11_ERR_ARG;
    uint32_t g = 0;
    const int st = stream_grid(grid, bytes / 16, &g);
    if (st != DF11_OK) return st;
    hipLaunchKernelGGL(df11_stream_copy_kernel, dim3(g), dim3(kStreamThreads), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<const u32x4 *>(src),
                       static_cast<u32x4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_ERR_HIP;
}
