// stream_read.hip -- plain HBM streaming kernels for the benchmark (not part of the attention
// library). The read kernel reads two device ranges once with non-temporal 16-byte loads, the
// access the decode kernels make to a KV cache, and does nothing else; the write kernel writes
// one range once with 16-byte stores, the access of a kernel whose output dominates its
// traffic (the probe producer). Their times for a given byte count are the floors the
// attention kernels of the same bytes are measured against (launch, ramp and the board's
// sustained rate included).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 at(const u32x4* a, size_t na, const u32x4* b, size_t i) {
    return __builtin_nontemporal_load(i < na ? a + i : b + (i - na));
}

// The virtual range [0, na + nb) of 16-byte elements (a first, then b) is cut into tiles of
// 8 * 256 elements (32 KB); workgroup w reads tiles w, w + grid, ..., each thread issuing its 8
// loads (one per 4 KB row of the tile, so every load instruction covers 4 KB contiguously)
// before using any. The XOR of everything read goes to sink only if it equals a value no
// input here produces, which keeps the loads alive.
constexpr int kUnroll = 8;
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ a, size_t na,
                                                          const u32x4* __restrict__ b, size_t nb,
                                                          uint32_t* __restrict__ sink) {
    const size_t n = na + nb;
    constexpr size_t tile = (size_t)kUnroll * 256;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t t0 = (size_t)blockIdx.x * tile; t0 < n; t0 += (size_t)gridDim.x * tile) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const size_t i = t0 + (size_t)j * 256 + threadIdx.x;
            x[j] = i < n ? at(a, na, b, i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) acc ^= x[j];
    }
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9E3779B9u) sink[blockIdx.x & 1023] = x;
}

// The same read restricted to the rows a decode call reads from a [B*H, L_max, 256-byte row]
// cache pair (L_max a multiple of 128, so that every 32 KB tile lies inside one (b, h)): the
// rows of a tile at or past the length of its (b, h) are skipped without a memory access, a
// tile wholly past it without a load. This is the floor of a decode call on the cache's own
// layout, where every (b, h) leaves the rows past its sequence end unread.
__global__ __launch_bounds__(256) void stream_read_rows_kernel(const u32x4* __restrict__ k,
                                                               const u32x4* __restrict__ v,
                                                               const int32_t* __restrict__ seqlens,
                                                               int H, int L_max, size_t na,
                                                               uint32_t* __restrict__ sink) {
    const size_t n = 2 * na;
    constexpr size_t tile = (size_t)kUnroll * 256;
    const size_t per_bh = (size_t)L_max * 16;  // 16-byte elements per (b, h)
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t t0 = (size_t)blockIdx.x * tile; t0 < n; t0 += (size_t)gridDim.x * tile) {
        const size_t e0 = t0 < na ? t0 : t0 - na;
        const u32x4* src = t0 < na ? k : v;
        const size_t bh = e0 / per_bh;  // the tile's (b, h), uniform
        const int row0 = (int)((e0 - bh * per_bh) >> 4);
        const int len = seqlens[bh / (size_t)H];
        if (row0 >= len) continue;
        u32x4 x[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int e = j * 256 + (int)threadIdx.x;
            x[j] = row0 + (e >> 4) < len ? __builtin_nontemporal_load(src + e0 + e)
                                          : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) acc ^= x[j];
    }
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9E3779B9u) sink[blockIdx.x & 1023] = x;
}

// Workgroup w writes tiles w, w + grid, ... of 32 KB (8 stores of 16 bytes per thread, each
// store instruction covering 4 KB contiguously); the value written is the tile index.
__global__ __launch_bounds__(256) void stream_write_kernel(u32x4* __restrict__ a, size_t n) {
    constexpr size_t tile = (size_t)kUnroll * 256;
    for (size_t t0 = (size_t)blockIdx.x * tile; t0 < n; t0 += (size_t)gridDim.x * tile) {
        const uint32_t v = (uint32_t)(t0 / tile);
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const size_t i = t0 + (size_t)j * 256 + threadIdx.x;
            if (i < n) a[i] = u32x4{v, v, v, v};
        }
    }
}

}  // namespace

// Writes bytes (a multiple of 16) at a (16-byte aligned) with `grid` workgroups of 256 threads
// on `stream`. Returns 0, or the HIP error code of the launch.
extern "C" int plx_bench_stream_write(void* a, size_t bytes, int grid, void* stream) {
    if (grid < 1 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_write_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (u32x4*)a, bytes / 16);
    return (int)hipGetLastError();
}

// Reads bytes_a bytes at a and bytes_b bytes at b (multiples of 16, 16-byte aligned) with
// `grid` workgroups of 256 threads on `stream`; sink holds at least 1024 words. Returns 0, or
// the HIP error code of the launch.
extern "C" int plx_bench_stream_read(const void* a, size_t bytes_a, const void* b,
                                     size_t bytes_b, void* sink, int grid, void* stream) {
    if (grid < 1 || (bytes_a | bytes_b) % 16 != 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)a, bytes_a / 16, (const u32x4*)b, bytes_b / 16,
                       (uint32_t*)sink);
    return (int)hipGetLastError();
}

// Reads the rows [0, min(seqlens[b], L_max)) of every (b, h) of the caches k and v, each
// [B, H, L_max, 128] bf16 (256-byte rows, L_max a multiple of 128), with `grid` workgroups on
// `stream`; sink holds at least 1024 words. Returns 0, or the HIP error code of the launch.
extern "C" int plx_bench_stream_read_rows(const void* k, const void* v, const int32_t* seqlens,
                                          int B, int H, int L_max, void* sink, int grid,
                                          void* stream) {
    if (grid < 1 || B < 1 || H < 1 || L_max < 128 || L_max % 128 != 0)
        return (int)hipErrorInvalidValue;
    const size_t na = (size_t)B * H * L_max * 16;
    hipLaunchKernelGGL(stream_read_rows_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)k, (const u32x4*)v, seqlens, H, L_max, na,
                       (uint32_t*)sink);
    return (int)hipGetLastError();
}
