// Read-only kernels that give the memory ceilings the GEMV is measured
// against (measurement only; the product library does not use them).
//
//   sgemv_bench_stream_read   every byte of a buffer, streamed with 16-byte
//                             non-temporal loads: the HBM read ceiling.
//   sgemv_bench_listed_read   the weight bytes a one-row sparse GEMV over a
//                             list reads from a packed blob (for every half
//                             tile, the 128-byte run of each listed column),
//                             with the same 16-byte lanes and the same grid
//                             of half tiles x 1024-column segments, and
//                             nothing else: no activations, no scales, no
//                             arithmetic, no sums across workgroups.
//
// Both fold what they read into one word per thread and store it only when
// it equals a value the data never produces, so the loads cannot be dropped
// and nothing is written.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kNever = 0x9E3779B9u;

__global__ __launch_bounds__(512) void k_stream_read(const u32x4* __restrict__ p, size_t n16,
                                                     uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    const uint32_t f = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (f == kNever) sink[threadIdx.x] = f;
}

// One workgroup per (half tile, 1024-column segment) of 8 wavefronts; the
// wavefront of group g reads, for each listed column of its 128 columns, 16
// bytes per lane (lane = slot c x block o: block o of the run, 8 columns per
// instruction), all issued before any is used, like the GEMV's loads.
__global__ __launch_bounds__(512) void k_listed_read(const uint8_t* __restrict__ w, const int32_t* __restrict__ starts,
                                                     const int32_t* __restrict__ idx, int K, int tiles,
                                                     uint32_t* __restrict__ sink) {
    const int vt = blockIdx.x % tiles, seg = blockIdx.x / tiles;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = seg * 8 + wave;
    if (g * 128 >= K) return;
    const int a = starts[g], b = starts[g + 1];   // the group's entries idx[a .. b)
    const uint8_t* run = w + (size_t)(vt >> 1) * K * 256 + (vt & 1) * 128 + 16 * (lane & 7);
    const int slot = lane >> 3;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int n = b - a;
    for (int j0 = 0; j0 < n; j0 += 8 * 8) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + 8 * u + slot;
            const int k = j < n ? idx[a + j] : idx[a];
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(run + (size_t)k * 256));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u];
    }
    const uint32_t f = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (f == kNever) sink[threadIdx.x] = f;
}

}  // namespace

// Streams bytes (a multiple of 16, 16-byte aligned) of device memory at p.
extern "C" int sgemv_bench_stream_read(const void* p, size_t bytes, void* sink, void* stream) {
    if (!p || !sink || bytes % 16 || (uintptr_t)p % 16) return -1;
    hipLaunchKernelGGL(k_stream_read, dim3(4096), dim3(512), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(p), bytes / 16, static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Reads the listed columns' runs of a packed weight region w (N x K codes,
// 512-output tiles): idx holds the ascending listed columns, starts[g] the
// position of group g's first entry (K / 128 + 1 entries, device memory).
extern "C" int sgemv_bench_listed_read(const void* w, const int32_t* starts, const int32_t* idx, int32_t K,
                                       int32_t N, void* sink, void* stream) {
    if (!w || !starts || !idx || !sink || K <= 0 || K % 128 || N <= 0 || N % 512) return -1;
    const int tiles = N / 256, segs = (K + 1023) / 1024;
    hipLaunchKernelGGL(k_listed_read, dim3(tiles * segs), dim3(512), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint8_t*>(w), starts, idx, (int)K, tiles, static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
