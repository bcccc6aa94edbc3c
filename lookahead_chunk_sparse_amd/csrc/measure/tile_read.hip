// Measurement only, not part of the decode path: the read bandwidth the HBM
// delivers for a stream of whole tiles at given positions, the access
// pattern of the gathered-chunk attention without its arithmetic.  The
// benchmark reads randomly placed 16 KB K/V tiles with it to state the
// practical ceiling beside the published peak.
//
// Each workgroup takes tiles t = blockIdx.x, +gridDim.x, ... and reads them
// whole with 16-byte loads carrying the non-temporal hint (as the attention's
// tile loads do), UNROLL loads in flight per thread; the data is XOR-folded
// into one word per thread so the loads stay live.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

template <int UNROLL>
__global__ __launch_bounds__(kThreads) void tile_read_kernel(const uint4* __restrict__ base,
                                                             const int64_t* __restrict__ tile_off, int n_tiles,
                                                             int tile_u4, unsigned* __restrict__ sink) {
    unsigned acc = 0;
    for (int t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const uint4* p = base + tile_off[t];
        for (int o = threadIdx.x; o < tile_u4; o += kThreads * UNROLL) {
            uint4 v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int i = o + u * kThreads;
                v[u] = __builtin_bit_cast(
                    uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + (i < tile_u4 ? i : tile_u4 - 1))));
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

// base: device buffer; tile_off: device int64 [n_tiles], offsets of the tiles
// in units of 16 bytes (each tile lies wholly inside the buffer); tile_u4:
// tile size in 16-byte units; sink: device uint32 [grid * 256].  unroll is
// 1, 2 or 4.  Returns the hipError_t of the launch.
extern "C" int lsa_measure_tile_read(const void* base, const int64_t* tile_off, int n_tiles, int tile_u4,
                                     unsigned* sink, int grid, int unroll, hipStream_t stream) {
    if (!base || !tile_off || !sink || n_tiles < 1 || tile_u4 < 1 || grid < 1) return (int)hipErrorInvalidValue;
    const auto* b = static_cast<const uint4*>(base);
    if (unroll == 1)
        hipLaunchKernelGGL(tile_read_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, b, tile_off, n_tiles, tile_u4, sink);
    else if (unroll == 2)
        hipLaunchKernelGGL(tile_read_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, b, tile_off, n_tiles, tile_u4, sink);
    else
        hipLaunchKernelGGL(tile_read_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, b, tile_off, n_tiles, tile_u4, sink);
    return (int)hipGetLastError();
}
