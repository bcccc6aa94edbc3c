// Host-tier fetch as a device-side gather over the host link: each
// workgroup copies whole 64-token chunks (K and V of every KV head) from
// pinned host memory, mapped into the GPU's address space, into their HBM
// pool slots (paperlayer.ai summary of "FlashMemory-DeepSeek-V4", 2.1
// Architecture: non-recalled entries are evicted to CPU; 3 Experiments /
// Experimental Setup: recalled chunks come back from CPU cold storage every
// tau = 64 steps).
//
// Why a kernel: every chunk is a separate 256 KB piece, and one DMA copy per
// piece costs more in per-copy overhead than the piece takes on the link
// (about 19 GB/s on one stream for 256 KB pieces, against about 56 GB/s for
// this gather and 58 GB/s for one contiguous copy, measured on MI355X).
// Reading the chunk ids from device memory also lets the fetch follow the
// top-k selection on the GPU with no host round trip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsa_kernels.h"

namespace lsa {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(kThreads) void fetch_pull_kernel(const uint4* __restrict__ host_kv, int64_t C,
                                                              const int32_t* __restrict__ ids,
                                                              const int32_t* __restrict__ slots,
                                                              uint4* __restrict__ pool, int64_t P, int k,
                                                              int64_t entries, int64_t chunk_u4) {
    for (int64_t e = blockIdx.x; e < entries; e += gridDim.x) {
        const int64_t b = e / k, j = e % k;
        const int64_t c = ids[e];
        const int64_t p = slots ? slots[e] : j;
        if (c < 0 || c >= C || p < 0 || p >= P) continue;  // invalid entry: its slot is left as it was
        const uint4* src = host_kv + (b * C + c) * chunk_u4;
        uint4* dst = pool + (b * P + p) * chunk_u4;
        for (int64_t o = threadIdx.x; o < chunk_u4; o += (int64_t)kThreads * kInFlight) {
            uint4 v[kInFlight];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) {
                const int64_t x = o + (int64_t)u * kThreads;
                v[u] = x < chunk_u4 ? src[x] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) {
                const int64_t x = o + (int64_t)u * kThreads;
                if (x < chunk_u4) dst[x] = v[u];
            }
        }
    }
}

}  // namespace

hipError_t launch_fetch_pull(const uint16_t* host_kv_dev, int64_t C, const int32_t* ids, const int32_t* slots,
                             uint16_t* pool, int64_t P, int B, int Hkv, int d, int k, int grid, hipStream_t stream) {
    const int64_t entries = (int64_t)B * k;
    const int64_t chunk_u4 = (int64_t)2 * Hkv * kChunkTokens * d * 2 / 16;
    const int64_t g = entries < grid ? entries : grid;
    hipLaunchKernelGGL(fetch_pull_kernel, dim3((unsigned)g), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(host_kv_dev), C, ids, slots, reinterpret_cast<uint4*>(pool),
                       P, k, entries, chunk_u4);
    return hipGetLastError();
}

}  // namespace lsa
