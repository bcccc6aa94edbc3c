// Opt-in validation of chunk lists (lsa_check_ids): the attention and fetch
// kernels trust their ids, so a caller can run this check first.  It reads
// only the id, store-position and count arrays.
//
// One 1024-thread workgroup per request:
//  * range: every used entry's chunk id in [0, C_ctx) and its store position
//    (the slot, or the id itself without slots) in [0, C_store);
//  * distinctness: the used entries' (value, entry) pairs are sorted in LDS
//    by a bitonic network, once for the ids and once for the slots; equal
//    neighbours are a value listed twice;
//  * counts in [0, k].
// Each rule keeps the first offending entry (b*k + j) with an atomic min,
// so the report names the same entry however the threads are scheduled.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "lsa_kernels.h"

namespace lsa {
namespace {

constexpr int kThreads = 1024;

__global__ void check_ids_init(int32_t* result) {
    if (threadIdx.x < kCheckResultWords) result[threadIdx.x] = INT32_MAX;
}

__global__ __launch_bounds__(kThreads) void check_ids_kernel(const int32_t* ids, const int32_t* slots,
                                                             const int32_t* counts, int k, int64_t C_ctx,
                                                             int64_t C_store, int32_t* result) {
    __shared__ uint64_t sm[kCheckMaxEntries];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int32_t* row = ids + (int64_t)b * k;
    const int32_t* srow = slots ? slots + (int64_t)b * k : nullptr;
    const int32_t first = b * k;  // B*k < 2^31 (checked on the host)
    int kb = k;
    if (counts) {
        const int32_t c = counts[b];
        if (c < 0 || c > k) {
            if (tid == 0) atomicMin(&result[3], b);
            kb = c < 0 ? 0 : k;  // the entries that can still be checked
        } else {
            kb = c;
        }
    }
    for (int j = tid; j < kb; j += kThreads) {
        const int64_t c = row[j];
        const int64_t p = srow ? (int64_t)srow[j] : c;
        if (c < 0 || c >= C_ctx || p < 0 || p >= C_store) atomicMin(&result[0], first + j);
    }
    int n = 1;
    while (n < kb) n <<= 1;
    for (int pass = 0; pass < (srow ? 2 : 1); ++pass) {
        const int32_t* src = pass == 0 ? row : srow;
        // order-preserving key of the value in the high word, the entry in the low word
        for (int j = tid; j < n; j += kThreads)
            sm[j] = j < kb ? ((uint64_t)((uint32_t)src[j] ^ 0x80000000u) << 32) | (uint32_t)j : ~0ull;
        __syncthreads();
        for (int size = 2; size <= n; size <<= 1)
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = tid; i < n / 2; i += kThreads) {
                    const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
                    const bool up = (lo & size) == 0;
                    const uint64_t x = sm[lo], y = sm[hi];
                    if ((x > y) == up) {
                        sm[lo] = y;
                        sm[hi] = x;
                    }
                }
                __syncthreads();
            }
        // equal values sit next to each other, the later entry second
        for (int j = tid + 1; j < kb; j += kThreads)
            if ((sm[j] >> 32) == (sm[j - 1] >> 32)) atomicMin(&result[1 + pass], first + (int32_t)(uint32_t)sm[j]);
        __syncthreads();  // sm is refilled by the next pass
    }
}

}  // namespace

hipError_t launch_check_ids(const int32_t* ids, const int32_t* slots, const int32_t* counts, int B, int k,
                            int64_t C_ctx, int64_t C_store, int32_t* result, hipStream_t stream) {
    hipLaunchKernelGGL(check_ids_init, dim3(1), dim3(64), 0, stream, result);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(check_ids_kernel, dim3((unsigned)B), dim3(kThreads), 0, stream, ids, slots, counts, k, C_ctx,
                       C_store, result);
    return hipGetLastError();
}

}  // namespace lsa
