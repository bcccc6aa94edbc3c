// Pool-slot assignment for a delta fetch: when the selection changes from
// S_prev to S_new, chunks in both keep their HBM pool slot and only the new
// ones are fetched, into slots S_prev does not use (S_prev is still being
// attended over while S_new arrives).  Non-recalled chunks simply drop out of
// the pool: the host copy stays the reference (paperlayer.ai summary of
// "FlashMemory-DeepSeek-V4", 2.1 Architecture: non-recalled entries are
// evicted to CPU; the handbook page's prefetching of only the critical
// chunks every 64 tokens).
//
// Rule (deterministic): the r-th chunk of S_new, in ascending id order, that
// is not in S_prev gets the r-th lowest slot that no entry of S_prev holds.
// An entry with a negative id is not in use (the -1 padding a threshold
// selection writes past its count): in S_prev it holds no slot, in S_new it
// gets slot -1 and is not fetched.
// One 1024-thread workgroup per request: S_prev's entries in use (id and
// slot, in list order) and a bitmap of their slots are staged in LDS; each
// thread takes a contiguous range of S_new (binary search in S_prev) and of
// the slots (free-slot compaction); block-wide exclusive scans compact
// S_prev and give every new chunk its rank and every free slot its position.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsa_kernels.h"

namespace lsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ inline int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off);
        if (lane >= off) v += u;
    }
    return v;
}

__device__ inline int block_excl_scan(int v, int* sm, int lane, int wave) {
    const int incl = wave_incl_scan(v, lane);
    if (lane == 63) sm[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += sm[w];
    __syncthreads();
    return before + incl - v;
}

// LDS use: prev ids and slots (2 n_prev ints) + free list (P ints) + slot bitmap (P bytes)
__global__ __launch_bounds__(kThreads) void pool_assign_kernel(const int32_t* __restrict__ prev_ids,
                                                               const int32_t* __restrict__ prev_slots, int n_prev,
                                                               const int32_t* __restrict__ new_ids, int k, int P,
                                                               int32_t* __restrict__ new_slots,
                                                               int32_t* __restrict__ fetch_slots) {
    extern __shared__ int lds[];
    __shared__ int sm_scan[kWaves];
    __shared__ int sm_nprev;
    int* s_prev = lds;                                            // [n_prev] ids in use, list order
    int* s_prev_slot = lds + n_prev;                              // [n_prev] their slots
    int* s_free = lds + 2 * n_prev;                               // [P]
    unsigned char* s_used = reinterpret_cast<unsigned char*>(lds + 2 * n_prev + P);  // [P]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const int32_t* pid = prev_ids + b * n_prev;
    const int32_t* psl = prev_slots + b * n_prev;
    const int32_t* nid = new_ids + b * k;

    for (int s = tid; s < P; s += kThreads) s_used[s] = 0;
    // S_prev's entries in use, compacted in list order (still ascending by id)
    {
        const int per_p = (n_prev + kThreads - 1) / kThreads;
        const int p0 = min(tid * per_p, n_prev), p1 = min(p0 + per_p, n_prev);
        int n_in = 0;
        for (int j = p0; j < p1; ++j) n_in += pid[j] >= 0;
        int at = block_excl_scan(n_in, sm_scan, lane, wave);
        for (int j = p0; j < p1; ++j)
            if (pid[j] >= 0) {
                s_prev[at] = pid[j];
                s_prev_slot[at] = psl[j];
                ++at;
            }
        if (tid == kThreads - 1) sm_nprev = at;  // the last thread's range ends the list
    }
    __syncthreads();
    const int np = sm_nprev;
    for (int j = tid; j < np; j += kThreads) {
        const int s = s_prev_slot[j];
        if (s >= 0 && s < P) s_used[s] = 1;
    }
    __syncthreads();

    // free slots in ascending order
    const int per_s = (P + kThreads - 1) / kThreads;
    const int s0 = tid * per_s, s1 = min(s0 + per_s, P);
    int n_free = 0;
    for (int s = s0; s < s1; ++s) n_free += !s_used[s];
    int pos = block_excl_scan(n_free, sm_scan, lane, wave);
    for (int s = s0; s < s1; ++s)
        if (!s_used[s]) s_free[pos++] = s;
    __syncthreads();

    // new entries: not in use, kept (found in S_prev) or fetched (next free slot)
    const int per_j = (k + kThreads - 1) / kThreads;
    const int j0 = min(tid * per_j, k), j1 = min(j0 + per_j, k);
    auto find = [&](int c) {  // index in S_prev of chunk c, or -1
        int lo = 0, hi = np;  // first prev index with id >= c
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_prev[mid] < c) lo = mid + 1; else hi = mid;
        }
        return lo < np && s_prev[lo] == c ? lo : -1;
    };
    int n_new = 0;
    for (int j = j0; j < j1; ++j) {
        const int c = nid[j];
        n_new += c >= 0 && find(c) < 0;
    }
    int rank = block_excl_scan(n_new, sm_scan, lane, wave);
    for (int j = j0; j < j1; ++j) {
        const int c = nid[j];
        if (c < 0) {
            new_slots[b * k + j] = -1;
            fetch_slots[b * k + j] = -1;
            continue;
        }
        const int at = find(c);
        if (at >= 0) {
            new_slots[b * k + j] = s_prev_slot[at];
            fetch_slots[b * k + j] = -1;
        } else {
            const int s = s_free[rank++];  // rank < number of free slots: P >= n_prev + k
            new_slots[b * k + j] = s;
            fetch_slots[b * k + j] = s;
        }
    }
}

}  // namespace

size_t pool_assign_lds_bytes(int n_prev, int P) {
    return (size_t)(2 * (int64_t)n_prev + P) * sizeof(int) + (size_t)P;
}

hipError_t launch_pool_assign(const int32_t* prev_ids, const int32_t* prev_slots, int n_prev, const int32_t* new_ids,
                              int B, int k, int P, int32_t* new_slots, int32_t* fetch_slots, hipStream_t stream) {
    hipLaunchKernelGGL(pool_assign_kernel, dim3((unsigned)B), dim3(kThreads), pool_assign_lds_bytes(n_prev, P),
                       stream, prev_ids, prev_slots, n_prev, new_ids, k, P, new_slots, fetch_slots);
    return hipGetLastError();
}

}  // namespace lsa
