// Fixed-budget chunk re-selection for gfx950: per row, the first k chunks of
// the order (logit descending, chunk index ascending), written in ascending
// chunk order (paperlayer.ai summary of "FlashMemory-DeepSeek-V4", 1
// Introduction and 2.1 Architecture: only the chunks the indexer ranks
// highest are kept; ties go to the lower chunk index).
//
// One 1024-thread workgroup per row; thread t keeps logits [t*KPT, (t+1)*KPT)
// in registers as order-preserving unsigned keys (logit XOR 0x80000000).
//  1. Radix select, one bit per pass, from the most significant bit where the
//     row's keys differ (a block-wide AND/OR finds the common leading bits):
//     a pass counts the keys of the current bucket whose next bit is set
//     (cross-lane reduction per wave, then LDS across the 16 waves) and
//     descends into the half that holds the k-th largest key.  The result is that key v* and
//     `need`, the number of keys equal to v* that belong to the selection.
//  2. Ordered compaction: keys > v* are taken; keys == v* are taken while
//     their rank among equal keys, in index order, is below `need`.  Two
//     block-wide exclusive scans (equal-key ranks, output offsets) in thread
//     order, which is index order, make the output ascending.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsa_kernels.h"

namespace lsa {
namespace {

constexpr int kThreads = kTopkThreads;
constexpr int kWaves = kThreads / 64;

__device__ inline int wave_sum(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ inline int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off);
        if (lane >= off) v += u;
    }
    return v;
}

// Block-wide sum; `sm` holds kWaves ints.  Two barriers so sm can be reused.
__device__ inline int block_sum(int v, int* sm, int lane, int wave) {
    v = wave_sum(v);
    if (lane == 0) sm[wave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += sm[w];
    __syncthreads();
    return t;
}

// Block-wide exclusive scan in thread order.
__device__ inline int block_excl_scan(int v, int* sm, int lane, int wave) {
    const int incl = wave_incl_scan(v, lane);
    if (lane == 63) sm[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += sm[w];
    __syncthreads();
    return before + incl - v;
}

__device__ inline uint32_t wave_or(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v |= (uint32_t)__shfl_xor((int)v, off);
    return v;
}
__device__ inline uint32_t wave_and(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v &= (uint32_t)__shfl_xor((int)v, off);
    return v;
}

// Threshold mode (counts != nullptr): the row keeps the chunks whose logit
// exceeds `thr`, at most k of them (the first k in the same order when more
// pass); the output row is padded with -1 and counts[row] = chunks kept.
template <int KPT>
__global__ __launch_bounds__(kThreads) void topk_kernel(const int32_t* __restrict__ logits, int C, int k,
                                                        int32_t* __restrict__ out, int32_t thr,
                                                        int32_t* __restrict__ counts) {
    __shared__ int sm_i[kWaves];
    __shared__ uint32_t sm_or[kWaves], sm_and[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t* row = logits + (int64_t)blockIdx.x * C;
    int32_t* dst = out + (int64_t)blockIdx.x * k;
    const int base = tid * KPT;

    uint32_t key[KPT];
    uint32_t lor = 0u, land = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const int idx = base + e;
        key[e] = idx < C ? ((uint32_t)row[idx] ^ 0x80000000u) : 0u;
        if (idx < C) {
            lor |= key[e];
            land &= key[e];
        }
    }
    lor = wave_or(lor);
    land = wave_and(land);
    if (lane == 0) {
        sm_or[wave] = lor;
        sm_and[wave] = land;
    }
    __syncthreads();
    lor = 0u;
    land = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        lor |= sm_or[w];
        land &= sm_and[w];
    }

    // --- how many to keep ---
    int kk = k;
    if (counts) {
        const uint32_t tkey = (uint32_t)thr ^ 0x80000000u;
        int above = 0;
#pragma unroll
        for (int e = 0; e < KPT; ++e) above += (base + e < C) && (key[e] > tkey);
        above = block_sum(above, sm_i, lane, wave);
        kk = above < k ? above : k;
        if (tid == 0) counts[blockIdx.x] = kk;
        for (int j = kk + tid; j < k; j += kThreads) dst[j] = -1;
        if (kk == 0) return;  // uniform: every thread saw the same sum
    }

    // --- radix select over the bits where keys differ ---
    uint32_t prefix = land;  // correct on every common bit
    int need = kk;
    const uint32_t diff = lor ^ land;
    if (diff != 0u) {
        const int top = 31 - __builtin_clz(diff);
        uint32_t mask = top == 31 ? 0u : ~((2u << top) - 1u);  // bits above `top`
        prefix &= mask;
        for (int bit = top; bit >= 0; --bit) {
            const uint32_t bitv = 1u << bit;
            const uint32_t cand = prefix | bitv;
            const uint32_t mb = mask | bitv;
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < KPT; ++e) cnt += (base + e < C) && ((key[e] & mb) == cand);
            cnt = block_sum(cnt, sm_i, lane, wave);
            if (cnt >= need)
                prefix = cand;
            else
                need -= cnt;
            mask = mb;
        }
    }
    const uint32_t vstar = prefix;

    // --- ordered compaction ---
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const bool valid = base + e < C;
        n_gt += valid && key[e] > vstar;
        n_eq += valid && key[e] == vstar;
    }
    const int eq_before = block_excl_scan(n_eq, sm_i, lane, wave);
    int take_eq = need - eq_before;
    take_eq = take_eq < 0 ? 0 : take_eq > n_eq ? n_eq : take_eq;
    int pos = block_excl_scan(n_gt + take_eq, sm_i, lane, wave);
    int eq_seen = eq_before;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const int idx = base + e;
        if (idx >= C) continue;
        // pos < kk holds by construction (|{> v*}| + need == kk); the test
        // keeps every store inside the row even so.
        if (key[e] > vstar) {
            if (pos < kk) dst[pos] = idx;
            ++pos;
        } else if (key[e] == vstar) {
            if (eq_seen < need) {
                if (pos < kk) dst[pos] = idx;
                ++pos;
            }
            ++eq_seen;
        }
    }
}

template <int KPT>
hipError_t launch(const int32_t* logits, int R, int C, int k, int32_t* ids, int32_t thr, int32_t* counts,
                  hipStream_t stream) {
    hipLaunchKernelGGL(topk_kernel<KPT>, dim3((unsigned)R), dim3(kThreads), 0, stream, logits, C, k, ids, thr, counts);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const int32_t* logits, int R, int C, int k, int32_t* chunk_ids, int32_t thr, int32_t* counts,
                       hipStream_t stream) {
    const int kpt = (C + kThreads - 1) / kThreads;
    if (kpt <= 1) return launch<1>(logits, R, C, k, chunk_ids, thr, counts, stream);
    if (kpt <= 2) return launch<2>(logits, R, C, k, chunk_ids, thr, counts, stream);
    if (kpt <= 4) return launch<4>(logits, R, C, k, chunk_ids, thr, counts, stream);
    if (kpt <= 8) return launch<8>(logits, R, C, k, chunk_ids, thr, counts, stream);
    if (kpt <= 16) return launch<16>(logits, R, C, k, chunk_ids, thr, counts, stream);
    if (kpt <= 32) return launch<32>(logits, R, C, k, chunk_ids, thr, counts, stream);
    if (kpt <= 64) return launch<64>(logits, R, C, k, chunk_ids, thr, counts, stream);
    return hipErrorInvalidValue;
}

}  // namespace lsa
