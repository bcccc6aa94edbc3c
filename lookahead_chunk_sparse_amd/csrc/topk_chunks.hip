// Fixed-budget chunk re-selection for gfx950: per row, the first k chunks of
// the order (logit descending, chunk index ascending), written in ascending
// chunk order (paperlayer.ai summary of "FlashMemory-DeepSeek-V4", 1
// Introduction and 2.1 Architecture: only the chunks the indexer ranks
// highest are kept; ties go to the lower chunk index).
//
// One 1024-thread workgroup per row; thread t keeps logits [t*KPT, (t+1)*KPT)
// in registers as order-preserving unsigned keys (logit XOR 0x80000000),
// offset by the row's smallest key so that only the bits spanning the row's
// range remain (logits of both signs would otherwise differ in every bit).
//  1. Radix select, 8 bits per pass from the top of the range: the keys of
//     the current bucket are counted per digit into an LDS histogram
//     (ds_add), then one wave finds, by a suffix scan over the 256 bins, the
//     digit that holds the k-th largest key.  The result is that key v* and
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

__device__ inline uint32_t wave_min(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}
__device__ inline uint32_t wave_max(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}

constexpr int kDigitBits = 8;
constexpr int kBins = 1 << kDigitBits;

// Threshold mode (counts != nullptr): the row keeps the chunks whose logit
// exceeds `thr`, at most k of them (the first k in the same order when more
// pass); the output row is padded with -1 and counts[row] = chunks kept.
template <int KPT>
__global__ __launch_bounds__(kThreads) void topk_kernel(const int32_t* __restrict__ logits, int C, int k,
                                                        int32_t* __restrict__ out, int32_t thr,
                                                        int32_t* __restrict__ counts) {
    __shared__ int sm_i[kWaves];
    __shared__ uint32_t sm_min[kWaves], sm_max[kWaves];
    __shared__ int sm_hist[kBins];
    __shared__ int sm_pick[2];  // digit chosen by the pass, keys still needed
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t* row = logits + (int64_t)blockIdx.x * C;
    int32_t* dst = out + (int64_t)blockIdx.x * k;
    const int base = tid * KPT;

    uint32_t key[KPT];
    uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const int idx = base + e;
        key[e] = idx < C ? ((uint32_t)row[idx] ^ 0x80000000u) : 0u;
        if (idx < C) {
            lmin = min(lmin, key[e]);
            lmax = max(lmax, key[e]);
        }
    }
    lmin = wave_min(lmin);
    lmax = wave_max(lmax);
    if (lane == 0) {
        sm_min[wave] = lmin;
        sm_max[wave] = lmax;
    }
    __syncthreads();
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        kmin = min(kmin, sm_min[w]);
        kmax = max(kmax, sm_max[w]);
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

    // --- radix select on key - kmin, 8 bits per pass ---
    // Keys of padding slots (index >= C) are never counted.
    uint32_t rel[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) rel[e] = key[e] - kmin;  // < 2^nb for valid keys
    const uint32_t range = kmax - kmin;
    const int nb = range == 0u ? 0 : 32 - __builtin_clz(range);
    uint64_t prefix = 0;  // digits chosen so far, as the value of key - kmin above bit `hi`
    int need = kk;
    for (int hi = nb; hi > 0; hi -= kDigitBits) {
        const int w = hi < kDigitBits ? hi : kDigitBits;
        const int sh = hi - w;
        for (int j = tid; j < kBins; j += kThreads) sm_hist[j] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const uint64_t r = rel[e];
            if (base + e < C && (r >> hi) == prefix)
                atomicAdd(&sm_hist[(int)((r >> sh) & ((1u << w) - 1u))], 1);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds bins 4l..4l+3; exclusive suffix sum over lanes
            int h[4], sl = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h[j] = sm_hist[4 * lane + j];
                sl += h[j];
            }
            int suf = sl;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int u = __shfl_down(suf, off);
                if (lane + off < 64) suf += u;
            }
            int above = suf - sl;  // keys of the bucket in higher digits
#pragma unroll
            for (int j = 3; j >= 0; --j) {
                if (above < need && need <= above + h[j]) {  // exactly one (lane, j) matches
                    sm_pick[0] = 4 * lane + j;
                    sm_pick[1] = need - above;
                }
                above += h[j];
            }
        }
        __syncthreads();
        prefix = (prefix << w) | (uint64_t)sm_pick[0];
        need = sm_pick[1];
    }
    const uint32_t vstar = kmin + (uint32_t)prefix;

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
