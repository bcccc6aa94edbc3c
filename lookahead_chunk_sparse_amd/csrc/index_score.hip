// Memory-indexer scan for gfx950: int8 dot products of the indexer query with
// every chunk's compressed indexer key, plus the sigmoid of the scaled logit
// (paperlayer.ai summary of "FlashMemory-DeepSeek-V4", 2.1 Architecture: the
// indexer reuses the compressed indexer keys and replaces a hard top-k by a
// sigmoid; 3 Experiments / Limitations: a shallow dot-product interaction).
//
// The scan reads every key byte once (HBM-bound, 1 byte per multiply-add),
// so it is a streaming GEMV on the vector ALUs, not an MFMA contraction:
// a key row of d_idx bytes is split over d_idx/16 lanes, each loading 16
// contiguous bytes (one wave instruction covers 1 KB of consecutive rows),
// doing 4 packed int8 dot products (v_dot4_i32_i8), and the lanes of a row
// reduce with cross-lane shuffles.  Logits are exact in int32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lsa_kernels.h"

namespace lsa {
namespace {

constexpr int kThreads = 256;

__device__ inline int dot16(const uint4& a, const uint4& b) {
    int acc = __builtin_amdgcn_sdot4((int)a.x, (int)b.x, 0, false);
    acc = __builtin_amdgcn_sdot4((int)a.y, (int)b.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)a.z, (int)b.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)a.w, (int)b.w, acc, false);
    return acc;
}

template <int DIDX>
__global__ __launch_bounds__(kThreads) void index_score_kernel(const int8_t* __restrict__ q,
                                                               const int8_t* __restrict__ keys, int B, int nq,
                                                               int C, float alpha, int32_t* __restrict__ logits,
                                                               float* __restrict__ scores) {
    constexpr int L = DIDX / 16;  // lanes per key row
    constexpr int RPB = kThreads / L;
    const int piece = threadIdx.x % L;
    const int64_t rows = (int64_t)B * C;
    for (int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / L; row < rows; row += (int64_t)gridDim.x * RPB) {
        const uint4 kk = *reinterpret_cast<const uint4*>(keys + row * DIDX + 16 * piece);
        const int64_t b = row / C, c = row % C;
        for (int r = 0; r < nq; ++r) {
            const uint4 qq = *reinterpret_cast<const uint4*>(q + ((b * nq + r) * DIDX) + 16 * piece);
            int acc = dot16(kk, qq);
#pragma unroll
            for (int off = L / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
            if (piece == 0) {
                const int64_t o = (b * nq + r) * (int64_t)C + c;
                logits[o] = acc;
                if (scores) {
                    const float x = alpha * (float)acc;
                    scores[o] = 1.0f / (1.0f + expf(-x));
                }
            }
        }
    }
}

template <int DIDX>
hipError_t launch(const int8_t* q, const int8_t* keys, int B, int nq, int C, float alpha, int32_t* logits,
                  float* scores, hipStream_t stream) {
    constexpr int RPB = kThreads / (DIDX / 16);
    const int64_t rows = (int64_t)B * C;
    int64_t blocks = (rows + RPB - 1) / RPB;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(index_score_kernel<DIDX>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, q, keys, B, nq,
                       C, alpha, logits, scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_index_score(const int8_t* q_idx, const int8_t* k_idx, int B, int nq, int C, int d_idx,
                              float alpha, int32_t* logits, float* scores, hipStream_t stream) {
    switch (d_idx) {
        case 16: return launch<16>(q_idx, k_idx, B, nq, C, alpha, logits, scores, stream);
        case 32: return launch<32>(q_idx, k_idx, B, nq, C, alpha, logits, scores, stream);
        case 64: return launch<64>(q_idx, k_idx, B, nq, C, alpha, logits, scores, stream);
        case 128: return launch<128>(q_idx, k_idx, B, nq, C, alpha, logits, scores, stream);
        case 256: return launch<256>(q_idx, k_idx, B, nq, C, alpha, logits, scores, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lsa
