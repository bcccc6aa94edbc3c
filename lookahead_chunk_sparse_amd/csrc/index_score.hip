// Memory-indexer scan for gfx950: int8 dot products of the indexer query with
// every chunk's compressed indexer key, plus the sigmoid of the scaled logit
// (paperlayer.ai summary of "FlashMemory-DeepSeek-V4", 2.1 Architecture: the
// indexer reuses the compressed indexer keys and replaces a hard top-k by a
// sigmoid; 3 Experiments / Limitations: a shallow dot-product interaction).
//
// Two kernels, both exact in int32:
//  * One query row per request (the decode case): the scan reads every key
//    byte once for one multiply-add (HBM-bound), so it is a streaming GEMV on
//    the vector ALUs: a key row of d_idx bytes is split over d_idx/16 lanes,
//    each loading 16 contiguous bytes (one wave instruction covers 1 KB of
//    consecutive rows) and doing 4 packed int8 dot products (v_dot4_i32_i8);
//    the lanes of a row reduce with cross-lane shuffles.
//  * Many query rows sharing a request's keys (nq >= a threshold): a real
//    dense contraction [nq x d_idx] . [d_idx x C], run on int8 MFMA
//    (v_mfma_i32_16x16x64_i8).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

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

// logit and, if wanted, sigmoid(alpha * logit) with the argument one fp32 product
__device__ inline void store_score(int32_t* logits, float* scores, int64_t o, int acc, float alpha) {
    logits[o] = acc;
    if (scores) {
        const float x = alpha * (float)acc;
        scores[o] = 1.0f / (1.0f + expf(-x));
    }
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
            if (piece == 0) store_score(logits, scores, (b * nq + r) * (int64_t)C + c, acc, alpha);
        }
    }
}

typedef __attribute__((ext_vector_type(4))) int i32x4;

// Batched scoring on int8 MFMA.  One MFMA tile: A = 16 key rows (chunks
// c0..c0+15), B = 16 query rows, contracting d_idx in steps of 64; lane
// (m = lane%16, g = lane/16) holds bytes [64s + 16g, +16) of its row for
// step s, the same byte positions for A and B, so each product pairs equal
// indices.  The 16x16 int32 result lands as lane (n, g), element r = logit of
// query n, chunk c0 + 4g + r.  A workgroup covers (request, QT*16 queries,
// a range of 16-chunk tiles); each wave keeps its QT query tiles in
// registers and reuses every key tile it loads QT times.
template <int DIDX, int QT>
__global__ __launch_bounds__(kThreads) void index_score_mfma_kernel(const int8_t* __restrict__ q,
                                                                    const int8_t* __restrict__ keys, int B, int nq,
                                                                    int C, float alpha, int n_qb, int n_cg, int tpw,
                                                                    int32_t* __restrict__ logits,
                                                                    float* __restrict__ scores) {
    constexpr int KS = DIDX / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    int blk = blockIdx.x;
    const int cg = blk % n_cg;
    blk /= n_cg;
    const int qb = blk % n_qb;
    const int b = blk / n_qb;
    const int r0 = qb * 16 * QT;

    i32x4 qop[QT][KS];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const int r = r0 + 16 * t + n;
        const int rr = r < nq ? r : nq - 1;
        const int8_t* qp = q + ((int64_t)b * nq + rr) * DIDX + 16 * g;
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            const i32x4 v = *reinterpret_cast<const i32x4*>(qp + 64 * st);
            qop[t][st] = r < nq ? v : i32x4{0, 0, 0, 0};
        }
    }
    // this workgroup's tiles [t0, t1); wave w takes a contiguous quarter, so
    // each output row is written in consecutive 64-byte pieces
    const int n_tiles = (C + 15) / 16;
    const int t0 = cg * tpw, t1 = min(t0 + tpw, n_tiles);
    const int per_wave = (t1 - t0 + kThreads / 64 - 1) / (kThreads / 64);
    const int w_end = min(t0 + (wave + 1) * per_wave, t1);
    const bool vec_ok = (C & 3) == 0;  // rows 16-byte aligned: int4/float4 stores
    for (int tile = t0 + wave * per_wave; tile < w_end; ++tile) {
        const int c0 = tile * 16;
        const int row = min(c0 + n, C - 1);  // rows past C load a valid row, never stored
        const int8_t* kp = keys + ((int64_t)b * C + row) * DIDX + 16 * g;
        i32x4 kop[KS];
#pragma unroll
        for (int st = 0; st < KS; ++st) kop[st] = *reinterpret_cast<const i32x4*>(kp + 64 * st);
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            i32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int st = 0; st < KS; ++st) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop[st], qop[t][st], acc, 0, 0, 0);
            const int r = r0 + 16 * t + n;
            if (r >= nq) continue;
            const int64_t base = ((int64_t)b * nq + r) * C;
            const int c = c0 + 4 * g;
            if (vec_ok && c + 4 <= C) {
                *reinterpret_cast<i32x4*>(logits + base + c) = acc;
                if (scores) {
                    float4 sv;
                    sv.x = 1.0f / (1.0f + expf(-(alpha * (float)acc[0])));
                    sv.y = 1.0f / (1.0f + expf(-(alpha * (float)acc[1])));
                    sv.z = 1.0f / (1.0f + expf(-(alpha * (float)acc[2])));
                    sv.w = 1.0f / (1.0f + expf(-(alpha * (float)acc[3])));
                    *reinterpret_cast<float4*>(scores + base + c) = sv;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c + e < C) store_score(logits, scores, base + c + e, acc[e], alpha);
            }
        }
    }
}

template <int DIDX>
hipError_t launch_mfma(const int8_t* q, const int8_t* keys, int B, int nq, int C, float alpha, int32_t* logits,
                       float* scores, hipStream_t stream) {
    constexpr int QT = 4;
    const int n_qb = (nq + 16 * QT - 1) / (16 * QT);
    const int n_tiles = (C + 15) / 16;
    // about 512 workgroups (two per CU), at least one 16-chunk tile per wave.
    // Measured at C = 16,384 against 1024 workgroups: 14.1 against 17.1 us
    // at nq = 512, 10.8 against 11.8 at nq = 256, level at 128 and 1024.
    // Other targets from 320 to 1024 gave 17.5-21.8 us at nq = 512.
    const int64_t groups = (int64_t)B * n_qb;
    int64_t n_cg = (512 + groups - 1) / groups;
    const int64_t max_cg = (n_tiles + 3) / 4;
    if (n_cg > max_cg) n_cg = max_cg;
    if (n_cg < 1) n_cg = 1;
    const int tpw = (int)((n_tiles + n_cg - 1) / n_cg);
    n_cg = (n_tiles + tpw - 1) / tpw;
    hipLaunchKernelGGL((index_score_mfma_kernel<DIDX, QT>), dim3((unsigned)(groups * n_cg)), dim3(kThreads), 0,
                       stream, q, keys, B, nq, C, alpha, n_qb, (int)n_cg, tpw, logits, scores);
    return hipGetLastError();
}

// Query rows per request from which the MFMA kernel is used: the
// LSA_TUNE_SCORE_MFMA_MIN_NQ knob, 16 by default (the crossover measured at
// C = 16,384).
int score_mfma_min_nq() { return tuning(LSA_TUNE_SCORE_MFMA_MIN_NQ); }

template <int DIDX>
hipError_t launch(const int8_t* q, const int8_t* keys, int B, int nq, int C, float alpha, int32_t* logits,
                  float* scores, hipStream_t stream) {
    // The MFMA grid has at least one workgroup per (request, 64 query rows):
    // beyond 2^22 of those its work-item count would pass 32 bits, and the
    // GEMV kernel (a capped grid that strides over the rows) takes over.
    if (DIDX % 64 == 0 && nq >= score_mfma_min_nq() && (int64_t)B * ((nq + 63) / 64) < ((int64_t)1 << 22))
        return launch_mfma<(DIDX % 64 == 0 ? DIDX : 64)>(q, keys, B, nq, C, alpha, logits, scores, stream);
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
