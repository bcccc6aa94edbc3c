// Internal launch interface of the HIP kernels behind the C ABI (include/lsa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <functional>

#include "../../include/lsa.h"

namespace lsa {

// Value of a tuning knob (lsa_tuning) for the calling thread: its override,
// else the environment's value read once per process, else the library's
// constant default (0 where the choice is made per call).
int32_t tuning(int knob);

// Records `fmt` as the calling thread's lsa_last_error() message and
// returns s (for entry points defined outside lsa_abi.hip).
lsa_status reject(lsa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

constexpr int kChunkTokens = 64;

// ---- index score (indexer dot product + sigmoid) ----
hipError_t launch_index_score(const int8_t* q_idx, const int8_t* k_idx, int B, int nq, int C, int d_idx,
                              float alpha, int32_t* logits, float* scores, hipStream_t stream);

// ---- top-k chunk selection ----
constexpr int kTopkThreads = 1024;
constexpr int kTopkRegisterMaxC = 65536;  // longer rows take the streaming kernel
constexpr int kTopkMaxC = 1 << 30;
// counts == nullptr: top-k; else keep logits > thr, at most k, counts[r] = kept
hipError_t launch_topk(const int32_t* logits, int R, int C, int k, int32_t* chunk_ids, int32_t thr, int32_t* counts,
                       hipStream_t stream);
// token stage: top k_tok of the usable list positions of each row's recalled
// chunks by float score; ascending, -1 padded, tok_counts[r] = kept.  With a
// workspace (topk_tokens_workspace_bytes, when nonzero) long rows run as
// slices + candidates over many workgroups per row.
struct TopkSplit {
    int slices;     // 0: no split
    int slice_len;  // positions per slice, a multiple of 64
};
TopkSplit topk_tokens_split(int n_list, int k_tok);
size_t topk_tokens_workspace_bytes(int R, int n_list, int k_tok);
hipError_t launch_topk_tokens(const float* scores, const int32_t* list_ids, const int32_t* list_counts,
                              const int32_t* ctx, int R, int n_list, int k_tok, int32_t* tok, int32_t* tok_counts,
                              void* workspace, hipStream_t stream);

// ---- gathered GQA decode attention ----
struct AttendArgs {
    const uint16_t* q;      // [B][Hq][d] bf16
    const uint16_t* kv;     // [B][C_store][2][Hkv][64][d] bf16
    int64_t C_store;
    const int32_t* ids;     // [B][k]
    const int32_t* slots;   // [B][k] or nullptr
    const int32_t* counts;  // [B] entries used per request, or nullptr (all k)
    const int32_t* ctx;     // [B]
    const uint16_t* seg_kv; // [B][2][Hkv][S_max][d] resident segment, or nullptr
    const int32_t* seg_len; // [B] tokens in the segment
    int S_max;
    const int32_t* tok;        // [B][k_tok] list positions j*64 + t to attend, or nullptr (every token)
    const int32_t* tok_counts; // [B] listed positions in use, or nullptr (all k_tok)
    int k_tok;
    int B, Hq, Hkv, G, d, k, n_split;
    int depth;              // chunks in flight per wave + 1 (register ring size)
    float scale_log2;       // sm_scale * log2(e)
    float* part_o;          // [B][Hkv][n_split][G][d]      (n_split > 1)
    float* part_ml;         // [B][Hkv][n_split][G][2]      (n_split > 1)
    float* out;             // [B][Hq][d]
};

int attend_default_splits(int B, int Hkv, int k);
int attend_pipeline_depth();
size_t attend_workspace_bytes(int B, int Hkv, int G, int d, int n_split);
void attend_workspace_carve(AttendArgs& a, void* workspace);
hipError_t launch_gather_attend(const AttendArgs& a, hipStream_t stream);

// ---- host-tier fetch as a device-side gather over the host link ----
hipError_t launch_fetch_pull(const uint16_t* host_kv_dev, int64_t C, const int32_t* ids, const int32_t* slots,
                             uint16_t* pool, int64_t P, int B, int Hkv, int d, int k, int grid, hipStream_t stream);

// ---- host-tier fetch through a staging buffer ----
// Chunks per staged copy: the scatter's destination list rides in its kernel
// arguments (4 bytes a chunk).
constexpr int kStagePiece = 512;
struct StageScatterArgs {
    const uint16_t* src;  // device staging: n consecutive chunks
    uint16_t* pool;       // [B][P] chunks
    int64_t chunk_u4;     // 16-byte words per chunk (16 * Hkv * d)
    int n;                // chunks staged
    int32_t dst[kStagePiece];  // pool chunk b * P + slot of staged chunk s
};
hipError_t launch_stage_scatter(const StageScatterArgs& a, hipStream_t stream);
// Runs fn(i) for every i in [0, n) on the library's host worker threads and
// the calling thread; returns when all have run.  One job at a time.
void host_parallel_for(int n, const std::function<void(int)>& fn);
// Copies host chunks src_chunks[0..n) of `store` (chunk_bytes each, a
// multiple of 64) to consecutive places of dst, on those threads.
void host_gather_chunks(char* dst, const char* store, const int64_t* src_chunks, int n, size_t chunk_bytes);

// ---- opt-in validation of chunk lists ----
constexpr int kCheckMaxEntries = 16384;  // entries per request the check sorts in LDS
constexpr int kCheckResultWords = 4;     // first bad entry: range, repeated id, repeated slot; first bad count
hipError_t launch_check_ids(const int32_t* ids, const int32_t* slots, const int32_t* counts, int B, int k,
                            int64_t C_ctx, int64_t C_store, int32_t* result, hipStream_t stream);

// ---- pool-slot assignment for a delta fetch ----
size_t pool_assign_lds_bytes(int n_prev, int P);
hipError_t launch_pool_assign(const int32_t* prev_ids, const int32_t* prev_slots, int n_prev, const int32_t* new_ids,
                              int B, int k, int P, int32_t* new_slots, int32_t* fetch_slots, hipStream_t stream);

}  // namespace lsa
