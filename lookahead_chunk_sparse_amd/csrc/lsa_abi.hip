// C-ABI entry points (include/lsa.h): argument validation, workspace
// layout and kernel launches; plus the host-tier fetch, which is pure
// host-to-device DMA on a side stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <limits.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/lsa.h"
#include "fetch_runs.h"
#include "lsa_kernels.h"

namespace {

thread_local std::string g_last_error;

lsa_status fail(lsa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lsa_status fail(lsa_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

}  // namespace

namespace lsa {
lsa_status reject(lsa_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}
}  // namespace lsa

namespace {

lsa_status ok() {
    g_last_error.clear();
    return LSA_OK;
}

lsa_status hip_fail(hipError_t e, const char* what) {
    return fail(LSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// ---- the DMA fetch's streams ----
constexpr int kFetchLanes = 16;  // library streams one lsa_fetch_chunks call may spread its copies over
constexpr int kMaxDevices = 64;
struct FetchLanes {
    std::mutex mu;  // one call at a time records and waits on the fork and join events
    hipStream_t s[kFetchLanes] = {};
    hipEvent_t fork = nullptr, join[kFetchLanes] = {};
};

// The current device's fetch streams and events (default priority, no
// timing; all kFetchLanes, of which a call uses LSA_TUNE_FETCH_LANES),
// created at the first use and kept until the process ends;
// nullptr if they cannot be created (the copies then stay on the caller's
// stream).
FetchLanes* fetch_lanes() {
    static std::mutex init_mu;
    static FetchLanes* per_dev[kMaxDevices] = {};
    static bool failed[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> g(init_mu);
    if (per_dev[dev] || failed[dev]) return per_dev[dev];
    auto* f = new FetchLanes();
    bool good = hipEventCreateWithFlags(&f->fork, hipEventDisableTiming) == hipSuccess;
    for (int l = 0; l < kFetchLanes && good; ++l)
        good = hipStreamCreateWithFlags(&f->s[l], hipStreamNonBlocking) == hipSuccess &&
               hipEventCreateWithFlags(&f->join[l], hipEventDisableTiming) == hipSuccess;
    if (!good) {
        (void)hipGetLastError();
        for (int l = 0; l < kFetchLanes; ++l) {
            if (f->s[l]) (void)hipStreamDestroy(f->s[l]);
            if (f->join[l]) (void)hipEventDestroy(f->join[l]);
        }
        if (f->fork) (void)hipEventDestroy(f->fork);
        delete f;
        failed[dev] = true;
        return nullptr;
    }
    per_dev[dev] = f;
    return f;
}

// A launch counts its work-items (workgroups x threads) in 32 bits: these
// bound the workgroups of the launches whose count follows the arguments.
constexpr int64_t kMaxRowGroups = (int64_t)1 << 22;    // 1024-thread top-k / pool workgroups
constexpr int64_t kMaxSplitGroups = (int64_t)1 << 24;  // 256-thread attention workgroups

// ---- tuning knobs (include/lsa.h, lsa_tuning) ----
constexpr const char* kTuneEnv[LSA_TUNE_COUNT] = {"LSA_ATTEND_DEPTH",     "LSA_SCORE_MFMA_MIN_NQ",
                                                  "LSA_TOPK_STREAM_MIN_C", "LSA_TOPK_SPLIT_MIN_N",
                                                  "LSA_TOPK_SPLIT_SLICES", "LSA_FETCH_LANES"};
// the library's own choice where it is a constant (0: chosen per call)
constexpr int32_t kTuneDefault[LSA_TUNE_COUNT] = {2, 16, lsa::kTopkRegisterMaxC + 1, 32769, 0, 4};

bool tune_value_ok(int knob, int32_t v) {
    if (v < 0) return false;
    if (knob == LSA_TUNE_ATTEND_DEPTH) return v == 0 || (v >= 2 && v <= 4);
    if (knob == LSA_TUNE_FETCH_LANES) return v <= 16;
    return true;
}

// The environment's values, read once per process (thread-safe static
// initialisation); values out of range are ignored.
const int32_t* env_tuning() {
    static const struct Env {
        int32_t v[LSA_TUNE_COUNT];
        Env() {
            for (int i = 0; i < LSA_TUNE_COUNT; ++i) {
                const char* e = getenv(kTuneEnv[i]);
                const long x = e ? strtol(e, nullptr, 10) : 0;
                v[i] = (x > 0 && x <= INT32_MAX && tune_value_ok(i, (int32_t)x)) ? (int32_t)x : 0;
            }
        }
    } env;
    return env.v;
}

thread_local int32_t t_tune[LSA_TUNE_COUNT] = {};

}  // namespace

namespace lsa {
int32_t tuning(int knob) {
    if (t_tune[knob] > 0) return t_tune[knob];
    const int32_t e = env_tuning()[knob];
    return e > 0 ? e : kTuneDefault[knob];
}
}  // namespace lsa

extern "C" {

lsa_status lsa_set_tuning(int32_t knob, int32_t value) {
    if (knob < 0 || knob >= LSA_TUNE_COUNT) return fail(LSA_ERR_INVALID_ARGUMENT, "unknown knob %d", knob);
    if (!tune_value_ok(knob, value))
        return fail(LSA_ERR_INVALID_ARGUMENT, "value %d out of range for %s", value, kTuneEnv[knob]);
    t_tune[knob] = value;
    return ok();
}

int32_t lsa_get_tuning(int32_t knob) {
    if (knob < 0 || knob >= LSA_TUNE_COUNT) return -1;
    return lsa::tuning(knob);
}

const char* lsa_status_string(int32_t s) {
    switch (s) {
        case LSA_OK: return "LSA_OK";
        case LSA_ERR_INVALID_ARGUMENT: return "LSA_ERR_INVALID_ARGUMENT";
        case LSA_ERR_UNSUPPORTED: return "LSA_ERR_UNSUPPORTED";
        case LSA_ERR_WORKSPACE: return "LSA_ERR_WORKSPACE";
        case LSA_ERR_HIP: return "LSA_ERR_HIP";
    }
    return "LSA_ERR_UNKNOWN";
}

const char* lsa_last_error(void) { return g_last_error.c_str(); }

lsa_status lsa_index_score(const int8_t* q_idx, const int8_t* k_idx, int32_t B, int32_t nq, int32_t C,
                           int32_t d_idx, float alpha, int32_t* logits, float* scores, hipStream_t stream) {
    if (!q_idx || !k_idx || !logits) return fail(LSA_ERR_INVALID_ARGUMENT, "q_idx, k_idx and logits are required");
    if (B < 1 || nq < 1 || C < 1)
        return fail(LSA_ERR_INVALID_ARGUMENT, "B=%d nq=%d C=%d must all be >= 1", B, nq, C);
    if ((int64_t)B * nq * C >= ((int64_t)1 << 31))
        return fail(LSA_ERR_INVALID_ARGUMENT, "B*nq*C=%lld must be < 2^31", (long long)B * nq * C);
    if (!std::isfinite(alpha)) return fail(LSA_ERR_INVALID_ARGUMENT, "alpha must be finite");
    if (d_idx != 16 && d_idx != 32 && d_idx != 64 && d_idx != 128 && d_idx != 256)
        return fail(LSA_ERR_UNSUPPORTED, "d_idx=%d: supported are 16, 32, 64, 128, 256", d_idx);
    if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(logits, 4) || (scores && !aligned(scores, 4)))
        return fail(LSA_ERR_INVALID_ARGUMENT, "q_idx/k_idx need 16-byte, logits/scores 4-byte alignment");
    hipError_t e = lsa::launch_index_score(q_idx, k_idx, B, nq, C, d_idx, alpha, logits, scores, stream);
    if (e != hipSuccess) return hip_fail(e, "index score launch");
    return ok();
}

lsa_status lsa_topk_chunks(const int32_t* logits, int32_t R, int32_t C, int32_t k, int32_t* chunk_ids,
                           hipStream_t stream) {
    if (!logits || !chunk_ids) return fail(LSA_ERR_INVALID_ARGUMENT, "logits and chunk_ids are required");
    if (R < 1 || C < 1) return fail(LSA_ERR_INVALID_ARGUMENT, "R=%d C=%d must be >= 1", R, C);
    if (k < 1 || k > C) return fail(LSA_ERR_INVALID_ARGUMENT, "k=%d must be in [1, C=%d]", k, C);
    if (C > lsa::kTopkMaxC) return fail(LSA_ERR_UNSUPPORTED, "C=%d exceeds %d", C, lsa::kTopkMaxC);
    if (R >= kMaxRowGroups) return fail(LSA_ERR_UNSUPPORTED, "R=%d: must be < 2^22", R);
    if (!aligned(logits, 4) || !aligned(chunk_ids, 4))
        return fail(LSA_ERR_INVALID_ARGUMENT, "logits and chunk_ids need 4-byte alignment");
    hipError_t e = lsa::launch_topk(logits, R, C, k, chunk_ids, 0, nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    return ok();
}

lsa_status lsa_threshold_chunks(const int32_t* logits, int32_t R, int32_t C, int32_t logit_threshold, int32_t k_max,
                                int32_t* chunk_ids, int32_t* counts, hipStream_t stream) {
    if (!logits || !chunk_ids || !counts)
        return fail(LSA_ERR_INVALID_ARGUMENT, "logits, chunk_ids and counts are required");
    if (R < 1 || C < 1) return fail(LSA_ERR_INVALID_ARGUMENT, "R=%d C=%d must be >= 1", R, C);
    if (k_max < 1 || k_max > C) return fail(LSA_ERR_INVALID_ARGUMENT, "k_max=%d must be in [1, C=%d]", k_max, C);
    if (C > lsa::kTopkMaxC) return fail(LSA_ERR_UNSUPPORTED, "C=%d exceeds %d", C, lsa::kTopkMaxC);
    if (R >= kMaxRowGroups) return fail(LSA_ERR_UNSUPPORTED, "R=%d: must be < 2^22", R);
    if (!aligned(logits, 4) || !aligned(chunk_ids, 4) || !aligned(counts, 4))
        return fail(LSA_ERR_INVALID_ARGUMENT, "logits, chunk_ids and counts need 4-byte alignment");
    hipError_t e = lsa::launch_topk(logits, R, C, k_max, chunk_ids, logit_threshold, counts, stream);
    if (e != hipSuccess) return hip_fail(e, "threshold-select launch");
    return ok();
}

static lsa_status check_attend_shape(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t k) {
    if (B < 1 || Hq < 1 || Hkv < 1 || k < 1)
        return fail(LSA_ERR_INVALID_ARGUMENT, "B=%d Hq=%d Hkv=%d k=%d must all be >= 1", B, Hq, Hkv, k);
    if (Hq % Hkv != 0) return fail(LSA_ERR_INVALID_ARGUMENT, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (Hq / Hkv > 16) return fail(LSA_ERR_UNSUPPORTED, "Hq/Hkv=%d: at most 16 query heads per KV head", Hq / Hkv);
    if (d != 64 && d != 128) return fail(LSA_ERR_UNSUPPORTED, "d=%d: supported head dims are 64 and 128", d);
    if ((int64_t)B * Hq >= ((int64_t)1 << 31) || (int64_t)B * k >= ((int64_t)1 << 31))
        return fail(LSA_ERR_INVALID_ARGUMENT, "B*Hq and B*k must be < 2^31");
    if ((int64_t)B * Hq >= ((int64_t)1 << 24))
        return fail(LSA_ERR_UNSUPPORTED, "B*Hq=%lld: must be < 2^24", (long long)B * Hq);
    return LSA_OK;
}

int32_t lsa_gather_attend_default_splits(int32_t B, int32_t Hkv, int32_t k) {
    if (B < 1 || Hkv < 1 || k < 1) return -1;
    return lsa::attend_default_splits(B, Hkv, k);
}

size_t lsa_topk_tokens_workspace_size(int32_t B, int32_t k, int32_t k_tok) {
    if (B < 1 || k < 1 || k_tok < 1 || (int64_t)k * lsa::kChunkTokens > lsa::kTopkMaxC) return (size_t)-1;
    return lsa::topk_tokens_workspace_bytes(B, k, k_tok);
}

lsa_status lsa_topk_tokens(const float* scores, const int32_t* chunk_ids, const int32_t* counts,
                           const int32_t* ctx_len, int32_t B, int32_t k, int32_t k_tok, int32_t* tok,
                           int32_t* tok_counts, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!scores || !chunk_ids || !ctx_len || !tok || !tok_counts)
        return fail(LSA_ERR_INVALID_ARGUMENT, "scores, chunk_ids, ctx_len, tok and tok_counts are required");
    if (B < 1 || k < 1 || k_tok < 1)
        return fail(LSA_ERR_INVALID_ARGUMENT, "B=%d k=%d k_tok=%d must all be >= 1", B, k, k_tok);
    if ((int64_t)k * lsa::kChunkTokens > lsa::kTopkMaxC)
        return fail(LSA_ERR_UNSUPPORTED, "k=%d: at most %d list positions (k <= %d)", k, lsa::kTopkMaxC,
                    lsa::kTopkMaxC / lsa::kChunkTokens);
    if ((int64_t)B * k * lsa::kChunkTokens >= ((int64_t)1 << 31) || (int64_t)B * k_tok >= ((int64_t)1 << 31))
        return fail(LSA_ERR_INVALID_ARGUMENT, "B*k*64 and B*k_tok must be < 2^31");
    if (!aligned(scores, 4) || !aligned(chunk_ids, 4) || !aligned(ctx_len, 4) || !aligned(tok, 4) ||
        !aligned(tok_counts, 4) || (counts && !aligned(counts, 4)))
        return fail(LSA_ERR_INVALID_ARGUMENT, "all pointers need 4-byte alignment");
    if (workspace) {
        const size_t need = lsa::topk_tokens_workspace_bytes(B, k, k_tok);
        if (workspace_bytes < need)
            return fail(LSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
        if (!aligned(workspace, 256)) return fail(LSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        if (need == 0) workspace = nullptr;  // no split for these sizes
    }
    const int64_t groups = (int64_t)B * (workspace ? lsa::topk_tokens_split(k, k_tok).slices : 1);
    if (groups >= kMaxRowGroups)
        return fail(LSA_ERR_UNSUPPORTED, "%lld select workgroups (B times the slices): must be < 2^22", (long long)groups);
    hipError_t e = lsa::launch_topk_tokens(scores, chunk_ids, counts, ctx_len, B, k, k_tok, tok, tok_counts, workspace,
                                           stream);
    if (e != hipSuccess) return hip_fail(e, "token top-k launch");
    return ok();
}

size_t lsa_gather_attend_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t k, int32_t n_split) {
    if (check_attend_shape(B, Hq, Hkv, d, k) != LSA_OK || n_split < 0) return (size_t)-1;
    if (n_split == 0) n_split = lsa::attend_default_splits(B, Hkv, k);
    if (n_split > k) n_split = k;
    if ((int64_t)B * Hkv * n_split >= kMaxSplitGroups) return (size_t)-1;
    return lsa::attend_workspace_bytes(B, Hkv, Hq / Hkv, d, n_split);
}

static lsa_status gather_attend_impl(const uint16_t* q, const uint16_t* kv, int64_t C_store, const int32_t* chunk_ids,
                                     const int32_t* slots, const int32_t* counts, const int32_t* ctx_len,
                                     const int32_t* tok, const int32_t* tok_counts, int32_t k_tok,
                                     const uint16_t* seg_kv, const int32_t* seg_len, int32_t S_max, int32_t B,
                                     int32_t Hq, int32_t Hkv, int32_t d, int32_t k, float sm_scale, void* workspace,
                                     size_t workspace_bytes, int32_t n_split, float* out, hipStream_t stream) {
    if (!q || !kv || !chunk_ids || !ctx_len || !out)
        return fail(LSA_ERR_INVALID_ARGUMENT, "q, kv, chunk_ids, ctx_len and out are required");
    lsa_status st = check_attend_shape(B, Hq, Hkv, d, k);
    if (st != LSA_OK) return st;
    if (C_store < 1) return fail(LSA_ERR_INVALID_ARGUMENT, "C_store=%lld must be >= 1", (long long)C_store);
    if (!std::isfinite(sm_scale)) return fail(LSA_ERR_INVALID_ARGUMENT, "sm_scale must be finite");
    if (n_split < 0) return fail(LSA_ERR_INVALID_ARGUMENT, "n_split=%d must be >= 0", n_split);
    if (seg_kv && (!seg_len || S_max < lsa::kChunkTokens || S_max % lsa::kChunkTokens != 0 || !aligned(seg_kv, 16)))
        return fail(LSA_ERR_INVALID_ARGUMENT,
                    "a segment needs seg_len, S_max a positive multiple of 64 (S_max=%d) and 16-byte alignment", S_max);
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16))
        return fail(LSA_ERR_INVALID_ARGUMENT, "q, kv and out need 16-byte alignment");
    // list entries split across workgroups: chunks, or blocks of 64 listed tokens
    int32_t entries = k;
    if (tok) {
        if (k_tok < 1) return fail(LSA_ERR_INVALID_ARGUMENT, "k_tok=%d must be >= 1", k_tok);
        if ((int64_t)B * k_tok >= ((int64_t)1 << 31)) return fail(LSA_ERR_INVALID_ARGUMENT, "B*k_tok must be < 2^31");
        // C_store * rows < 2^31 (row indices are int32), tested without forming the product
        const int64_t rows = 2 * (int64_t)Hkv * lsa::kChunkTokens;
        if (C_store >= ((((int64_t)1 << 31) + rows - 1) / rows))
            return fail(LSA_ERR_UNSUPPORTED, "token lists need C_store*2*Hkv*64 < 2^31 (C_store=%lld)",
                        (long long)C_store);
        if (!aligned(tok, 4) || (tok_counts && !aligned(tok_counts, 4)))
            return fail(LSA_ERR_INVALID_ARGUMENT, "tok and tok_counts need 4-byte alignment");
        entries = (k_tok + lsa::kChunkTokens - 1) / lsa::kChunkTokens;
    }
    if (n_split == 0) n_split = lsa::attend_default_splits(B, Hkv, entries);
    if (n_split > entries) n_split = entries;
    if ((int64_t)B * Hkv * n_split >= kMaxSplitGroups)
        return fail(LSA_ERR_UNSUPPORTED, "B*Hkv*n_split=%lld workgroups: must be < 2^24", (long long)B * Hkv * n_split);
    const int G = Hq / Hkv;
    const size_t need = lsa::attend_workspace_bytes(B, Hkv, G, d, n_split);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(LSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    if (need > 0 && !aligned(workspace, 256)) return fail(LSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

    lsa::AttendArgs a;
    a.q = q;
    a.kv = kv;
    a.C_store = C_store;
    a.ids = chunk_ids;
    a.slots = slots;
    a.counts = counts;
    a.ctx = ctx_len;
    a.seg_kv = seg_kv;
    a.seg_len = seg_kv ? seg_len : nullptr;
    a.S_max = seg_kv ? S_max : 0;
    a.tok = tok;
    a.tok_counts = tok ? tok_counts : nullptr;
    a.k_tok = tok ? k_tok : 0;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = G;
    a.d = d;
    a.k = k;
    a.n_split = n_split;
    a.depth = lsa::attend_pipeline_depth();
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    a.out = out;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    if (need > 0) lsa::attend_workspace_carve(a, workspace);
    hipError_t e = lsa::launch_gather_attend(a, stream);
    if (e != hipSuccess) return hip_fail(e, "gather-attend launch");
    return ok();
}

lsa_status lsa_gather_attend(const uint16_t* q, const uint16_t* kv, int64_t C_store, const int32_t* chunk_ids,
                             const int32_t* slots, const int32_t* counts, const int32_t* ctx_len,
                             const uint16_t* seg_kv, const int32_t* seg_len, int32_t S_max, int32_t B,
                             int32_t Hq, int32_t Hkv,
                             int32_t d, int32_t k, float sm_scale, void* workspace, size_t workspace_bytes,
                             int32_t n_split, float* out, hipStream_t stream) {
    return gather_attend_impl(q, kv, C_store, chunk_ids, slots, counts, ctx_len, nullptr, nullptr, 0, seg_kv, seg_len,
                              S_max, B, Hq, Hkv, d, k, sm_scale, workspace, workspace_bytes, n_split, out, stream);
}

lsa_status lsa_gather_attend_tokens(const uint16_t* q, const uint16_t* kv, int64_t C_store, const int32_t* chunk_ids,
                                    const int32_t* slots, const int32_t* counts, const int32_t* ctx_len,
                                    const int32_t* tok, const int32_t* tok_counts, int32_t k_tok,
                                    const uint16_t* seg_kv, const int32_t* seg_len, int32_t S_max, int32_t B,
                                    int32_t Hq, int32_t Hkv, int32_t d, int32_t k, float sm_scale, void* workspace,
                                    size_t workspace_bytes, int32_t n_split, float* out, hipStream_t stream) {
    if (!tok) return fail(LSA_ERR_INVALID_ARGUMENT, "tok is required");
    return gather_attend_impl(q, kv, C_store, chunk_ids, slots, counts, ctx_len, tok, tok_counts, k_tok, seg_kv,
                              seg_len, S_max, B, Hq, Hkv, d, k, sm_scale, workspace, workspace_bytes, n_split, out,
                              stream);
}

lsa_status lsa_fetch_chunks(const uint16_t* host_kv, int64_t C, const int32_t* host_chunk_ids,
                            const int32_t* host_slots, uint16_t* pool_kv, int64_t P, int32_t B, int32_t Hkv,
                            int32_t d, int32_t k, hipStream_t side_stream, hipEvent_t done) {
    if (!host_kv || !host_chunk_ids || !pool_kv)
        return fail(LSA_ERR_INVALID_ARGUMENT, "host_kv, host_chunk_ids and pool_kv are required");
    if (C < 1 || P < 1 || B < 1 || Hkv < 1 || d < 1 || k < 1)
        return fail(LSA_ERR_INVALID_ARGUMENT, "C, P, B, Hkv, d, k must all be >= 1");
    if (!host_slots && k > P) return fail(LSA_ERR_INVALID_ARGUMENT, "k=%d > P=%lld with default slots", k, (long long)P);
    for (int64_t e = 0; e < (int64_t)B * k; ++e) {
        if (host_slots && host_slots[e] < 0) continue;  // not copied: its id is not read
        if (host_chunk_ids[e] < 0 || host_chunk_ids[e] >= C)
            return fail(LSA_ERR_INVALID_ARGUMENT, "chunk id %d at entry %lld outside [0, %lld)", host_chunk_ids[e],
                        (long long)e, (long long)C);
        if (host_slots && host_slots[e] >= P)
            return fail(LSA_ERR_INVALID_ARGUMENT, "slot %d at entry %lld outside [0, %lld)", host_slots[e],
                        (long long)e, (long long)P);
    }
    // The copies must come from pinned memory to be asynchronous DMA.
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof attr);
    hipError_t pe = hipPointerGetAttributes(&attr, host_kv);
    if (pe != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();  // clear the error a pageable pointer leaves behind
        return fail(LSA_ERR_INVALID_ARGUMENT, "host_kv is not pinned host memory (allocate it with hipHostMalloc)");
    }
    const size_t chunk_bytes = (size_t)2 * Hkv * lsa::kChunkTokens * d * sizeof(uint16_t);
    // The copies go round-robin onto kFetchLanes library streams that start
    // after, and rejoin, side_stream: one stream's copies run one after the
    // other with a fixed cost each (about 20 GB/s in 256 KB copies), several
    // streams overlap it.  Under graph capture they stay on side_stream.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    const hipError_t ce = hipStreamIsCapturing(side_stream, &cap);
    if (ce != hipSuccess) return hip_fail(ce, "capture status");
    // The library's streams belong to the current device: a side_stream of
    // another device keeps its copies.
    const int n_lanes = lsa::tuning(LSA_TUNE_FETCH_LANES);
    bool fan_out = cap == hipStreamCaptureStatusNone && n_lanes > 1;
    if (fan_out) {
        int cur_dev = -1;
        hipDevice_t stream_dev = -1;
        if (hipGetDevice(&cur_dev) != hipSuccess || hipStreamGetDevice(side_stream, &stream_dev) != hipSuccess) {
            (void)hipGetLastError();  // a failed query only keeps the copies on side_stream
            fan_out = false;
        } else {
            fan_out = stream_dev == cur_dev;
        }
    }
    FetchLanes* lanes = fan_out ? fetch_lanes() : nullptr;
    std::unique_lock<std::mutex> hold;
    if (lanes) {
        hold = std::unique_lock<std::mutex>(lanes->mu);
        hipError_t e = hipEventRecord(lanes->fork, side_stream);
        for (int l = 0; l < n_lanes && e == hipSuccess; ++l) e = hipStreamWaitEvent(lanes->s[l], lanes->fork, 0);
        if (e != hipSuccess) return hip_fail(e, "fetch fork");
    }
    hipError_t copy_err = hipSuccess;
    int n_run = 0;
    lsa::coalesce_fetch_runs(host_chunk_ids, host_slots, B, k, [&](int32_t b, int64_t c0, int64_t p0, int32_t run) {
        const char* src = reinterpret_cast<const char*>(host_kv) + ((int64_t)b * C + c0) * chunk_bytes;
        char* dst = reinterpret_cast<char*>(pool_kv) + ((int64_t)b * P + p0) * chunk_bytes;
        copy_err = hipMemcpyAsync(dst, src, run * chunk_bytes, hipMemcpyHostToDevice,
                                  lanes ? lanes->s[n_run++ % n_lanes] : side_stream);
        return copy_err == hipSuccess;
    });
    if (lanes) {  // rejoin, also after a failed copy, so side_stream never runs ahead of what was issued
        hipError_t e = hipSuccess;
        for (int l = 0; l < n_lanes && e == hipSuccess; ++l) {
            e = hipEventRecord(lanes->join[l], lanes->s[l]);
            if (e == hipSuccess) e = hipStreamWaitEvent(side_stream, lanes->join[l], 0);
        }
        if (e != hipSuccess && copy_err == hipSuccess) copy_err = e;
    }
    if (copy_err != hipSuccess) return hip_fail(copy_err, "fetch copy");
    if (done) {
        hipError_t e = hipEventRecord(done, side_stream);
        if (e != hipSuccess) return hip_fail(e, "fetch event record");
    }
    return ok();
}

lsa_status lsa_fetch_chunks_staged(const uint16_t* host_kv, int64_t C, const int32_t* host_chunk_ids,
                                   const int32_t* host_slots, uint16_t* pool_kv, int64_t P, int32_t B, int32_t Hkv,
                                   int32_t d, int32_t k, uint16_t* host_staging, uint16_t* dev_staging,
                                   int64_t stage_chunks, hipStream_t side_stream, hipEvent_t done) {
    if (!host_kv || !host_chunk_ids || !pool_kv || !host_staging || !dev_staging)
        return fail(LSA_ERR_INVALID_ARGUMENT, "host_kv, host_chunk_ids, pool_kv and both staging buffers are required");
    if (C < 1 || P < 1 || B < 1 || Hkv < 1 || d < 1 || k < 1)
        return fail(LSA_ERR_INVALID_ARGUMENT, "C, P, B, Hkv, d, k must all be >= 1");
    if (stage_chunks < 2) return fail(LSA_ERR_INVALID_ARGUMENT, "stage_chunks=%lld: at least 2", (long long)stage_chunks);
    if (!host_slots && k > P) return fail(LSA_ERR_INVALID_ARGUMENT, "k=%d > P=%lld with default slots", k, (long long)P);
    if ((int64_t)B * P >= ((int64_t)1 << 31) || (int64_t)B * C >= ((int64_t)1 << 40))
        return fail(LSA_ERR_UNSUPPORTED, "B*P must be < 2^31 and B*C < 2^40");
    if (!aligned(host_kv, 16) || !aligned(pool_kv, 16) || !aligned(host_staging, 16) || !aligned(dev_staging, 16))
        return fail(LSA_ERR_INVALID_ARGUMENT, "host_kv, pool_kv and the staging buffers need 16-byte alignment");
    for (int64_t e = 0; e < (int64_t)B * k; ++e) {
        if (host_slots && host_slots[e] < 0) continue;  // not copied: its id is not read
        if (host_chunk_ids[e] < 0 || host_chunk_ids[e] >= C)
            return fail(LSA_ERR_INVALID_ARGUMENT, "chunk id %d at entry %lld outside [0, %lld)", host_chunk_ids[e],
                        (long long)e, (long long)C);
        if (host_slots && host_slots[e] >= P)
            return fail(LSA_ERR_INVALID_ARGUMENT, "slot %d at entry %lld outside [0, %lld)", host_slots[e],
                        (long long)e, (long long)P);
    }
    // both host buffers pinned (the staging buffer is read by asynchronous
    // DMA, the store is read by the gather threads), the staging on the
    // device in device memory
    for (const void* hp : {(const void*)host_kv, (const void*)host_staging}) {
        hipPointerAttribute_t attr;
        memset(&attr, 0, sizeof attr);
        const hipError_t pe = hipPointerGetAttributes(&attr, hp);
        if (pe != hipSuccess || attr.type != hipMemoryTypeHost) {
            (void)hipGetLastError();
            return fail(LSA_ERR_INVALID_ARGUMENT,
                        "host_kv and host_staging must be pinned host memory (allocate them with hipHostMalloc)");
        }
    }
    {
        hipPointerAttribute_t attr;
        memset(&attr, 0, sizeof attr);
        const hipError_t pe = hipPointerGetAttributes(&attr, dev_staging);
        if (pe != hipSuccess || attr.type != hipMemoryTypeDevice) {
            (void)hipGetLastError();
            return fail(LSA_ERR_INVALID_ARGUMENT, "dev_staging must be device memory");
        }
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    const hipError_t ce = hipStreamIsCapturing(side_stream, &cap);
    if (ce != hipSuccess) return hip_fail(ce, "capture status");
    if (cap != hipStreamCaptureStatusNone)
        return fail(LSA_ERR_UNSUPPORTED, "the staged fetch waits on the host for its copies: not under graph capture");

    const size_t chunk_bytes = (size_t)2 * Hkv * lsa::kChunkTokens * d * sizeof(uint16_t);
    // the entries to copy: store chunk b * C + id into pool chunk b * P + slot
    std::vector<int64_t> src;
    std::vector<int32_t> dst;
    src.reserve((size_t)B * k);
    dst.reserve((size_t)B * k);
    for (int32_t b = 0; b < B; ++b)
        for (int32_t j = 0; j < k; ++j) {
            const int64_t e = (int64_t)b * k + j;
            const int32_t slot = host_slots ? host_slots[e] : j;
            if (slot < 0) continue;
            src.push_back((int64_t)b * C + host_chunk_ids[e]);
            dst.push_back((int32_t)((int64_t)b * P + slot));
        }
    // Pieces of up to `piece` chunks alternate between the two halves of the
    // staging buffers: the host gathers piece p + 1 while piece p crosses
    // the link, and waits for the copy out of a half before filling it again.
    const int64_t piece = std::min<int64_t>(stage_chunks / 2, lsa::kStagePiece);
    hipEvent_t ev[2] = {nullptr, nullptr};
    bool used[2] = {false, false};
    hipError_t err = hipSuccess;
    for (int h = 0; h < 2 && err == hipSuccess; ++h) err = hipEventCreateWithFlags(&ev[h], hipEventDisableTiming);
    int h = 0;
    for (size_t p0 = 0; p0 < src.size() && err == hipSuccess; p0 += (size_t)piece, h ^= 1) {
        const int n = (int)std::min<size_t>((size_t)piece, src.size() - p0);
        if (used[h] && (err = hipEventSynchronize(ev[h])) != hipSuccess) break;
        char* hs = reinterpret_cast<char*>(host_staging) + (size_t)h * piece * chunk_bytes;
        char* ds = reinterpret_cast<char*>(dev_staging) + (size_t)h * piece * chunk_bytes;
        lsa::host_gather_chunks(hs, reinterpret_cast<const char*>(host_kv), src.data() + p0, n, chunk_bytes);
        if ((err = hipMemcpyAsync(ds, hs, (size_t)n * chunk_bytes, hipMemcpyHostToDevice, side_stream)) != hipSuccess)
            break;
        if ((err = hipEventRecord(ev[h], side_stream)) != hipSuccess) break;
        used[h] = true;
        lsa::StageScatterArgs sa{};
        sa.src = reinterpret_cast<const uint16_t*>(ds);
        sa.pool = pool_kv;
        sa.chunk_u4 = (int64_t)(chunk_bytes / 16);
        sa.n = n;
        for (int i = 0; i < n; ++i) sa.dst[i] = dst[p0 + i];
        err = lsa::launch_stage_scatter(sa, side_stream);
    }
    // the host staging buffer is the caller's again once every copy out of it
    // has finished (also after a failure, so no copy still reads it)
    for (int hh = 0; hh < 2; ++hh) {
        if (used[hh]) {
            const hipError_t e = hipEventSynchronize(ev[hh]);
            if (err == hipSuccess) err = e;
        }
        if (ev[hh]) (void)hipEventDestroy(ev[hh]);
    }
    if (err != hipSuccess) return hip_fail(err, "staged fetch");
    if (done) {
        const hipError_t e = hipEventRecord(done, side_stream);
        if (e != hipSuccess) return hip_fail(e, "fetch event record");
    }
    return ok();
}

lsa_status lsa_fetch_chunks_pull(const uint16_t* host_kv, int64_t C, const int32_t* chunk_ids, const int32_t* slots,
                                 uint16_t* pool_kv, int64_t P, int32_t B, int32_t Hkv, int32_t d, int32_t k,
                                 int32_t grid, hipStream_t stream) {
    if (!host_kv || !chunk_ids || !pool_kv)
        return fail(LSA_ERR_INVALID_ARGUMENT, "host_kv, chunk_ids and pool_kv are required");
    if (C < 1 || P < 1 || B < 1 || Hkv < 1 || k < 1 || grid < 0 || grid >= (1 << 24))
        return fail(LSA_ERR_INVALID_ARGUMENT, "C, P, B, Hkv, k must be >= 1 and 0 <= grid < 2^24");
    if (d != 64 && d != 128) return fail(LSA_ERR_UNSUPPORTED, "d=%d: supported head dims are 64 and 128", d);
    if (!slots && k > P) return fail(LSA_ERR_INVALID_ARGUMENT, "k=%d > P=%lld with default slots", k, (long long)P);
    if ((int64_t)B * k >= ((int64_t)1 << 31)) return fail(LSA_ERR_INVALID_ARGUMENT, "B*k must be < 2^31");
    if (!aligned(host_kv, 16) || !aligned(pool_kv, 16) || !aligned(chunk_ids, 4) || (slots && !aligned(slots, 4)))
        return fail(LSA_ERR_INVALID_ARGUMENT, "host_kv/pool_kv need 16-byte, ids/slots 4-byte alignment");
    // The kernel reads host_kv through the GPU's mapping of pinned memory.
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof attr);
    hipError_t pe = hipPointerGetAttributes(&attr, host_kv);
    if (pe != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fail(LSA_ERR_INVALID_ARGUMENT, "host_kv is not pinned host memory (allocate it with hipHostMalloc)");
    }
    void* dev_view = nullptr;
    pe = hipHostGetDevicePointer(&dev_view, const_cast<uint16_t*>(host_kv), 0);
    if (pe != hipSuccess || !dev_view) {
        (void)hipGetLastError();
        return fail(LSA_ERR_INVALID_ARGUMENT, "host_kv is not mapped into the device address space");
    }
    hipError_t e = lsa::launch_fetch_pull(static_cast<const uint16_t*>(dev_view), C, chunk_ids, slots, pool_kv, P, B,
                                          Hkv, d, k, grid ? grid : 16, stream);
    if (e != hipSuccess) return hip_fail(e, "fetch-pull launch");
    return ok();
}

lsa_status lsa_check_ids(const int32_t* chunk_ids, const int32_t* slots, const int32_t* counts, int32_t B, int32_t k,
                         int64_t C_ctx, int64_t C_store, int32_t* result, hipStream_t stream) {
    if (!chunk_ids || !result) return fail(LSA_ERR_INVALID_ARGUMENT, "chunk_ids and result are required");
    if (B < 1 || k < 1 || C_ctx < 1 || C_store < 1)
        return fail(LSA_ERR_INVALID_ARGUMENT, "B=%d, k=%d, C_ctx=%lld, C_store=%lld must all be >= 1", B, k,
                    (long long)C_ctx, (long long)C_store);
    if (k > lsa::kCheckMaxEntries)
        return fail(LSA_ERR_UNSUPPORTED, "k=%d: the check handles at most %d entries per request", k,
                    lsa::kCheckMaxEntries);
    if (B >= kMaxRowGroups || (int64_t)B * k >= ((int64_t)1 << 31))
        return fail(LSA_ERR_UNSUPPORTED, "B=%d, k=%d: B must be < 2^22 and B*k < 2^31", B, k);
    if (!aligned(chunk_ids, 4) || !aligned(result, 4) || (slots && !aligned(slots, 4)) || (counts && !aligned(counts, 4)))
        return fail(LSA_ERR_INVALID_ARGUMENT, "all pointers need 4-byte alignment");
    hipError_t e = lsa::launch_check_ids(chunk_ids, slots, counts, B, k, C_ctx, C_store, result, stream);
    if (e != hipSuccess) return hip_fail(e, "id-check launch");
    int32_t r[lsa::kCheckResultWords];
    e = hipMemcpyAsync(r, result, sizeof r, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "id-check result copy");
    auto value_at = [](const int32_t* p, int32_t at) {
        int32_t v = 0;
        (void)hipMemcpy(&v, p + at, sizeof v, hipMemcpyDeviceToHost);
        return v;
    };
    if (r[3] != INT32_MAX) {
        const int32_t c = value_at(counts, r[3]);
        return fail(LSA_ERR_INVALID_ARGUMENT, "request %d: count %d outside [0, k=%d]", r[3], c, k);
    }
    if (r[0] != INT32_MAX) {
        const int32_t c = value_at(chunk_ids, r[0]);
        const int32_t p = slots ? value_at(slots, r[0]) : c;
        return fail(LSA_ERR_INVALID_ARGUMENT,
                    "request %d entry %d: chunk id %d (must be in [0, %lld)) at store position %d (must be in [0, %lld))",
                    r[0] / k, r[0] % k, c, (long long)C_ctx, p, (long long)C_store);
    }
    if (r[1] != INT32_MAX)
        return fail(LSA_ERR_INVALID_ARGUMENT, "request %d entry %d: chunk id %d listed twice", r[1] / k, r[1] % k,
                    value_at(chunk_ids, r[1]));
    if (r[2] != INT32_MAX)
        return fail(LSA_ERR_INVALID_ARGUMENT, "request %d entry %d: store position %d listed twice", r[2] / k, r[2] % k,
                    value_at(slots, r[2]));
    return ok();
}

lsa_status lsa_pool_assign(const int32_t* prev_ids, const int32_t* prev_slots, int32_t n_prev, const int32_t* new_ids,
                           int32_t B, int32_t k, int64_t P, int32_t* new_slots, int32_t* fetch_slots,
                           hipStream_t stream) {
    if (!new_ids || !new_slots || !fetch_slots || (n_prev > 0 && (!prev_ids || !prev_slots)))
        return fail(LSA_ERR_INVALID_ARGUMENT, "new_ids, new_slots, fetch_slots (and prev_* when n_prev > 0) are required");
    if (B < 1 || k < 1 || n_prev < 0) return fail(LSA_ERR_INVALID_ARGUMENT, "B, k must be >= 1 and n_prev >= 0");
    if (B >= kMaxRowGroups) return fail(LSA_ERR_UNSUPPORTED, "B=%d: must be < 2^22", B);
    if (P < (int64_t)n_prev + k)
        return fail(LSA_ERR_INVALID_ARGUMENT, "P=%lld must be >= n_prev + k = %d", (long long)P, n_prev + k);
    if (P > INT32_MAX || lsa::pool_assign_lds_bytes(n_prev, (int)P) > 65536)
        return fail(LSA_ERR_UNSUPPORTED, "n_prev=%d, P=%lld: the assignment needs (2 n_prev + P) * 4 + P <= 65536 bytes",
                    n_prev, (long long)P);
    hipError_t e = lsa::launch_pool_assign(prev_ids, prev_slots, n_prev, new_ids, B, k, (int)P, new_slots, fetch_slots,
                                           stream);
    if (e != hipSuccess) return hip_fail(e, "pool-assign launch");
    return ok();
}

}  // extern "C"
