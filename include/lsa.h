/*
 * lsa.h -- C ABI of the MI355X (gfx950) library for the decode-time hot path
 * of Lookahead Sparse Attention (LSA, "FlashMemory").
 *
 * The pages describe the problem as: keep on the GPU only the KV chunks the
 * next decode window needs, predict them every tau = 64 steps with a neural
 * memory indexer whose score is a sigmoid of a dot product between the
 * current indexer query and each chunk's frozen compressed key, fetch them
 * ahead of use, and attend over them (paperlayer.ai summary of
 * "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via Lookahead
 * Sparse Attention", Abstract, 1 Introduction and 2.1 Architecture; the
 * sergiiob.dev handbook "DeepSeek-V4: Architecting for Ultra-Long Contexts",
 * The Neural Memory Indexer).  The four calls below are those steps.
 *
 * Conventions shared by every call
 *  - Pointers marked "device" must point to memory of the current HIP device;
 *    "host" pointers to host memory.  The caller owns every buffer; the
 *    library never allocates, frees, or keeps a pointer past the call.
 *  - Work is enqueued on `stream` (0 = the null stream) and is asynchronous:
 *    outputs are valid once the stream has reached the call.
 *  - Arguments are validated before any HIP call.  A rejected call enqueues
 *    nothing and returns LSA_ERR_INVALID_ARGUMENT, LSA_ERR_UNSUPPORTED or
 *    LSA_ERR_WORKSPACE; lsa_last_error() then holds a message (per thread).
 *    A failed launch or copy returns LSA_ERR_HIP.  Faults inside a kernel
 *    surface at the caller's next synchronisation, as with any HIP kernel.
 *  - Chunk ids that are out of range, or duplicated, are caller errors the
 *    kernels do not check (the ids produced by lsa_topk_chunks are always in
 *    range and distinct); lsa_check_ids checks a list on request.
 *  - A chunk is LSA_CHUNK_TOKENS = 64 consecutive tokens.
 *  - bf16 values are passed as their raw 16-bit patterns (uint16_t).
 *  - Calls keep no mutable global state that a result depends on: per
 *    device the library holds only the copy streams of lsa_fetch_chunks and
 *    the scratch array of lsa_gather_attend_noalloc, and per process the
 *    host worker threads of lsa_fetch_chunks_staged, set up at their first
 *    use and kept until the process ends; the tuning overrides below are per
 *    thread.  Calls may be issued from several host threads on different
 *    streams.
 *  - Tuning knobs (lsa_tuning below) choose among kernels and launch shapes;
 *    none changes a result.
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LSA_CHUNK_TOKENS 64

typedef enum lsa_status {
    LSA_OK = 0,
    LSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, size out of range, inconsistent shape */
    LSA_ERR_UNSUPPORTED = 2,      /* well-formed but outside what the kernels implement */
    LSA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
    LSA_ERR_HIP = 4               /* a HIP launch or copy failed */
} lsa_status;

/*
 * Tuning knobs.  The value in effect for a call is the calling thread's
 * override (lsa_set_tuning), else the environment variable named beside the
 * knob (read once per process, at the library's first use of any knob), else
 * the library's own choice.  No knob changes a result; the top-k split knobs
 * change what lsa_topk_tokens_workspace_size returns, so a thread sets them
 * before querying it.
 */
typedef enum lsa_tuning {
    LSA_TUNE_ATTEND_DEPTH = 0,      /* LSA_ATTEND_DEPTH: register ring depth of the
                                       attention's tile loads, 2-4 (default 2) */
    LSA_TUNE_SCORE_MFMA_MIN_NQ = 1, /* LSA_SCORE_MFMA_MIN_NQ: query rows per request from
                                       which lsa_index_score uses the int8 MFMA kernel (16) */
    LSA_TUNE_TOPK_STREAM_MIN_C = 2, /* LSA_TOPK_STREAM_MIN_C: row length from which the
                                       selects stream the row from memory (65537) */
    LSA_TUNE_TOPK_SPLIT_MIN_N = 3,  /* LSA_TOPK_SPLIT_MIN_N: token-list length from which
                                       lsa_topk_tokens splits a row over workgroups */
    LSA_TUNE_TOPK_SPLIT_SLICES = 4, /* LSA_TOPK_SPLIT_SLICES: slices of such a split
                                       (default: chosen from the sizes) */
    LSA_TUNE_FETCH_LANES = 5,       /* LSA_FETCH_LANES: copy streams lsa_fetch_chunks
                                       spreads its copies over, 1-16 (4) */
    LSA_TUNE_COUNT = 6
} lsa_tuning;

/* Override a knob (an lsa_tuning value) for the calling thread; value 0
 * drops the override.  LSA_ERR_INVALID_ARGUMENT for an unknown knob or a
 * value out of range (negative; ring depth other than 2-4; more than 16
 * fetch streams).  The knob is passed as int32_t so that any integer a
 * caller passes is well defined. */
lsa_status lsa_set_tuning(int32_t knob, int32_t value);

/* The value in effect for the calling thread (0: chosen per call from the
 * sizes), or -1 for an unknown knob. */
int32_t lsa_get_tuning(int32_t knob);

/* Static string naming a status code (an lsa_status value; any other
 * integer gives "LSA_ERR_UNKNOWN"). */
const char* lsa_status_string(int32_t s);

/* Message describing the last rejected call made by this host thread
 * ("" if none).  Valid until the thread's next call into the library. */
const char* lsa_last_error(void);

/*
 * lsa_index_score -- the memory indexer's score of every chunk.
 *
 * Defined by: the indexer scores chunks by a dot product between the indexer
 * query (from the current hidden state) and each chunk's frozen compressed
 * indexer key, passed through a sigmoid (paperlayer.ai summary, 2.1
 * Architecture and 3 Experiments / Limitations; Korean review, 1. Key Terms &
 * Definitions).  For request b, query row r < nq and chunk c:
 *     logits[b][r][c] = sum_i q_idx[b][r][i] * k_idx[b][c][i]   exact int32
 *     scores[b][r][c] = 1 / (1 + exp(-x)),  x = alpha * (float)logits[b][r][c]
 * with x formed as one fp32 product; scores are fp32 within 1e-6 relative
 * (plus 2^-126 absolute where the sigmoid underflows).
 *
 *  q_idx   device int8  [B][nq][d_idx]   indexer queries
 *  k_idx   device int8  [B][C][d_idx]    indexer keys, one row per chunk
 *  B, nq, C  >= 1 (nq rows share their request's keys; B*nq*C < 2^31)
 *  d_idx   16, 32, 64, 128 or 256 (LSA_ERR_UNSUPPORTED otherwise)
 *  alpha   scale of the sigmoid argument (finite)
 *  logits  device int32 [B][nq][C]       required output
 *  scores  device fp32  [B][nq][C]       optional output (NULL: not written)
 *  stream  HIP stream
 * Pointers to device buffers need 16-byte alignment for q_idx and k_idx,
 * 4-byte for logits and scores.
 */
lsa_status lsa_index_score(const int8_t* q_idx, const int8_t* k_idx, int32_t B, int32_t nq, int32_t C,
                           int32_t d_idx, float alpha, int32_t* logits, float* scores, hipStream_t stream);

/*
 * lsa_topk_chunks -- the fixed-budget re-selection.
 *
 * Defined by: every tau steps LSA keeps only the chunks the indexer ranks
 * highest (paperlayer.ai summary, 1 Introduction and 2.1 Architecture, where
 * the native indexer's selection is a top-k).  For each row r the selected
 * set is the first k chunks of the total order "logit descending, then chunk
 * index ascending" (ties go to the lower chunk index), written in ascending
 * chunk order.  The set is unique, so the output is bit-exact.
 *
 *  logits     device int32 [R][C]   (any int32 values)
 *  1 <= R < 2^22, 1 <= C <= 2^30, 1 <= k <= C (rows up to 65536 chunks keep their
 *  keys in registers; longer ones stream from memory in every pass)
 *  chunk_ids  device int32 [R][k]   output, ascending within each row
 *  stream     HIP stream
 */
lsa_status lsa_topk_chunks(const int32_t* logits, int32_t R, int32_t C, int32_t k, int32_t* chunk_ids,
                           hipStream_t stream);

/*
 * lsa_threshold_chunks -- the pages' own selection rule: sigmoid gating with
 * a variable budget.
 *
 * Defined by: the memory indexer keeps every chunk whose sigmoid score
 * passes a threshold (0.5 in the reported configuration) instead of a fixed
 * top-k (paperlayer.ai summary, 2.1 Architecture and 2.4 Configuration).  The
 * budget per request is then variable, here capped at k_max (the HBM pool
 * size).  For each row r: the chunks with logit > logit_threshold; if more
 * than k_max pass, the first k_max of the order (logit descending, chunk
 * index ascending).  Written in ascending chunk order into
 * chunk_ids[r][0..counts[r]), the rest of the row set to -1.
 * With scores sigma(alpha * logit), alpha > 0: sigma > 0.5 exactly when
 * alpha * logit > 0, i.e. logit > 0, so the 0.5 threshold is
 * logit_threshold = 0.  Another score threshold s maps to the largest
 * integer logit whose score does not exceed s.
 *
 *  logits      device int32 [R][C]
 *  1 <= R < 2^22, 1 <= C <= 2^30, 1 <= k_max <= C
 *  chunk_ids   device int32 [R][k_max] output
 *  counts      device int32 [R] output, chunks kept per row (0..k_max)
 */
lsa_status lsa_threshold_chunks(const int32_t* logits, int32_t R, int32_t C, int32_t logit_threshold, int32_t k_max,
                                int32_t* chunk_ids, int32_t* counts, hipStream_t stream);

/*
 * lsa_topk_tokens -- the token-level second stage inside the recalled chunks.
 *
 * Defined by: after the chunk recall, the model's native token-level scoring
 * picks a fine-grained top-k among the recalled entries only, not over the
 * whole context (paperlayer.ai summary, 2.1 Architecture).  The pages give
 * no formula for those token scores, so they are an input here.  List
 * position p = j*64 + t names token t of list entry j (chunk
 * chunk_ids[b][j]); it competes iff j < counts[b] (all k when counts is
 * NULL) and chunk_ids[b][j]*64 + t < ctx_len[b].  Among the competing
 * positions the first min(k_tok, competing) of the order "score descending,
 * then position ascending" are kept (scores compare as values: -0 equals
 * +0, subnormals are not flushed), written in ascending position order
 * into tok[b][0..tok_counts[b]),
 * the rest of the row set to -1.  The set is unique: bit-exact.
 *
 *  scores      device fp32 [B][k*64], no NaN among competing positions
 *  chunk_ids   device int32 [B][k]
 *  counts      device int32 [B] entries in use, or NULL (all k)
 *  ctx_len     device int32 [B]
 *  B >= 1, k >= 1 with k*64 <= 2^30, k_tok >= 1; B < 2^22, and B times
 *  the slices < 2^22 when the list is split (LSA_ERR_UNSUPPORTED otherwise)
 *  tok         device int32 [B][k_tok] output: list positions
 *  tok_counts  device int32 [B] output: positions kept per request
 *  workspace   device buffer of lsa_topk_tokens_workspace_size(B, k, k_tok)
 *              bytes, 256-byte aligned, or NULL.  With it, lists of more
 *              than 32768 positions are selected by many workgroups per
 *              request: each slice of the list keeps its own top k_tok,
 *              then the top k_tok of those candidates are taken (the same
 *              set, since every position of the request's top k_tok is in
 *              its slice's).  NULL: one workgroup per request.  Scratch
 *              only; calls sharing a workspace must not overlap in time.
 * All other pointers need 4-byte alignment.
 */
lsa_status lsa_topk_tokens(const float* scores, const int32_t* chunk_ids, const int32_t* counts,
                           const int32_t* ctx_len, int32_t B, int32_t k, int32_t k_tok, int32_t* tok,
                           int32_t* tok_counts, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace lsa_topk_tokens can use for these sizes: 0 when the
 * select runs as one workgroup per request anyway, (size_t)-1 when the
 * arguments are invalid. */
size_t lsa_topk_tokens_workspace_size(int32_t B, int32_t k, int32_t k_tok);

/*
 * Number of bytes of workspace lsa_gather_attend needs for these sizes and
 * this split count (n_split = 0: the library's own choice).  Returns 0 when
 * no workspace is needed, (size_t)-1 when the arguments are invalid or the
 * launch would exceed 2^24 split workgroups (B*Hkv*min(n_split, k)).
 */
size_t lsa_gather_attend_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t k,
                                        int32_t n_split);

/* The split count lsa_gather_attend uses for n_split = 0 (>= 1), or -1 when
 * the arguments are invalid. */
int32_t lsa_gather_attend_default_splits(int32_t B, int32_t Hkv, int32_t k);

/*
 * lsa_gather_attend -- GQA decode attention over the retained chunks only.
 *
 * Defined by: attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V, with query
 * heads in groups that share one KV head (sergiiob.dev handbook, "Grouped
 * Query Attention (GQA) vs. Multi-Head Attention (MHA)": 64 query heads, 8 KV
 * heads, d_k = 128, every 8 query heads one KV head), restricted to the
 * tokens of the chunks LSA kept in GPU memory (paperlayer.ai summary,
 * Abstract and 2.1 Architecture).  For request b and query head h, with KV
 * head g = h / (Hq/Hkv):
 *     tokens  = { chunk_ids[b][j]*64 + t : j < k, t < 64, that position < ctx_len[b] }
 *     out[b][h] = sum_tok softmax_tok(sm_scale * q[b][h].K[tok]) * V[tok]
 * where K/V of list entry j are read from store position slots[b][j]
 * (slots == NULL: position chunk_ids[b][j]).  Products and sums in fp32
 * (bf16 inputs are exact in fp32); the softmax weights enter the V product
 * as a two-term bf16 split, about 16 significant bits.
 *
 *  q          device bf16 [B][Hq][d]
 *  kv         device bf16 [B][C_store][2][Hkv][64][d]: chunk-major; index 2
 *             selects K (0) or V (1); every stored chunk holds 64 token rows,
 *             also past ctx_len (those rows are read, then ignored)
 *  C_store    chunk positions per request in `kv` (>= 1)
 *  chunk_ids  device int32 [B][k]: context chunk index of each list entry
 *             (decides which tokens are < ctx_len)
 *  slots      device int32 [B][k] store position of each entry, or NULL
 *  counts     device int32 [B]: entries in use per request (the first
 *             counts[b] of the row; as lsa_threshold_chunks writes them), or
 *             NULL: all k
 *  ctx_len    device int32 [B]: valid tokens per request; a request whose
 *             listed chunks (and segment) hold no valid token gets out = 0
 *  seg_kv     device bf16 [B][2][Hkv][S_max][d], or NULL: a resident segment
 *             attended in the same softmax as the chunks -- the local
 *             sliding window and the freshly decoded tokens the pages always
 *             keep in GPU memory (paperlayer.ai summary, 2.1 Architecture:
 *             the recalled chunks join the local window's KV, which is never
 *             offloaded; 3 Experiments / Experimental Setup: the local 8K /
 *             decoded window is retained).  Its tokens are not
 *             chunk tokens: ctx_len bounds only the chunks, so a caller
 *             passes the length of the offloadable history there.
 *  seg_len    device int32 [B]: tokens of the segment in use (<= S_max)
 *  S_max      segment capacity, a multiple of 64 (ignored without seg_kv)
 *  B >= 1; Hq % Hkv == 0; 1 <= Hq/Hkv <= 16; d = 64 or 128; 1 <= k;
 *  B*Hq < 2^24
 *  sm_scale   softmax scale, normally 1/sqrt(d)
 *  workspace  device buffer of at least
 *             lsa_gather_attend_workspace_size(B, Hq, Hkv, d, k, n_split)
 *             bytes, 256-byte aligned (NULL allowed when that size is 0);
 *             scratch for the per-split partial results, no state is kept
 *             in it between calls.  Calls sharing a workspace must not
 *             overlap in time (same stream, or otherwise ordered).
 *  n_split    chunk-list splits per (request, KV head); 0 = library choice;
 *             B*Hkv*min(n_split, k) <= 2^24 (LSA_ERR_UNSUPPORTED otherwise)
 *  out        device fp32 [B][Hq][d]
 *  stream     HIP stream
 * q, kv and out need 16-byte alignment.
 */
lsa_status lsa_gather_attend(const uint16_t* q, const uint16_t* kv, int64_t C_store, const int32_t* chunk_ids,
                             const int32_t* slots, const int32_t* counts, const int32_t* ctx_len,
                             const uint16_t* seg_kv, const int32_t* seg_len, int32_t S_max, int32_t B,
                             int32_t Hq, int32_t Hkv,
                             int32_t d, int32_t k, float sm_scale, void* workspace, size_t workspace_bytes,
                             int32_t n_split, float* out, hipStream_t stream);

/*
 * lsa_gather_attend_noalloc -- lsa_gather_attend without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, result and validation as lsa_gather_attend, minus the
 * workspace.  The split partials live in a static device buffer of
 * LSA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; its device address is looked up on the first call
 * made with that GPU current.  The call allocates nothing.  Sizes whose
 * partials exceed the buffer (lsa_gather_attend_workspace_size(...) >
 * LSA_NOALLOC_SCRATCH_BYTES) are rejected with LSA_ERR_WORKSPACE before any
 * HIP call.  All calls on one GPU share that GPU's buffer: calls whose
 * executions overlap in time on one GPU (different streams, different host
 * threads without ordering) race and give wrong results; calls ordered on
 * one stream are safe.
 */
#define LSA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
lsa_status lsa_gather_attend_noalloc(const uint16_t* q, const uint16_t* kv, int64_t C_store,
                                     const int32_t* chunk_ids, const int32_t* slots, const int32_t* counts,
                                     const int32_t* ctx_len, const uint16_t* seg_kv, const int32_t* seg_len,
                                     int32_t S_max, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t k,
                                     float sm_scale, int32_t n_split, float* out, hipStream_t stream);

/*
 * lsa_gather_attend_tokens -- lsa_gather_attend over a listed subset of the
 * chunk tokens (the output of lsa_topk_tokens).
 *
 * Defined by: the same attention as lsa_gather_attend, with the chunk tokens
 * restricted to those the token-level top-k kept (paperlayer.ai summary, 2.1
 * Architecture: the fine-grained entries picked from the recalled subset,
 * combined with the sliding-window KV).  The chunk tokens are
 *     { chunk_ids[b][j]*64 + t : p = j*64 + t in tok[b][0..tok_counts[b]),
 *       j < counts[b], that position < ctx_len[b] }
 * each listed position counted once per listing (positions outside the used
 * entries or past ctx_len are left out); the resident segment, if given, is
 * attended in full as in lsa_gather_attend.  Every other argument has the
 * meaning it has there.
 *
 *  tok         device int32 [B][k_tok] list positions (ascending is the
 *              efficient order; any order gives the same result up to
 *              rounding)
 *  tok_counts  device int32 [B] positions in use, or NULL (all k_tok)
 *  k_tok >= 1
 *  kv          the store of lsa_gather_attend; C_store * 2*Hkv*64 < 2^31
 *  workspace   lsa_gather_attend_workspace_size(B, Hq, Hkv, d, ceil(k_tok/64),
 *              n_split) bytes; n_split splits the token list into contiguous
 *              parts (0 = library choice for ceil(k_tok/64) blocks of 64
 *              listed tokens)
 */
lsa_status lsa_gather_attend_tokens(const uint16_t* q, const uint16_t* kv, int64_t C_store, const int32_t* chunk_ids,
                                    const int32_t* slots, const int32_t* counts, const int32_t* ctx_len,
                                    const int32_t* tok, const int32_t* tok_counts, int32_t k_tok,
                                    const uint16_t* seg_kv, const int32_t* seg_len, int32_t S_max, int32_t B,
                                    int32_t Hq, int32_t Hkv, int32_t d, int32_t k, float sm_scale, void* workspace,
                                    size_t workspace_bytes, int32_t n_split, float* out, hipStream_t stream);

/*
 * lsa_check_ids -- opt-in check of a chunk list before it is attended over or
 * fetched (the kernels trust their ids; no page passage defines this call).
 *
 * Reads only chunk_ids, slots and counts.  For every request b, over its used
 * entries j < counts[b] (all k when counts is NULL; entries past the count,
 * such as the -1 padding of lsa_threshold_chunks, are not looked at):
 *   - 0 <= chunk_ids[b][j] < C_ctx (the request's context chunks);
 *   - its store position, slots[b][j] (or chunk_ids[b][j] when slots is
 *     NULL), in [0, C_store);
 *   - no chunk id and no store position listed twice;
 *   - counts[b] in [0, k].
 * Synchronous: enqueues the check on `stream`, waits for the stream, and
 * returns LSA_OK, or LSA_ERR_INVALID_ARGUMENT with lsa_last_error() naming
 * the first offending request and entry and the rule it breaks.
 *
 *  chunk_ids  device int32 [B][k]
 *  slots      device int32 [B][k] or NULL
 *  counts     device int32 [B] or NULL
 *  1 <= B < 2^22, 1 <= k <= 16384, B*k < 2^31; C_ctx, C_store >= 1
 *  result     device int32 [4], scratch the check writes (owned by the
 *             caller, so that the call allocates nothing)
 *  stream     HIP stream (not under graph capture: the call waits for it)
 */
lsa_status lsa_check_ids(const int32_t* chunk_ids, const int32_t* slots, const int32_t* counts, int32_t B, int32_t k,
                         int64_t C_ctx, int64_t C_store, int32_t* result, hipStream_t stream);

/*
 * lsa_fetch_chunks -- host-tier fetch of the selected chunks into HBM.
 *
 * Defined by: non-recalled entries live in CPU memory and the recalled
 * chunks are brought back from that cold storage every tau = 64 steps,
 * asynchronously, ahead of use (paperlayer.ai summary, 2.1 Architecture and
 * 3 Experiments / Experimental Setup; sergiiob.dev handbook, The Neural Memory
 * Indexer, item 3).  For every request b and entry j:
 *     pool_kv[b][slot] := host_kv[b][chunk_ids[b][j]]   (K and V, all heads)
 * with slot = host_slots[b][j] (NULL: slot j), as host-to-device copies
 * ordered on `side_stream`; entries whose chunk ids and slots both run on
 * consecutively are merged into one copy, and an entry with a negative slot
 * is not copied (its id is not read): the fetch_slots of lsa_pool_assign
 * (-1 for a chunk already in the pool, or an entry not in use) give a delta
 * fetch.  The copies are spread round-robin over LSA_TUNE_FETCH_LANES (4)
 * streams of the library's own (created for the current device at the first
 * call, default priority, kept until the process ends) that start after the
 * work already on `side_stream` and that `side_stream` waits for again, so
 * several DMA copies are in flight at once; under graph capture, or when
 * `side_stream` belongs to another device than the current one, they stay
 * on `side_stream`.  If
 * `done` is not NULL it is recorded on `side_stream` after the last copy, so
 * a compute stream can wait on it (hipStreamWaitEvent) before attending over
 * the pool.
 *
 *  host_kv         host bf16 [B][C][2][Hkv][64][d], pinned (hipHostMalloc);
 *                  pageable memory is rejected with LSA_ERR_INVALID_ARGUMENT
 *  C               chunks per request in host_kv
 *  host_chunk_ids  host int32 [B][k], each in [0, C) (checked) where copied
 *  host_slots      host int32 [B][k], each < P (checked; negative: not
 *                  copied), or NULL
 *  pool_kv         device bf16 [B][P][2][Hkv][64][d]
 *  P               chunk slots per request in the pool (k <= P when slots is NULL)
 *  B, Hkv, d, k    >= 1
 *  side_stream     HIP stream the copies go on
 *  done            HIP event or NULL
 * The id and slot arrays are read during the call and may be reused at once.
 */
lsa_status lsa_fetch_chunks(const uint16_t* host_kv, int64_t C, const int32_t* host_chunk_ids,
                            const int32_t* host_slots, uint16_t* pool_kv, int64_t P, int32_t B, int32_t Hkv,
                            int32_t d, int32_t k, hipStream_t side_stream, hipEvent_t done);

/*
 * lsa_fetch_chunks_staged -- the fetch of lsa_fetch_chunks (the same
 * definition, arguments and result in the pool), sent over the host link
 * in large copies: the selected chunks lie scattered over the host store,
 * and one copy per 256 KB chunk carries a fixed cost that keeps the link
 * below half its rate.  Here the library's host worker threads gather the
 * chunks to copy into consecutive places of a pinned staging buffer, each
 * piece of up to stage_chunks / 2 chunks (at most 512) crosses the link as
 * one hipMemcpyAsync on `side_stream`, and a kernel on `side_stream` moves
 * the piece's chunks from the device staging buffer into their pool slots.
 * Pieces alternate between the two halves of the staging buffers, so the
 * host gathers one piece while the previous one is on the link.
 *
 * Defined by: as lsa_fetch_chunks (paperlayer.ai summary, 2.1 Architecture
 * and 3 Experiments / Experimental Setup; sergiiob.dev handbook, The Neural
 * Memory Indexer, item 3 and its closing paragraph on host-to-device
 * bandwidth).
 *
 *  host_kv, C, host_chunk_ids, host_slots, pool_kv, P, B, Hkv, d, k, done:
 *                 as for lsa_fetch_chunks (negative slots: not copied);
 *                 also B*P < 2^31
 *  host_staging   pinned host memory (hipHostMalloc) of stage_chunks chunks
 *                 (2*Hkv*64*d bf16 each), owned by the caller
 *  dev_staging    device memory of stage_chunks chunks, owned by the caller
 *  stage_chunks   >= 2
 *  side_stream    HIP stream the copies and the scatter kernels go on
 * Unlike lsa_fetch_chunks the call waits on the host: before it refills a
 * staging half for the copy out of it, and before it returns for every
 * copy, so host_staging is the caller's again on return; side_stream must
 * therefore not wait for work that is enqueued after the call.  dev_staging
 * is read by the scatter kernels in side_stream's order: a later use on
 * another stream waits for `done` or side_stream first.  Under graph
 * capture it returns LSA_ERR_UNSUPPORTED.  Calls from several threads each
 * need their own staging buffers; their gathers share the worker threads
 * one call at a time.
 */
lsa_status lsa_fetch_chunks_staged(const uint16_t* host_kv, int64_t C, const int32_t* host_chunk_ids,
                                   const int32_t* host_slots, uint16_t* pool_kv, int64_t P, int32_t B, int32_t Hkv,
                                   int32_t d, int32_t k, uint16_t* host_staging, uint16_t* dev_staging,
                                   int64_t stage_chunks, hipStream_t side_stream, hipEvent_t done);

/*
 * lsa_fetch_chunks_pull -- the same host-tier fetch as lsa_fetch_chunks, done
 * by a kernel that reads the pinned host memory through the GPU's mapping of
 * it (a gather over the host link) instead of one DMA copy per run.
 *
 * Defined by: the same passages as lsa_fetch_chunks.  For every request b
 * and entry j:  pool_kv[b][slot] := host_kv[b][chunk_ids[b][j]]  with
 * slot = slots[b][j] (NULL: slot j).  The ids and slots are read on the GPU,
 * so the fetch can follow lsa_topk_chunks on the device with no host round
 * trip, and can be captured in a HIP graph.  An entry whose id is outside
 * [0, C) or whose slot is outside [0, P) is skipped (its slot is left as it
 * was); the kernel never reads or writes outside the two buffers.
 *
 *  host_kv    pinned host bf16 [B][C][2][Hkv][64][d] (hipHostMalloc; its
 *             device mapping is looked up with hipHostGetDevicePointer)
 *  C          chunks per request in host_kv
 *  chunk_ids  device int32 [B][k]
 *  slots      device int32 [B][k] or NULL (k <= P then)
 *  pool_kv    device bf16 [B][P][2][Hkv][64][d]
 *  B, Hkv, k >= 1; d = 64 or 128
 *  grid       workgroups of the gather, < 2^24 (0 = 16).  The link is the bound:
 *             8-16 workgroups already reach it (about 57 GB/s on MI355X),
 *             and every workgroup parked on long host-link reads slows the
 *             kernels that share its compute unit
 *  stream     HIP stream (normally a side stream, so the copy overlaps
 *             attention on the main stream)
 * host_kv and pool_kv need 16-byte alignment.
 */
lsa_status lsa_fetch_chunks_pull(const uint16_t* host_kv, int64_t C, const int32_t* chunk_ids, const int32_t* slots,
                                 uint16_t* pool_kv, int64_t P, int32_t B, int32_t Hkv, int32_t d, int32_t k,
                                 int32_t grid, hipStream_t stream);

/*
 * lsa_pool_assign -- HBM pool slots for a delta fetch.
 *
 * Defined by: LSA keeps in GPU memory only the recalled chunks and evicts the
 * others to CPU memory (paperlayer.ai summary, 2.1 Architecture), fetching
 * the critical chunks ahead of the next window (sergiiob.dev handbook, The
 * Neural Memory Indexer, item 3).  Between two selections, the chunks kept
 * by both need no copy.  For every request b, with S_prev = prev_ids[b]
 * held at prev_slots[b] and S_new = new_ids[b]:
 *   - a chunk of S_new that is also in S_prev keeps its slot
 *     (new_slots = that slot, fetch_slots = -1: nothing to copy);
 *   - the r-th chunk of S_new, in ascending id order, that is not in S_prev
 *     gets the r-th lowest slot of [0, P) that no entry of S_prev holds
 *     (new_slots = fetch_slots = that slot).
 * Passing fetch_slots as the slots of lsa_fetch_chunks_pull then copies
 * exactly the new chunks (entries with slot -1 are skipped), and new_slots
 * are the slots lsa_gather_attend reads S_new from.  S_prev's slots stay
 * untouched, so attention over S_prev may run while S_new is fetched.
 * An entry with a negative chunk id is not in use: the -1 padding that
 * lsa_threshold_chunks writes past each request's count.  In S_prev it holds
 * no slot (its slot is not read); in S_new it gets new_slots = fetch_slots
 * = -1, so the pull fetch skips it (and attention, given the counts, never
 * reads it).  Variable-size selections thus go through unchanged.
 *
 *  prev_ids    device int32 [B][n_prev], ascending within each row among the
 *              entries in use (as lsa_topk_chunks and lsa_threshold_chunks
 *              write them); may be NULL when n_prev = 0
 *  prev_slots  device int32 [B][n_prev], distinct within a row and in
 *              [0, P) for the entries in use
 *  n_prev      0 for the first selection (every chunk is new)
 *  new_ids     device int32 [B][k], ascending within each row among the
 *              entries in use
 *  B           requests, 1 <= B < 2^22
 *  P           pool slots per request, >= n_prev + k;
 *              (2 n_prev + P) * 4 + P <= 65536 (LSA_ERR_UNSUPPORTED otherwise)
 *  new_slots, fetch_slots  device int32 [B][k] outputs
 */
lsa_status lsa_pool_assign(const int32_t* prev_ids, const int32_t* prev_slots, int32_t n_prev, const int32_t* new_ids,
                           int32_t B, int32_t k, int64_t P, int32_t* new_slots, int32_t* fetch_slots,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
