/*
 * CPU oracle for the decode path of Lookahead Sparse Attention (LSA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code with the HIP library.
 *
 * Each function is the plain definition of one step, in exact integers or in
 * IEEE double, with no blocking, fusion or reordering beyond the definition:
 *
 *  1. Indexer logits: the dot product of the indexer query with each chunk's
 *     compressed indexer key ("FlashMemory-DeepSeek-V4 ... Lookahead Sparse
 *     Attention", paperlayer.ai summary, 2 Methodology / 2.1 Architecture and
 *     3 Experiments / Limitations, which name a dot-product interaction; the
 *     Korean review, 1. Key Terms & Definitions, "Neural Memory Indexer").
 *     Exact in int64.
 *  2. Indexer score: a sigmoid of the logit (same 2.1 Architecture bullet and
 *     the review's definition).  The argument is alpha*logit formed as one
 *     IEEE single-precision product, then 1/(1+exp(-x)) in double.
 *  3. Chunk selection: a fixed budget of k chunks, the first k of the order
 *     "key descending, then chunk index ascending", returned in ascending
 *     chunk order.  Written as a rank count: chunk c is kept iff fewer than k
 *     chunks precede it in that order.
 *  4. Gathered GQA decode attention: softmax(q K^T / sqrt(d_k)) V over the
 *     tokens of the kept chunks (sergiiob.dev handbook "DeepSeek-V4:
 *     Architecting for Ultra-Long Contexts", section "Grouped Query Attention
 *     (GQA) vs. Multi-Head Attention (MHA)", the attention formula; the same
 *     section: 64 query heads share 8 KV heads, every 8 consecutive query
 *     heads one KV head).  bf16 inputs widened exactly to double; every sum
 *     in double; tokens at or past the request's context length are left out.
 *  5. Host-tier fetch: a byte copy of each selected chunk into its pool slot
 *     (paperlayer.ai summary, 2.1 Architecture: non-recalled entries are
 *     evicted to CPU; 3 Experiments / Experimental Setup: recalled chunks are
 *     retrieved from CPU cold storage every tau = 64 steps).
 *  6. Pool slots of a delta fetch (the same passages: only the chunks not
 *     already recalled need fetching): a chunk kept from the previous
 *     selection keeps its slot; the r-th new chunk in ascending id order takes
 *     the r-th lowest slot the previous selection does not hold.  Entries
 *     with a negative id (the padding of a variable-size selection) are not
 *     in use.
 *  7. Threshold selection (summary 2.1 Architecture, 2.4 Configuration:
 *     sigmoid gating at 0.5 instead of a fixed top-k): the chunks whose logit
 *     exceeds a threshold, capped at k_max by the same order as item 3.
 *  8. Token selection inside the recalled chunks (summary 2.1 Architecture:
 *     after the chunk recall, the model's own token-level scores pick a
 *     fine-grained top-k among the recalled entries only).  The scores are an
 *     input: the pages do not give the scoring function.  Same order as item
 *     3 over the usable tokens of the recalled chunks, by list position.
 *     Item 4 then attends over exactly the listed tokens.
 *
 * Layouts (row-major):
 *   q_idx  int8   [B][nq][d_idx]        K_idx int8 [B][C][d_idx]
 *   logits int64  [B*nq][C]             ids   int32 [B][k]
 *   q      bf16   [B][Hq][d]            kv    bf16 [B][C_store][2][Hkv][T][d]
 *   out    double [B][Hq][d]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* 1. logits[b*nq + r][c] = sum_i q_idx[b][r][i] * K_idx[b][c][i]  (exact). */
void oracle_index_logits(const int8_t* q_idx, const int8_t* k_idx, int64_t B, int64_t nq, int64_t C,
                         int64_t d_idx, int64_t* logits) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < C; ++c)
            for (int64_t r = 0; r < nq; ++r) {
                const int8_t* qv = q_idx + (b * nq + r) * d_idx;
                const int8_t* kv = k_idx + (b * C + c) * d_idx;
                int64_t acc = 0;
                for (int64_t i = 0; i < d_idx; ++i) acc += (int64_t)qv[i] * (int64_t)kv[i];
                logits[(b * nq + r) * C + c] = acc;
            }
}

/* 2. scores[j] = 1 / (1 + exp(-x)),  x = alpha * (float)logit in IEEE fp32. */
void oracle_index_scores(const int64_t* logits, int64_t n, float alpha, double* scores) {
    for (int64_t j = 0; j < n; ++j) {
        volatile float xl = (float)logits[j];
        volatile float x = alpha * xl; /* one single-precision product */
        scores[j] = 1.0 / (1.0 + exp(-(double)x));
    }
}

/* 3. Budgeted selection.  Chunk c precedes chunk c' when key[c] > key[c'],
 *    or key[c] == key[c'] and c < c'.  Chunk c is kept iff
 *    #{c' : c' precedes c} < k.  Ids are written in ascending order.
 *    Returns 0, or -1 if k is out of [1, C]. */
int oracle_topk_i64(const int64_t* keys, int64_t R, int64_t C, int64_t k, int32_t* ids) {
    if (k < 1 || k > C) return -1;
    unsigned char* keep = (unsigned char*)malloc((size_t)C);
    int status = 0;
    for (int64_t r = 0; r < R && status == 0; ++r) {
        const int64_t* row = keys + r * C;
        /* each chunk's rank is counted on its own, so the counts run in
         * parallel; the kept chunks are then listed in ascending order */
#pragma omp parallel for schedule(dynamic, 64)
        for (int64_t c = 0; c < C; ++c) {
            int64_t before = 0;
            for (int64_t c2 = 0; c2 < C; ++c2)
                if (row[c2] > row[c] || (row[c2] == row[c] && c2 < c)) ++before;
            keep[c] = before < k;
        }
        int64_t n_out = 0;
        for (int64_t c = 0; c < C; ++c) n_out += keep[c];
        if (n_out != k) status = -2; /* cannot happen: the order is total */
        n_out = 0;
        for (int64_t c = 0; c < C && status == 0; ++c)
            if (keep[c]) ids[r * k + n_out++] = (int32_t)c;
    }
    free(keep);
    return status;
}

/* Same rule on double keys (used to compare selection by score with
 * selection by logit). */
int oracle_topk_f64(const double* keys, int64_t R, int64_t C, int64_t k, int32_t* ids) {
    if (k < 1 || k > C) return -1;
    for (int64_t r = 0; r < R; ++r) {
        const double* row = keys + r * C;
        int64_t n_out = 0;
        for (int64_t c = 0; c < C; ++c) {
            int64_t before = 0;
            for (int64_t c2 = 0; c2 < C; ++c2)
                if (row[c2] > row[c] || (row[c2] == row[c] && c2 < c)) ++before;
            if (before < k) ids[r * k + n_out++] = (int32_t)c;
        }
        if (n_out != k) return -2;
    }
    return 0;
}

/* 4. Gathered GQA decode attention.
 *    For request b and query head h (KV head g = h / (Hq/Hkv)), the tokens
 *    are those of the listed chunks: list entry j names chunk chunk_ids[b][j]
 *    stored at position slots[b][j] of the store (slots == NULL: the chunk's
 *    own index); token t of that chunk is at context position
 *    chunk_ids[b][j]*T + t and is used iff that position < ctx_len[b] and
 *    j < counts[b] (counts may be NULL: all k entries).  If seg_kv is not
 *    NULL the first seg_len[b] tokens of the resident segment
 *    seg_kv[b][K|V][g][0..S_max) join them (the local window and decoded
 *    tokens, always kept).
 *      z  = (q[b][h] . K[token]) * sm_scale
 *      w  = exp(z - max z)
 *      out[b][h] = sum_token w * V[token] / sum_token w
 *    If `tok` is not NULL only the listed tokens of the chunks are used:
 *    tok[b][0..tok_counts[b]) (all k_tok when tok_counts is NULL) are list
 *    positions p = j*T + t, each naming token t of list entry j; a position
 *    whose entry is unused or whose token is at or past ctx_len[b] is left
 *    out.  The resident segment, if any, is used in full as above.
 *    If `weights` is not NULL it receives the normalised softmax weight of
 *    every (list entry, token) pair, [B][Hq][k*T + S_max] (segment token t at
 *    k*T + t), 0 for unused tokens.
 *    Returns 0, -1 on bad arguments, -3 if a request has no usable token. */
int oracle_gather_attend(const uint16_t* q, const uint16_t* kv, int64_t C_store, const int32_t* chunk_ids,
                         const int32_t* slots, const int32_t* counts, const int32_t* ctx_len,
                         const uint16_t* seg_kv, const int32_t* seg_len, int64_t S_max, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t d, int64_t k, int64_t T, double sm_scale, double* out, double* weights,
                         const int32_t* tok, const int32_t* tok_counts, int64_t k_tok) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || d < 1 || k < 1 || T < 1) return -1;
    if (seg_kv && (!seg_len || S_max < 1)) return -1;
    if (tok && k_tok < 1) return -1;
    const int64_t group = Hq / Hkv;
    const int64_t tile = T * d;              /* one (K|V, head) tile          */
    const int64_t chunk = 2 * Hkv * tile;    /* one chunk, K and V, all heads */
    const int64_t n_slot = k * T + (seg_kv ? S_max : 0);
    const int64_t n_list = (tok && k_tok > k * T ? k_tok : k * T) + (seg_kv ? S_max : 0);
    int status = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t g = h / group;
            const uint16_t* qh = q + (b * Hq + h) * d;
            /* the token list: K and V row of every used token, and its slot in `weights` */
            const uint16_t** Kr = (const uint16_t**)malloc(sizeof(uint16_t*) * (size_t)n_list);
            const uint16_t** Vr = (const uint16_t**)malloc(sizeof(uint16_t*) * (size_t)n_list);
            int64_t* where = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_list);
            double* z = (double*)malloc(sizeof(double) * (size_t)n_list);
            int64_t n = 0;
            const int64_t kb = counts ? (counts[b] < k ? counts[b] : k) : k;
            if (tok) {
                /* the listed tokens: list position p = j*T + t names token t
                   of list entry j; positions outside the used entries or at
                   or past the context length are left out */
                const int64_t tc = tok_counts ? tok_counts[b] : k_tok;
                for (int64_t u = 0; u < tc && u < k_tok; ++u) {
                    const int64_t pos = tok[b * k_tok + u];
                    if (pos < 0 || pos >= kb * T) continue;
                    const int64_t j = pos / T, t = pos % T;
                    const int64_t c = chunk_ids[b * k + j];
                    if (c * T + t >= (int64_t)ctx_len[b]) continue;
                    const int64_t p = slots ? slots[b * k + j] : c;
                    Kr[n] = kv + (b * C_store + p) * chunk + (0 * Hkv + g) * tile + t * d;
                    Vr[n] = kv + (b * C_store + p) * chunk + (1 * Hkv + g) * tile + t * d;
                    where[n++] = pos;
                }
            }
            for (int64_t j = 0; !tok && j < kb; ++j) {
                const int64_t c = chunk_ids[b * k + j];
                const int64_t p = slots ? slots[b * k + j] : c;
                const uint16_t* K = kv + (b * C_store + p) * chunk + (0 * Hkv + g) * tile;
                const uint16_t* V = kv + (b * C_store + p) * chunk + (1 * Hkv + g) * tile;
                for (int64_t t = 0; t < T; ++t)
                    if (c * T + t < (int64_t)ctx_len[b]) {
                        Kr[n] = K + t * d;
                        Vr[n] = V + t * d;
                        where[n++] = j * T + t;
                    }
            }
            if (seg_kv) {
                const uint16_t* K = seg_kv + ((b * 2 + 0) * Hkv + g) * S_max * d;
                const uint16_t* V = seg_kv + ((b * 2 + 1) * Hkv + g) * S_max * d;
                for (int64_t t = 0; t < seg_len[b] && t < S_max; ++t) {
                    Kr[n] = K + t * d;
                    Vr[n] = V + t * d;
                    where[n++] = k * T + t;
                }
            }
            double* o = out + (b * Hq + h) * d;
            for (int64_t i = 0; i < d; ++i) o[i] = 0.0;
            if (n == 0) {
#pragma omp atomic write
                status = -3;
            } else {
                double m = -INFINITY;
                for (int64_t e = 0; e < n; ++e) {
                    double dot = 0.0;
                    for (int64_t i = 0; i < d; ++i) dot += bf16_to_double(qh[i]) * bf16_to_double(Kr[e][i]);
                    z[e] = dot * sm_scale;
                    if (z[e] > m) m = z[e];
                }
                double l = 0.0;
                for (int64_t e = 0; e < n; ++e) {
                    z[e] = exp(z[e] - m); /* z now holds the unnormalised weight */
                    l += z[e];
                }
                for (int64_t e = 0; e < n; ++e)
                    for (int64_t i = 0; i < d; ++i) o[i] += z[e] * bf16_to_double(Vr[e][i]);
                for (int64_t i = 0; i < d; ++i) o[i] /= l;
                if (weights) {
                    double* wrow = weights + (b * Hq + h) * n_slot;
                    for (int64_t e = 0; e < n_slot; ++e) wrow[e] = 0.0;
                    for (int64_t e = 0; e < n; ++e) wrow[where[e]] += z[e] / l;
                }
            }
            free(Kr);
            free(Vr);
            free(where);
            free(z);
        }
    return status;
}

/* 5. Host-tier fetch: pool[b][slots[b][j]] := host[b][chunk_ids[b][j]]
 *    (whole chunk: K and V of every KV head).  slots == NULL means slot j. */
int oracle_fetch_chunks(const uint16_t* host_kv, int64_t C, const int32_t* chunk_ids, const int32_t* slots,
                        uint16_t* pool_kv, int64_t P, int64_t B, int64_t Hkv, int64_t d, int64_t k, int64_t T) {
    const int64_t chunk = 2 * Hkv * T * d;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < k; ++j) {
            const int64_t c = chunk_ids[b * k + j];
            const int64_t p = slots ? slots[b * k + j] : j;
            if (c < 0 || c >= C || p < 0 || p >= P) return -1;
            memcpy(pool_kv + (b * P + p) * chunk, host_kv + (b * C + c) * chunk, sizeof(uint16_t) * (size_t)chunk);
        }
    return 0;
}

/* 6. Delta-fetch slots.  For each request: chunk new_ids[j] found among
 *    prev_ids keeps that entry's slot (fetch_slots[j] = -1); otherwise it
 *    takes the next slot, in ascending order, held by no entry of the
 *    previous selection (fetch_slots[j] = that slot).  new_ids is walked in
 *    the order given (ascending for selections).  An entry with a negative
 *    chunk id is not in use (the -1 padding of a threshold selection past its
 *    count): in prev_ids it holds no slot, and in new_ids it gets
 *    new_slots[j] = fetch_slots[j] = -1.
 *    Returns 0; -1 for a previous slot outside [0, P); -2 if the free slots
 *    run out. */
int oracle_pool_assign(const int32_t* prev_ids, const int32_t* prev_slots, int64_t n_prev, const int32_t* new_ids,
                       int64_t B, int64_t k, int64_t P, int32_t* new_slots, int32_t* fetch_slots) {
    unsigned char* held = (unsigned char*)malloc((size_t)P);
    int rc = 0;
    for (int64_t b = 0; b < B && rc == 0; ++b) {
        memset(held, 0, (size_t)P);
        for (int64_t j = 0; j < n_prev; ++j) {
            if (prev_ids[b * n_prev + j] < 0) continue; /* not in use */
            const int64_t sl = prev_slots[b * n_prev + j];
            if (sl < 0 || sl >= P) { rc = -1; break; }
            held[sl] = 1;
        }
        int64_t next = 0;
        for (int64_t j = 0; j < k && rc == 0; ++j) {
            const int32_t c = new_ids[b * k + j];
            if (c < 0) { /* not in use */
                new_slots[b * k + j] = -1;
                fetch_slots[b * k + j] = -1;
                continue;
            }
            int64_t found = -1;
            for (int64_t q = 0; q < n_prev; ++q)
                if (prev_ids[b * n_prev + q] == c) { found = q; break; }
            if (found >= 0) {
                new_slots[b * k + j] = prev_slots[b * n_prev + found];
                fetch_slots[b * k + j] = -1;
            } else {
                while (next < P && held[next]) ++next;
                if (next >= P) { rc = -2; break; }
                new_slots[b * k + j] = (int32_t)next;
                fetch_slots[b * k + j] = (int32_t)next;
                ++next;
            }
        }
    }
    free(held);
    return rc;
}

/* 7. Threshold selection: in row r, count the keys above thr; keep
 *    kk = min(count, k_max) chunks, those that fewer than kk chunks precede
 *    in the order of item 3 (they are exactly the keys above thr when
 *    count <= k_max).  Ascending ids, then -1 up to k_max; counts[r] = kk. */
int oracle_threshold_i64(const int64_t* keys, int64_t R, int64_t C, int64_t thr, int64_t k_max, int32_t* ids,
                         int32_t* counts) {
    if (k_max < 1 || k_max > C) return -1;
    unsigned char* keep = (unsigned char*)malloc((size_t)C);
    int status = 0;
    for (int64_t r = 0; r < R && status == 0; ++r) {
        const int64_t* row = keys + r * C;
        int64_t above = 0;
        for (int64_t c = 0; c < C; ++c) above += row[c] > thr;
        const int64_t kk = above < k_max ? above : k_max;
        /* ranks counted in parallel iterations, as in item 3 */
#pragma omp parallel for schedule(dynamic, 64)
        for (int64_t c = 0; c < C; ++c) {
            int64_t before = 0;
            for (int64_t c2 = 0; c2 < C; ++c2)
                if (row[c2] > row[c] || (row[c2] == row[c] && c2 < c)) ++before;
            keep[c] = before < kk;
        }
        int64_t n_out = 0;
        for (int64_t c = 0; c < C; ++c) n_out += keep[c];
        if (n_out != kk) status = -2;
        n_out = 0;
        for (int64_t c = 0; c < C && status == 0; ++c)
            if (keep[c]) ids[r * k_max + n_out++] = (int32_t)c;
        if (status == 0) {
            for (int64_t j = n_out; j < k_max; ++j) ids[r * k_max + j] = -1;
            counts[r] = (int32_t)kk;
        }
    }
    free(keep);
    return status;
}

/* 8. Token selection inside the recalled chunks.  List position p = j*T + t
 *    (token t of list entry j) is usable iff j < counts[b] (all k entries
 *    when counts is NULL) and chunk_ids[b][j]*T + t < ctx_len[b].  Among the
 *    usable positions, p precedes p' when score[p] > score[p'] (compared as
 *    values: -0 equals +0), or the scores are equal and p < p'.  With
 *    kt = min(k_tok, number usable), position p is kept iff fewer than kt
 *    usable positions precede it.  tok[b] receives the kept positions in
 *    ascending order, then -1 up to k_tok; tok_counts[b] = kt.
 *    scores float [B][k*T].  Returns 0; -1 on bad sizes or a NaN score. */
int oracle_topk_tokens(const float* scores, const int32_t* chunk_ids, const int32_t* counts, const int32_t* ctx_len,
                       int64_t B, int64_t k, int64_t T, int64_t k_tok, int32_t* tok, int32_t* tok_counts) {
    if (B < 1 || k < 1 || T < 1 || k_tok < 1) return -1;
    const int64_t n = k * T;
    int status = 0;
    unsigned char* usable = (unsigned char*)malloc((size_t)n);
    unsigned char* keep = (unsigned char*)malloc((size_t)n);
    for (int64_t b = 0; b < B; ++b) {
        const float* row = scores + b * n;
        const int64_t kb = counts ? (counts[b] < 0 ? 0 : counts[b] < k ? counts[b] : k) : k;
        int64_t n_use = 0;
        for (int64_t p = 0; p < n; ++p) {
            const int64_t j = p / T, t = p % T;
            usable[p] = j < kb && (int64_t)chunk_ids[b * k + j] * T + t < (int64_t)ctx_len[b];
            if (usable[p] && isnan(row[p])) status = -1;
            n_use += usable[p];
        }
        const int64_t kt = k_tok < n_use ? k_tok : n_use;
        /* each usable position's rank is counted on its own, so the counts
         * run in parallel; the kept positions are then listed in order */
#pragma omp parallel for schedule(dynamic, 64)
        for (int64_t p = 0; p < n; ++p) {
            int64_t before = 0;
            if (usable[p])
                for (int64_t p2 = 0; p2 < n; ++p2)
                    if (usable[p2] && (row[p2] > row[p] || (row[p2] == row[p] && p2 < p))) ++before;
            keep[p] = usable[p] && before < kt;
        }
        int64_t n_out = 0;
        for (int64_t p = 0; p < n; ++p)  /* at most kt, unless a NaN broke the order */
            if (keep[p] && n_out < k_tok) tok[b * k_tok + n_out++] = (int32_t)p;
        for (int64_t u = n_out; u < k_tok; ++u) tok[b * k_tok + u] = -1;
        tok_counts[b] = (int32_t)n_out;
    }
    free(usable);
    free(keep);
    return status;
}
