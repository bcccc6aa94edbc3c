/*
 * Runs every function of the CPU oracle (oracle/lsa_oracle.c) and of the
 * seeded input generator (synth/synth.c) on small inputs that reach their
 * edge cases, built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py: an out-of-bounds access, a use of freed memory,
 * a signed overflow or a misaligned access in either aborts the program.
 * A few invariants are checked on the way, so that a run that merely does
 * not crash does not pass.  Prints "sanitize_oracle: ok" at the end.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle */
void oracle_index_logits(const int8_t*, const int8_t*, int64_t, int64_t, int64_t, int64_t, int64_t*);
void oracle_index_scores(const int64_t*, int64_t, float, double*);
int oracle_topk_i64(const int64_t*, int64_t, int64_t, int64_t, int32_t*);
int oracle_topk_f64(const double*, int64_t, int64_t, int64_t, int32_t*);
int oracle_gather_attend(const uint16_t*, const uint16_t*, int64_t, const int32_t*, const int32_t*, const int32_t*,
                         const int32_t*, const uint16_t*, const int32_t*, int64_t, int64_t, int64_t, int64_t, int64_t,
                         int64_t, int64_t, double, double*, double*, const int32_t*, const int32_t*, int64_t);
int oracle_fetch_chunks(const uint16_t*, int64_t, const int32_t*, const int32_t*, uint16_t*, int64_t, int64_t, int64_t,
                        int64_t, int64_t, int64_t);
int oracle_pool_assign(const int32_t*, const int32_t*, int64_t, const int32_t*, int64_t, int64_t, int64_t, int32_t*,
                       int32_t*);
int oracle_threshold_i64(const int64_t*, int64_t, int64_t, int64_t, int64_t, int32_t*, int32_t*);
int oracle_topk_tokens(const float*, const int32_t*, const int32_t*, const int32_t*, int64_t, int64_t, int64_t, int64_t,
                       int32_t*, int32_t*);
/* generator */
uint64_t synth_key(uint64_t, uint64_t);
uint64_t synth_draw(uint64_t, uint64_t);
void synth_fill_i8(int8_t*, int64_t, uint64_t, int64_t, int32_t, int32_t);
void synth_fill_i32(int32_t*, int64_t, uint64_t, int64_t, int32_t, int32_t);
void synth_fill_u64(uint64_t*, int64_t, uint64_t, int64_t);
void synth_fill_normal_bf16(uint16_t*, int64_t, uint64_t, int64_t, double);
void synth_fill_normal_bf16_runs(uint16_t*, const int64_t*, int64_t, int64_t, uint64_t, double);
int64_t synth_choose(int32_t*, int64_t, int64_t, const uint8_t*, uint64_t, int32_t*);

static int failures = 0;
#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

/* heap copies of exactly the needed size, so that ASan sees every overrun */
static void* dup_bytes(const void* p, size_t n) {
    void* q = malloc(n ? n : 1);
    memcpy(q, p, n);
    return q;
}

static void generator(void) {
    const uint64_t key = synth_key(0, 7);
    CHECK(synth_draw(key, 0) != synth_draw(key, 1));
    int8_t* i8 = malloc(1000);
    synth_fill_i8(i8, 1000, key, 0, -128, 127);
    synth_fill_i8(i8, 1000, key, 123456789, -16, 15);
    for (int i = 0; i < 1000; ++i) CHECK(i8[i] >= -16 && i8[i] <= 15);
    synth_fill_i8(i8, 1, key, 0, 5, 5);
    CHECK(i8[0] == 5);
    free(i8);
    int32_t* i32 = malloc(4 * 333);
    synth_fill_i32(i32, 333, key, 5, INT32_MIN, INT32_MAX);
    synth_fill_i32(i32, 333, key, 5, -3, 3);
    for (int i = 0; i < 333; ++i) CHECK(i32[i] >= -3 && i32[i] <= 3);
    free(i32);
    uint64_t* u64 = malloc(8 * 17);
    synth_fill_u64(u64, 17, key, 0);
    free(u64);
    uint16_t* bf = malloc(2 * 1001);
    synth_fill_normal_bf16(bf, 1001, key, 0, 1.0);
    synth_fill_normal_bf16(bf, 1001, key, 3, 8.0);
    int64_t firsts[3] = {0, 5000, 77};
    uint16_t* runs = malloc(2 * 3 * 64);
    synth_fill_normal_bf16_runs(runs, firsts, 3, 64, key, 1.0);
    synth_fill_normal_bf16(bf, 64, key, 5000, 1.0);
    CHECK(memcmp(bf, runs + 64, 2 * 64) == 0); /* a run equals the stream at its offset */
    free(runs);
    free(bf);
    /* partial Fisher-Yates: distinct draws, with and without exclusions */
    int32_t* out = malloc(4 * 50);
    int32_t* work = malloc(4 * 200);
    uint8_t* excl = calloc(200, 1);
    for (int i = 0; i < 200; i += 3) excl[i] = 1;
    int64_t got = synth_choose(out, 50, 200, excl, key, work);
    CHECK(got == 50);
    for (int i = 0; i < 50; ++i) {
        CHECK(out[i] >= 0 && out[i] < 200 && !excl[out[i]]);
        for (int j = 0; j < i; ++j) CHECK(out[i] != out[j]);
    }
    got = synth_choose(out, 50, 50, NULL, key, work);
    CHECK(got == 50);
    free(excl);
    free(work);
    free(out);
}

static void scan_and_select(void) {
    enum { B = 2, NQ = 3, C = 5, D = 16 };
    int8_t q[B * NQ * D], k[B * C * D];
    for (int i = 0; i < B * NQ * D; ++i) q[i] = (int8_t)(i % 2 ? -128 : 127);
    for (int i = 0; i < B * C * D; ++i) k[i] = (int8_t)((i * 7) % 256 - 128);
    int8_t* qh = dup_bytes(q, sizeof q);
    int8_t* kh = dup_bytes(k, sizeof k);
    int64_t* logits = malloc(sizeof(int64_t) * B * NQ * C);
    oracle_index_logits(qh, kh, B, NQ, C, D, logits);
    double* sc = malloc(sizeof(double) * B * NQ * C);
    oracle_index_scores(logits, B * NQ * C, 1.0f / 256, sc);
    for (int i = 0; i < B * NQ * C; ++i) CHECK(sc[i] >= 0.0 && sc[i] <= 1.0);
    int64_t zero = 0;
    double s0;
    oracle_index_scores(&zero, 1, 0.5f, &s0);
    CHECK(s0 == 0.5);
    /* top-k: k = 1 and k = C, all-equal keys, rejection of k out of range */
    int32_t* ids = malloc(sizeof(int32_t) * B * NQ * C);
    CHECK(oracle_topk_i64(logits, B * NQ, C, 1, ids) == 0);
    CHECK(oracle_topk_i64(logits, B * NQ, C, C, ids) == 0);
    for (int r = 0; r < B * NQ; ++r)
        for (int c = 0; c < C; ++c) CHECK(ids[r * C + c] == c);
    CHECK(oracle_topk_i64(logits, B * NQ, C, 0, ids) == -1);
    CHECK(oracle_topk_i64(logits, B * NQ, C, C + 1, ids) == -1);
    int64_t eq[7] = {3, 3, 3, 3, 3, 3, 3};
    int64_t* eqh = dup_bytes(eq, sizeof eq);
    CHECK(oracle_topk_i64(eqh, 1, 7, 4, ids) == 0);
    for (int j = 0; j < 4; ++j) CHECK(ids[j] == j); /* ties go to the lower index */
    CHECK(oracle_topk_f64(sc, B * NQ, C, 2, ids) == 0);
    /* threshold: none above, all above, capped */
    int32_t* cnt = malloc(sizeof(int32_t) * B * NQ);
    CHECK(oracle_threshold_i64(logits, B * NQ, C, INT64_MAX, C, ids, cnt) == 0);
    for (int r = 0; r < B * NQ; ++r) CHECK(cnt[r] == 0 && ids[r * C] == -1);
    CHECK(oracle_threshold_i64(logits, B * NQ, C, INT64_MIN, 2, ids, cnt) == 0);
    for (int r = 0; r < B * NQ; ++r) CHECK(cnt[r] == 2);
    CHECK(oracle_threshold_i64(logits, B * NQ, C, 0, 0, ids, cnt) == -1);
    free(cnt);
    free(eqh);
    free(ids);
    free(sc);
    free(logits);
    free(kh);
    free(qh);
}

static void attention_and_tokens(void) {
    enum { B = 2, HQ = 6, HKV = 2, D = 8, T = 4, CS = 5, K = 3, S = 8 };
    const int64_t chunk = 2 * HKV * T * D;
    uint16_t* q = malloc(2 * B * HQ * D);
    uint16_t* kv = malloc(2 * B * CS * chunk);
    uint16_t* seg = malloc(2 * B * 2 * HKV * S * D);
    synth_fill_normal_bf16(q, B * HQ * D, synth_key(1, 1), 0, 1.0);
    synth_fill_normal_bf16(kv, B * CS * chunk, synth_key(1, 2), 0, 1.0);
    synth_fill_normal_bf16(seg, B * 2 * HKV * S * D, synth_key(1, 3), 0, 1.0);
    int32_t ids_s[B * K] = {0, 2, 4, 1, 3, 4};
    int32_t slots_s[B * K] = {4, 0, 2, 1, 3, 0};
    int32_t ctx_s[B] = {4 * T + 1, 3 * T + 2}; /* partial last chunks */
    int32_t counts_s[B] = {3, 2};
    int32_t seg_len_s[B] = {S, 3};
    int32_t* ids = dup_bytes(ids_s, sizeof ids_s);
    int32_t* slots = dup_bytes(slots_s, sizeof slots_s);
    int32_t* ctx = dup_bytes(ctx_s, sizeof ctx_s);
    int32_t* counts = dup_bytes(counts_s, sizeof counts_s);
    int32_t* seg_len = dup_bytes(seg_len_s, sizeof seg_len_s);
    double* out = malloc(sizeof(double) * B * HQ * D);
    double* w = malloc(sizeof(double) * B * HQ * (K * T + S));
    CHECK(oracle_gather_attend(q, kv, CS, ids, NULL, NULL, ctx, NULL, NULL, 0, B, HQ, HKV, D, K, T, 0.35, out, w, NULL,
                               NULL, 0) == 0);
    CHECK(oracle_gather_attend(q, kv, CS, ids, slots, counts, ctx, seg, seg_len, S, B, HQ, HKV, D, K, T, 0.35, out, w,
                               NULL, NULL, 0) == 0);
    for (int bh = 0; bh < B * HQ; ++bh) {
        double sum = 0.0;
        for (int e = 0; e < K * T + S; ++e) sum += w[bh * (K * T + S) + e];
        CHECK(fabs(sum - 1.0) < 1e-12); /* softmax weights sum to one */
    }
    /* token lists: unsorted, -1, positions of unused entries and past the
       context, a repeat; counts cut the list */
    enum { KT = 9 };
    int32_t tok_s[B * KT] = {5, -1, 11, 0, 0, 12 * T, 3, 7, 2, 1, 2, 3, 4, 9, 100, -5, 8, 6};
    int32_t tok_counts_s[B] = {KT, 5};
    int32_t* tok = dup_bytes(tok_s, sizeof tok_s);
    int32_t* tok_counts = dup_bytes(tok_counts_s, sizeof tok_counts_s);
    CHECK(oracle_gather_attend(q, kv, CS, ids, slots, counts, ctx, NULL, NULL, 0, B, HQ, HKV, D, K, T, 0.35, out, w, tok,
                               tok_counts, KT) == 0);
    /* a request with no usable token is reported */
    int32_t zero_ctx_s[B] = {0, 0};
    int32_t* zero_ctx = dup_bytes(zero_ctx_s, sizeof zero_ctx_s);
    CHECK(oracle_gather_attend(q, kv, CS, ids, NULL, NULL, zero_ctx, NULL, NULL, 0, B, HQ, HKV, D, K, T, 0.35, out,
                               NULL, NULL, NULL, 0) == -3);
    CHECK(oracle_gather_attend(q, kv, CS, ids, NULL, NULL, ctx, NULL, NULL, 0, B, 5, HKV, D, K, T, 0.35, out, NULL,
                               NULL, NULL, 0) == -1); /* Hq not a multiple of Hkv */
    /* token selection: ragged counts, partial context, k_tok above the usable count */
    float* scores = malloc(sizeof(float) * B * K * T);
    for (int i = 0; i < B * K * T; ++i) scores[i] = (float)((i * 37) % 11) * 0.25f - 1.0f;
    scores[3] = -0.0f;
    scores[4] = 0.0f;
    scores[5] = INFINITY;
    int32_t* sel = malloc(sizeof(int32_t) * B * 50);
    int32_t* sel_n = malloc(sizeof(int32_t) * B);
    CHECK(oracle_topk_tokens(scores, ids, counts, ctx, B, K, T, 50, sel, sel_n) == 0);
    for (int b = 0; b < B; ++b) {
        for (int u = 1; u < sel_n[b]; ++u) CHECK(sel[b * 50 + u] > sel[b * 50 + u - 1]);
        for (int u = sel_n[b]; u < 50; ++u) CHECK(sel[b * 50 + u] == -1);
    }
    CHECK(oracle_topk_tokens(scores, ids, NULL, ctx, B, K, T, 1, sel, sel_n) == 0);
    scores[0] = NAN;
    CHECK(oracle_topk_tokens(scores, ids, NULL, ctx, B, K, T, 3, sel, sel_n) == -1);
    free(sel_n);
    free(sel);
    free(scores);
    free(zero_ctx);
    free(tok_counts);
    free(tok);
    free(w);
    free(out);
    free(seg_len);
    free(counts);
    free(ctx);
    free(slots);
    free(ids);
    free(seg);
    free(kv);
    free(q);
}

static void fetch_and_pool(void) {
    enum { B = 2, C = 6, P = 4, HKV = 1, D = 4, T = 2, K = 3 };
    const int64_t chunk = 2 * HKV * T * D;
    uint16_t* host = malloc(2 * B * C * chunk);
    uint16_t* pool = calloc(B * P * chunk, 2);
    for (int64_t i = 0; i < B * C * chunk; ++i) host[i] = (uint16_t)i;
    int32_t ids_s[B * K] = {0, 1, 5, 2, 3, 4};
    int32_t slots_s[B * K] = {3, 0, 1, 0, 1, 2};
    int32_t* ids = dup_bytes(ids_s, sizeof ids_s);
    int32_t* slots = dup_bytes(slots_s, sizeof slots_s);
    CHECK(oracle_fetch_chunks(host, C, ids, slots, pool, P, B, HKV, D, K, T) == 0);
    CHECK(memcmp(pool + (0 * P + 3) * chunk, host + (0 * C + 0) * chunk, 2 * chunk) == 0);
    CHECK(oracle_fetch_chunks(host, C, ids, NULL, pool, P, B, HKV, D, K, T) == 0);
    ids[4] = C; /* out of range: rejected, nothing read past the store */
    CHECK(oracle_fetch_chunks(host, C, ids, slots, pool, P, B, HKV, D, K, T) == -1);
    ids[4] = 3;
    slots[2] = P;
    CHECK(oracle_fetch_chunks(host, C, ids, slots, pool, P, B, HKV, D, K, T) == -1);
    /* pool slots: first selection, a delta, free slots running out, a bad previous slot */
    int32_t* ns = malloc(sizeof(int32_t) * B * K);
    int32_t* fs = malloc(sizeof(int32_t) * B * K);
    CHECK(oracle_pool_assign(NULL, NULL, 0, ids, B, K, 2 * K, ns, fs) == 0);
    int32_t prev_s[B * K] = {0, 1, 2, 2, 3, 9};
    int32_t prev_slots_s[B * K] = {0, 1, 2, 5, 4, 3};
    int32_t* prev = dup_bytes(prev_s, sizeof prev_s);
    int32_t* prev_slots = dup_bytes(prev_slots_s, sizeof prev_slots_s);
    CHECK(oracle_pool_assign(prev, prev_slots, K, ids, B, K, 2 * K, ns, fs) == 0);
    for (int e = 0; e < B * K; ++e) CHECK(fs[e] == -1 || fs[e] == ns[e]);
    CHECK(oracle_pool_assign(prev, prev_slots, K, ids, B, K, K, ns, fs) == -2);
    prev_slots[1] = 2 * K;
    CHECK(oracle_pool_assign(prev, prev_slots, K, ids, B, K, 2 * K, ns, fs) == -1);
    free(prev_slots);
    free(prev);
    free(fs);
    free(ns);
    free(slots);
    free(ids);
    free(pool);
    free(host);
}

int main(void) {
    generator();
    scan_and_select();
    attention_and_tokens();
    fetch_and_pool();
    if (failures) {
        fprintf(stderr, "sanitize_oracle: %d checks failed\n", failures);
        return 1;
    }
    printf("sanitize_oracle: ok\n");
    return 0;
}
