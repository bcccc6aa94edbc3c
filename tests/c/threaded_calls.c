/* The library's threading promise, checked from plain C11 + pthreads: calls
 * may be issued from several host threads on different streams, and the
 * message behind lsa_last_error() belongs to the calling thread.
 *
 * The main thread first runs every problem once on its own stream (the
 * serial reference).  Then NT threads each take one problem and repeat
 * scan -> select -> attend on their own stream and workspace, comparing
 * every repetition's ids and output bit for bit with the reference (the
 * kernels are deterministic for fixed inputs and split count).  Thread 0
 * also makes a call the library must reject and checks that its own
 * message says why, while the other threads' messages stay empty after
 * their successful calls.
 *
 * Inputs come from a fixed linear congruential generator: no method
 * arithmetic is needed, only equality between runs.
 * usage: threaded_calls   (prints "threaded_calls: ok", exit status 0) */
#include <pthread.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lsa.h"

enum { NT = 4, REPS = 12, B = 2, C = 96, D_IDX = 128, K = 20, HQ = 64, HKV = 8, D = 128, N_SPLIT = 2 };

#define CHECK_HIP(x)                                                                          \
    do {                                                                                      \
        hipError_t e_ = (x);                                                                  \
        if (e_ != hipSuccess) {                                                               \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            exit(2);                                                                          \
        }                                                                                     \
    } while (0)

typedef struct {
    int8_t *q_idx, *k_idx;
    uint16_t *q, *kv;
    int32_t *ctx, *logits, *ids;
    float* out;
    void* ws;
    size_t ws_bytes;
    hipStream_t stream;
    int32_t ref_ids[B * K];
    float ref_out[B * HQ * D];
    int failures;
    char note[256];
} Problem;

static uint32_t lcg(uint32_t* s) {
    *s = *s * 1664525u + 1013904223u;
    return *s >> 8;
}

static void* dev_fill(size_t bytes, uint32_t seed, int kind) {
    unsigned char* h = malloc(bytes);
    if (!h) exit(4);
    uint32_t s = seed;
    if (kind == 0) { /* int8 in [-16, 15] */
        for (size_t i = 0; i < bytes; ++i) h[i] = (unsigned char)(int8_t)((int)(lcg(&s) % 32) - 16);
    } else { /* bf16 with exponents near 1: sign, 2^-2..2^1, random mantissa */
        uint16_t* v = (uint16_t*)h;
        for (size_t i = 0; i < bytes / 2; ++i) {
            const uint32_t r = lcg(&s);
            v[i] = (uint16_t)(((r & 1u) << 15) | ((125u + (r >> 1) % 4u) << 7) | ((r >> 3) & 0x7Fu));
        }
    }
    void* p = NULL;
    CHECK_HIP(hipMalloc(&p, bytes));
    CHECK_HIP(hipMemcpy(p, h, bytes, hipMemcpyHostToDevice));
    free(h);
    return p;
}

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    CHECK_HIP(hipMalloc(&p, bytes));
    return p;
}

/* scan -> select -> attend on the problem's stream; 0 on success */
static int run_once(Problem* p) {
    lsa_status s = lsa_index_score(p->q_idx, p->k_idx, B, 1, C, D_IDX, 1.0f / (16 * D_IDX), p->logits, NULL,
                                   p->stream);
    if (s == LSA_OK) s = lsa_topk_chunks(p->logits, B, C, K, p->ids, p->stream);
    if (s == LSA_OK)
        s = lsa_gather_attend(p->q, p->kv, C, p->ids, NULL, NULL, p->ctx, NULL, NULL, 0, B, HQ, HKV, D, K,
                              0.08838834764831845f, p->ws, p->ws_bytes, N_SPLIT, p->out, p->stream);
    if (s != LSA_OK) {
        snprintf(p->note, sizeof p->note, "%s: %s", lsa_status_string(s), lsa_last_error());
        return 1;
    }
    return 0;
}

static void* worker(void* arg) {
    Problem* p = arg;
    int32_t* ids = malloc(sizeof p->ref_ids);
    float* out = malloc(sizeof p->ref_out);
    if (!ids || !out) exit(4);
    for (int r = 0; r < REPS && !p->failures; ++r) {
        if (run_once(p)) {
            p->failures++;
            break;
        }
        CHECK_HIP(hipMemcpyAsync(ids, p->ids, sizeof p->ref_ids, hipMemcpyDeviceToHost, p->stream));
        CHECK_HIP(hipMemcpyAsync(out, p->out, sizeof p->ref_out, hipMemcpyDeviceToHost, p->stream));
        CHECK_HIP(hipStreamSynchronize(p->stream));
        if (memcmp(ids, p->ref_ids, sizeof p->ref_ids) || memcmp(out, p->ref_out, sizeof p->ref_out)) {
            snprintf(p->note, sizeof p->note, "repetition %d differs from the serial run", r);
            p->failures++;
        }
        if (lsa_last_error()[0] != '\0') {
            snprintf(p->note, sizeof p->note, "message after a successful call: %s", lsa_last_error());
            p->failures++;
        }
    }
    free(ids);
    free(out);
    return NULL;
}

static void* rejecting_worker(void* arg) {
    Problem* p = arg;
    /* k > C: rejected before any HIP call, with this thread's message */
    if (lsa_topk_chunks(p->logits, B, C, C + 1, p->ids, p->stream) != LSA_ERR_INVALID_ARGUMENT ||
        strstr(lsa_last_error(), "k=") == NULL) {
        snprintf(p->note, sizeof p->note, "rejected call: status or message wrong (%s)", lsa_last_error());
        p->failures++;
        return NULL;
    }
    return worker(arg);
}

int main(void) {
    static Problem pr[NT];
    const size_t ws_bytes = lsa_gather_attend_workspace_size(B, HQ, HKV, D, K, N_SPLIT);
    if (ws_bytes == (size_t)-1) {
        fprintf(stderr, "workspace query rejected the sizes\n");
        return 3;
    }
    int32_t ctx_h[B] = {C * 64, C * 64 - 29};
    for (int t = 0; t < NT; ++t) {
        Problem* p = &pr[t];
        p->q_idx = dev_fill((size_t)B * D_IDX, 11u + 7u * t, 0);
        p->k_idx = dev_fill((size_t)B * C * D_IDX, 101u + 7u * t, 0);
        p->q = dev_fill((size_t)B * HQ * D * 2, 1001u + 7u * t, 1);
        p->kv = dev_fill((size_t)B * C * 2 * HKV * 64 * D * 2, 10001u + 7u * t, 1);
        p->ctx = dev_alloc(sizeof ctx_h);
        CHECK_HIP(hipMemcpy(p->ctx, ctx_h, sizeof ctx_h, hipMemcpyHostToDevice));
        p->logits = dev_alloc((size_t)B * C * 4);
        p->ids = dev_alloc((size_t)B * K * 4);
        p->out = dev_alloc((size_t)B * HQ * D * 4);
        p->ws_bytes = ws_bytes;
        p->ws = ws_bytes ? dev_alloc(ws_bytes) : NULL;
        CHECK_HIP(hipStreamCreate(&p->stream));
        /* serial reference, one problem after another */
        if (run_once(p)) {
            fprintf(stderr, "serial run of problem %d failed: %s\n", t, p->note);
            return 3;
        }
        CHECK_HIP(hipMemcpyAsync(p->ref_ids, p->ids, sizeof p->ref_ids, hipMemcpyDeviceToHost, p->stream));
        CHECK_HIP(hipMemcpyAsync(p->ref_out, p->out, sizeof p->ref_out, hipMemcpyDeviceToHost, p->stream));
        CHECK_HIP(hipStreamSynchronize(p->stream));
    }
    pthread_t th[NT];
    for (int t = 0; t < NT; ++t)
        if (pthread_create(&th[t], NULL, t == 0 ? rejecting_worker : worker, &pr[t]) != 0) {
            fprintf(stderr, "pthread_create failed\n");
            return 5;
        }
    for (int t = 0; t < NT; ++t) pthread_join(th[t], NULL);
    int bad = 0;
    for (int t = 0; t < NT; ++t) {
        if (pr[t].failures) {
            printf("FAIL thread %d: %s\n", t, pr[t].note);
            bad = 1;
        }
        CHECK_HIP(hipStreamDestroy(pr[t].stream));
        CHECK_HIP(hipFree(pr[t].q_idx));
        CHECK_HIP(hipFree(pr[t].k_idx));
        CHECK_HIP(hipFree(pr[t].q));
        CHECK_HIP(hipFree(pr[t].kv));
        CHECK_HIP(hipFree(pr[t].ctx));
        CHECK_HIP(hipFree(pr[t].logits));
        CHECK_HIP(hipFree(pr[t].ids));
        CHECK_HIP(hipFree(pr[t].out));
        if (pr[t].ws) CHECK_HIP(hipFree(pr[t].ws));
    }
    if (bad) return 1;
    printf("threaded_calls: ok (%d threads x %d repetitions)\n", NT, REPS);
    return 0;
}
