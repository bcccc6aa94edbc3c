/* Two re-selection intervals of the decode path, driven from plain C11
 * through include/lsa.h with device memory from the HIP runtime and nothing
 * else: no PyTorch, no Python.  tests/test_gpu_c_client.py writes the inputs,
 * runs this program and checks every file it writes against the oracle.
 *
 * Per interval i (0, then 1), all on one compute stream unless noted:
 *   lsa_index_score      scan of the indexer keys with query i
 *   lsa_topk_chunks      the k kept chunks
 *   lsa_pool_assign      pool slots against interval i-1's chunks (none at 0)
 *   lsa_fetch_chunks_pull  copy of the new chunks only, from pinned host
 *                        memory, on a side stream the compute stream waits on
 *   lsa_gather_attend    attention of step query i over the pool
 * Then interval 0 again with the DMA fetch: the ids go back to the host,
 * lsa_fetch_chunks copies every kept chunk into a second pool (slot j for
 * entry j), and lsa_gather_attend attends over it.
 *
 * usage: decode_interval DIR B C d_idx k Hq Hkv d alpha sm_scale
 * reads  DIR/q_idx.bin  int8   [2][B][d_idx]   indexer query per interval
 *        DIR/k_idx.bin  int8   [B][C][d_idx]
 *        DIR/q.bin      bf16   [2][B][Hq][d]   step query per interval
 *        DIR/kv.bin     bf16   [B][C][2][Hkv][64][d]
 *        DIR/ctx.bin    int32  [B]
 * writes DIR/{logits,scores,ids,slots,fslots,out}{0,1}.bin, DIR/out0_dma.bin
 *        and DIR/pool.bin (bf16 [B][2k][2][Hkv][64][d], after interval 1).
 * Exit status 0 on success; any failed call prints its message and exits
 * with 2 (HIP) or 3 (library). */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lsa.h"

#define CHECK_HIP(x)                                                                                 \
    do {                                                                                             \
        hipError_t e_ = (x);                                                                         \
        if (e_ != hipSuccess) {                                                                      \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_));        \
            exit(2);                                                                                 \
        }                                                                                            \
    } while (0)

#define CHECK_LSA(x)                                                                                 \
    do {                                                                                             \
        lsa_status s_ = (x);                                                                         \
        if (s_ != LSA_OK) {                                                                          \
            fprintf(stderr, "%s:%d %s: %s (%s)\n", __FILE__, __LINE__, #x, lsa_status_string(s_),   \
                    lsa_last_error());                                                               \
            exit(3);                                                                                 \
        }                                                                                            \
    } while (0)

static const char* g_dir;

static FILE* open_in_dir(const char* name, const char* mode) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    FILE* f = fopen(path, mode);
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        exit(4);
    }
    return f;
}

static void read_all(const char* name, void* dst, size_t bytes) {
    FILE* f = open_in_dir(name, "rb");
    if (fread(dst, 1, bytes, f) != bytes || fgetc(f) != EOF) {
        fprintf(stderr, "%s does not hold exactly %zu bytes\n", name, bytes);
        exit(4);
    }
    fclose(f);
}

/* Copies `bytes` of device memory at `src` to DIR/name. */
static void write_device(const char* name, const void* src, size_t bytes) {
    void* h = malloc(bytes);
    if (!h) {
        fprintf(stderr, "out of host memory\n");
        exit(4);
    }
    CHECK_HIP(hipMemcpy(h, src, bytes, hipMemcpyDeviceToHost));
    FILE* f = open_in_dir(name, "wb");
    if (fwrite(h, 1, bytes, f) != bytes) {
        fprintf(stderr, "short write of %s\n", name);
        exit(4);
    }
    fclose(f);
    free(h);
}

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    CHECK_HIP(hipMalloc(&p, bytes ? bytes : 1));
    return p;
}

/* Host bytes -> new device buffer. */
static void* dev_upload(const void* src, size_t bytes) {
    void* p = dev_alloc(bytes);
    CHECK_HIP(hipMemcpy(p, src, bytes, hipMemcpyHostToDevice));
    return p;
}

int main(int argc, char** argv) {
    if (argc != 11) {
        fprintf(stderr, "usage: %s DIR B C d_idx k Hq Hkv d alpha sm_scale\n", argv[0]);
        return 1;
    }
    g_dir = argv[1];
    const int32_t B = atoi(argv[2]), C = atoi(argv[3]), d_idx = atoi(argv[4]), k = atoi(argv[5]);
    const int32_t Hq = atoi(argv[6]), Hkv = atoi(argv[7]), d = atoi(argv[8]);
    const float alpha = strtof(argv[9], NULL), sm_scale = strtof(argv[10], NULL);
    if (B < 1 || C < 1 || d_idx < 1 || k < 1 || k > C || Hq < 1 || Hkv < 1 || d < 1) {
        fprintf(stderr, "bad sizes\n");
        return 1;
    }
    const int64_t P = 2 * (int64_t)k; /* room for both intervals' chunks */
    const size_t n_qidx = (size_t)B * d_idx, n_kidx = (size_t)B * C * d_idx, n_q = (size_t)B * Hq * d;
    const size_t chunk_elems = (size_t)2 * Hkv * LSA_CHUNK_TOKENS * d;
    const size_t n_sel = (size_t)B * k;

    /* inputs */
    int8_t* h_qidx = malloc(2 * n_qidx);
    int8_t* h_kidx = malloc(n_kidx);
    uint16_t* h_q = malloc(2 * n_q * sizeof(uint16_t));
    int32_t* h_ctx = malloc(B * sizeof(int32_t));
    int32_t* h_ident = malloc(n_sel * sizeof(int32_t));
    int32_t* h_ids = malloc(n_sel * sizeof(int32_t));
    if (!h_qidx || !h_kidx || !h_q || !h_ctx || !h_ident || !h_ids) {
        fprintf(stderr, "out of host memory\n");
        return 4;
    }
    read_all("q_idx.bin", h_qidx, 2 * n_qidx);
    read_all("k_idx.bin", h_kidx, n_kidx);
    read_all("q.bin", h_q, 2 * n_q * sizeof(uint16_t));
    read_all("ctx.bin", h_ctx, B * sizeof(int32_t));
    uint16_t* host_kv = NULL; /* the host tier: pinned and mapped for the pull fetch */
    CHECK_HIP(hipHostMalloc((void**)&host_kv, (size_t)B * C * chunk_elems * sizeof(uint16_t), hipHostMallocMapped));
    read_all("kv.bin", host_kv, (size_t)B * C * chunk_elems * sizeof(uint16_t));
    for (size_t e = 0; e < n_sel; ++e) h_ident[e] = (int32_t)(e % (size_t)k);

    int8_t* d_kidx = dev_upload(h_kidx, n_kidx);
    int32_t* d_ctx = dev_upload(h_ctx, B * sizeof(int32_t));
    int32_t* d_ident = dev_upload(h_ident, n_sel * sizeof(int32_t));
    int8_t* d_qidx[2];
    uint16_t* d_q[2];
    int32_t *d_logits[2], *d_ids[2], *d_slots[2], *d_fslots[2];
    float *d_scores[2], *d_out[2];
    for (int i = 0; i < 2; ++i) {
        d_qidx[i] = dev_upload(h_qidx + i * n_qidx, n_qidx);
        d_q[i] = dev_upload(h_q + i * n_q, n_q * sizeof(uint16_t));
        d_logits[i] = dev_alloc((size_t)B * C * sizeof(int32_t));
        d_scores[i] = dev_alloc((size_t)B * C * sizeof(float));
        d_ids[i] = dev_alloc(n_sel * sizeof(int32_t));
        d_slots[i] = dev_alloc(n_sel * sizeof(int32_t));
        d_fslots[i] = dev_alloc(n_sel * sizeof(int32_t));
        d_out[i] = dev_alloc(n_q * sizeof(float));
    }
    uint16_t* d_pool = dev_alloc((size_t)B * P * chunk_elems * sizeof(uint16_t));
    uint16_t* d_pool_dma = dev_alloc((size_t)B * k * chunk_elems * sizeof(uint16_t));
    float* d_out_dma = dev_alloc(n_q * sizeof(float));
    const size_t ws_bytes = lsa_gather_attend_workspace_size(B, Hq, Hkv, d, k, 0);
    if (ws_bytes == (size_t)-1) {
        fprintf(stderr, "workspace query rejected the sizes: %s\n", lsa_last_error());
        return 3;
    }
    void* ws = ws_bytes ? dev_alloc(ws_bytes) : NULL;

    hipStream_t s, side;
    hipEvent_t selected, fetched;
    CHECK_HIP(hipStreamCreate(&s));
    CHECK_HIP(hipStreamCreate(&side));
    CHECK_HIP(hipEventCreateWithFlags(&selected, hipEventDisableTiming));
    CHECK_HIP(hipEventCreateWithFlags(&fetched, hipEventDisableTiming));

    for (int i = 0; i < 2; ++i) {
        CHECK_LSA(lsa_index_score(d_qidx[i], d_kidx, B, 1, C, d_idx, alpha, d_logits[i], d_scores[i], s));
        CHECK_LSA(lsa_topk_chunks(d_logits[i], B, C, k, d_ids[i], s));
        CHECK_LSA(lsa_pool_assign(i ? d_ids[i - 1] : NULL, i ? d_slots[i - 1] : NULL, i ? k : 0, d_ids[i], B, k, P,
                                  d_slots[i], d_fslots[i], s));
        CHECK_HIP(hipEventRecord(selected, s));
        CHECK_HIP(hipStreamWaitEvent(side, selected, 0));
        CHECK_LSA(lsa_fetch_chunks_pull(host_kv, C, d_ids[i], d_fslots[i], d_pool, P, B, Hkv, d, k, 0, side));
        CHECK_HIP(hipEventRecord(fetched, side));
        CHECK_HIP(hipStreamWaitEvent(s, fetched, 0));
        CHECK_LSA(lsa_gather_attend(d_q[i], d_pool, P, d_ids[i], d_slots[i], NULL, d_ctx, NULL, NULL, 0, B, Hq, Hkv,
                                    d, k, sm_scale, ws, ws_bytes, 0, d_out[i], s));
    }

    /* interval 0 through the DMA fetch: host ids, slot j for entry j */
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(h_ids, d_ids[0], n_sel * sizeof(int32_t), hipMemcpyDeviceToHost));
    CHECK_LSA(lsa_fetch_chunks(host_kv, C, h_ids, NULL, d_pool_dma, k, B, Hkv, d, k, side, fetched));
    CHECK_HIP(hipStreamWaitEvent(s, fetched, 0));
    CHECK_LSA(lsa_gather_attend(d_q[0], d_pool_dma, k, d_ids[0], d_ident, NULL, d_ctx, NULL, NULL, 0, B, Hq, Hkv, d,
                                k, sm_scale, ws, ws_bytes, 0, d_out_dma, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipStreamSynchronize(side));

    static const char* digits[2] = {"0", "1"};
    for (int i = 0; i < 2; ++i) {
        char name[64];
        snprintf(name, sizeof name, "logits%s.bin", digits[i]);
        write_device(name, d_logits[i], (size_t)B * C * sizeof(int32_t));
        snprintf(name, sizeof name, "scores%s.bin", digits[i]);
        write_device(name, d_scores[i], (size_t)B * C * sizeof(float));
        snprintf(name, sizeof name, "ids%s.bin", digits[i]);
        write_device(name, d_ids[i], n_sel * sizeof(int32_t));
        snprintf(name, sizeof name, "slots%s.bin", digits[i]);
        write_device(name, d_slots[i], n_sel * sizeof(int32_t));
        snprintf(name, sizeof name, "fslots%s.bin", digits[i]);
        write_device(name, d_fslots[i], n_sel * sizeof(int32_t));
        snprintf(name, sizeof name, "out%s.bin", digits[i]);
        write_device(name, d_out[i], n_q * sizeof(float));
    }
    write_device("out0_dma.bin", d_out_dma, n_q * sizeof(float));
    write_device("pool.bin", d_pool, (size_t)B * P * chunk_elems * sizeof(uint16_t));

    CHECK_HIP(hipEventDestroy(selected));
    CHECK_HIP(hipEventDestroy(fetched));
    CHECK_HIP(hipStreamDestroy(s));
    CHECK_HIP(hipStreamDestroy(side));
    for (int i = 0; i < 2; ++i) {
        CHECK_HIP(hipFree(d_qidx[i]));
        CHECK_HIP(hipFree(d_q[i]));
        CHECK_HIP(hipFree(d_logits[i]));
        CHECK_HIP(hipFree(d_scores[i]));
        CHECK_HIP(hipFree(d_ids[i]));
        CHECK_HIP(hipFree(d_slots[i]));
        CHECK_HIP(hipFree(d_fslots[i]));
        CHECK_HIP(hipFree(d_out[i]));
    }
    CHECK_HIP(hipFree(d_kidx));
    CHECK_HIP(hipFree(d_ctx));
    CHECK_HIP(hipFree(d_ident));
    CHECK_HIP(hipFree(d_pool));
    CHECK_HIP(hipFree(d_pool_dma));
    CHECK_HIP(hipFree(d_out_dma));
    if (ws) CHECK_HIP(hipFree(ws));
    CHECK_HIP(hipHostFree(host_kv));
    free(h_qidx);
    free(h_kidx);
    free(h_q);
    free(h_ctx);
    free(h_ident);
    free(h_ids);
    printf("decode_interval: ok\n");
    return 0;
}
