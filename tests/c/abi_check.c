/* Compiled as C11 against include/lsa.h and linked to liblsa.so by
 * tests/test_abi_c.py: the header is plain C, every entry point resolves at
 * link time, and rejected calls return their status before any HIP call
 * (so this runs without a GPU). */
#include <stdio.h>
#include <string.h>

#include "lsa.h"

static int expect(const char* what, lsa_status got, lsa_status want) {
    if (got != want) {
        printf("FAIL %s: %s (%s), wanted %s\n", what, lsa_status_string(got), lsa_last_error(),
               lsa_status_string(want));
        return 1;
    }
    return 0;
}

int main(void) {
    int bad = 0;
    void* bogus = (void*)(size_t)(1u << 20);
    int32_t ids[2] = {0, 5};
    bad += expect("index_score null", lsa_index_score(NULL, bogus, 1, 1, 4, 64, 1.0f, bogus, NULL, NULL),
                  LSA_ERR_INVALID_ARGUMENT);
    bad += expect("index_score d_idx", lsa_index_score(bogus, bogus, 1, 1, 4, 48, 1.0f, bogus, NULL, NULL),
                  LSA_ERR_UNSUPPORTED);
    bad += expect("topk k", lsa_topk_chunks(bogus, 1, 8, 9, bogus, NULL), LSA_ERR_INVALID_ARGUMENT);
    bad += expect("threshold k_max", lsa_threshold_chunks(bogus, 1, 8, 0, 0, bogus, bogus, NULL),
                  LSA_ERR_INVALID_ARGUMENT);
    bad += expect("attend heads", lsa_gather_attend(bogus, bogus, 4, bogus, NULL, NULL, bogus, NULL, NULL, 0, 1, 60, 8,
                                                    128, 2, 0.1f, NULL, 0, 1, bogus, NULL),
                  LSA_ERR_INVALID_ARGUMENT);
    bad += expect("attend workspace", lsa_gather_attend(bogus, bogus, 4, bogus, NULL, NULL, bogus, NULL, NULL, 0, 2, 64,
                                                        8, 128, 4, 0.1f, NULL, 0, 2, bogus, NULL),
                  LSA_ERR_WORKSPACE);
    bad += expect("fetch id", lsa_fetch_chunks(bogus, 4, ids, NULL, bogus, 2, 1, 1, 64, 2, NULL, NULL),
                  LSA_ERR_INVALID_ARGUMENT);
    bad += expect("fetch pull null", lsa_fetch_chunks_pull(NULL, 4, bogus, NULL, bogus, 2, 1, 1, 64, 2, 0, NULL),
                  LSA_ERR_INVALID_ARGUMENT);
    bad += expect("pool assign P", lsa_pool_assign(bogus, bogus, 4, bogus, 1, 4, 7, bogus, bogus, NULL),
                  LSA_ERR_INVALID_ARGUMENT);
    bad += expect("token top-k k", lsa_topk_tokens(bogus, bogus, NULL, bogus, 2, (1 << 24) + 1, 8, bogus, bogus,
                                                                   NULL, 0, NULL),
                  LSA_ERR_UNSUPPORTED);
    bad += expect("token attend tok", lsa_gather_attend_tokens(bogus, bogus, 4, bogus, NULL, NULL, bogus, NULL, NULL,
                                                               128, NULL, NULL, 0, 2, 64, 8, 128, 4, 0.1f, NULL, 0, 1,
                                                               bogus, NULL),
                  LSA_ERR_INVALID_ARGUMENT);
    bad += expect("token top-k workspace", lsa_topk_tokens(bogus, bogus, NULL, bogus, 4, 1638, 2048, bogus, bogus,
                                                             bogus, 64, NULL),
                  LSA_ERR_WORKSPACE);
    if (lsa_topk_tokens_workspace_size(4, 12, 500) != 0) { puts("FAIL token workspace size"); ++bad; }
    if (lsa_gather_attend_workspace_size(16, 64, 8, 128, 276, 1) != 0) { puts("FAIL workspace size"); ++bad; }
    if (lsa_gather_attend_default_splits(16, 8, 276) < 1) { puts("FAIL default splits"); ++bad; }
    if (strcmp(lsa_status_string(LSA_OK), "LSA_OK") != 0) { puts("FAIL status string"); ++bad; }
    printf(bad ? "abi_check: %d failures\n" : "abi_check: ok\n", bad);
    return bad != 0;
}
