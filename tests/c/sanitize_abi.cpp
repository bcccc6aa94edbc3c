// Host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_sanitizers.py builds it with the library's sources, the
// sanitizers on the host pass only).  No GPU is used: every entry point is
// called with arguments its validation rejects before any HIP call, the size
// queries run over extreme values (a signed overflow in them aborts the run),
// the tuning knobs are set and read, and the fetch's run coalescing is
// checked against a brute-force expansion on random id and slot lists.
// Prints "sanitize_abi: ok" at the end.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <random>
#include <vector>

#include "../../include/lsa.h"
#include "../../lookahead_chunk_sparse_amd/csrc/fetch_runs.h"

static int failures = 0;
#define CHECK(cond)                                                           \
    do {                                                                      \
        if (!(cond)) {                                                        \
            fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #cond, lsa_last_error()); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

// non-null, aligned addresses that the rejected calls never dereference
static void* const P = reinterpret_cast<void*>(uintptr_t(1) << 20);
static const int8_t* const I8 = static_cast<const int8_t*>(P);
static const uint16_t* const U16 = static_cast<const uint16_t*>(P);
static const int32_t* const CI32 = static_cast<const int32_t*>(P);
static int32_t* const I32 = static_cast<int32_t*>(P);
static float* const F32 = static_cast<float*>(P);

static void rejected_calls() {
    CHECK(lsa_index_score(nullptr, I8, 1, 1, 1, 64, 1.f, I32, F32, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_index_score(I8, I8, 1, 1, 1, 48, 1.f, I32, F32, nullptr) == LSA_ERR_UNSUPPORTED);
    CHECK(lsa_index_score(I8, I8, 65536, 65536, 2, 64, 1.f, I32, F32, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_index_score(I8, I8, 1, 1, 1, 64, __builtin_inff(), I32, F32, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_topk_chunks(CI32, 1, 10, 11, I32, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_topk_chunks(CI32, 1 << 22, 10, 1, I32, nullptr) == LSA_ERR_UNSUPPORTED);
    CHECK(lsa_topk_chunks(CI32, INT32_MAX, INT32_MAX, INT32_MAX, I32, nullptr) != LSA_OK);
    CHECK(lsa_threshold_chunks(CI32, 1, 10, 0, 0, I32, I32, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_topk_tokens(F32, CI32, nullptr, CI32, 1, (1 << 24) + 1, 10, I32, I32, nullptr, 0, nullptr) ==
          LSA_ERR_UNSUPPORTED);
    CHECK(lsa_topk_tokens(F32, CI32, nullptr, CI32, INT32_MAX, INT32_MAX / 64, INT32_MAX, I32, I32, nullptr, 0,
                          nullptr) != LSA_OK);
    CHECK(lsa_gather_attend(U16, U16, 10, CI32, nullptr, nullptr, CI32, nullptr, nullptr, 0, 2, 64, 7, 128, 4, 0.1f,
                            nullptr, 0, 0, F32, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_gather_attend(U16, U16, 10, CI32, nullptr, nullptr, CI32, nullptr, nullptr, 0, 2, 64, 8, 96, 4, 0.1f,
                            nullptr, 0, 0, F32, nullptr) == LSA_ERR_UNSUPPORTED);
    CHECK(lsa_gather_attend(U16, U16, 10, CI32, nullptr, nullptr, CI32, nullptr, nullptr, 0, 16, 64, 8, 128, 276, 0.1f,
                            nullptr, 0, 0, F32, nullptr) == LSA_ERR_WORKSPACE);
    CHECK(lsa_gather_attend(U16, U16, 10, CI32, nullptr, nullptr, CI32, U16, CI32, 65, 2, 64, 8, 128, 4, 0.1f, nullptr,
                            0, 1, F32, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_gather_attend(U16, U16, 10, CI32, nullptr, nullptr, CI32, nullptr, nullptr, 0, INT32_MAX, INT32_MAX, 1,
                            128, INT32_MAX, 0.1f, nullptr, 0, INT32_MAX, F32, nullptr) != LSA_OK);
    CHECK(lsa_gather_attend_tokens(U16, U16, 10, CI32, nullptr, nullptr, CI32, nullptr, nullptr, 5, nullptr, nullptr, 0,
                                   2, 64, 8, 128, 4, 0.1f, nullptr, 0, 1, F32, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_gather_attend_tokens(U16, U16, INT64_MAX / 4, CI32, nullptr, nullptr, CI32, CI32, nullptr, 5, nullptr,
                                   nullptr, 0, 2, 64, 8, 128, 4, 0.1f, nullptr, 0, 1, F32, nullptr) != LSA_OK);
    CHECK(lsa_gather_attend_noalloc(U16, U16, 100, CI32, nullptr, nullptr, CI32, nullptr, nullptr, 0, 64, 64, 8, 128,
                                    64, 0.1f, 16, F32, nullptr) == LSA_ERR_WORKSPACE);
    CHECK(lsa_pool_assign(CI32, CI32, 5, CI32, 2, 4, 8, I32, I32, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_pool_assign(CI32, CI32, 16000, CI32, 2, 4, 16004, I32, I32, nullptr) == LSA_ERR_UNSUPPORTED);
    CHECK(lsa_fetch_chunks_pull(U16, 10, CI32, nullptr, const_cast<uint16_t*>(U16), 4, 2, 8, 96, 4, 0, nullptr) ==
          LSA_ERR_UNSUPPORTED);
    // the DMA fetch checks every id and slot on the host before any copy
    std::vector<int32_t> ids = {0, 1, 2, 3, 4, 99}, slots = {0, 1, 2, 0, 1, 2};
    std::vector<uint16_t> host(16);
    uint16_t* pool = const_cast<uint16_t*>(U16);
    CHECK(lsa_fetch_chunks(host.data(), 10, ids.data(), slots.data(), pool, 3, 2, 1, 64, 3, nullptr, nullptr) ==
          LSA_ERR_INVALID_ARGUMENT);
    CHECK(strstr(lsa_last_error(), "99") != nullptr);
    ids[5] = 5;
    slots[4] = 3;  // a slot past the pool
    CHECK(lsa_fetch_chunks(host.data(), 10, ids.data(), slots.data(), pool, 3, 2, 1, 64, 3, nullptr, nullptr) ==
          LSA_ERR_INVALID_ARGUMENT);
    CHECK(strstr(lsa_last_error(), "slot 3") != nullptr);
    // a negative slot is not copied, so its id is not checked: the call gets as
    // far as the pinned-memory test, which this (pageable) buffer fails
    slots[4] = -1;
    ids[4] = 99;
    CHECK(lsa_fetch_chunks(host.data(), 10, ids.data(), slots.data(), pool, 3, 2, 1, 64, 3, nullptr, nullptr) ==
          LSA_ERR_INVALID_ARGUMENT);
    CHECK(strstr(lsa_last_error(), "99") == nullptr);
    CHECK(lsa_fetch_chunks(host.data(), 10, ids.data(), nullptr, pool, 2, 2, 1, 64, 3, nullptr, nullptr) ==
          LSA_ERR_INVALID_ARGUMENT);
    // the staged fetch: staging buffers required, at least 2 chunks of them,
    // the same id and slot checks, and pageable host memory refused
    uint16_t* stage = const_cast<uint16_t*>(U16);
    CHECK(lsa_fetch_chunks_staged(host.data(), 10, ids.data(), slots.data(), pool, 3, 2, 1, 64, 3, nullptr, stage, 4,
                                  nullptr, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_fetch_chunks_staged(host.data(), 10, ids.data(), slots.data(), pool, 3, 2, 1, 64, 3, stage, stage, 1,
                                  nullptr, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(strstr(lsa_last_error(), "stage_chunks") != nullptr);
    CHECK(lsa_fetch_chunks_staged(host.data(), 10, ids.data(), slots.data(), pool, 1 << 30, 4, 1, 64, 1, stage, stage,
                                  4, nullptr, nullptr) == LSA_ERR_UNSUPPORTED);
    ids[4] = 4;
    slots[4] = 3;  // a slot past the pool
    CHECK(lsa_fetch_chunks_staged(host.data(), 10, ids.data(), slots.data(), pool, 3, 2, 1, 64, 3, stage, stage, 4,
                                  nullptr, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(strstr(lsa_last_error(), "slot 3") != nullptr);
    slots[4] = -1;  // not copied: its id 99 is not read; the pageable store is refused next
    ids[4] = 99;
    CHECK(lsa_fetch_chunks_staged(host.data(), 10, ids.data(), slots.data(), pool, 3, 2, 1, 64, 3, stage, stage, 4,
                                  nullptr, nullptr) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(strstr(lsa_last_error(), "pinned") != nullptr);
    for (int32_t s : {0, 1, 2, 3, 4, 5, -1, 99, INT32_MIN}) CHECK(lsa_status_string(s) != nullptr);
    CHECK(strcmp(lsa_status_string(99), "LSA_ERR_UNKNOWN") == 0);
}

static void size_queries() {
    const int32_t v[] = {INT32_MIN, -1, 0, 1, 2, 7, 8, 63, 64, 65, 128, 1000, 65535, 65536, 1 << 20, 1 << 24,
                         INT32_MAX / 2, INT32_MAX - 1, INT32_MAX};
    size_t n_ok = 0;
    for (int32_t B : v)
        for (int32_t k : v)
            for (int32_t ns : {0, 1, 3, 64, INT32_MAX}) {
                const size_t w = lsa_gather_attend_workspace_size(B, 64, 8, 128, k, ns);
                const size_t t = lsa_topk_tokens_workspace_size(B, k, ns ? ns : 1);
                const int32_t s = lsa_gather_attend_default_splits(B, 8, k);
                n_ok += (w != (size_t)-1) + (t != (size_t)-1) + (s > 0);
            }
    CHECK(n_ok > 0);
}

static void tuning() {
    CHECK(lsa_get_tuning(99) == -1);
    CHECK(lsa_set_tuning(-1, 1) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_set_tuning(LSA_TUNE_ATTEND_DEPTH, 5) == LSA_ERR_INVALID_ARGUMENT);
    CHECK(lsa_set_tuning(LSA_TUNE_ATTEND_DEPTH, 3) == LSA_OK && lsa_get_tuning(LSA_TUNE_ATTEND_DEPTH) == 3);
    CHECK(lsa_set_tuning(LSA_TUNE_ATTEND_DEPTH, 0) == LSA_OK);
    // with the split knobs forced, the token workspace query changes and stays consistent
    const size_t before = lsa_topk_tokens_workspace_size(4, 1638, 2048);
    CHECK(lsa_set_tuning(LSA_TUNE_TOPK_SPLIT_SLICES, 3) == LSA_OK);
    const size_t forced = lsa_topk_tokens_workspace_size(4, 1638, 2048);
    CHECK(forced != before);
    CHECK(lsa_set_tuning(LSA_TUNE_TOPK_SPLIT_SLICES, 0) == LSA_OK);
    CHECK(lsa_topk_tokens_workspace_size(4, 1638, 2048) == before);
}

static void run_coalescing() {
    std::mt19937 rng(7);
    for (int trial = 0; trial < 2000; ++trial) {
        const int32_t B = 1 + (int32_t)(rng() % 4), k = 1 + (int32_t)(rng() % 40);
        const bool with_slots = rng() % 2;
        std::vector<int32_t> ids((size_t)B * k), slots((size_t)B * k);
        for (auto& x : ids) x = (int32_t)(rng() % 60);
        for (auto& x : slots) x = (int32_t)(rng() % 60);
        const bool with_skips = with_slots && rng() % 2;  // negative slots: entries not copied
        if (trial % 3 == 0)  // long runs
            for (int32_t b = 0; b < B; ++b)
                for (int32_t j = 1; j < k; ++j)
                    if (rng() % 4) {
                        ids[(size_t)b * k + j] = ids[(size_t)b * k + j - 1] + 1;
                        slots[(size_t)b * k + j] = slots[(size_t)b * k + j - 1] + 1;
                    }
        if (with_skips)
            for (auto& x : slots)
                if (rng() % 4 == 0) x = -1 - (int32_t)(rng() % 3);
        // expanding the runs gives back every entry with a slot >= 0 (all of
        // them without slots), in order, exactly once
        std::vector<int64_t> got_c, got_p, got_b;
        int calls = 0;
        const bool done = lsa::coalesce_fetch_runs(ids.data(), with_slots ? slots.data() : nullptr, B, k,
                                                   [&](int32_t b, int64_t c0, int64_t p0, int32_t run) {
                                                       ++calls;
                                                       if (run < 1) return false;
                                                       for (int32_t i = 0; i < run; ++i) {
                                                           got_b.push_back(b);
                                                           got_c.push_back(c0 + i);
                                                           got_p.push_back(p0 + i);
                                                       }
                                                       return true;
                                                   });
        CHECK(done);
        size_t n_copied = 0;
        for (size_t e = 0; e < ids.size(); ++e) n_copied += !(with_slots && slots[e] < 0);
        CHECK(got_c.size() == n_copied);
        int expected_runs = 0;
        size_t g = 0;  // next expanded entry
        for (int32_t b = 0; b < B && got_c.size() == n_copied; ++b)
            for (int32_t j = 0; j < k; ++j) {
                const size_t e = (size_t)b * k + j;
                if (with_slots && slots[e] < 0) continue;
                const int64_t p = with_slots ? slots[e] : j;
                CHECK(got_b[g] == b && got_c[g] == ids[e] && got_p[g] == p);
                ++g;
                const bool cont = j > 0 && !(with_slots && slots[e - 1] < 0) && ids[e] == ids[e - 1] + 1 &&
                                  p == (with_slots ? (int64_t)slots[e - 1] : (int64_t)j - 1) + 1;
                expected_runs += !cont;
            }
        CHECK(calls == expected_runs);  // and the runs are maximal
    }
    // stopping early
    std::vector<int32_t> ids = {0, 5, 9};
    int calls = 0;
    CHECK(!lsa::coalesce_fetch_runs(ids.data(), nullptr, 1, 3, [&](int32_t, int64_t, int64_t, int32_t) {
        return ++calls < 2;
    }));
    CHECK(calls == 2);
}

int main() {
    rejected_calls();
    size_queries();
    tuning();
    run_coalescing();
    if (failures) {
        fprintf(stderr, "sanitize_abi: %d checks failed\n", failures);
        return 1;
    }
    printf("sanitize_abi: ok\n");
    return 0;
}
