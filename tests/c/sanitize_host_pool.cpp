// Host gather threads of the staged host-tier fetch under the sanitizers
// (tests/test_sanitizers.py builds this with fetch_staged.hip, the
// sanitizers on the host pass only: ThreadSanitizer in one build,
// AddressSanitizer with UndefinedBehaviorSanitizer in another).  No GPU is
// used: lsa::host_gather_chunks only reads and writes host memory.
//
// Each gather copies the listed chunks of a host store into consecutive
// places of a destination buffer; every copied byte is checked.  Gathers of
// 0, 1 and more chunks than there are worker threads run back to back, and
// then three threads gather at once (the pool runs one job at a time and the
// others wait for it).  Prints "sanitize_host_pool: ok" at the end.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <thread>
#include <vector>

#include "../../lookahead_chunk_sparse_amd/csrc/lsa_kernels.h"

namespace {

constexpr size_t kChunk = 4096;  // bytes per chunk: a multiple of 64
constexpr int kStoreChunks = 97;

unsigned char byte_of(int64_t chunk, size_t i) { return (unsigned char)(chunk * 131 + i * 7 + (i >> 9)); }

// One gather of n random chunks (with repeats) into a fresh buffer; returns
// the number of wrong bytes.
long gather_and_check(const char* store, int n, uint32_t seed) {
    std::mt19937 rng(seed);
    std::vector<int64_t> src((size_t)n);
    for (auto& s : src) s = (int64_t)(rng() % kStoreChunks);
    char* dst = static_cast<char*>(aligned_alloc(64, (size_t)(n ? n : 1) * kChunk));
    lsa::host_gather_chunks(dst, store, src.data(), n, kChunk);
    long bad = 0;
    for (int i = 0; i < n; ++i)
        for (size_t b = 0; b < kChunk; ++b) bad += (unsigned char)dst[(size_t)i * kChunk + b] != byte_of(src[(size_t)i], b);
    free(dst);
    return bad;
}

}  // namespace

int main() {
    char* store = static_cast<char*>(aligned_alloc(64, (size_t)kStoreChunks * kChunk));
    for (int64_t c = 0; c < kStoreChunks; ++c)
        for (size_t b = 0; b < kChunk; ++b) store[(size_t)c * kChunk + b] = (char)byte_of(c, b);

    long bad = 0;
    int calls = 0;
    for (int round = 0; round < 20; ++round)
        for (int n : {0, 1, 2, 9, 33, 200}) {
            bad += gather_and_check(store, n, (uint32_t)(round * 1000 + n));
            ++calls;
        }

    long bad_t[3] = {0, 0, 0};
    std::vector<std::thread> threads;
    for (int t = 0; t < 3; ++t)
        threads.emplace_back([&, t] {
            for (int r = 0; r < 15; ++r) bad_t[t] += gather_and_check(store, 5 + 11 * t + r, (uint32_t)(77 * t + r));
        });
    for (auto& th : threads) th.join();
    calls += 45;
    bad += bad_t[0] + bad_t[1] + bad_t[2];

    free(store);
    if (bad) {
        fprintf(stderr, "sanitize_host_pool: %ld wrong bytes over %d gathers\n", bad, calls);
        return 1;
    }
    printf("sanitize_host_pool: ok (%d gathers)\n", calls);
    return 0;
}
