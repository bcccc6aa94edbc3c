// Run coalescing of the host-tier DMA fetch (lsa_fetch_chunks): entries
// whose chunk ids and pool slots both run on consecutively become one copy.
// Pure host code, shared by the library and its sanitizer test.
#pragma once

#include <stdint.h>

namespace lsa {

// For every request b and every maximal run of entries j..j+n-1 with
// ids[j+i] = ids[j] + i and slot(j+i) = slot(j) + i (slot(j) = slots[b][j],
// or j when slots is null), calls emit(b, ids[j], slot(j), n) in entry order.
// An entry with a negative slot is not copied (a delta fetch's chunk that is
// already in the pool, or an entry not in use) and ends a run.  emit returns
// false to stop; the function then returns false.
template <class Emit>
bool coalesce_fetch_runs(const int32_t* ids, const int32_t* slots, int32_t B, int32_t k, Emit&& emit) {
    for (int32_t b = 0; b < B; ++b) {
        const int32_t* id = ids + (int64_t)b * k;
        const int32_t* sl = slots ? slots + (int64_t)b * k : nullptr;
        int32_t j = 0;
        while (j < k) {
            if (sl && sl[j] < 0) {
                ++j;
                continue;
            }
            const int64_t c0 = id[j];
            const int64_t p0 = sl ? sl[j] : j;
            int32_t run = 1;
            while (j + run < k && (int64_t)id[j + run] == c0 + run && (sl ? (int64_t)sl[j + run] : (int64_t)j + run) == p0 + run)
                ++run;
            if (!emit(b, c0, p0, run)) return false;
            j += run;
        }
    }
    return true;
}

}  // namespace lsa
