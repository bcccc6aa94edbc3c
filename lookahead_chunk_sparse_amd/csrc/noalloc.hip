// lsa_gather_attend_noalloc: lsa_gather_attend for callers that cannot
// allocate device memory.  The split-K partial results, which
// lsa_gather_attend keeps in a caller-supplied workspace, live here in a
// file-scope device array of fixed size instead; each GPU the library runs
// on holds its own copy until the process ends.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/lsa.h"
#include "lsa_kernels.h"

namespace {

constexpr size_t kScratchBytes = LSA_NOALLOC_SCRATCH_BYTES;

// The partial (m, l, o) triples of every split.  Nothing in it needs to start
// at zero: the split kernel writes every partial the combine reads.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on each GPU (in host code the array's
// name is only a stand-in for it), looked up once per device with that
// device current.
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

lsa_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LSA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LSA_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return LSA_OK;
}

}  // namespace

extern "C" lsa_status lsa_gather_attend_noalloc(const uint16_t* q, const uint16_t* kv, int64_t C_store,
                                                const int32_t* chunk_ids, const int32_t* slots, const int32_t* counts,
                                                const int32_t* ctx_len, const uint16_t* seg_kv,
                                                const int32_t* seg_len, int32_t S_max, int32_t B, int32_t Hq,
                                                int32_t Hkv, int32_t d, int32_t k, float sm_scale, int32_t n_split,
                                                float* out, hipStream_t stream) {
    // sizes first, on the host: an invalid shape is reported by
    // lsa_gather_attend's own validation, which runs before any HIP call
    const size_t need = lsa_gather_attend_workspace_size(B, Hq, Hkv, d, k, n_split);
    if (need == (size_t)-1)
        return lsa_gather_attend(q, kv, C_store, chunk_ids, slots, counts, ctx_len, seg_kv, seg_len, S_max, B, Hq,
                                 Hkv, d, k, sm_scale, nullptr, 0, n_split, out, stream);
    if (need > kScratchBytes)
        return lsa::reject(LSA_ERR_WORKSPACE,
                           "these sizes need %zu bytes of split partials; the static scratch holds %zu "
                           "(use lsa_gather_attend with a workspace, or fewer splits)",
                           need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        if (scratch_of_current_device(&ws) != LSA_OK)
            return lsa::reject(LSA_ERR_HIP, "the static scratch buffer's device address could not be looked up");
    }
    return lsa_gather_attend(q, kv, C_store, chunk_ids, slots, counts, ctx_len, seg_kv, seg_len, S_max, B, Hq, Hkv,
                             d, k, sm_scale, ws, need > 0 ? kScratchBytes : 0, n_split, out, stream);
}
