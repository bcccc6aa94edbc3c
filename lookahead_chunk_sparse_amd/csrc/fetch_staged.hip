// Host-tier fetch through a staging buffer (paperlayer.ai summary of
// "FlashMemory-DeepSeek-V4", 2.1 Architecture: non-recalled entries are
// evicted to CPU; 3 Experiments / Experimental Setup: the recalled chunks
// come back from CPU cold storage every tau = 64 steps; sergiiob.dev
// handbook, The Neural Memory Indexer, item 3 and its closing paragraph:
// the transfer is bound by host-to-device bandwidth).
//
// A selection's chunks are scattered over the host store, so a copy per
// chunk moves 256 KB with a fixed cost each and stays far below the link's
// rate.  Here the host gathers the chunks to fetch into consecutive places
// of a pinned staging buffer (worker threads, plain memcpy), the staging
// buffer crosses the link in large copies, and a device kernel moves each
// staged chunk into its pool slot at HBM speed.
//
// This file holds the device side (the scatter kernel) and the host worker
// threads; the entry point that orders them is lsa_fetch_chunks_staged in
// lsa_abi.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "lsa_kernels.h"

namespace lsa {
namespace {

constexpr int kScatterThreads = 256;
constexpr int kScatterParts = 4;  // workgroups per staged chunk

// Workgroup (s, part) copies part `part` of staged chunk s into pool chunk
// dst[s] (= b * P + slot).  A chunk is 16 * Hkv * d 16-byte words, so it
// splits into kScatterParts equal parts; each round issues its loads before
// its stores, and every access is bounded by the part's end.
__global__ __launch_bounds__(kScatterThreads) void stage_scatter_kernel(StageScatterArgs a) {
    const int s = blockIdx.x / kScatterParts, part = blockIdx.x % kScatterParts;
    const uint4* __restrict__ src = reinterpret_cast<const uint4*>(a.src) + (int64_t)s * a.chunk_u4;
    uint4* __restrict__ dst = reinterpret_cast<uint4*>(a.pool) + (int64_t)a.dst[s] * a.chunk_u4;
    const int64_t per = a.chunk_u4 / kScatterParts;
    const int64_t o0 = part * per, o1 = o0 + per;
    constexpr int kIn = 4;
    for (int64_t base = o0 + threadIdx.x; base < o1; base += (int64_t)kScatterThreads * kIn) {
        uint4 v[kIn];
#pragma unroll
        for (int u = 0; u < kIn; ++u) {
            const int64_t o = base + u * kScatterThreads;
            if (o < o1) v[u] = src[o];
        }
#pragma unroll
        for (int u = 0; u < kIn; ++u) {
            const int64_t o = base + u * kScatterThreads;
            if (o < o1) dst[o] = v[u];
        }
    }
}

// Host worker threads for the gather, created at the first use and kept
// until the process ends.  One job at a time: a job is a count of items and
// a function, and the calling thread works on it too.
class HostPool {
  public:
    explicit HostPool(int n_workers) {
        for (int t = 0; t < n_workers; ++t) workers_.emplace_back([this] { run(); });
    }
    ~HostPool() {
        {
            std::lock_guard<std::mutex> g(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& w : workers_) w.join();
    }
    void parallel_for(int n, const std::function<void(int)>& fn) {
        std::lock_guard<std::mutex> one_job(job_mu_);
        {
            std::lock_guard<std::mutex> g(mu_);
            fn_ = &fn;
            n_ = n;
            next_.store(0);
            busy_ = (int)workers_.size();
            ++generation_;
        }
        cv_.notify_all();
        work();
        std::unique_lock<std::mutex> g(mu_);
        done_cv_.wait(g, [this] { return busy_ == 0; });
        fn_ = nullptr;
    }

  private:
    void work() {
        for (int i = next_.fetch_add(1); i < n_; i = next_.fetch_add(1)) (*fn_)(i);
    }
    void run() {
        uint64_t seen = 0;
        for (;;) {
            {
                std::unique_lock<std::mutex> g(mu_);
                cv_.wait(g, [&] { return stop_ || generation_ != seen; });
                if (stop_) return;
                seen = generation_;
            }
            work();
            std::lock_guard<std::mutex> g(mu_);
            if (--busy_ == 0) done_cv_.notify_all();
        }
    }

    std::vector<std::thread> workers_;
    std::mutex job_mu_;  // one parallel_for at a time
    std::mutex mu_;
    std::condition_variable cv_, done_cv_;
    const std::function<void(int)>* fn_ = nullptr;
    int n_ = 0;
    std::atomic<int> next_{0};
    int busy_ = 0;
    uint64_t generation_ = 0;
    bool stop_ = false;
};

}  // namespace

void host_parallel_for(int n, const std::function<void(int)>& fn) {
    // 8 workers beside the caller: the gather reads and writes host memory,
    // so a few threads already draw on its bandwidth
    static HostPool pool(8);
    pool.parallel_for(n, fn);
}

namespace {

// One chunk into the staging buffer with non-temporal 16-byte stores: the
// staging buffer is read next by the DMA engine, not by this core, so the
// stores skip the cache (no read for ownership of the destination lines).
// bytes is a multiple of 64 and both addresses are 16-byte aligned.
void stream_copy(char* dst, const char* src, size_t bytes) {
    typedef long long v2i64 __attribute__((vector_size(16)));
    const v2i64* s = reinterpret_cast<const v2i64*>(src);
    v2i64* d = reinterpret_cast<v2i64*>(dst);
    for (size_t i = 0; i < bytes / 16; i += 4) {
        const v2i64 a = s[i], b = s[i + 1], c = s[i + 2], e = s[i + 3];
        __builtin_nontemporal_store(a, d + i);
        __builtin_nontemporal_store(b, d + i + 1);
        __builtin_nontemporal_store(c, d + i + 2);
        __builtin_nontemporal_store(e, d + i + 3);
    }
    __builtin_ia32_sfence();  // the stores are visible before the copy is issued
}

}  // namespace

void host_gather_chunks(char* dst, const char* store, const int64_t* src_chunks, int n, size_t chunk_bytes) {
    host_parallel_for(n, [&](int i) {
        stream_copy(dst + (size_t)i * chunk_bytes, store + (size_t)src_chunks[i] * chunk_bytes, chunk_bytes);
    });
}

hipError_t launch_stage_scatter(const StageScatterArgs& a, hipStream_t stream) {
    if (a.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(stage_scatter_kernel, dim3((unsigned)a.n * kScatterParts), dim3(kScatterThreads), 0, stream,
                       a);
    return hipGetLastError();
}

}  // namespace lsa
