// Gathered-chunk GQA decode attention for gfx950 (split-K flash decode).
//
// What it computes: for request b and query head h (KV head g = h / G),
// softmax(q K^T * sm_scale) V over the 64-token chunks listed for b, leaving
// out tokens at or past ctx_len[b] (attention formula and GQA grouping:
// sergiiob.dev handbook "DeepSeek-V4: Architecting for Ultra-Long Contexts",
// "Grouped Query Attention (GQA) vs. Multi-Head Attention (MHA)"; retained
// chunks only: paperlayer.ai summary of "FlashMemory-DeepSeek-V4", Abstract
// and 2.1 Architecture).
//
// How, on CDNA4:
//  * One workgroup = (request b, KV head g, split s) owns a contiguous slice
//    of b's chunk list; its 4 waves each take 16 of every chunk's 64 tokens.
//    Every K/V byte of the group is read from HBM once and serves all G query
//    heads of the group (G <= 16 fills the N side of a 16-wide MFMA tile).
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: A = 16 token rows of K (each
//    lane loads 16 contiguous bytes of a row), B = the group's queries, kept
//    in registers for the whole loop.
//  * O^T += V^T P^T on v_mfma_f32_16x16x16_bf16: the S^T accumulator layout
//    (lane = head + 16*(slot/4), element = slot%4) is exactly the B-operand
//    layout P^T needs, so P never leaves registers.  V^T needs each lane to
//    hold 4 tokens of one d column: lanes load 16 contiguous bytes of 4 rows
//    (4 consecutive rows per load instruction, fully coalesced) and a v_perm
//    per output dword transposes them in registers, so no LDS is used on the
//    streaming path.  Which slot carries which token is a free choice; slot
//    4i+r carries token 4r+i of the wave's 16, making each load instruction
//    cover 4 whole consecutive rows.
//  * P enters the V product as hi + lo bf16 parts (two MFMAs), keeping about
//    16 significant bits of the softmax weights; all accumulation is fp32.
//  * Online softmax per wave in the log2 domain; the 4 waves merge through
//    LDS at the end; splits merge in a second small kernel.
//  * Token-list mode (TOK): after the chunk recall, a token-level top-k
//    keeps only some tokens of the recalled chunks (paperlayer.ai summary,
//    2.1 Architecture).  The workgroup's list is then blocks of 64 listed
//    tokens; each token's K/V row index is staged in LDS (-1: masked) and
//    every lane loads its own rows, 64 contiguous bytes per lane and row
//    instead of whole 16 KB tiles.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "lsa_kernels.h"

namespace lsa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

// Chunk mode's K/V tile loads carry the non-temporal hint: every byte is
// read once, and the hint lifts the HBM read rate of random 16 KB tiles from
// about 6.0 to 6.8 TB/s (measured with the tile-read kernel over data that
// cannot be cached between reads).  The token-list mode's 64-byte pieces of
// scattered rows measured 1-2 us slower with it, so they load plainly.
__device__ inline uint4 load_nt(const uint16_t* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ inline uint2 load_nt2(const uint16_t* p) {
    return __builtin_bit_cast(uint2, __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)));
}

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kSliceTokens = 16;
constexpr int kListCache = 512;  // list entries staged in LDS at a time
constexpr int kTokCache = 32;    // token blocks (of 64 rows) staged in LDS at a time

template <int D>
struct VRow;  // one lane's share of one V row: D/16 bf16 values
template <>
struct VRow<128> {
    uint4 v;
};
template <>
struct VRow<64> {
    uint2 v;
};

template <int D, bool NT>
__device__ inline VRow<D> load_vrow(const uint16_t* p) {
    if constexpr (D == 128)
        return VRow<128>{NT ? load_nt(p) : *reinterpret_cast<const uint4*>(p)};
    else
        return VRow<64>{NT ? load_nt2(p) : *reinterpret_cast<const uint2*>(p)};
}

__device__ inline uint32_t vrow_dword(const VRow<128>& r, int w) {
    return w == 0 ? r.v.x : w == 1 ? r.v.y : w == 2 ? r.v.z : r.v.w;
}
__device__ inline uint32_t vrow_dword(const VRow<64>& r, int w) { return w == 0 ? r.v.x : r.v.y; }


// Registers of one wave's 16-token slice of one chunk.
template <int D>
struct Slice {
    uint4 k[D / 32];   // K: row pi(lane%16), 8 bf16 per MFMA step
    VRow<D> v[4];      // V: rows 4r + lane/16, d range [D/16 * (lane%16), +D/16)
};

template <int D>
__device__ inline void load_slice(Slice<D>& s, const uint16_t* ktile, const uint16_t* vtile, int wave, int lane) {
    const int n = lane & 15, i = lane >> 4;
    const int tk = wave * kSliceTokens + 4 * (n & 3) + (n >> 2);  // token of A row n
    const uint16_t* kp = ktile + (size_t)tk * D + 8 * i;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) s.k[st] = load_nt(kp + 32 * st);
    constexpr int DPL = D / 16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tv = wave * kSliceTokens + 4 * r + i;
        s.v[r] = load_vrow<D, true>(vtile + (size_t)tv * D + DPL * n);
    }
}

// Same register layout as load_slice, from per-row addresses: krow is the K
// row of this lane's A row, vrow[r] the V row of its token 4r + lane/16.
template <int D>
__device__ inline void load_slice_rows(Slice<D>& s, const uint16_t* krow, const uint16_t* const* vrow, int lane) {
    const int n = lane & 15, i = lane >> 4;
    const uint16_t* kp = krow + 8 * i;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) s.k[st] = *reinterpret_cast<const uint4*>(kp + 32 * st);
    constexpr int DPL = D / 16;
#pragma unroll
    for (int r = 0; r < 4; ++r) s.v[r] = load_vrow<D, false>(vrow[r] + DPL * n);
}

// Across the 4 rows of 16 lanes: every lane gets the maximum (sum) of its
// column, lanes l, l^16, l^32 and l^48.  gfx950's row-swap moves exchange
// rows between two registers, so a copy of v swapped with itself puts lane
// l^16 (then l^32) beside lane l with no LDS round trip.  Each step combines
// the same two values per lane as a butterfly over l^16 and l^32, so the
// results are the same bits.
__device__ inline float max_over_rows(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_over_rows(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ inline short bf16_bits(float x) { return __builtin_bit_cast(short, (__bf16)x); }
__device__ inline float bf16_value(short b) { return (float)__builtin_bit_cast(__bf16, b); }

__device__ inline uint4 select4(bool ok, uint4 v) {
    return ok ? v : make_uint4(0, 0, 0, 0);
}
__device__ inline void vrow_mask(VRow<128>& r, bool ok) { r.v = select4(ok, r.v); }
__device__ inline void vrow_mask(VRow<64>& r, bool ok) { r.v = ok ? r.v : make_uint2(0, 0); }

// Online-softmax update of one wave with one 16-token slice; tokens at or
// past `nvalid` (chunk-relative), and token 4r + lane/16 when bit r of
// `vmask` is clear, are masked.  Straight-line code except for
// the rescale of O, which only runs when some head's running max grows and
// issues no memory operation, so the loads in flight are never waited on
// early.
template <int D>
__device__ inline void process_slice(Slice<D>& sl, int nvalid, uint32_t vmask, int first_tok, int i, const bf16x8* qb,
                                     float scale_log2, float& m_run, float& l_run, f32x4* oacc) {
    constexpr int KS = D / 32;
    constexpr int DPL = D / 16;
    // S^T[slot][head] for this wave's 16 tokens
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KS; ++st)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, sl.k[st]), qb[st], sacc, 0, 0, 0);
    // lane holds head n, slots 4i+r = tokens first_tok + 4r + i; the K and V
    // rows of masked tokens may hold anything, so S is replaced and V zeroed
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool ok = first_tok + 4 * r + i < nvalid && ((vmask >> r) & 1u);
        sv[r] = ok ? sacc[r] * scale_log2 : -INFINITY;
        vrow_mask(sl.v[r], ok);
    }
    const float mx = max_over_rows(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    if (__any(mx > m_run)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 while m_run = -inf
        l_run *= alpha;
#pragma unroll
        for (int jj = 0; jj < DPL; ++jj) oacc[jj] *= alpha;
        m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;  // nothing valid yet: every p is 0
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sv[r] - m_use);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    i16x4 phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const short h = bf16_bits(p[r]);
        phi[r] = h;
        plo[r] = bf16_bits(p[r] - bf16_value(h));
    }
    // A operand of O^T += V^T P^T: element r = V[token 4r+i][DPL*n + jj]
#pragma unroll
    for (int jj = 0; jj < DPL; ++jj) {
        const int w = jj >> 1;
        const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(vrow_dword(sl.v[1], w), vrow_dword(sl.v[0], w), sel);
        const uint32_t hi = __builtin_amdgcn_perm(vrow_dword(sl.v[3], w), vrow_dword(sl.v[2], w), sel);
        const i16x4 av = __builtin_bit_cast(i16x4, make_uint2(lo, hi));
        oacc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, phi, oacc[jj], 0, 0, 0);
        oacc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, plo, oacc[jj], 0, 0, 0);
    }
}

// Merge the 4 waves' (m, l, o) of head h, column dd (log2-domain maxima).
__device__ inline void merge_waves(const float (*sm_m)[16], const float (*sm_l)[16], const float* sm_o, int h, int dd,
                                   int D, float& o, float& l, float& mstar) {
    mstar = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mstar = fmaxf(mstar, sm_m[w][h]);
    o = 0.f;
    l = 0.f;
    if (mstar != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = __builtin_amdgcn_exp2f(sm_m[w][h] - mstar);
            o += sc * sm_o[w * 16 * D + h * D + dd];
            l += sc * sm_l[w][h];
        }
    }
}

template <int D, int NBUF, bool TOK>
__global__ __launch_bounds__(kThreads) void attend_split_kernel(AttendArgs a) {
    constexpr int KS = D / 32;   // QK MFMA steps over d
    constexpr int DPL = D / 16;  // PV MFMAs (d values per lane per V row)
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15, i = lane >> 4;

    // Workgroup i runs on XCD i % 8, so with 2 splits the even XCDs hold the
    // first half of every list and the odd ones the second.  Rotating the
    // split index per group to mix them on every XCD measured 0.2% slower at
    // 128K (5,811 against 5,824 steps/s on one box), so the plain order stays.
    int blk = blockIdx.x;
    const int s = blk % a.n_split;
    blk /= a.n_split;
    const int g = blk % a.Hkv;
    const int b = blk / a.Hkv;
    const int G = a.G;

    // entries of this request's list in use (variable with threshold selection)
    int64_t kb = a.k;
    if (a.counts) {
        const int64_t cnt = a.counts[b];
        kb = cnt < 0 ? 0 : cnt > a.k ? a.k : cnt;
    }
    // then the resident segment (local window + decoded tokens) as 64-token blocks
    int seg_len = 0;
    if (a.seg_kv) {
        const int sl = a.seg_len[b];
        seg_len = sl < 0 ? 0 : sl > a.S_max ? a.S_max : sl;
    }
    // list entries before the segment: chunks, or blocks of 64 listed tokens
    int64_t n_main = kb, n_tok = 0;
    if constexpr (TOK) {
        n_tok = a.k_tok;
        if (a.tok_counts) {
            const int64_t tc = a.tok_counts[b];
            n_tok = tc < 0 ? 0 : tc > a.k_tok ? a.k_tok : tc;
        }
        n_main = (n_tok + kChunkTokens - 1) / kChunkTokens;
    }
    const int64_t total = n_main + (seg_len + kChunkTokens - 1) / kChunkTokens;
    const int64_t j0 = ((int64_t)s * total) / a.n_split;
    const int64_t j1 = ((int64_t)(s + 1) * total) / a.n_split;
    const int ctx = a.ctx[b];
    const int32_t* ids = a.ids + (int64_t)b * a.k;

    // B operand of S^T = K Q^T: lane (head n, group i) holds q[n][32*st + 8*i .. +8].
    bf16x8 qb[KS];
    {
        const bool live = n < G;  // lanes of padding heads read head 0 and use zeros
        const uint16_t* qp = a.q + ((int64_t)b * a.Hq + (int64_t)g * G + (live ? n : 0)) * D + 8 * i;
#pragma unroll
        for (int st = 0; st < KS; ++st)
            qb[st] = __builtin_bit_cast(bf16x8, select4(live, *reinterpret_cast<const uint4*>(qp + 32 * st)));
    }

    const int64_t chunk_elems = (int64_t)2 * a.Hkv * kChunkTokens * D;
    const int64_t tile_elems = (int64_t)kChunkTokens * D;
    const uint16_t* kv_b = a.kv + (int64_t)b * a.C_store * chunk_elems + (int64_t)g * tile_elems;
    const int64_t v_off = (int64_t)a.Hkv * tile_elems;
    const int first_tok = wave * kSliceTokens;

    f32x4 oacc[DPL];
#pragma unroll
    for (int jj = 0; jj < DPL; ++jj) oacc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max (log2 domain) of head n
    float l_run = 0.f;        // this lane's share of the running sum of head n

    // The workgroup's list entries (K tile offset, valid tokens, source) are
    // staged in LDS, up to kListCache entries at a time (TOK: the row index
    // of every token of up to kTokCache blocks), so computing a prefetch
    // address never waits behind the K/V loads in flight.  Entry j < n_main
    // is gathered chunk j (TOK: block j of the token list); entry n_main + m
    // is block m of the segment (flag kSegBit in sm_nv).  Offsets, not pointers, are staged: addresses
    // formed from the kernel's own buffer arguments stay in the global
    // address space, whose loads only count against vmcnt.
    constexpr int kSegBit = 1 << 16;
    constexpr int kCache = TOK ? kTokCache : kListCache;
    __shared__ int64_t sm_off[TOK ? 1 : kListCache];
    __shared__ int sm_nv[kCache];
    // TOK: row index of every staged token, in D-element rows from the
    // K base of its source (-1: masked)
    __shared__ int sm_row[TOK ? kTokCache * kChunkTokens : 1];
    const int32_t* tok_b = TOK ? a.tok + (int64_t)b * a.k_tok : nullptr;
    const int rows_per_chunk = 2 * a.Hkv * kChunkTokens;
    const int32_t* pos_src = a.slots ? a.slots + (int64_t)b * a.k : ids;
    // TOK: the request's list (chunk ids, store positions) staged in LDS once
    // when it fits; the staging of every round then looks positions up there
    constexpr int kTokPerThread = kTokCache * kChunkTokens / kThreads;
    static_assert(kTokCache * kChunkTokens % kThreads == 0, "whole staging rounds per thread");
    constexpr int kIdCache = 1024;
    __shared__ int sm_cid[TOK ? kIdCache : 1];
    __shared__ int sm_pos[TOK ? kIdCache : 1];
    const bool list_in_lds = TOK && kb <= kIdCache;
    // listed positions of a staging round, loaded clamped and unconditionally;
    // the first round's loads are issued here, before the list staging, so
    // the two round trips overlap
    int32_t pv[TOK ? kTokPerThread : 1];
    auto load_positions = [&](int64_t seg) {
#pragma unroll
        for (int r = 0; r < kTokPerThread; ++r) {
            const int64_t u = seg * kChunkTokens + threadIdx.x + r * kThreads;
            pv[r] = tok_b[u < a.k_tok ? u : a.k_tok - 1];
        }
    };
    if (TOK && j0 < j1) load_positions(j0);
    if (list_in_lds)
        for (int j = threadIdx.x; j < kb; j += kThreads) {
            sm_cid[j] = ids[j];
            sm_pos[j] = pos_src[j];
        }  // read after the first barrier of the staging loop
    const uint16_t* seg_b =
        a.seg_kv ? a.seg_kv + ((int64_t)b * 2 * a.Hkv + g) * (int64_t)a.S_max * D : kv_b;  // kv_b: never used
    const int64_t seg_v_off = (int64_t)a.Hkv * a.S_max * D;

    // Ring of NBUF register buffers: entry e of a segment lives in
    // buf[e % NBUF]; NBUF - 1 entries are in flight while one is processed.
    Slice<D> buf[NBUF];
    int nv[NBUF];
    uint32_t vm[NBUF];
    // Loads are counted in issue order (vmcnt), so the groups of loads are
    // kept in program order: a buffer's loads must be older than those of
    // every buffer issued after it for the waits to stay partial.
    auto issue = [&](int e, int bi) {
        const int f = sm_nv[e];
        const bool in_seg = (f & kSegBit) != 0;
        nv[bi] = f & (kSegBit - 1);
        if constexpr (TOK) {
            const uint16_t* bp = in_seg ? seg_b : kv_b;
            const int64_t vo = in_seg ? seg_v_off : v_off;
            const int* rows = sm_row + e * kChunkTokens + wave * kSliceTokens;
            const int rk = rows[4 * (n & 3) + (n >> 2)];
            const uint16_t* vrow[4];
            uint32_t m = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rv = rows[4 * r + i];
                m |= (uint32_t)(rv >= 0) << r;
                vrow[r] = bp + vo + (int64_t)(rv < 0 ? 0 : rv) * D;  // masked rows read row 0, never used
            }
            vm[bi] = m;
            const uint16_t* krow = bp + (int64_t)(rk < 0 ? 0 : rk) * D;
            __builtin_amdgcn_sched_barrier(0);
            load_slice_rows<D>(buf[bi], krow, vrow, lane);
            __builtin_amdgcn_sched_barrier(0);
        } else {
            vm[bi] = 0xFu;
            const uint16_t* kt = (in_seg ? seg_b : kv_b) + sm_off[e];
            const uint16_t* vt = kt + (in_seg ? seg_v_off : v_off);
            __builtin_amdgcn_sched_barrier(0);
            load_slice<D>(buf[bi], kt, vt, wave, lane);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int64_t seg = j0; seg < j1; seg += kCache) {
        const int segn = (int)(j1 - seg < kCache ? j1 - seg : kCache);
        __syncthreads();  // the previous segment's entries are no longer read
        if constexpr (TOK) {
            // Each thread stages kTokPerThread tokens: the listed positions
            // (loaded already for the first round), looked up in the list
            // staged in LDS.
            if (seg != j0) load_positions(seg);
#pragma unroll
            for (int r = 0; r < kTokPerThread; ++r) {
                const int x = threadIdx.x + r * kThreads;
                if (x >= segn * kChunkTokens) break;
                const int e = x / kChunkTokens, t = x % kChunkTokens;
                const int64_t jb = seg + e;
                int row = -1;
                if (jb < n_main) {
                    const int64_t u = jb * kChunkTokens + t;
                    const int64_t p = pv[r];
                    if (u < n_tok && p >= 0 && p < kb * kChunkTokens) {
                        const int j = (int)(p / kChunkTokens), tt = (int)(p % kChunkTokens);
                        const int64_t cid = list_in_lds ? sm_cid[j] : ids[j];
                        const int64_t pos = list_in_lds ? sm_pos[j] : pos_src[j];
                        if (cid * kChunkTokens + tt < ctx) row = (int)(pos * rows_per_chunk + tt);
                    }
                } else {
                    const int64_t sidx = (jb - n_main) * kChunkTokens + t;
                    if (sidx < seg_len) row = (int)sidx;
                }
                sm_row[x] = row;
                if (t == 0) sm_nv[e] = kChunkTokens | (jb < n_main ? 0 : kSegBit);
            }
        }
        for (int e = threadIdx.x; !TOK && e < segn; e += kThreads) {
            const int64_t j = seg + e;
            int64_t v;
            int flag = 0;
            if (j < kb) {
                const int64_t c = ids[j];
                v = (int64_t)ctx - c * kChunkTokens;
                sm_off[e] = (int64_t)pos_src[j] * chunk_elems;
            } else {
                const int64_t m = j - kb;
                v = (int64_t)seg_len - m * kChunkTokens;
                sm_off[e] = m * kChunkTokens * D;
                flag = kSegBit;
            }
            sm_nv[e] = (v < 0 ? 0 : v > kChunkTokens ? kChunkTokens : (int)v) | flag;
        }
        __syncthreads();
        // Every step issues one prefetch (past the segment's end it re-reads
        // the last entry, never used) and processes one buffer, so the
        // compiler can count the loads in flight exactly.  Full rounds of
        // NBUF steps run in a loop with no early exit; the remainder follows.
        auto step = [&](int e, int u) {
            const int ep = e + NBUF - 1;
            issue(ep < segn ? ep : segn - 1, (u + NBUF - 1) % NBUF);
            process_slice<D>(buf[u], nv[u], vm[u], first_tok, i, qb, a.scale_log2, m_run, l_run, oacc);
        };
#pragma unroll
        for (int u = 0; u < NBUF - 1; ++u) issue(u < segn ? u : segn - 1, u);
        int e = 0;
        for (; e + NBUF <= segn; e += NBUF) {
#pragma unroll
            for (int u = 0; u < NBUF; ++u) step(e + u, u);
        }
#pragma unroll
        for (int u = 0; u < NBUF - 1; ++u)
            if (e + u < segn) step(e + u, u);
    }

    // ---- merge the 4 waves of the workgroup through LDS ----
    __shared__ float sm_m[kWaves][16];
    __shared__ float sm_l[kWaves][16];
    __shared__ float sm_o[kWaves * 16 * D];
    const float l_tot = sum_over_rows(l_run);
    if (n < G) {
        if (i == 0) {
            sm_m[wave][n] = m_run;
            sm_l[wave][n] = l_tot;
        }
        // lane holds O[n][DPL*(4i + r) + jj]
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int jj = 0; jj < DPL; ++jj) sm_o[wave * 16 * D + n * D + DPL * (4 * i + r) + jj] = oacc[jj][r];
    }
    __syncthreads();

    const int64_t grp = (int64_t)b * a.Hkv + g;
    if (a.n_split == 1) {
        for (int e = threadIdx.x; e < G * D; e += kThreads) {
            const int h = e / D, dd = e % D;
            float o, l, mstar;
            merge_waves(sm_m, sm_l, sm_o, h, dd, D, o, l, mstar);
            a.out[((int64_t)b * a.Hq + (int64_t)g * G + h) * D + dd] = l > 0.f ? o / l : 0.f;
        }
        return;
    }
    const int64_t part = grp * a.n_split + s;
    for (int e = threadIdx.x; e < G * D; e += kThreads) {
        const int h = e / D, dd = e % D;
        float o, l, mstar;
        merge_waves(sm_m, sm_l, sm_o, h, dd, D, o, l, mstar);
        a.part_o[(part * G + h) * D + dd] = o;
        if (dd == 0) {
            a.part_ml[(part * G + h) * 2 + 0] = mstar;
            a.part_ml[(part * G + h) * 2 + 1] = l;
        }
    }
}

// Merge the n_split partial (m, l, o) triples of every (request, head):
// m* = max m_s, o = sum_s 2^(m_s - m*) o_s / sum_s 2^(m_s - m*) l_s.
// One workgroup of d threads per (request, query head).  For NS > 0 (the
// split count known at compile time) every partial is loaded up front, so
// the kernel costs one memory latency.  A separate launch: merging inside
// the split kernel would need agent-scope fences across the XCDs' L2
// caches, which measured far slower than this launch.
template <int NS>
__global__ __launch_bounds__(128) void attend_combine_kernel(AttendArgs a) {
    const int bh = blockIdx.x;  // b * Hq + h
    const int b = bh / a.Hq, h = bh % a.Hq;
    const int g = h / a.G, hh = h % a.G;
    const int dd = threadIdx.x;
    const int64_t base = ((int64_t)b * a.Hkv + g) * a.n_split;
    float mstar = -INFINITY, o = 0.f, l = 0.f;
    if constexpr (NS > 0) {
        float pm[NS], pl[NS], po[NS];
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) {
            const int64_t ps = (base + sp) * a.G + hh;
            pm[sp] = a.part_ml[ps * 2];
            pl[sp] = a.part_ml[ps * 2 + 1];
            po[sp] = a.part_o[ps * a.d + dd];
        }
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) mstar = fmaxf(mstar, pm[sp]);
        // Branch-free, so that every load above is issued before any result is
        // needed (loads used only under a branch move into it, a second round
        // trip).  A split with no valid token has m = -inf and weight 0; when
        // all have, every weight is 0 and so is the output.
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) {
            const float sc = pm[sp] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pm[sp] - mstar);
            l += sc * pl[sp];
            o += sc * po[sp];
        }
    } else {
        for (int sp = 0; sp < a.n_split; ++sp) mstar = fmaxf(mstar, a.part_ml[((base + sp) * a.G + hh) * 2]);
        if (mstar != -INFINITY) {
            for (int sp = 0; sp < a.n_split; ++sp) {
                const int64_t ps = (base + sp) * a.G + hh;
                const float sc = __builtin_amdgcn_exp2f(a.part_ml[ps * 2] - mstar);
                l += sc * a.part_ml[ps * 2 + 1];
                o += sc * a.part_o[ps * a.d + dd];
            }
        }
    }
    a.out[(int64_t)bh * a.d + dd] = l > 0.f ? o / l : 0.f;
}

}  // namespace

// Register-ring size of the split kernel: 2 unless the LSA_TUNE_ATTEND_DEPTH
// knob (2, 3 or 4) says otherwise.  With the non-temporal tile loads one
// slice in flight per wave beside the one being processed measured fastest
// (128K: 172.9 us at 2, 175.2 at 3, 177.2 at 4).
int attend_pipeline_depth() { return tuning(LSA_TUNE_ATTEND_DEPTH); }

int attend_default_splits(int B, int Hkv, int k) {
    // About one workgroup per CU (256): with every K/V byte read exactly once,
    // fewer and longer streams keep HBM fuller than more and shorter ones
    // (measured on the 128K workload: 256 workgroups beat 128 and 512+).
    const int64_t groups = (int64_t)B * Hkv;
    int64_t s = (256 + groups / 2) / groups;
    if (s < 1) s = 1;
    if (s > k) s = k;
    return (int)s;
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: [partial O][partial (m, l)], the second region 256-byte
// aligned; nothing when there is a single split.
size_t attend_workspace_bytes(int B, int Hkv, int G, int d, int n_split) {
    if (n_split <= 1) return 0;
    const size_t parts = (size_t)B * Hkv * n_split * G;
    return round256(parts * d * sizeof(float)) + parts * 2 * sizeof(float);
}

void attend_workspace_carve(AttendArgs& a, void* workspace) {
    char* p = static_cast<char*>(workspace);
    const size_t parts = (size_t)a.B * a.Hkv * a.n_split * a.G;
    a.part_o = reinterpret_cast<float*>(p);
    p += round256(parts * a.d * sizeof(float));
    a.part_ml = reinterpret_cast<float*>(p);
}

template <int D, bool TOK>
void launch_split_mode(const AttendArgs& a, dim3 grid, hipStream_t stream) {
    switch (a.depth) {
        case 2: hipLaunchKernelGGL((attend_split_kernel<D, 2, TOK>), grid, dim3(kThreads), 0, stream, a); break;
        case 4: hipLaunchKernelGGL((attend_split_kernel<D, 4, TOK>), grid, dim3(kThreads), 0, stream, a); break;
        default: hipLaunchKernelGGL((attend_split_kernel<D, 3, TOK>), grid, dim3(kThreads), 0, stream, a); break;
    }
}

template <int D>
void launch_split(const AttendArgs& a, dim3 grid, hipStream_t stream) {
    if (a.tok)
        launch_split_mode<D, true>(a, grid, stream);
    else
        launch_split_mode<D, false>(a, grid, stream);
}

hipError_t launch_gather_attend(const AttendArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)a.B * a.Hkv * a.n_split));
    if (a.d == 128)
        launch_split<128>(a, grid, stream);
    else
        launch_split<64>(a, grid, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    const dim3 cgrid((unsigned)((int64_t)a.B * a.Hq)), cblock(a.d);
    switch (a.n_split) {
        case 2: hipLaunchKernelGGL(attend_combine_kernel<2>, cgrid, cblock, 0, stream, a); break;
        case 3: hipLaunchKernelGGL(attend_combine_kernel<3>, cgrid, cblock, 0, stream, a); break;
        case 4: hipLaunchKernelGGL(attend_combine_kernel<4>, cgrid, cblock, 0, stream, a); break;
        case 5: hipLaunchKernelGGL(attend_combine_kernel<5>, cgrid, cblock, 0, stream, a); break;
        case 6: hipLaunchKernelGGL(attend_combine_kernel<6>, cgrid, cblock, 0, stream, a); break;
        case 7: hipLaunchKernelGGL(attend_combine_kernel<7>, cgrid, cblock, 0, stream, a); break;
        case 8: hipLaunchKernelGGL(attend_combine_kernel<8>, cgrid, cblock, 0, stream, a); break;
        default: hipLaunchKernelGGL(attend_combine_kernel<0>, cgrid, cblock, 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace lsa
