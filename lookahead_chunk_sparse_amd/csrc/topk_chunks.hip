// Fixed-budget chunk re-selection for gfx950: per row, the first k chunks of
// the order (logit descending, chunk index ascending), written in ascending
// chunk order (paperlayer.ai summary of "FlashMemory-DeepSeek-V4", 1
// Introduction and 2.1 Architecture: only the chunks the indexer ranks
// highest are kept; ties go to the lower chunk index).
//
// One 1024-thread workgroup per row; wave w keeps positions
// [64*KPT*w, 64*KPT*(w+1)) in registers, lane l every 64th of them from l
// (coalesced loads), as order-preserving unsigned keys (logit XOR 0x80000000);
// digits are taken of key - (the row's smallest key), so that only the bits
// spanning the row's range remain (logits of both signs would otherwise
// differ in every bit).
//  1. Radix select from the top of the range.  A pass counts the keys of the
//     current bucket per 8-bit digit into an LDS histogram (ds_add, one copy
//     per lane against same-word conflicts); one wave then finds, by a suffix
//     scan over the 256 bins, the digit that holds the k-th largest key, and
//     that digit's keys become the bucket.  Every pass over the registers
//     costs the whole row's keys in VALU work on one CU, so once the bucket
//     fits (8192 keys) it moves into LDS and later passes read only it; once
//     it is down to 256 keys one wave decides the remaining bits one at a
//     time from ballots (a bit of the k-th key is 1 iff at least `need` keys
//     of the bucket have it set).  The result is that key v*, the number of
//     keys equal to v*, and `need`, how many of those belong to the selection.
//  2. Ordered compaction: keys > v* are taken; keys == v* are taken while
//     their rank among equal keys, in index order, is below `need` (all of
//     them when need is their number: then simply the keys >= v*).  Each
//     wave appends its keys >= v* to its own LDS region in index order;
//     scans of the per-wave totals then place every wave's outputs, so the
//     output is ascending.
// Rows too long for registers stream from memory instead (the same select
// with a 16-copy histogram and no LDS bucket), and very long token rows are
// split into slices whose top k are merged by a candidates pass.
//
// The same select serves the token-level stage: after the chunk recall the
// model's own token scores pick a fine-grained top-k among the recalled
// tokens only (same summary, 2.1 Architecture); there the keys are float
// scores over the list positions of the recalled chunks.  Token rows held in
// registers first try a fast select (tokens_fast_select): a sampled bound,
// the keys above it copied to LDS, a 12-bit histogram and an ordered
// compaction of those keys only; the radix select above is its fallback.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "lsa_kernels.h"

namespace lsa {
namespace {

constexpr int kThreads = kTopkThreads;
constexpr int kWaves = kThreads / 64;

// Minimum and maximum over the 64 lanes of a wave, the same in every lane:
// the DPP steps of an inclusive scan (row shifts of 1, 2, 4, 8, then the
// row broadcasts of lanes 15 and 31), where a lane with no source takes the
// operation's identity, leave the whole wave's result in lane 63.  Register
// moves only: no LDS round trip per step, as a shuffle would take.
__device__ inline uint32_t wave_min(uint32_t v) {
    int x = (int)v;
    const int id = -1;  // 0xFFFFFFFF, the identity of an unsigned minimum
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(id, x, 0x111, 0xF, 0xF, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(id, x, 0x112, 0xF, 0xF, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(id, x, 0x114, 0xF, 0xF, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(id, x, 0x118, 0xF, 0xF, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(id, x, 0x142, 0xA, 0xF, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(id, x, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}
__device__ inline uint32_t wave_max(uint32_t v) {
    int x = (int)v;  // identity 0
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}

constexpr int kDigitBits = 8;
constexpr int kBins = 1 << kDigitBits;
// Copies of the streaming kernel's histogram: lane l counts into copy
// l % kCopies, so lanes whose keys share a bin hit kCopies different words
// (scores crowd into a few bins, and same-word LDS atomics serialise).
constexpr int kCopies = 16;

// After a histogram pass (and its barrier): sums the COPIES copies of every
// bin ([bin][copy] layout) and picks the digit holding the need-th largest
// key of the bucket; sm_pick = {digit, keys still needed within it, keys in
// it}.  Ends with a barrier.
template <int COPIES>
__device__ inline void pick_digit(const int* sm_hist, int* sm_tot, int* sm_pick, int tid, int lane, int wave,
                                  int need) {
    {
        // every thread sums COPIES/4 copies of bin tid/4; 4 neighbouring
        // lanes complete the bin
        static_assert(kThreads == 4 * kBins && COPIES % 16 == 0, "copy reduction layout");
        constexpr int kPer = COPIES / 4;
        const int4* p = reinterpret_cast<const int4*>(&sm_hist[kPer * tid]);
        int t = 0;
#pragma unroll
        for (int i = 0; i < kPer / 4; ++i) {
            const int4 v = p[i];
            t += (v.x + v.y) + (v.z + v.w);
        }
        // quad sums by DPP lane swaps (quad_perm [1,0,3,2], then [2,3,0,1])
        t += __builtin_amdgcn_update_dpp(0, t, 0xB1, 0xF, 0xF, false);
        t += __builtin_amdgcn_update_dpp(0, t, 0x4E, 0xF, 0xF, false);
        if ((tid & 3) == 0) sm_tot[tid >> 2] = t;
    }
    __syncthreads();
    if (wave == 0) {
        // lane l holds bins 4l..4l+3; exclusive suffix sum over lanes
        int h[4], sl = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h[j] = sm_tot[4 * lane + j];
            sl += h[j];
        }
        int suf = sl;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_down(suf, off);
            if (lane + off < 64) suf += u;
        }
        int above = suf - sl;  // keys of the bucket in higher digits
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            if (above < need && need <= above + h[j]) {  // exactly one (lane, j) matches
                sm_pick[0] = 4 * lane + j;
                sm_pick[1] = need - above;
                sm_pick[2] = h[j];
            }
            above += h[j];
        }
    }
    __syncthreads();
}

// Order-preserving unsigned key of a float score: equal values give equal
// keys (-0 is taken as +0: adding +0 maps -0 to +0 and leaves every other
// value as it is), larger values larger keys.  NaN is not a score.
__device__ inline uint32_t score_key(float x) {
    const uint32_t u = __float_as_uint(x + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // negative: ~u; else u | 2^31
}

// One row (or row slice) per workgroup.  Modes:
//  * kModeLogits, budget (counts == nullptr): the first k of C int32 logits;
//  * kModeLogits, threshold (counts != nullptr): the logits above thr, at
//    most k; the row is padded with -1 and counts[row] = chunks kept;
//  * kModeTokens: float scores of the C = 64 * n_list list positions of a
//    row's recalled chunks; only usable positions compete (entry j < the
//    row's list count, context position ids[j]*64 + t < ctx); at most k are
//    kept, -1 padding, counts[row] = kept;
//  * kModeSlice: the same on slice s of the row (positions [s*L, s*L + L),
//    L a multiple of 64), workgroup r*n_slices + s; the slice's top k go to
//    the candidate arrays as (position, key), ascending, padded (-1, 0);
//  * kModeCand: row r's n_slices*k candidates (key 0: none) in position
//    order; the top k of them are written as positions, -1 padding,
//    counts[row] = kept.
// Slice + candidates give the tokens mode's result with many workgroups per
// row: every position of the row's top k is in its slice's top k.
enum : int { kModeLogits = 0, kModeTokens = 1, kModeSlice = 2, kModeCand = 3 };

struct TopkArgs {
    const int32_t* logits;      // [R][C] (logits)
    const float* scores;        // [R][64 * n_list] (tokens, slice)
    const int32_t* list_ids;    // [R][n_list] recalled chunk ids (tokens, slice)
    const int32_t* list_counts; // [R] entries in use, may be null (tokens, slice)
    const int32_t* ctx;         // [R] context length (tokens, slice)
    int n_list;
    int C, k;                   // positions per workgroup's row (slice mode: the slice length L), kept
    int32_t thr;
    int32_t* out;               // [R][k] (logits, tokens, candidates)
    int32_t* counts;            // [R] or null (logits budget)
    int n_slices;               // slice, candidates
    int32_t* cand_pos;          // [R][n_slices][k] positions (written by slice, read by candidates)
    uint32_t* cand_key;         // [R][n_slices][k] keys, 0 = none
    int sample_rank;            // tokens mode: rank of the sample key that bounds the candidates (0: off)
};

// A bucket of at most kListCap keys moves from registers into LDS; one of at
// most kBallotMax keys is finished bit by bit by one wave.
constexpr int kListCap = 8192;
constexpr int kBallotMax = 256;
constexpr int kBallotSlots = kBallotMax / 64;
// The register kernel's histogram has one copy per lane: keys of one digit in
// one load instruction then never share an LDS word.
constexpr int kLaneCopies = 64;

// Rank of this lane among the set bits of m below it.
__device__ inline int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers: within
// each row of 16 lanes by shifts of 1, 2, 4 and 8 lanes, then across rows by
// adding lane 15 of row 0 to row 1 and lane 47 to row 3, then lane 31 to
// rows 2 and 3 (DPP row_shr and row_bcast; a lane with no source adds 0).
__device__ inline int wave_incl_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// OR over the 64 lanes of a wave, the same in every lane (DPP, as above).
__device__ inline uint32_t wave_or(uint32_t v) {
    int x = (int)v;
    x |= __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
    x |= __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
    x |= __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
    x |= __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
    x |= __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
    x |= __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
    return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}

// Sum of per-wave totals tot[0..wave), the same in every lane.
__device__ inline int sum_below(const int* tot, int wave, int lane) {
    const int x = lane < wave ? tot[lane & (kThreads / 64 - 1)] : 0;
    return __builtin_amdgcn_readlane(wave_incl_sum(x), 63);
}

// The rank-th largest (1-based) of the values v0 and v1 held by the lanes of
// one wave (128 values, all below 2^bits, bits even), decided two bits at a
// time from the top: among the values still agreeing with the decided bits,
// the digit is the largest d whose count of digits >= d reaches `rank`.  The
// three counts of a step are independent ballots, so the dependent chain is
// half as long as bit by bit.
__device__ inline uint32_t wave_rank_value2(uint32_t v0, uint32_t v1, int bits, int rank) {
    uint64_t c0 = ~0ull, c1 = ~0ull;
    uint32_t r = 0;
    for (int b = bits - 2; b >= 0; b -= 2) {
        const uint32_t d0 = (v0 >> b) & 3u, d1 = (v1 >> b) & 3u;
        const uint64_t g3a = c0 & __ballot(d0 == 3u), g3b = c1 & __ballot(d1 == 3u);
        const uint64_t g2a = c0 & __ballot(d0 >= 2u), g2b = c1 & __ballot(d1 >= 2u);
        const uint64_t g1a = c0 & __ballot(d0 >= 1u), g1b = c1 & __ballot(d1 >= 1u);
        const int n3 = __popcll(g3a) + __popcll(g3b), n2 = __popcll(g2a) + __popcll(g2b),
                  n1 = __popcll(g1a) + __popcll(g1b);
        if (n3 >= rank) {
            c0 = g3a; c1 = g3b; r |= 3u << b;
        } else if (n2 >= rank) {
            c0 = g2a & ~g3a; c1 = g2b & ~g3b; rank -= n3; r |= 2u << b;
        } else if (n1 >= rank) {
            c0 = g1a & ~g2a; c1 = g1b & ~g2b; rank -= n2; r |= 1u << b;
        } else {
            c0 &= ~g1a; c1 &= ~g1b; rank -= n1;
        }
    }
    return r;
}

// The rank-th largest (1-based) of the values v held by the lanes of one
// wave, all below 2^bits, decided bit by bit from the top: the bit is 1 iff
// at least `rank` of the values still agreeing with the decided bits have it.
__device__ inline uint32_t wave_rank_value(uint32_t v, int bits, int rank) {
    uint64_t cand = ~0ull;
    uint32_t r = 0;
    for (int b = bits - 1; b >= 0; --b) {
        const uint64_t one = cand & __ballot((v >> b) & 1u);
        const int c1 = __popcll(one);
        const bool set = rank <= c1;
        cand = set ? one : cand & ~one;
        rank = set ? rank : rank - c1;
        r |= set ? 1u << b : 0u;
    }
    return r;
}

// One wave finishes a select on the cnt <= 64*NS keys of lst (all agreeing
// above bit hi): bit by bit from bit hi-1 down, the bit of the need-th
// largest key is 1 iff at least `need` of the remaining candidates have it
// set, and the candidates keep the keys that agree with it.  Writes
// sm_pick = {the decided low bits, keys still needed, keys equal to the
// result}.  Branch-free inner loop: the masks live in scalar registers.
template <int NS>
__device__ inline void ballot_finish(const uint32_t* lst, int cnt, int hi, int need, int lane, int* sm_pick) {
    uint32_t v[NS];
    uint64_t cand[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int i = 64 * s + lane;
        v[s] = lst[i < cnt ? i : 0];
        cand[s] = __ballot(i < cnt);
    }
    uint32_t low = 0;
    int nd = need;
    for (int b = hi - 1; b >= 0; --b) {
        uint64_t one[NS];
        int c1 = 0;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            one[s] = cand[s] & __ballot((v[s] >> b) & 1u);
            c1 += __popcll(one[s]);
        }
        const bool set = nd <= c1;
#pragma unroll
        for (int s = 0; s < NS; ++s) cand[s] = set ? one[s] : (cand[s] & ~one[s]);
        nd = set ? nd : nd - c1;
        low |= set ? (1u << b) : 0u;
    }
    int ceq = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) ceq += __popcll(cand[s]);
    if (lane == 0) {
        sm_pick[0] = (int)low;
        sm_pick[1] = nd;
        sm_pick[2] = ceq;
    }
}

// The fast select of score rows (token rows, their slices and their
// candidates): wave 0 draws kSamples keys spread over the workgroup's
// positions (two per lane) while the other waves form their keys; the 12-bit
// key prefix of the sample key of rank sample_rank bounds a candidate set
// (every key at or above that prefix) that holds the kept keys whenever it
// has at least k members; it is then selected from in LDS.
constexpr int kSamples = 128;
constexpr int kSampleBits = 12;        // key prefix the sample decides
constexpr int kRegion = 768;           // (key, position) pairs each wave holds in LDS
constexpr int kRegionStride = kRegion + 64;  // and one spare pair per lane: the writes need no branch
constexpr int kCandWord0 = 4352;       // first word of the waves' regions in sm_raw
constexpr int kTokBinBits = 12;        // digit width of the candidates' histogram
constexpr int kTokBins = 1 << kTokBinBits;
constexpr int kSmallCap = 64;          // a bin this small is ranked by one wave

// LDS word of histogram bin b: the low 5 bits are XORed with the next 5, a
// bijection on [0, 4096) that spreads bins at power-of-two strides (scores
// with few mantissa bits fill every 8th or 16th bin) over the LDS banks.
__device__ inline int hist_word(uint32_t b) { return (int)(b ^ ((b >> 5) & 31u)); }
// Word 3 of a buffer resource on this GPU family: 32-bit raw data, no swizzle.
constexpr int kBufferWord3 = 0x00020000;

// Score row (token, slice or candidates mode), register-resident, KPT keys
// per thread, kk < competing keys; pos_of(e) is the position slot e's key is
// written as, dst_key (slices only) receives the kept keys too.  The cost of
// this one-workgroup select is set by the issue rate of its one compute unit
// (16 waves share 4 SIMDs, one scalar unit and the LDS), so every step below
// is a few instructions per wave between barriers:
//  1. The bound pv (taken by the caller from the 128-key sample) splits off
//     the candidates, every key >= pv: each wave copies its own to its LDS
//     region as (key, position) pairs, in position order.  If fewer than kk
//     keys reach pv in all, or some wave has more than its region holds,
//     false is returned (uniformly) and the full select runs instead.
//  2. A 4096-bin histogram of the candidates' top 12 bits above pv
//     (key - pv >> sh, sh = bits of kmax - pv beyond 12) and a block-wide
//     suffix scan find the bin of the kk-th largest candidate.  A bin that
//     holds a single value (width 1, or every candidate's bits below the bin
//     width equal to pv's) decides v* outright; a bin of at most 64 keys is
//     gathered and finished by one wave, bit by bit; a larger bin is
//     histogrammed again on its next 12 bits.
//  3. Ordered compaction: candidates > v*, and the first `keep` candidates
//     equal to v* in position order.  Waves cover the row in position order,
//     so one exclusive scan of per-wave counts places all outputs in
//     ascending position order.
// The row's counts and -1 padding are the caller's.  The histogram's 4096
// words at the start of sm_raw must be zero on entry.  Uses sm_raw: [0,
// 4096) histogram (bin b at word hist_word(b)), [4096, 4160) small bucket,
// from kCandWord0 the waves' regions of kRegion pairs.
template <int KPT, class PosOf>
__device__ __forceinline__ bool tokens_fast_select(const uint32_t (&key)[KPT], PosOf pos_of, int kk, uint32_t kmax,
                                                   uint32_t pv, int tid, int lane, int wave, uint32_t* sm_raw,
                                                   int* sm_i, int* sm_j, int* sm_cnt, int* sm_pick, int32_t* dst,
                                                   uint32_t* dst_key) {
    int* const hist = reinterpret_cast<int*>(sm_raw);   // [kTokBins]
    uint32_t* const small = sm_raw + kTokBins;           // [kSmallCap]
    uint2* const reg = reinterpret_cast<uint2*>(sm_raw + kCandWord0) + wave * kRegionStride;  // this wave's pairs
    static_assert(kTokBins + kSmallCap <= kCandWord0 && kCandWord0 % 4 == 0, "histogram and bucket below the pairs");
    static_assert(kCandWord0 + 2 * kWaves * kRegionStride <= kBins * kLaneCopies + 2 * kListCap, "regions fit sm_raw");
    static_assert(kThreads * 4 == kTokBins && kRegion % 64 == 0, "scan layout: 4 bins per thread; whole runs");

    // --- 1. the candidates ---
    // The wave's count comes first (ballots and scalar counts only); if it
    // fits the region, every lane writes at every slot, a key that is not a
    // candidate to the lane's spare pair (a select instead of a branch around
    // the store).  A wave whose candidates overflow writes nothing (the full
    // select then runs).
    uint64_t in_m[KPT];
    uint32_t n_before[KPT];
    uint32_t n = 0;  // this wave's candidates
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        in_m[e] = __ballot(key[e] >= pv);
        n_before[e] = n;
        n += (uint32_t)__popcll(in_m[e]);
    }
    if (n <= (uint32_t)kRegion) {  // uniform
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            // the lane's bit of the kept mask selects, without a second compare
            const uint32_t at = n_before[e] + (uint32_t)lanes_below(in_m[e]);
            reg[__builtin_amdgcn_inverse_ballot_w64(in_m[e]) ? at : (uint32_t)(kRegion + lane)] =
                make_uint2(key[e], pos_of(e));
        }
    }
    if (lane == 0) sm_i[wave] = (int)n;
    if (tid == 0) sm_cnt[1] = 0;  // small bucket fill, used after later barriers
    __syncthreads();
    const int cw = lane < kWaves ? sm_i[lane & (kWaves - 1)] : 0;
    const int c = __builtin_amdgcn_readlane(wave_incl_sum(cw), 63);
    if (c < kk || __ballot(cw > kRegion) != 0) return false;  // uniform
    const int nw = (int)n, nruns = (nw + 63) / 64;  // this wave's pairs and runs of 64 (uniform)

    const uint32_t range = kmax - pv;  // kmax >= pv: some key reaches pv
    int hi = range == 0u ? 0 : 32 - __builtin_clz(range);
    int sh = hi > kTokBinBits ? hi - kTokBinBits : 0;
    // the histogram, and the OR of every candidate's bits below the bin
    // width: 0 when each bin holds a single value (as for scores rounded to
    // few mantissa bits)
    // (plain loops over the wave's runs: every instruction a wave issues here
    // costs the compute unit about 16 cycles, as all 16 waves issue it)
    uint32_t below = 0;
    {
        const uint32_t low = (1u << sh) - 1u;
#pragma unroll 1
        for (int i = lane; i < nw; i += 64) {
            const uint32_t x = reg[i].x - pv;
            atomicAdd(&hist[hist_word(x >> sh)], 1);
            below |= x & low;
        }
    }
    below = wave_or(below);
    if (lane == 0) sm_cnt[2 + wave] = (int)below;
    __syncthreads();
    below = wave_or(lane < kWaves ? (uint32_t)sm_cnt[2 + (lane & (kWaves - 1))] : 0u);

    // --- 2. v* and how many keys equal to it are kept ---
    uint32_t base = pv, vstar;
    int need = kk, keep;
    for (;;) {
        // thread t holds bins 4095 - 4t down to 4092 - 4t: a prefix sum over
        // threads is a suffix sum over bins
        const int b0 = kTokBins - 1 - 4 * tid;
        const int h3 = hist[hist_word(b0)], h2 = hist[hist_word(b0 - 1)], h1 = hist[hist_word(b0 - 2)],
                  h0 = hist[hist_word(b0 - 3)];
        const int sum = (h0 + h1) + (h2 + h3);
        const int incl = wave_incl_sum(sum);
        if (lane == 63) sm_j[wave] = incl;
        __syncthreads();
        const int excl = incl - sum + sum_below(sm_j, wave, lane);
        if (excl < need && need <= excl + sum) {  // exactly one thread
            int b = b0 - 3, nd = need - excl - h3 - h2 - h1, cb = h0;
            if (excl + h3 >= need) {
                b = b0; nd = need - excl; cb = h3;
            } else if (excl + h3 + h2 >= need) {
                b = b0 - 1; nd = need - excl - h3; cb = h2;
            } else if (excl + h3 + h2 + h1 >= need) {
                b = b0 - 2; nd = need - excl - h3 - h2; cb = h1;
            }
            sm_pick[0] = b;
            sm_pick[1] = nd;
            sm_pick[2] = cb;
        }
        __syncthreads();
        const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane(sm_pick[0]);
        need = __builtin_amdgcn_readfirstlane(sm_pick[1]);
        const int cb = __builtin_amdgcn_readfirstlane(sm_pick[2]);
        if (sh == 0 || below == 0u) {  // the bin holds one value: base + (b << sh)
            vstar = base + (b << sh);
            keep = need;
            break;
        }
        const uint32_t lo = base + (b << sh);  // the bin holds keys in [lo, lo + 2^sh)
        if (cb <= kSmallCap) {
            // gather the bin's keys (as offsets from lo), then one wave
            // decides their need-th largest bit by bit
#pragma unroll 1
            for (int r = 0; r < nruns; ++r) {
                const int i = 64 * r + lane;
                const uint32_t x = reg[i].x - lo;
                const bool in = i < nw && (x >> sh) == 0u;
                const uint64_t m = __ballot(in);
                if (m) {  // uniform
                    int at = 0;
                    if (lane == 0) at = atomicAdd(&sm_cnt[1], __popcll(m));
                    at = __builtin_amdgcn_readfirstlane(at);
                    if (in) small[at + lanes_below(m)] = x;
                }
            }
            __syncthreads();
            if (wave == 0) {
                // lanes past the bin hold 0, below every offset that can be picked
                const uint32_t di = lane < cb ? small[lane] : 0u;
                uint32_t dv;
                if (cb <= 16) {  // few keys: count, for every lane's key, the keys above it and at or above it
                    int gt = 0, ge = 0;
                    for (int j = 0; j < cb; ++j) {
                        const uint32_t dj = (uint32_t)__builtin_amdgcn_readlane((int)di, j);
                        gt += dj > di;
                        ge += dj >= di;
                    }
                    const uint64_t hm = __ballot(lane < cb && gt < need && need <= ge);  // the lanes holding v*
                    dv = (uint32_t)__builtin_amdgcn_readlane((int)di, __builtin_ctzll(hm | (1ull << 63)));
                } else {
                    dv = wave_rank_value(di, sh, need);
                }
                const int n_gt = __popcll(__ballot(lane < cb && di > dv));
                if (lane == 0) {
                    sm_pick[0] = (int)(lo + dv);
                    sm_pick[1] = need - n_gt;
                }
            }
            __syncthreads();
            vstar = (uint32_t)__builtin_amdgcn_readfirstlane(sm_pick[0]);
            keep = __builtin_amdgcn_readfirstlane(sm_pick[1]);
            break;
        }
        // a crowded bin: histogram its keys on their next bits
        base = lo;
        hi = sh;
        sh = hi > kTokBinBits ? hi - kTokBinBits : 0;
        reinterpret_cast<int4*>(hist)[tid] = make_int4(0, 0, 0, 0);
        __syncthreads();
        below = 0u;
        for (int i = lane; i < nw; i += 64) {
            const uint32_t x = reg[i].x - base;
            if ((x >> hi) == 0u) {
                atomicAdd(&hist[hist_word(x >> sh)], 1);
                below |= x & ((1u << sh) - 1u);
            }
        }
        below = wave_or(below);
        if (lane == 0) sm_cnt[2 + wave] = (int)below;
        __syncthreads();
        below = wave_or(lane < kWaves ? (uint32_t)sm_cnt[2 + (lane & (kWaves - 1))] : 0u);
    }

    // --- 3. ordered compaction, each wave over its own region ---
    // Two runs per trip with both loads issued first; the loads are
    // unconditional (a run past nw reads stale words of the wave's stride,
    // masked by i < nw), so no load waits behind a branch.
    static_assert(kRegion + 64 <= kRegionStride, "a run past the region stays in the wave's stride");
    int n_gt = 0, n_eq = 0;
#pragma unroll 1
    for (int r = 0; r < nruns; r += 2) {  // uniform trip count: the ballots see every lane
        const int i0 = 64 * r + lane, i1 = i0 + 64;
        const uint32_t x0 = reg[i0].x, x1 = reg[i1].x;
        const uint32_t k0 = i0 < nw ? x0 : 0u, k1 = i1 < nw ? x1 : 0u;  // key 0 < pv <= v*: neither
        n_gt += __popcll(__ballot(k0 > vstar)) + __popcll(__ballot(k1 > vstar));
        n_eq += __popcll(__ballot(k0 == vstar)) + __popcll(__ballot(k1 == vstar));
    }
    if (lane == 0) {
        sm_i[wave] = n_gt;
        sm_j[wave] = n_eq;
    }
    __syncthreads();
    const int gt_before = sum_below(sm_i, wave, lane), eq_before = sum_below(sm_j, wave, lane);
    int out = gt_before + min(eq_before, keep);
    int eq_seen = eq_before;
    // the outputs as buffers of kk words: a store's offset is a lane's rank
    // among the run's kept keys, its base the run's first output
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(dst, 0, kk * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(dst_key ? dst_key : reinterpret_cast<uint32_t*>(dst), 0, kk * 4,
                                          kBufferWord3);
    // The masks are combined as lane masks (ballots of plain compares and
    // scalar logic), so no bool is rebuilt from a mask and balloted again.
    auto emit = [&](const uint2 p, const bool valid) {
        const uint64_t vm = __ballot(valid);
        const uint64_t em = vm & __ballot(p.x == vstar);
        const uint64_t gm = vm & __ballot(p.x > vstar);
        const uint64_t lm = __ballot(lanes_below(em) < keep - eq_seen);  // within the keys equal to v* kept
        const uint64_t tm = gm | (em & lm);
        if (__builtin_amdgcn_inverse_ballot_w64(tm)) {
            const int at = 4 * lanes_below(tm);
            __builtin_amdgcn_raw_buffer_store_b32(p.y, ors, at, 4 * out, 0);
            if (dst_key) __builtin_amdgcn_raw_buffer_store_b32(p.x, krs, at, 4 * out, 0);  // slices hand their keys on
        }
        out += __popcll(tm);
        eq_seen += __popcll(em);
    };
#pragma unroll 1
    for (int r = 0; r < nruns; r += 2) {
        const int i0 = 64 * r + lane, i1 = i0 + 64;
        const uint2 p0 = reg[i0], p1 = reg[i1];
        // both pairs whole in registers here: a position used only under the
        // store's branch would otherwise be loaded there and waited for
        asm volatile("" ::"v"(p0.y), "v"(p1.y));
        emit(p0, i0 < nw);
        emit(p1, i1 < nw);
    }
    return true;
}

template <int KPT, int MODE>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
    constexpr bool kScoreKeys = MODE != kModeLogits;  // key 0 marks a position that does not compete
    __shared__ int sm_i[kWaves];
    __shared__ int sm_j[kWaves];
    __shared__ int sm_avail[kWaves];
    __shared__ uint32_t sm_min[kWaves], sm_max[kWaves];
    // While selecting: the histogram ([bin][copy]) and two lists that hold a
    // bucket's keys as r (below), in no particular order.  Afterwards the
    // same words hold the per-wave output regions of the compaction.
    constexpr int kRawWords = kBins * kLaneCopies + 2 * kListCap;
    __shared__ __align__(16) uint32_t sm_raw[kRawWords];
    int* const sm_hist = reinterpret_cast<int*>(sm_raw);
    uint32_t* const sm_lists = sm_raw + kBins * kLaneCopies;  // list s: sm_lists + s * kListCap
    __shared__ int sm_tot[kBins];
    __shared__ int sm_pick[3];  // digit chosen by a pass, keys still needed, keys in the digit
    __shared__ int sm_cnt[2 + kWaves];  // list fills; token rows: small-bin fill, per-wave ORs
    __shared__ uint32_t sm_pv;  // token rows: the fast select's bound
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int k = a.k;
    // the workgroup's row, slice and positions
    const int row = MODE == kModeSlice ? (int)blockIdx.x / a.n_slices : (int)blockIdx.x;
    const int slice = MODE == kModeSlice ? (int)blockIdx.x % a.n_slices : 0;
    const int row_len = MODE == kModeSlice ? a.n_list * kChunkTokens
                        : MODE == kModeCand ? a.n_slices * k : a.C;
    const int off = MODE == kModeSlice ? slice * a.C : 0;  // first position of the slice
    const int C = MODE == kModeSlice ? min(a.C, row_len - off) : row_len;  // positions here (may be <= 0 for a slice)
    int32_t* dst = MODE == kModeSlice ? a.cand_pos + (int64_t)blockIdx.x * k : a.out + (int64_t)row * k;
    uint32_t* dst_key = MODE == kModeSlice ? a.cand_key + (int64_t)blockIdx.x * k : nullptr;
    // wave w owns positions [w*64*KPT, (w+1)*64*KPT); slot e of lane l is
    // position w*64*KPT + 64*e + l, so every load instruction reads 64
    // consecutive positions
    const int wbase = wave * 64 * KPT;

    // Loads are unconditional, from clamped in-bounds indices, and all issued
    // before any is used; keys are formed without branches (a load whose
    // only use sits under a branch moves into it and waits there).
    uint32_t key[KPT];
    uint32_t cpos_e[MODE == kModeCand ? KPT : 1];  // candidates: row position of each slot's key
    int lim_l = 0;        // list rows: usable tokens of the wave's entry `lane` (lane < KPT)
    if constexpr (MODE == kModeTokens || MODE == kModeSlice) {
        // slot e of wave w is exactly list entry j = off/64 + w*KPT + e (64 tokens)
        const float* srow = a.scores + (int64_t)row * row_len;
        const int32_t* ids = a.list_ids + (int64_t)row * a.n_list;
        int kb = a.n_list;
        if (a.list_counts) {
            const int cnt = a.list_counts[row];
            kb = cnt < 0 ? 0 : cnt > a.n_list ? a.n_list : cnt;
        }
        // usable tokens of chunk c: 64 below chunk ctx/64, ctx%64 in it, none above
        const int ctx_row = a.ctx[row] > 0 ? a.ctx[row] : 0;
        const uint32_t ctx_chunk = (uint32_t)ctx_row / kChunkTokens;
        const int ctx_rem = ctx_row % kChunkTokens;
        const int j0 = off / kChunkTokens;
        // entries of this workgroup in use: j0 <= j < jend (C is a multiple of 64)
        const int jend = C > 0 ? min(kb, j0 + C / kChunkTokens) : 0;
        // lane e < KPT loads the id of the wave's slot e (KPT <= 64)
        const int jl = j0 + wave * KPT + lane;
        // Buffer loads with the row as the buffer: a position past the row's
        // end reads 0 (it lies in no entry in use, so it never competes), and
        // slot e's offset is an immediate: no address arithmetic per slot.
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(srow), 0, row_len * 4, kBufferWord3);
        // The fast select's sample, drawn by wave 0 ahead of its own keys so
        // that its rank is found while the row's loads are in flight: lane
        // l takes token (29 l + 7) mod 64 of list entry l * n_list / 64, as a
        // 12-bit key prefix (0 where the token is not usable).
        const bool sampler = wave == 0 && a.sample_rank > 0;  // uniform
        // sample s = lane and lane + 64: token (29 s + 7) mod 64 of list entry
        // j0 + s * E / 128 of the workgroup's E = C / 64 entries
        const int n_ent = C > 0 ? C / kChunkTokens : 0;
        const int js0 = j0 + (int)(((int64_t)lane * n_ent) / kSamples);
        const int js1 = j0 + (int)(((int64_t)(lane + 64) * n_ent) / kSamples);
        const int ts0 = (29 * lane + 7) & (kChunkTokens - 1), ts1 = (29 * (lane + 64) + 7) & (kChunkTokens - 1);
        uint32_t cs0 = 0, cs1 = 0;
        float vs0 = 0.0f, vs1 = 0.0f;
        if (sampler && n_ent > 0) {
            cs0 = (uint32_t)ids[js0];
            cs1 = (uint32_t)ids[js1];
            vs0 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (64 * js0 + ts0) * 4, 0, 0));
            vs1 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (64 * js1 + ts1) * 4, 0, 0));
        }
        const int32_t cidv = ids[jl < a.n_list ? jl : a.n_list - 1];
        const int vo = (off + wbase + lane) * 4;  // byte offset of slot 0
        float sc[KPT];
#pragma unroll
        for (int e = 0; e < KPT; ++e)
            sc[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, vo + 256 * e, 0, 0));
        if (sampler) {
            auto prefix = [&](int js, int ts, uint32_t cs, float vs) {  // 0 where the token is not usable
                const int lims = js < jend ? (cs < ctx_chunk ? kChunkTokens : cs == ctx_chunk ? ctx_rem : 0) : 0;
                return ts < lims ? score_key(vs) >> (32 - kSampleBits) : 0u;
            };
            const uint32_t p = wave_rank_value2(prefix(js0, ts0, cs0, vs0), prefix(js1, ts1, cs1, vs1), kSampleBits,
                                                a.sample_rank);
            if (lane == 0) sm_pv = p << (32 - kSampleBits);
        }
        // tokens of entry j below the context length: 64 below chunk ctx/64,
        // ctx%64 in it, none above it or in an entry not in use
        const uint32_t cidl = (uint32_t)cidv;
        lim_l = lane < KPT && jl < jend ? (cidl < ctx_chunk ? kChunkTokens : cidl == ctx_chunk ? ctx_rem : 0) : 0;
        if (__ballot(lane < KPT && lim_l != kChunkTokens) == 0) {  // uniform: every slot of the wave usable
#pragma unroll
            for (int e = 0; e < KPT; ++e) key[e] = score_key(sc[e]);
        } else {
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const int lim = __builtin_amdgcn_readlane(lim_l, e);
                key[e] = lane < lim ? score_key(sc[e]) : 0u;
            }
        }
    } else if constexpr (MODE == kModeCand) {
        const uint32_t* krow = a.cand_key + (int64_t)row * C;
        const int32_t* prow = a.cand_pos + (int64_t)row * C;
        // the fast select's sample: keys s * C / 128 for s = lane, lane + 64
        const bool sampler = wave == 0 && a.sample_rank > 0;  // uniform
        uint32_t ks0 = 0, ks1 = 0;
        if (sampler) {
            ks0 = krow[(int)(((int64_t)lane * C) / kSamples)];
            ks1 = krow[(int)(((int64_t)(lane + 64) * C) / kSamples)];
        }
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int idx = wbase + 64 * e + lane;
            key[e] = krow[idx < C ? idx : C - 1];
        }
        if (a.sample_rank > 0) {  // the fast select keeps each key's row position with it
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const int idx = wbase + 64 * e + lane;
                cpos_e[e] = (uint32_t)prow[idx < C ? idx : C - 1];
            }
        }
        if (sampler) {
            const uint32_t p = wave_rank_value2(ks0 >> (32 - kSampleBits), ks1 >> (32 - kSampleBits), kSampleBits,
                                                a.sample_rank);
            if (lane == 0) sm_pv = p << (32 - kSampleBits);
        }
#pragma unroll
        for (int e = 0; e < KPT; ++e) key[e] &= 0u - (uint32_t)(wbase + 64 * e + lane < C);
    } else {
        const int32_t* lrow = a.logits + (int64_t)row * C;
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int idx = wbase + 64 * e + lane;
            key[e] = (uint32_t)lrow[idx < C ? idx : C - 1] ^ 0x80000000u;
        }
    }

    if constexpr (!kScoreKeys) {
        // A position past the row takes key 0, the smallest key, behind every
        // real key of that value in position order: it is never selected (at
        // most the C real keys are) and moves no pick (it can only add to the
        // lowest bucket); the range below is taken over real keys only.
#pragma unroll
        for (int e = 0; e < KPT; ++e) key[e] = wbase + 64 * e + lane < C ? key[e] : 0u;
    }

    // --- range and keep count ---
    // Score keys: the minimum is taken over key - 1, so that key 0 (not
    // competing) wraps to the top and drops out; 1 is added back below.
    const bool capped = kScoreKeys || a.counts != nullptr;
    const uint32_t tkey = kScoreKeys ? 0u : ((uint32_t)a.thr ^ 0x80000000u);
    // List rows: the competing keys are exactly the usable positions (no
    // score is NaN, so no usable position has key 0), counted from lim_l.
    // Token rows take the minimum only if the full select runs (below).
    constexpr bool kListRows = MODE == kModeTokens || MODE == kModeSlice;
    uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
    int avail = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        if constexpr (kListRows) {
            if constexpr (MODE == kModeSlice) lmin = min(lmin, key[e] - 1u);
            lmax = max(lmax, key[e]);
        } else if constexpr (kScoreKeys) {
            lmin = min(lmin, key[e] - 1u);
            lmax = max(lmax, key[e]);
            avail += __popcll(__ballot(key[e] != 0u));
        } else {
            const bool o = wbase + 64 * e + lane < C;
            lmin = min(lmin, o ? key[e] : 0xFFFFFFFFu);
            lmax = max(lmax, o ? key[e] : 0u);
            if (capped) avail += __popcll(__ballot(o && key[e] > tkey));
        }
    }
    if constexpr (kListRows) avail = __builtin_amdgcn_readlane(wave_incl_sum(lim_l), 63);
    if constexpr (MODE != kModeTokens) lmin = wave_min(lmin);
    lmax = wave_max(lmax);
    if (lane == 0) {
        if constexpr (MODE != kModeTokens) sm_min[wave] = lmin;
        sm_max[wave] = lmax;
        sm_avail[wave] = avail;
    }
    if (tid == 0) sm_cnt[0] = 0;
    if constexpr (MODE != kModeLogits) {
        // the fast select's histogram starts at zero
        if (a.sample_rank > 0) reinterpret_cast<int4*>(sm_raw)[tid] = make_int4(0, 0, 0, 0);
    }
    __syncthreads();
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    avail = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if constexpr (MODE != kModeTokens) kmin = min(kmin, sm_min[w]);
        kmax = max(kmax, sm_max[w]);
        avail += sm_avail[w];
    }
    // values read back from LDS are the same in every lane: say so, so that
    // they live in scalar registers and the control flow on them stays scalar
    kmin = __builtin_amdgcn_readfirstlane(kmin);
    kmax = __builtin_amdgcn_readfirstlane(kmax);
    avail = __builtin_amdgcn_readfirstlane(avail);
    if constexpr (kScoreKeys) kmin += 1u;  // (no competing key: avail == 0, unused)

    // --- how many to keep ---
    int kk = k;
    if (capped) {
        kk = avail < k ? avail : k;
        if (MODE != kModeSlice && tid == 0) a.counts[row] = kk;
        for (int j = kk + tid; j < k; j += kThreads) {
            dst[j] = -1;
            if constexpr (MODE == kModeSlice) dst_key[j] = 0u;
        }
        if (kk == 0) return;  // uniform: every thread saw the same sum
    }
    const int n_ok = kScoreKeys ? avail : C;  // competing keys

    if constexpr (MODE != kModeLogits) {
        // the position a kept key is written as
        auto pos_of = [&](int e) -> uint32_t {
            if constexpr (MODE == kModeCand) return cpos_e[e];
            else return (uint32_t)(off + wbase + 64 * e + lane);
        };
        if (a.sample_rank > 0 && kk < n_ok &&
            tokens_fast_select<KPT>(key, pos_of, kk, kmax, sm_pv ? sm_pv : 1u, tid, lane, wave, sm_raw, sm_i, sm_j,
                                    sm_cnt, sm_pick, dst, dst_key))
            return;
    }
    if constexpr (MODE == kModeTokens) {
        // the full select below works on key - (the smallest competing key)
        uint32_t m = 0xFFFFFFFFu;
#pragma unroll
        for (int e = 0; e < KPT; ++e) m = min(m, key[e] - 1u);
        m = wave_min(m);
        if (lane == 0) sm_min[wave] = m;
        __syncthreads();
        kmin = 0xFFFFFFFFu;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) kmin = min(kmin, sm_min[w]);
        kmin = __builtin_amdgcn_readfirstlane(kmin) + 1u;
    }

    // --- radix select ---
    // On r = key - kmin: a competing key has r in [0, range].  A score key
    // that does not compete is 0, so r wraps above range (kmin >= 1 and
    // kmax < 2^32), and every test below bounds r by range; a logits position
    // past the row has key 0 too: outside every bucket unless kmin is 0, and
    // then the smallest value, as above.
    const uint32_t range = kmax - kmin;
    // The bits of r* (the kk-th largest r) are decided from the top; the
    // current bucket holds the keys that agree with r* on the decided bits
    // (cnt keys, of which `need` are kept): r in [rstar, rstar + ub].
    int hi = range == 0u ? 0 : 32 - __builtin_clz(range);  // bits [0, hi) of r* are undecided
    if (kk == n_ok) hi = 0;  // every competing key is kept: r* = 0 will do
    uint32_t rstar = 0;      // decided bits of r*, in place
    int need = kk, cnt = n_ok;
    int src = -1;            // the bucket is in registers (-1) or in list src
    auto bucket_ub = [&](int h) {  // key - (kmin + rstar) <= ub <=> key in the bucket (and r <= range)
        const uint32_t span = h >= 32 ? 0xFFFFFFFFu : (1u << h) - 1u;
        return min(span, range - rstar);
    };
    while (hi > 0) {
        if (src >= 0 && cnt <= kBallotMax) {
            // one wave decides the remaining bits, high to low: with c1 keys
            // of the bucket having the bit set, the bit of r* is 1 iff
            // need <= c1; the bucket keeps the keys that agree
            if (wave == 0) {
                if (cnt <= 64)
                    ballot_finish<1>(sm_lists + src * kListCap, cnt, hi, need, lane, sm_pick);
                else
                    ballot_finish<kBallotSlots>(sm_lists + src * kListCap, cnt, hi, need, lane, sm_pick);
            }
            __syncthreads();
            rstar |= (uint32_t)__builtin_amdgcn_readfirstlane(sm_pick[0]);
            need = __builtin_amdgcn_readfirstlane(sm_pick[1]);
            cnt = __builtin_amdgcn_readfirstlane(sm_pick[2]);
            break;
        }
        // one histogram pass over the next (up to) 8 bits
        const int w = hi < kDigitBits ? hi : kDigitBits;
        const int sh = hi - w;
        const uint32_t dmask = (1u << w) - 1u;
        const int nxt = src < 0 ? 0 : 1 - src;  // list the next bucket may move to
        {
            int4* h4 = reinterpret_cast<int4*>(sm_hist);
            for (int j = tid; j < kBins * kLaneCopies / 4; j += kThreads) h4[j] = make_int4(0, 0, 0, 0);
        }
        __syncthreads();
        if (tid == 0) sm_cnt[nxt] = 0;  // ordered before its use by the barriers of pick_digit
        if (src < 0) {
            const uint32_t ub = bucket_ub(hi);
            const uint32_t base = kmin + rstar;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const uint32_t d = key[e] - base;
                if (d <= ub) atomicAdd(&sm_hist[(int)(d >> sh) * kLaneCopies + lane], 1);
            }
        } else {
            const uint32_t* lst = sm_lists + src * kListCap;
            for (int i = tid; i < cnt; i += kThreads)
                atomicAdd(&sm_hist[(int)((lst[i] >> sh) & dmask) * kLaneCopies + lane], 1);
        }
        __syncthreads();
        pick_digit<kLaneCopies>(sm_hist, sm_tot, sm_pick, tid, lane, wave, need);
        const uint32_t dg = (uint32_t)__builtin_amdgcn_readfirstlane(sm_pick[0]);
        const int cnt_in = cnt;
        need = __builtin_amdgcn_readfirstlane(sm_pick[1]);
        cnt = __builtin_amdgcn_readfirstlane(sm_pick[2]);
        rstar |= dg << sh;
        hi = sh;
        if (hi > 0 && cnt <= kListCap) {
            // move the new bucket into list nxt: per wave, one LDS atomic
            // reserves the places of its keys (the bucket tests are
            // recomputed rather than kept, to spare scalar registers)
            uint32_t* out = sm_lists + nxt * kListCap;
            if (src < 0) {
                const uint32_t ub = bucket_ub(hi);
                const uint32_t base = kmin + rstar;
                int n = 0;
#pragma unroll
                for (int e = 0; e < KPT; ++e) n += __popcll(__ballot(key[e] - base <= ub));
                int at = 0;
                if (lane == 0 && n > 0) at = atomicAdd(&sm_cnt[nxt], n);
                at = __builtin_amdgcn_readfirstlane(at);
#pragma unroll
                for (int e = 0; e < KPT; ++e) {
                    const bool in = key[e] - base <= ub;
                    const uint64_t mk = __ballot(in);
                    if (in) out[at + lanes_below(mk)] = key[e] - kmin;
                    at += __popcll(mk);
                }
            } else {
                const uint32_t* in = sm_lists + src * kListCap;
                for (int i0 = 0; i0 < cnt_in; i0 += kThreads) {
                    const int i = i0 + tid;
                    const uint32_t r = in[i < cnt_in ? i : 0];
                    const bool match = i < cnt_in && ((r >> sh) & dmask) == dg;
                    const uint64_t mk = __ballot(match);
                    int base = 0;
                    if (lane == 0 && mk != 0) base = atomicAdd(&sm_cnt[nxt], __popcll(mk));
                    base = __builtin_amdgcn_readfirstlane(base);
                    if (match) out[base + lanes_below(mk)] = r;
                }
            }
            src = nxt;
            __syncthreads();
        }
    }
    // every key equal to r* is kept: the selection is exactly the keys >= r*
    const bool all_eq = need == cnt;

    // --- ordered compaction ---
    // ge <=> v* <= key <= kmax, gt <=> v* < key <= kmax, eq <=> key == v*.
    const uint32_t vstar = kmin + rstar;
    const uint32_t top = kmax - vstar;
    auto ge = [&](int e) { return key[e] - vstar <= top; };
    auto gt = [&](int e) { return key[e] - vstar - 1u < top; };
    auto eq = [&](int e) { return key[e] == vstar; };
    // the output of slot e taken at place p
    auto emit = [&](int p, int e) {
        const int idx = wbase + 64 * e + lane;
        if constexpr (MODE == kModeSlice) {
            dst[p] = off + idx;
            dst_key[p] = key[e];
        } else if constexpr (MODE == kModeCand) {
            dst[p] = a.cand_pos[(int64_t)row * C + idx];
        } else {
            dst[p] = idx;
        }
    };
    // The selection in position order: keys > r*, and the first `need` keys
    // == r* (all of them when all_eq).  Waves come one after the other in
    // position order, so exclusive scans over per-wave totals place each
    // wave's outputs.  The select reads the histogram and the lists no more
    // (its last step ended with a barrier): their words take the regions.
    constexpr int kEntryWords = MODE == kModeSlice ? 2 : 1;  // position (and key)
    constexpr int kRegionWords = 64 * KPT * kEntryWords;
    if constexpr (kWaves * kRegionWords <= kRawWords) {
        // One sweep: every wave appends its keys >= r* to its own region in
        // position order (an equal key flagged in bit 31; positions < 2^30),
        // then, after one barrier, copies the ones taken to the output with
        // coalesced stores.
        uint32_t* reg = sm_raw + wave * kRegionWords;
        int n_ge = 0, n_eq = 0;
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const bool in = ge(e);
            const uint64_t m = __ballot(in);
            if (in) {
                const int i = n_ge + lanes_below(m);
                const uint32_t idx = (uint32_t)(wbase + 64 * e + lane);
                const uint32_t ent = all_eq || !eq(e) ? idx : idx | 0x80000000u;
                if constexpr (MODE == kModeSlice) {
                    reg[2 * i] = ent;
                    reg[2 * i + 1] = key[e];
                } else {
                    reg[i] = ent;
                }
            }
            n_ge += __popcll(m);
            if (!all_eq) n_eq += __popcll(__ballot(eq(e)));
        }
        if (lane == 0) {
            sm_i[wave] = n_ge;
            sm_j[wave] = n_eq;
        }
        __syncthreads();
        int ge_before = 0, eq_before = 0;
        for (int w = 0; w < wave; ++w) {
            ge_before += sm_i[w];
            eq_before += sm_j[w];
        }
        ge_before = __builtin_amdgcn_readfirstlane(ge_before);
        eq_before = __builtin_amdgcn_readfirstlane(eq_before);
        // equal keys are taken in position order: min(eq_before, need) of them precede
        int pos = all_eq ? ge_before : ge_before - eq_before + (eq_before < need ? eq_before : need);
        int eq_seen = eq_before;
        for (int i0 = 0; i0 < n_ge; i0 += 64) {
            const int i = i0 + lane;
            const bool valid = i < n_ge;
            const uint32_t v = reg[kEntryWords * (valid ? i : 0)];
            bool take = valid;
            if (!all_eq) {
                const bool is_eq = valid && (v >> 31) != 0u;
                const uint64_t eqm = __ballot(is_eq);
                take = valid && (!is_eq || eq_seen + lanes_below(eqm) < need);
                eq_seen += __popcll(eqm);
            }
            const uint64_t tm = __ballot(take);
            const int p = pos + lanes_below(tm);
            // p < kk for every real key; the test also drops a logits position past the row
            if (take && p < kk) {
                const int idx = (int)(v & 0x7FFFFFFFu);
                if constexpr (MODE == kModeSlice) {
                    dst[p] = off + idx;
                    dst_key[p] = reg[2 * i + 1];
                } else if constexpr (MODE == kModeCand) {
                    dst[p] = a.cand_pos[(int64_t)row * C + idx];
                } else {
                    dst[p] = idx;
                }
            }
            pos += __popcll(tm);
        }
    } else {
        // Two sweeps over the registers: per-wave totals (keys taken when
        // all_eq, else keys > r* and keys == r*), then the outputs.
        int n_a = 0, n_b = 0;
        if (all_eq) {
#pragma unroll
            for (int e = 0; e < KPT; ++e) n_a += __popcll(__ballot(ge(e)));
        } else {
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                n_a += __popcll(__ballot(gt(e)));
                n_b += __popcll(__ballot(eq(e)));
            }
        }
        if (lane == 0) {
            sm_i[wave] = n_a;
            sm_j[wave] = n_b;
        }
        __syncthreads();
        int a_before = 0, b_before = 0;
        for (int w = 0; w < wave; ++w) {
            a_before += sm_i[w];
            b_before += sm_j[w];
        }
        a_before = __builtin_amdgcn_readfirstlane(a_before);
        b_before = __builtin_amdgcn_readfirstlane(b_before);
        // p < kk holds for every real key by construction; the tests keep every
        // store inside the row even so (and drop a logits position past the row)
        if (all_eq) {
            int pos = a_before;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const bool take = ge(e);
                const uint64_t tm = __ballot(take);
                const int p = pos + lanes_below(tm);
                if (take && p < kk) emit(p, e);
                pos += __popcll(tm);
            }
        } else {
            // equal keys are taken in position order: min(b_before, need) of them precede
            int pos = a_before + (b_before < need ? b_before : need);
            int eq_seen = b_before;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                bool take = gt(e);
                const uint64_t eqm = __ballot(eq(e));
                if (eqm != 0) {
                    take = take || (eq(e) && eq_seen + lanes_below(eqm) < need);
                    eq_seen += __popcll(eqm);
                }
                const uint64_t tm = __ballot(take);
                const int p = pos + lanes_below(tm);
                if (take && p < kk) emit(p, e);
                pos += __popcll(tm);
            }
        }
    }
}

// Rows too long for the keys to stay in registers (more than 64 per
// thread): the same select, streaming the row from memory in every phase
// instead (it stays in L2 between phases).  Wave w owns positions
// [64*S*w, 64*S*(w+1)), S = slots per wave; slot e of lane l is position
// 64*S*w + 64e + l, loaded in batches of kBatch slots (clamped,
// unconditional loads issued before use).
constexpr int kBatch = 8;

template <bool TOK>
__global__ __launch_bounds__(kThreads) void topk_stream_kernel(TopkArgs a) {
    __shared__ int sm_i[kWaves];
    __shared__ int sm_j[kWaves];
    __shared__ int sm_avail[kWaves];
    __shared__ uint32_t sm_min[kWaves], sm_max[kWaves];
    __shared__ __align__(16) int sm_hist[kBins * kCopies];  // [bin][copy]
    __shared__ int sm_tot[kBins];
    __shared__ int sm_pick[3];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int C = a.C, k = a.k;
    int32_t* dst = a.out + (int64_t)blockIdx.x * k;
    const int S = (C + 64 * kWaves - 1) / (64 * kWaves);
    const int wbase = wave * 64 * S;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    const float* srow = TOK ? a.scores + (int64_t)blockIdx.x * C : nullptr;
    const int32_t* lrow = TOK ? nullptr : a.logits + (int64_t)blockIdx.x * C;
    const int32_t* ids = TOK ? a.list_ids + (int64_t)blockIdx.x * a.n_list : nullptr;
    int kb = 0;
    int64_t ctx = 0;
    if constexpr (TOK) {
        kb = a.n_list;
        if (a.list_counts) {
            const int cnt = a.list_counts[blockIdx.x];
            kb = cnt < 0 ? 0 : cnt > a.n_list ? a.n_list : cnt;
        }
        ctx = a.ctx[blockIdx.x];
    }
    // body(e, key, ok) for every slot e of this wave, in slot order
    auto for_each_slot = [&](auto&& body) {
        for (int e0 = 0; e0 < S; e0 += kBatch) {
            uint32_t key[kBatch];
            bool ok[kBatch];
            if constexpr (TOK) {
                float v[kBatch];
                int32_t cid[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int p = wbase + 64 * (e0 + u) + lane;
                    v[u] = srow[p < C ? p : C - 1];
                    const int j = wave * S + e0 + u;  // list entry of the slot (position 64j + lane)
                    cid[u] = ids[j < a.n_list ? j : a.n_list - 1];
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int j = wave * S + e0 + u;
                    ok[u] = e0 + u < S && j < kb && (int64_t)cid[u] * kChunkTokens + lane < ctx;
                    key[u] = ok[u] ? score_key(v[u]) : 0u;
                }
            } else {
                int32_t v[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int p = wbase + 64 * (e0 + u) + lane;
                    v[u] = lrow[p < C ? p : C - 1];
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    ok[u] = e0 + u < S && wbase + 64 * (e0 + u) + lane < C;
                    key[u] = (uint32_t)v[u] ^ 0x80000000u;
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (e0 + u < S) body(e0 + u, key[u], ok[u]);  // wave-uniform condition
        }
    };

    // --- range and keep count ---
    const bool capped = TOK || a.counts != nullptr;
    const uint32_t tkey = TOK ? 0u : ((uint32_t)a.thr ^ 0x80000000u);
    uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
    int avail = 0;
    for_each_slot([&](int, uint32_t key, bool ok) {
        if (ok) {
            lmin = min(lmin, key);
            lmax = max(lmax, key);
        }
        if (capped) avail += __popcll(__ballot(ok && (TOK || key > tkey)));
    });
    lmin = wave_min(lmin);
    lmax = wave_max(lmax);
    if (lane == 0) {
        sm_min[wave] = lmin;
        sm_max[wave] = lmax;
        sm_avail[wave] = avail;
    }
    __syncthreads();
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    avail = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        kmin = min(kmin, sm_min[w]);
        kmax = max(kmax, sm_max[w]);
        avail += sm_avail[w];
    }
    kmin = __builtin_amdgcn_readfirstlane(kmin);  // the same in every lane
    kmax = __builtin_amdgcn_readfirstlane(kmax);
    avail = __builtin_amdgcn_readfirstlane(avail);
    int kk = k;
    if (capped) {
        kk = avail < k ? avail : k;
        if (tid == 0) a.counts[blockIdx.x] = kk;
        for (int j = kk + tid; j < k; j += kThreads) dst[j] = -1;
        if (kk == 0) return;  // uniform
    }

    // --- radix select on key - kmin, 8 bits per pass ---
    const uint32_t range = kmax - kmin;
    const int nb = range == 0u ? 0 : 32 - __builtin_clz(range);
    uint64_t prefix = 0;
    int need = kk;
    const int copy = lane % kCopies;
    for (int hi = nb; hi > 0; hi -= kDigitBits) {
        const int w = hi < kDigitBits ? hi : kDigitBits;
        const int sh = hi - w;
        for (int j = tid; j < kBins * kCopies; j += kThreads) sm_hist[j] = 0;
        __syncthreads();
        for_each_slot([&](int, uint32_t key, bool ok) {
            const uint64_t r = key - kmin;
            if (ok && (r >> hi) == prefix) atomicAdd(&sm_hist[(int)((r >> sh) & ((1u << w) - 1u)) * kCopies + copy], 1);
        });
        __syncthreads();
        pick_digit<kCopies>(sm_hist, sm_tot, sm_pick, tid, lane, wave, need);
        prefix = (prefix << w) | (uint64_t)__builtin_amdgcn_readfirstlane(sm_pick[0]);
        need = __builtin_amdgcn_readfirstlane(sm_pick[1]);
    }
    const uint32_t vstar = kmin + (uint32_t)prefix;

    // --- ordered compaction ---
    int n_gt = 0, n_eq = 0;
    for_each_slot([&](int, uint32_t key, bool ok) {
        n_gt += __popcll(__ballot(ok && key > vstar));
        n_eq += __popcll(__ballot(ok && key == vstar));
    });
    if (lane == 0) {
        sm_i[wave] = n_gt;
        sm_j[wave] = n_eq;
    }
    __syncthreads();
    int gt_before = 0, eq_before = 0;
    for (int w = 0; w < wave; ++w) {
        gt_before += sm_i[w];
        eq_before += sm_j[w];
    }
    gt_before = __builtin_amdgcn_readfirstlane(gt_before);  // the same in every lane
    eq_before = __builtin_amdgcn_readfirstlane(eq_before);
    int pos = gt_before + (eq_before < need ? eq_before : need);
    int eq_seen = eq_before;
    for_each_slot([&](int e, uint32_t key, bool ok) {
        const bool gt = ok && key > vstar;
        const bool eq = ok && key == vstar;
        const uint64_t eqm = __ballot(eq);
        const bool take = gt || (eq && eq_seen + __popcll(eqm & below) < need);
        const uint64_t tm = __ballot(take);
        const int p = pos + __popcll(tm & below);
        if (take && p < kk) dst[p] = wbase + 64 * e + lane;  // p < kk by construction
        pos += __popcll(tm);
        eq_seen += __popcll(eqm);
    });
}

// Rows of at least this many positions stream from memory (the
// LSA_TUNE_TOPK_STREAM_MIN_C knob; by default rows beyond the register
// kernel's 65536 positions).
int stream_min_c() { return tuning(LSA_TUNE_TOPK_STREAM_MIN_C); }

template <int MODE>
hipError_t launch_mode(const TopkArgs& a, int grid, int positions, hipStream_t stream) {
    const int kpt = (positions + kThreads - 1) / kThreads;
    const dim3 g((unsigned)grid), block(kThreads);
    if (kpt <= 1) hipLaunchKernelGGL((topk_kernel<1, MODE>), g, block, 0, stream, a);
    else if (kpt <= 2) hipLaunchKernelGGL((topk_kernel<2, MODE>), g, block, 0, stream, a);
    else if (kpt <= 4) hipLaunchKernelGGL((topk_kernel<4, MODE>), g, block, 0, stream, a);
    else if (kpt <= 8) hipLaunchKernelGGL((topk_kernel<8, MODE>), g, block, 0, stream, a);
    else if (kpt <= 12) hipLaunchKernelGGL((topk_kernel<12, MODE>), g, block, 0, stream, a);
    else if (kpt <= 13) hipLaunchKernelGGL((topk_kernel<13, MODE>), g, block, 0, stream, a);
    else if (kpt <= 14) hipLaunchKernelGGL((topk_kernel<14, MODE>), g, block, 0, stream, a);
    else if (kpt <= 15) hipLaunchKernelGGL((topk_kernel<15, MODE>), g, block, 0, stream, a);
    else if (kpt <= 16) hipLaunchKernelGGL((topk_kernel<16, MODE>), g, block, 0, stream, a);
    else if (kpt <= 18) hipLaunchKernelGGL((topk_kernel<18, MODE>), g, block, 0, stream, a);
    else if (kpt <= 20) hipLaunchKernelGGL((topk_kernel<20, MODE>), g, block, 0, stream, a);
    else if (kpt <= 24) hipLaunchKernelGGL((topk_kernel<24, MODE>), g, block, 0, stream, a);
    else if (kpt <= 32) hipLaunchKernelGGL((topk_kernel<32, MODE>), g, block, 0, stream, a);
    else if (kpt <= 48) hipLaunchKernelGGL((topk_kernel<48, MODE>), g, block, 0, stream, a);
    else if (kpt <= 64) hipLaunchKernelGGL((topk_kernel<64, MODE>), g, block, 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Rank, among the 128 sample keys, whose 12-bit prefix bounds the token
// candidates: the expected rank of the k_tok-th largest key (128 k/n), plus
// three binomial standard deviations and 4, so that fewer than k_tok keys
// reach the bound only rarely (the full select then runs).  0 (no candidate
// path) when the bound would keep most of the row anyway.
int token_sample_rank(int n, int k_tok) {
    if (n <= 0 || k_tok >= n) return 0;
    const double S = kSamples, p = (double)k_tok / n;
    const double r = S * p + 3.0 * sqrt(S * p * (1.0 - p)) + 4.0;
    return r > 0.75 * S ? 0 : (int)ceil(r);
}

}  // namespace

// Split of a token row of 64*n_list positions into slices for the
// slice + candidates path, for rows of more than 32768 positions (measured:
// at 17,664 positions one workgroup per row is faster, 19.5 against 23.8 us
// for 16 rows; at 50,048 the split takes 36 against 73 us, at 104,832 43
// against 165 us); the LSA_TUNE_TOPK_SPLIT_MIN_N knob moves the bound for
// testing.  About n / (8 k_tok) slices (at most 16), each a multiple of 64
// positions; none (slices = 0) when that gives fewer than 2 or the slices or
// candidates would not fit the register-resident kernel.
TopkSplit topk_tokens_split(int n_list, int k_tok) {
    TopkSplit sp{0, 0};
    const int64_t n = (int64_t)n_list * kChunkTokens;
    const int64_t min_n = tuning(LSA_TUNE_TOPK_SPLIT_MIN_N);  // 32769 unless overridden
    if (n < min_n) return sp;
    // ceil(n / (8 k_tok)) slices: a sweep at 8 x 50,048 and 4 x 104,832
    // positions (k_tok = 2048) was fastest at 4-6 slices (more slices grow
    // the candidates' select, fewer the slices'); the
    // LSA_TUNE_TOPK_SPLIT_SLICES knob overrides the count for tuning
    int64_t P = (n + 8 * (int64_t)k_tok - 1) / (8 * (int64_t)k_tok);
    if (P > 16) P = 16;
    if (const int32_t ov = tuning(LSA_TUNE_TOPK_SPLIT_SLICES)) P = ov;
    if (P < 2) return sp;
    int64_t L = (n + P - 1) / P;
    L = (L + kChunkTokens - 1) / kChunkTokens * kChunkTokens;
    P = (n + L - 1) / L;
    if (P < 2 || L > kTopkRegisterMaxC || P * k_tok > kTopkRegisterMaxC) return sp;
    sp.slices = (int)P;
    sp.slice_len = (int)L;
    return sp;
}

size_t topk_tokens_workspace_bytes(int R, int n_list, int k_tok) {
    const TopkSplit sp = topk_tokens_split(n_list, k_tok);
    if (sp.slices == 0) return 0;
    const size_t n = (size_t)R * sp.slices * k_tok;
    return round256(n * sizeof(int32_t)) + n * sizeof(uint32_t);
}

hipError_t launch_topk(const int32_t* logits, int R, int C, int k, int32_t* chunk_ids, int32_t thr, int32_t* counts,
                       hipStream_t stream) {
    TopkArgs a{};
    a.logits = logits;
    a.C = C;
    a.k = k;
    a.thr = thr;
    a.out = chunk_ids;
    a.counts = counts;
    if (C >= stream_min_c()) {
        hipLaunchKernelGGL((topk_stream_kernel<false>), dim3((unsigned)R), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
    }
    return launch_mode<kModeLogits>(a, R, C, stream);
}

hipError_t launch_topk_tokens(const float* scores, const int32_t* list_ids, const int32_t* list_counts,
                              const int32_t* ctx, int R, int n_list, int k_tok, int32_t* tok, int32_t* tok_counts,
                              void* workspace, hipStream_t stream) {
    TopkArgs a{};
    a.scores = scores;
    a.list_ids = list_ids;
    a.list_counts = list_counts;
    a.ctx = ctx;
    a.n_list = n_list;
    a.C = n_list * kChunkTokens;
    a.k = k_tok;
    a.out = tok;
    a.counts = tok_counts;
    const TopkSplit sp = workspace ? topk_tokens_split(n_list, k_tok) : TopkSplit{0, 0};
    if (sp.slices > 0) {
        // every slice's top k_tok, then the top k_tok of those candidates
        char* w = static_cast<char*>(workspace);
        const size_t n = (size_t)R * sp.slices * k_tok;
        a.cand_pos = reinterpret_cast<int32_t*>(w);
        a.cand_key = reinterpret_cast<uint32_t*>(w + round256(n * sizeof(int32_t)));
        a.n_slices = sp.slices;
        a.C = sp.slice_len;
        a.sample_rank = token_sample_rank(sp.slice_len, k_tok);
        hipError_t e = launch_mode<kModeSlice>(a, R * sp.slices, sp.slice_len, stream);
        if (e != hipSuccess) return e;
        a.sample_rank = token_sample_rank(sp.slices * k_tok, k_tok);
        return launch_mode<kModeCand>(a, R, sp.slices * k_tok, stream);
    }
    if (a.C >= stream_min_c()) {
        hipLaunchKernelGGL((topk_stream_kernel<true>), dim3((unsigned)R), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
    }
    a.sample_rank = token_sample_rank(a.C, k_tok);
    return launch_mode<kModeTokens>(a, R, a.C, stream);
}

}  // namespace lsa
