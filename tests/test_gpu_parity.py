"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the same
seeded inputs: logits and selections bit-exact, sigmoid scores within 1e-6
relative, attention within max-abs 1e-2 / mean-abs 1e-3 of fp64."""
import math

import numpy as np
import pytest

from conftest import gpu_available
from helpers import check_attention, check_scores, to_dev, to_dev_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def lsa():
    import lookahead_chunk_sparse_amd as m
    return m


@pytest.fixture(scope="module")
def W():
    from synth import workloads
    return workloads


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ index score

@pytest.mark.parametrize("B,nq,C,d_idx,lo,hi", [
    (1, 1, 64, 64, -16, 15),
    (3, 1, 65, 128, -16, 15),
    (2, 3, 1, 128, -128, 127),
    (2, 2, 1000, 16, -128, 127),
    (1, 1, 777, 32, -128, 127),
    (4, 1, 513, 256, -128, 127),
    (1, 5, 129, 64, -128, 127),
])
def test_index_score_shapes(lsa, oracle_lib, synth_lib, B, nq, C, d_idx, lo, hi):
    say("index_score", B, nq, C, d_idx)
    s = synth_lib.stream
    q = synth_lib.uniform_i8((B, nq, d_idx), 21, s(synth_lib.TAG_MISC, 500 + C), lo, hi)
    K = synth_lib.uniform_i8((B, C, d_idx), 21, s(synth_lib.TAG_MISC, 600 + C), lo, hi)
    alpha = 1.0 / (16 * d_idx)
    logits, scores = lsa.lsa_index_score(to_dev(q), to_dev(K), alpha)
    L_ref = oracle_lib.index_logits(q, K)
    assert np.array_equal(logits.cpu().numpy().reshape(L_ref.shape), L_ref)
    check_scores(scores.cpu().numpy().reshape(L_ref.shape), oracle_lib.index_scores(L_ref, alpha))


def test_index_score_extremes(lsa, oracle_lib):
    """Largest-magnitude logits (+-2^21) and a non-power-of-two alpha."""
    q = np.full((1, 1, 128), -128, dtype=np.int8)
    K = np.stack([np.full(128, -128), np.full(128, 127), np.zeros(128), np.full(128, 1)]).astype(np.int8)[None]
    for alpha in (2.0 ** -11, 0.1, 3e-5):
        logits, scores = lsa.lsa_index_score(to_dev(q), to_dev(K), alpha)
        L_ref = oracle_lib.index_logits(q, K)
        assert np.array_equal(logits.cpu().numpy().reshape(L_ref.shape), L_ref)
        check_scores(scores.cpu().numpy().reshape(L_ref.shape), oracle_lib.index_scores(L_ref, alpha))


@pytest.mark.parametrize("name", ["tiny", "32k", "128k", "500k", "1m_host"])
def test_index_score_and_selection_workloads(lsa, oracle_lib, W, name):
    """Every re-selection of every workload: logits and ids bit-exact."""
    w = W.WORKLOADS[name]
    K = W.indexer_keys(w)
    Kd = to_dev(K)
    for it in range(w.intervals if w.drift else 1):
        say(name, "interval", it)
        q = W.indexer_query(w, it)
        logits, scores = lsa.lsa_index_score(to_dev(q), Kd, w.alpha)
        ids = lsa.lsa_topk_chunks(logits.view(w.B, w.C), w.k)
        L_ref, S_ref, ids_ref = oracle_lib.select(q, K, w.k, w.alpha)
        assert np.array_equal(logits.cpu().numpy().reshape(L_ref.shape), L_ref)
        check_scores(scores.cpu().numpy().reshape(S_ref.shape), S_ref)
        got = ids.cpu().numpy()
        assert np.array_equal(got, ids_ref), f"{name}: {np.sum(got != ids_ref)} ids differ"


@pytest.mark.parametrize("path", ["gemv", "mfma"])
@pytest.mark.parametrize("B,nq,C,d_idx", [
    (1, 16, 1, 128), (2, 17, 15, 128), (1, 64, 1000, 128), (3, 65, 17, 64), (1, 256, 16384, 128),
    (2, 33, 513, 256), (1, 128, 2048, 64),
])
def test_batched_scoring(lsa, oracle_lib, synth_lib, tune, path, B, nq, C, d_idx):
    """Many query rows sharing a request's keys: the int8-MFMA kernel and the
    GEMV kernel (forced through the dispatch threshold) both match."""
    tune(score_mfma_min_nq=1 if path == "mfma" else 1000000)
    s = synth_lib.stream
    q = synth_lib.uniform_i8((B, nq, d_idx), 23, s(synth_lib.TAG_MISC, 1500 + nq), -128, 127)
    K = synth_lib.uniform_i8((B, C, d_idx), 23, s(synth_lib.TAG_MISC, 1600 + C), -128, 127)
    K[0, 0] = -128
    q[0, 0] = -128  # the largest logit, 2^21 at d_idx = 128
    alpha = 0.1 / d_idx
    logits, scores = lsa.lsa_index_score(to_dev(q), to_dev(K), alpha)
    L_ref = oracle_lib.index_logits(q, K)
    assert np.array_equal(logits.cpu().numpy().reshape(L_ref.shape), L_ref)
    check_scores(scores.cpu().numpy().reshape(L_ref.shape), oracle_lib.index_scores(L_ref, alpha))
    # each row's selection too (the oracle's rank-count top-k is quadratic in
    # C: on the largest rows only the first 4 are compared)
    ids = lsa.lsa_topk_chunks(logits, max(1, C // 10)).cpu().numpy().reshape(B * nq, -1)
    rows = B * nq if C <= 2048 else 4
    assert np.array_equal(ids[:rows], oracle_lib.topk_chunks(L_ref[:rows], max(1, C // 10)))


# ------------------------------------------------------------------ top-k

def _rows(synth_lib, kind, R, C, seed):
    s = synth_lib.stream(synth_lib.TAG_MISC, 700 + seed)
    if kind == "random":
        return synth_lib.uniform_i32((R, C), seed, s, -(2 ** 31), 2 ** 31 - 1)
    if kind == "narrow":
        return synth_lib.uniform_i32((R, C), seed, s, -3000, 3000)
    if kind == "few":
        return synth_lib.uniform_i32((R, C), seed, s, -2, 2)
    if kind == "equal":
        return np.full((R, C), 7, dtype=np.int32)
    if kind == "extremes":
        v = synth_lib.uniform_i32((R, C), seed, s, 0, 3)
        return np.choose(v, [-(2 ** 31), 2 ** 31 - 1, 0, -1]).astype(np.int32)
    if kind == "crowded":
        # a wide range (outliers at both ends) with nearly every value in a
        # narrow band: most keys share their top bits, and the band's
        # buckets stay large for several digits
        v = synth_lib.uniform_i32((R, C), seed, s, 0, 999)
        v[:, 0] = 2 ** 30
        v[:, -1] = -(2 ** 30)
        return v.astype(np.int32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["random", "narrow", "few", "equal", "extremes", "crowded"])
@pytest.mark.parametrize("C", [1, 2, 63, 64, 65, 1000, 1024, 1025, 2048, 7813, 16384])
def test_topk_parity(lsa, oracle_lib, synth_lib, kind, C):
    R = 3 if C <= 2048 else 1
    rows = _rows(synth_lib, kind, R, C, seed=C)
    dl = to_dev(rows)
    for k in sorted({1, C, max(1, C // 7), max(1, C - 1)}):
        got = lsa.lsa_topk_chunks(dl, k).cpu().numpy()
        ref = oracle_lib.topk_chunks(rows.astype(np.int64), k)
        assert np.array_equal(got, ref), (kind, C, k)


@pytest.mark.parametrize("C", [32768, 40000, 65536])
def test_topk_large_rows(lsa, oracle_lib, synth_lib, C):
    rows = _rows(synth_lib, "narrow", 1, C, seed=C)
    for k in (1, C // 10, C):
        got = lsa.lsa_topk_chunks(to_dev(rows), k).cpu().numpy()
        assert np.array_equal(got, oracle_lib.topk_chunks(rows.astype(np.int64), k)), (C, k)


@pytest.mark.parametrize("C", [40000, 65536])
def test_topk_large_rows_crowded(lsa, oracle_lib, synth_lib, C):
    """Long rows whose buckets stay larger than LDS holds for a digit or two."""
    rows = _rows(synth_lib, "crowded", 1, C, seed=C + 9)
    for k in (C // 10, C // 2 + 3):
        got = lsa.lsa_topk_chunks(to_dev(rows), k).cpu().numpy()
        assert np.array_equal(got, oracle_lib.topk_chunks(rows.astype(np.int64), k)), (C, k)


@pytest.mark.parametrize("kind", ["random", "few", "equal", "extremes"])
@pytest.mark.parametrize("C", [1, 65, 1025, 7813])
def test_topk_streaming_parity(lsa, oracle_lib, synth_lib, tune, kind, C):
    """The streaming kernel (rows read from memory in every pass), forced on
    rows that would otherwise keep their keys in registers."""
    tune(topk_stream_min_c=1)
    rows = _rows(synth_lib, kind, 2, C, seed=C + 50)
    dl = to_dev(rows)
    for k in sorted({1, C, max(1, C // 7), max(1, C - 1)}):
        got = lsa.lsa_topk_chunks(dl, k).cpu().numpy()
        assert np.array_equal(got, oracle_lib.topk_chunks(rows.astype(np.int64), k)), (kind, C, k)
    for k_max, thr in ((max(1, C // 3), 0), (C, -5)):
        ids, counts = lsa.lsa_threshold_chunks(dl, k_max, thr)
        ref_ids, ref_counts = oracle_lib.threshold_chunks(rows.astype(np.int64), k_max, thr)
        assert np.array_equal(counts.cpu().numpy(), ref_counts) and np.array_equal(ids.cpu().numpy(), ref_ids)


def test_topk_rows_beyond_registers(lsa, oracle_lib, synth_lib):
    """A row of 100,000 chunks: longer than the register-resident kernel takes."""
    C = 100000
    rows = _rows(synth_lib, "narrow", 1, C, seed=7)
    for k in (1, 10000):
        got = lsa.lsa_topk_chunks(to_dev(rows), k).cpu().numpy()
        assert np.array_equal(got, oracle_lib.topk_chunks(rows.astype(np.int64), k)), k


@pytest.mark.parametrize("kind", ["random", "few", "equal", "extremes", "crowded", "none", "all"])
@pytest.mark.parametrize("C", [1, 64, 1000, 2048, 16384])
def test_threshold_parity(lsa, oracle_lib, synth_lib, kind, C):
    """Sigmoid gating with a cap: ids, padding and counts bit-exact."""
    R = 3 if C <= 2048 else 1
    if kind == "none":
        rows = -np.abs(_rows(synth_lib, "narrow", R, C, seed=C + 1)) - 1
    elif kind == "all":
        rows = np.abs(_rows(synth_lib, "narrow", R, C, seed=C + 2)) + 1
    else:
        rows = _rows(synth_lib, kind if kind != "random" else "narrow", R, C, seed=C + 3)
    dl = to_dev(rows.astype(np.int32))
    for k_max in sorted({1, C, max(1, C // 7)}):
        for thr in (0, 5, -(2 ** 31)):
            ids, counts = lsa.lsa_threshold_chunks(dl, k_max, thr)
            ref_ids, ref_counts = oracle_lib.threshold_chunks(rows.astype(np.int64), k_max, thr)
            assert np.array_equal(counts.cpu().numpy(), ref_counts), (kind, C, k_max, thr)
            assert np.array_equal(ids.cpu().numpy(), ref_ids), (kind, C, k_max, thr)


# ------------------------------------------------------------------ attention

def _problem(synth_lib, B, Hq, Hkv, d, C, seed, qscale=1.0):
    s = synth_lib.stream
    q = synth_lib.normal_bf16((B, Hq, d), seed, s(synth_lib.TAG_MISC, 800), scale=qscale)
    kv = synth_lib.normal_bf16((B, C, 2, Hkv, 64, d), seed, s(synth_lib.TAG_MISC, 801))
    return q, kv


def _ids(synth_lib, B, C, k, seed):
    """Ascending distinct chunk ids per request; chunk 0 is always listed so a
    request with a short context still has a valid token."""
    out = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        out[b] = np.sort(synth_lib.choose(k, C, seed, synth_lib.stream(synth_lib.TAG_MISC, 900 + b)))
        out[b, 0] = 0
    return out


ATTEND_CASES = [
    # B, Hq, Hkv, d, C, k, ctx (None = full), n_split, qscale
    (1, 8, 1, 64, 64, 8, None, 0, 1.0),        # tiny workload shape
    (4, 64, 8, 128, 40, 32, None, 0, 1.0),     # DeepSeek-V4 GQA shape
    (4, 64, 8, 128, 40, 32, None, 1, 1.0),     # no split
    (4, 64, 8, 128, 40, 32, None, 7, 1.0),     # ragged split
    (4, 64, 8, 128, 40, 32, None, 32, 1.0),    # one chunk per split
    (2, 64, 8, 128, 20, 20, [1270, 1281], 3, 1.0),  # partial last chunk in both requests
    (2, 64, 8, 128, 20, 5, [1, 65], 2, 1.0),   # a single valid token / one token past a chunk
    (3, 64, 8, 128, 30, 1, None, 0, 1.0),      # k = 1
    (2, 64, 8, 128, 30, 12, None, 0, 8.0),     # sharpened softmax
    (2, 16, 16, 128, 10, 6, None, 2, 2.0),     # MHA (one query head per KV head)
    (2, 32, 2, 128, 10, 6, None, 2, 2.0),      # 16 query heads per KV head
    (2, 12, 4, 64, 10, 6, [600, 333], 2, 2.0), # group of 3, d = 64, partial chunks
]


@pytest.mark.parametrize("B,Hq,Hkv,d,C,k,ctx,n_split,qscale", ATTEND_CASES)
def test_attend_parity(lsa, oracle_lib, synth_lib, B, Hq, Hkv, d, C, k, ctx, n_split, qscale):
    say("attend", B, Hq, Hkv, d, C, k, ctx, n_split, qscale)
    q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=31 + k, qscale=qscale)
    ids = _ids(synth_lib, B, C, k, seed=41 + k)
    ctx = np.full(B, C * 64, dtype=np.int32) if ctx is None else np.array(ctx, dtype=np.int32)
    scale = 1.0 / math.sqrt(d)
    out = lsa.lsa_gather_attend(to_dev_bf16(q), to_dev_bf16(kv), to_dev(ids), to_dev(ctx), scale, n_split=n_split)
    ref = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, scale)
    # requests without any valid token give 0 on the GPU; the oracle rejects them
    stats = check_attention(out.cpu().numpy(), ref, "attend")
    say("  ", stats)


@pytest.mark.parametrize("n_split", [0, 1, 3])
def test_attend_counts_parity(lsa, oracle_lib, synth_lib, n_split):
    """Variable list lengths per request (threshold selection), including an
    empty list (output 0)."""
    B, Hq, Hkv, d, C, k = 4, 64, 8, 128, 30, 12
    q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=55, qscale=2.0)
    ids = _ids(synth_lib, B, C, k, seed=56)
    counts = np.array([12, 5, 0, 1], dtype=np.int32)
    for b in range(B):
        ids[b, counts[b]:] = -1  # unused entries, as the threshold selection writes them
    ctx = np.full(B, C * 64, dtype=np.int32)
    out = lsa.lsa_gather_attend(to_dev_bf16(q), to_dev_bf16(kv), to_dev(ids), to_dev(ctx), 1 / math.sqrt(d),
                                n_split=n_split, counts=to_dev(counts)).cpu().numpy()
    assert (out[2] == 0).all()
    live = [0, 1, 3]
    ref = oracle_lib.gather_attend(q[live], kv[live], np.where(ids[live] < 0, 0, ids[live]), ctx[live], Hkv,
                                   1 / math.sqrt(d), counts=counts[live])
    check_attention(out[live], ref, "counts")


@pytest.mark.parametrize("S,seg_lens,counts,n_split", [
    (8192, [8192, 8000, 1, 0], [12, 12, 12, 12], 0),   # a full 8K window, partial blocks, empty
    (256, [200, 256, 64, 65], [3, 0, 12, 7], 3),       # a request with the window only
    (128, [128, 1, 127, 2], [12, 12, 12, 12], 1),      # no split
])
def test_attend_segment_parity(lsa, oracle_lib, synth_lib, S, seg_lens, counts, n_split):
    """Recalled chunks plus the resident local window / decoded tokens in
    one softmax."""
    B, Hq, Hkv, d, C, k = 4, 64, 8, 128, 30, 12
    q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=60, qscale=2.0)
    seg = synth_lib.normal_bf16((B, 2, Hkv, S, d), 61, synth_lib.stream(synth_lib.TAG_MISC, 2700 + S))
    ids = _ids(synth_lib, B, C, k, seed=62)
    counts = np.array(counts, dtype=np.int32)
    seg_len = np.array(seg_lens, dtype=np.int32)
    ctx = np.full(B, C * 64 - 17, dtype=np.int32)
    out = lsa.lsa_gather_attend(to_dev_bf16(q), to_dev_bf16(kv), to_dev(ids), to_dev(ctx), 1 / math.sqrt(d),
                                n_split=n_split, counts=to_dev(counts), seg_kv=to_dev_bf16(seg),
                                seg_len=to_dev(seg_len)).cpu().numpy()
    live = [b for b in range(B) if counts[b] > 0 or seg_len[b] > 0]
    ref = oracle_lib.gather_attend(q[live], kv[live], ids[live], ctx[live], Hkv, 1 / math.sqrt(d),
                                   counts=counts[live], seg_kv=seg[live], seg_len=seg_len[live])
    check_attention(out[live], ref, "segment")
    for b in range(B):
        if b not in live:
            assert (out[b] == 0).all()


def test_attend_no_valid_token_gives_zero(lsa, synth_lib):
    q, kv = _problem(synth_lib, 2, 8, 1, 64, 4, seed=3)
    ids = np.array([[2, 3], [0, 1]], dtype=np.int32)
    ctx = np.array([100, 0], dtype=np.int32)  # request 0: chunks 2,3 start at 128 > 100; request 1: empty
    out = lsa.lsa_gather_attend(to_dev_bf16(q), to_dev_bf16(kv), to_dev(ids), to_dev(ctx), 0.125, n_split=2)
    assert (out.cpu().numpy() == 0).all()


def test_attend_slots_pool(lsa, oracle_lib, synth_lib):
    """K/V read from a compact pool at explicit slots, masking by chunk id."""
    B, Hq, Hkv, d, C, k = 2, 64, 8, 128, 30, 9
    q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=5)
    ids = _ids(synth_lib, B, C, k, seed=6)
    ids[0, -1] = C - 1
    ctx = np.array([C * 64 - 20, C * 64], dtype=np.int32)
    perm = np.array([[(j * 4) % k for j in range(k)]] * B, dtype=np.int32)  # slots, a permutation
    pool = np.zeros((B, k, 2, Hkv, 64, d), dtype=np.uint16)
    for b in range(B):
        pool[b, perm[b]] = kv[b, ids[b]]
    out = lsa.lsa_gather_attend(to_dev_bf16(q), to_dev_bf16(pool), to_dev(ids), to_dev(ctx), 1 / math.sqrt(d),
                                slots=to_dev(perm))
    ref = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / math.sqrt(d))
    check_attention(out.cpu().numpy(), ref, "slots")


def test_attend_deterministic(lsa, synth_lib):
    """Same inputs, same bits (fixed reduction order)."""
    B, Hq, Hkv, d, C, k = 4, 64, 8, 128, 40, 32
    q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=77)
    ids = _ids(synth_lib, B, C, k, seed=78)
    args = (to_dev_bf16(q), to_dev_bf16(kv), to_dev(ids), to_dev(np.full(B, C * 64, dtype=np.int32)))
    a = lsa.lsa_gather_attend(*args, n_split=5).cpu().numpy()
    b = lsa.lsa_gather_attend(*args, n_split=5).cpu().numpy()
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ token-level stage

def _token_scores(synth_lib, B, n, seed):
    """bf16-rounded normals coarsened to quarters (long runs of equal scores),
    with signed zeros, subnormals and infinities planted."""
    s = synth_lib.bf16_bits_to_f32(synth_lib.normal_bf16((B, n), seed, synth_lib.stream(synth_lib.TAG_MISC, 4000)))
    s = np.round(s * 4) / 4
    s[:, 3::17] = 0.0
    s[:, 5::19] = -0.0
    s[:, 7::41] = np.inf
    s[:, 11::43] = -np.inf
    s[:, 13::47] = np.float32(1e-40)    # subnormals of both signs: ordered like any value,
    s[:, 15::53] = np.float32(-1e-40)   # and apart from zero
    s[:, 19::59] = np.float32(1.4e-45)
    return np.ascontiguousarray(s, dtype=np.float32)


@pytest.mark.parametrize("B,C,k,k_tok", [
    (4, 12, 5, 7),        # tiny
    (4, 12, 5, 400),      # budget above the usable tokens: padding
    (3, 64, 40, 600),
    (4, 2048, 276, 2048),  # the 128K recall, a 2048-token budget
    (2, 4096, 1024, 2048),  # the largest list: 65536 positions
    (2, 600, 500, 3000),   # 32000 positions: 32 per thread, the most whose output regions fit LDS
])
def test_topk_tokens_parity(lsa, oracle_lib, synth_lib, tune, B, C, k, k_tok):
    say("token top-k", B, C, k, k_tok)
    tune(topk_split_min_n=1)  # the slice + candidates path on every size it can split
    scores = _token_scores(synth_lib, B, k * 64, seed=k)
    ids = np.stack([np.sort(synth_lib.choose(k, C, 9, synth_lib.stream(synth_lib.TAG_MISC, 4010 + b)))
                    for b in range(B)]).astype(np.int32)
    ctx = np.full(B, C * 64, dtype=np.int32)
    ctx[0] = ids[0, -1] * 64 + 17                  # the last listed chunk is partial
    if B > 2:
        ctx[2] = ids[2, k // 2] * 64               # half the list lies past the context
    counts = np.full(B, k, dtype=np.int32)
    counts[1] = max(1, k - 3)
    for cn in (None, counts):
        ref, rc = oracle_lib.topk_tokens(scores, ids, ctx, k_tok, counts=cn)
        # "auto": the slice + candidates path where the library splits; None: one workgroup per request
        for ws in ("auto", None):
            tok, tc = lsa.lsa_topk_tokens(to_dev(scores), to_dev(ids), to_dev(ctx), k_tok,
                                          counts=None if cn is None else to_dev(cn), workspace=ws)
            assert np.array_equal(tc.cpu().numpy(), rc), (B, C, k, k_tok, ws)
            assert np.array_equal(tok.cpu().numpy(), ref), (B, C, k, k_tok, ws)


@pytest.mark.parametrize("B,C,k,k_tok", [(3, 2048, 276, 2048), (2, 4096, 1024, 5000), (2, 64, 3, 17)])
def test_topk_tokens_crowded_scores(lsa, oracle_lib, synth_lib, B, C, k, k_tok):
    """Scores spread evenly over [1, 2) with infinities at both ends: the
    whole list shares its top key bits, so the select keeps working on a
    crowded bucket for several digits (in registers while it is larger than
    LDS holds), with runs of equal scores at the end."""
    say("token top-k crowded", B, C, k, k_tok)
    s = synth_lib.stream(synth_lib.TAG_MISC, 4050)
    u = synth_lib.uniform_i32((B, k * 64), k, s, 0, 2 ** 16 - 1)
    scores = (1.0 + u.astype(np.float64) / 2 ** 16).astype(np.float32)  # 65536 distinct values, many repeats
    scores[:, 1] = np.inf
    scores[:, -2] = -np.inf
    ids = np.stack([np.sort(synth_lib.choose(k, C, 9, synth_lib.stream(synth_lib.TAG_MISC, 4060 + b)))
                    for b in range(B)]).astype(np.int32)
    ctx = np.full(B, C * 64, dtype=np.int32)
    ctx[-1] = ids[-1, -1] * 64 + 9
    ref, rc = oracle_lib.topk_tokens(scores, ids, ctx, k_tok)
    for ws in ("auto", None):
        tok, tc = lsa.lsa_topk_tokens(to_dev(scores), to_dev(ids), to_dev(ctx), k_tok, workspace=ws)
        assert np.array_equal(tc.cpu().numpy(), rc) and np.array_equal(tok.cpu().numpy(), ref), ws


@pytest.mark.parametrize("slices,k_tok", [(2, 2048), (12, 4096)])
def test_topk_tokens_split_shapes(lsa, oracle_lib, synth_lib, tune, slices, k_tok):
    """The 500K recall (782 chunks, 50,048 positions) split into 2 long slices
    (32 positions per thread in the slice select, which keeps keys too: its
    output takes two sweeps over the registers) or 12 slices with a 4096-token
    budget (49,152 candidates, 48 per thread: the same in the candidates
    select)."""
    say("token top-k split shapes", slices, k_tok)
    tune(topk_split_slices=slices)
    B, C, k = 2, 7813, 782
    scores = _token_scores(synth_lib, B, k * 64, seed=slices)
    ids = np.stack([np.sort(synth_lib.choose(k, C, 9, synth_lib.stream(synth_lib.TAG_MISC, 4070 + b)))
                    for b in range(B)]).astype(np.int32)
    ctx = np.array([500000, ids[1, -1] * 64 + 33], dtype=np.int32)
    ref, rc = oracle_lib.topk_tokens(scores, ids, ctx, k_tok)
    tok, tc = lsa.lsa_topk_tokens(to_dev(scores), to_dev(ids), to_dev(ctx), k_tok, workspace="auto")
    assert np.array_equal(tc.cpu().numpy(), rc) and np.array_equal(tok.cpu().numpy(), ref)


@pytest.mark.parametrize("B,C,k,k_tok", [(4, 12, 5, 7), (3, 64, 40, 600), (4, 2048, 276, 2048)])
def test_topk_tokens_streaming_parity(lsa, oracle_lib, synth_lib, tune, B, C, k, k_tok):
    """Token selection through the streaming kernel, forced on short lists."""
    tune(topk_stream_min_c=1)
    scores = _token_scores(synth_lib, B, k * 64, seed=k + 1)
    ids = np.stack([np.sort(synth_lib.choose(k, C, 9, synth_lib.stream(synth_lib.TAG_MISC, 4030 + b)))
                    for b in range(B)]).astype(np.int32)
    ctx = np.full(B, C * 64, dtype=np.int32)
    ctx[0] = ids[0, -1] * 64 + 17
    counts = np.full(B, k, dtype=np.int32)
    counts[1] = max(1, k - 3)
    tok, tc = lsa.lsa_topk_tokens(to_dev(scores), to_dev(ids), to_dev(ctx), k_tok, counts=to_dev(counts),
                                  workspace=None)  # no workspace: the streaming kernel, not the split
    ref, rc = oracle_lib.topk_tokens(scores, ids, ctx, k_tok, counts=counts)
    assert np.array_equal(tc.cpu().numpy(), rc) and np.array_equal(tok.cpu().numpy(), ref)


def test_topk_tokens_1m_recall(lsa, oracle_lib, synth_lib):
    """The 1M workload's recall (1638 chunks = 104,832 token positions):
    beyond the register-resident kernel.  With a workspace it runs as 16
    slices + candidates; without, the streaming kernel runs."""
    B, C, k, k_tok = 2, 16384, 1638, 2048
    scores = _token_scores(synth_lib, B, k * 64, seed=11)
    ids = np.stack([np.sort(synth_lib.choose(k, C, 9, synth_lib.stream(synth_lib.TAG_MISC, 4040 + b)))
                    for b in range(B)]).astype(np.int32)
    ctx = np.array([C * 64, ids[1, -1] * 64 + 5], dtype=np.int32)
    ref, rc = oracle_lib.topk_tokens(scores, ids, ctx, k_tok)
    for ws in ("auto", None):
        tok, tc = lsa.lsa_topk_tokens(to_dev(scores), to_dev(ids), to_dev(ctx), k_tok, workspace=ws)
        assert np.array_equal(tc.cpu().numpy(), rc) and np.array_equal(tok.cpu().numpy(), ref), ws


TOKEN_CASES = [
    # B, Hq, Hkv, d, C, k, k_tok, n_split, with slots, segment length (0: none)
    (2, 64, 8, 128, 30, 12, 100, 0, False, 0),
    (2, 64, 8, 128, 30, 12, 64, 1, False, 0),
    (3, 64, 8, 128, 40, 20, 700, 5, True, 0),
    (2, 16, 2, 64, 20, 8, 130, 2, False, 0),
    (2, 64, 8, 128, 30, 12, 300, 3, False, 200),
]


@pytest.mark.parametrize("B,Hq,Hkv,d,C,k,k_tok,n_split,use_slots,seg_n", TOKEN_CASES)
def test_attend_tokens_parity(lsa, oracle_lib, synth_lib, B, Hq, Hkv, d, C, k, k_tok, n_split, use_slots, seg_n):
    """Attention over listed tokens: unsorted lists with invalid entries
    (-1, positions of unused entries, tokens past the context), ragged
    counts, a compact pool with slots, a resident segment."""
    say("token attend", B, Hq, Hkv, d, C, k, k_tok, n_split, use_slots, seg_n)
    q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=70 + k_tok, qscale=4.0)
    ids = _ids(synth_lib, B, C, k, seed=71)
    counts = np.full(B, k, dtype=np.int32)
    counts[-1] = k - 2
    ctx = np.full(B, C * 64, dtype=np.int32)
    ctx[0] = ids[0, -1] * 64 + 30
    rng = np.random.default_rng(k_tok)
    tok = np.stack([rng.permutation(k * 64)[:k_tok] if k_tok <= k * 64 else rng.integers(0, k * 64, k_tok)
                    for _ in range(B)]).astype(np.int32)
    tok[:, 1] = -1
    tok[:, 2] = k * 64 + 5
    tok_counts = np.full(B, k_tok, dtype=np.int32)
    tok_counts[0] = max(1, k_tok - 37)
    store, slots = kv, None
    if use_slots:  # a compact pool in permuted slot order
        perm = np.array([[(j * 7) % k for j in range(k)]] * B, dtype=np.int32)
        store = np.zeros((B, k, 2, Hkv, 64, d), dtype=np.uint16)
        for b in range(B):
            store[b, perm[b]] = kv[b, ids[b]]
        slots = perm
    seg = seg_len = None
    kw = {}
    if seg_n:
        seg = synth_lib.normal_bf16((B, 2, Hkv, 256, d), 72, synth_lib.stream(synth_lib.TAG_MISC, 4020))
        seg_len = np.array([seg_n, 1] + [0] * (B - 2), dtype=np.int32)
        kw = dict(seg_kv=to_dev_bf16(seg), seg_len=to_dev(seg_len))
    out = lsa.lsa_gather_attend_tokens(to_dev_bf16(q), to_dev_bf16(store), to_dev(ids), to_dev(ctx), to_dev(tok),
                                       to_dev(tok_counts), sm_scale=1 / math.sqrt(d), n_split=n_split,
                                       counts=to_dev(counts), slots=None if slots is None else to_dev(slots), **kw)
    ref = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / math.sqrt(d), counts=counts, tok=tok,
                                   tok_counts=tok_counts, seg_kv=seg, seg_len=seg_len)
    say("  ", check_attention(out.cpu().numpy(), ref, "token attend"))


@pytest.mark.parametrize("n_split,seg_n", [(2, 0), (4, 0), (7, 0), (3, 256), (5, 128)])
def test_attend_tokens_counts_move_split_start(lsa, oracle_lib, synth_lib, n_split, seg_n):
    """Token counts far below the list length (down to 0 and 1) and partly
    filled segments, over several split counts: many splits start at another
    block than a full list and a full segment would give them, and some hold
    only segment blocks or nothing."""
    B, Hq, Hkv, d, C, k, k_tok = 5, 64, 8, 128, 40, 16, 900
    q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=90 + n_split, qscale=4.0)
    ids = _ids(synth_lib, B, C, k, seed=91)
    ctx = np.full(B, C * 64, dtype=np.int32)
    rng = np.random.default_rng(92 + n_split)
    tok = np.stack([rng.permutation(k * 64)[:k_tok] for _ in range(B)]).astype(np.int32)
    # request 3 lists no token when its segment gives it some (the oracle's
    # softmax needs at least one usable token per request)
    tok_counts = np.array([k_tok, k_tok // 3, 1, 0 if seg_n else 2, 450], dtype=np.int32)
    kw, seg, seg_len = {}, None, None
    if seg_n:
        seg = synth_lib.normal_bf16((B, 2, Hkv, seg_n, d), 93, synth_lib.stream(synth_lib.TAG_MISC, 4030))
        seg_len = np.array([seg_n, seg_n // 2, 1, 17, 0], dtype=np.int32)
        kw = dict(seg_kv=to_dev_bf16(seg), seg_len=to_dev(seg_len))
    say("token attend counts", n_split, seg_n, tok_counts.tolist())
    out = lsa.lsa_gather_attend_tokens(to_dev_bf16(q), to_dev_bf16(kv), to_dev(ids), to_dev(ctx), to_dev(tok),
                                       to_dev(tok_counts), sm_scale=1 / math.sqrt(d), n_split=n_split, **kw)
    ref = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / math.sqrt(d), tok=tok, tok_counts=tok_counts,
                                   seg_kv=seg, seg_len=seg_len)
    say("  ", check_attention(out.cpu().numpy(), ref, "token attend counts"))


def test_attend_tokens_all_listed_equals_chunk_attention(lsa, synth_lib):
    """Listing every token of the chunks reproduces chunk attention up to
    rounding order (same tokens, blocks of 64 listed rows instead of tiles)."""
    B, Hq, Hkv, d, C, k = 2, 64, 8, 128, 30, 10
    q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=80)
    ids = _ids(synth_lib, B, C, k, seed=81)
    ctx = np.array([ids[0, -1] * 64 + 9, C * 64], dtype=np.int32)
    args = (to_dev_bf16(q), to_dev_bf16(kv), to_dev(ids), to_dev(ctx))
    a = lsa.lsa_gather_attend(*args, n_split=1).cpu().numpy()
    tok = np.tile(np.arange(k * 64, dtype=np.int32), (B, 1))
    t = lsa.lsa_gather_attend_tokens(*args, to_dev(tok), None, n_split=1).cpu().numpy()
    np.testing.assert_allclose(t, a, rtol=0, atol=2e-6)


# ------------------------------------------------------------------ fetch

@pytest.mark.parametrize("lanes", [0, 1, 3, 16])
def test_fetch_byte_exact(lsa, oracle_lib, synth_lib, tune, lanes):
    """The DMA fetch with its copies on 1 stream (the caller's), on the
    library's default of 4 copy streams, and on 3 and 16 of them: the same pool
    bytes as the oracle's copy."""
    import torch
    if lanes:
        tune(fetch_lanes=lanes)
    B, C, Hkv, d, k, P = 2, 12, 2, 64, 5, 7
    host = synth_lib.normal_bf16((B, C, 2, Hkv, 64, d), 9, synth_lib.stream(synth_lib.TAG_MISC, 950))
    ids = np.array([[0, 1, 2, 7, 11], [3, 4, 6, 8, 9]], dtype=np.int32)
    slots = np.array([[0, 1, 2, 5, 6], [6, 5, 4, 0, 1]], dtype=np.int32)
    host_t = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).pin_memory()
    pool = torch.zeros((B, P, 2, Hkv, 64, d), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    done = torch.cuda.Event()
    lsa.lsa_fetch_chunks(host_t, torch.from_numpy(ids), pool, host_slots=torch.from_numpy(slots), stream=side)
    done.record(side)
    done.synchronize()
    ref = oracle_lib.fetch_chunks(host, ids, P, slots=slots)
    assert np.array_equal(pool.cpu().view(torch.int16).numpy().view(np.uint16), ref)
    # default slots (entry j -> slot j) and the done event of the ABI
    pool2 = torch.zeros((B, k, 2, Hkv, 64, d), dtype=torch.bfloat16, device="cuda")
    ev = torch.cuda.Event()
    ev.record(side)  # create the event before handing it to the library
    lsa.lsa_fetch_chunks(host_t, torch.from_numpy(ids), pool2, stream=side, done=ev)
    ev.synchronize()
    assert np.array_equal(pool2.cpu().view(torch.int16).numpy().view(np.uint16), oracle_lib.fetch_chunks(host, ids, k))


def test_fetch_concurrent_threads_byte_exact(lsa, oracle_lib, synth_lib):
    """Two host threads fetch at once, each on its own stream into its own
    pool, both through the library's shared copy streams (each call holds the
    fork and join events for its own use): every pool gets exactly its chunks
    at their slots, and an entry with a negative slot (a chunk already in the
    pool, as the delta fetch passes it) leaves the pool as it was."""
    import threading

    import torch
    B, C, Hkv, d, k, P = 2, 64, 2, 64, 24, 48
    host = synth_lib.normal_bf16((B, C, 2, Hkv, 64, d), 23, synth_lib.stream(synth_lib.TAG_MISC, 970))
    host_t = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).pin_memory()
    rng = np.random.default_rng(970)
    jobs = []
    for _ in range(2):
        ids = np.stack([np.sort(rng.choice(C, k, replace=False)) for _ in range(B)]).astype(np.int32)
        slots = np.stack([rng.choice(P, k, replace=False) for _ in range(B)]).astype(np.int32)
        slots[:, ::5] = -1  # not copied
        jobs.append((ids, slots))
    one = np.uint16(0x3F80)  # bf16 1.0
    pools = [torch.full((B, P, 2, Hkv, 64, d), 1.0, dtype=torch.bfloat16, device="cuda") for _ in jobs]
    torch.cuda.synchronize()
    errors = []

    def work(t):
        try:
            side = torch.cuda.Stream()
            for _ in range(5):
                lsa.lsa_fetch_chunks(host_t, torch.from_numpy(jobs[t][0]), pools[t],
                                     host_slots=torch.from_numpy(jobs[t][1]), stream=side)
            side.synchronize()
        except Exception as e:  # reported below, in the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(t,)) for t in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (ids, slots), pool in zip(jobs, pools):
        want = np.full((B, P, 2, Hkv, 64, d), one, dtype=np.uint16)
        want = oracle_lib.fetch_chunks(host, ids, P, slots=slots, pool=want, skip_negative_slots=True)
        assert np.array_equal(pool.cpu().view(torch.int16).numpy().view(np.uint16), want)


@pytest.mark.parametrize("stage,Hkv,d", [(2, 2, 64), (5, 2, 64), (64, 2, 64), (8, 8, 128)])
def test_fetch_staged_byte_exact(lsa, oracle_lib, synth_lib, stage, Hkv, d):
    """The staged fetch (host gather into pinned staging, large copies,
    scatter into the pool on the device) leaves the oracle's bytes in the
    pool: pieces of stage // 2 chunks (one chunk at a time for stage 2 and
    3), entries with a negative slot leave their slots as they were, two
    calls in a row reuse the staging buffers, and default slots put entry j
    at slot j."""
    import torch
    B, C, k, P = 2, 64, 24, 48
    host = synth_lib.normal_bf16((B, C, 2, Hkv, 64, d), 29, synth_lib.stream(synth_lib.TAG_MISC, 980 + stage))
    host_t = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).pin_memory()
    staging = lsa.alloc_fetch_staging(host_t, stage)
    rng = np.random.default_rng(980 + stage)
    one = np.uint16(0x3F80)  # bf16 1.0
    pool = torch.full((B, P, 2, Hkv, 64, d), 1.0, dtype=torch.bfloat16, device="cuda")
    want = np.full(tuple(pool.shape), one, dtype=np.uint16)
    side = torch.cuda.Stream()
    for rep in range(2):
        ids = np.stack([np.sort(rng.choice(C, k, replace=False)) for _ in range(B)]).astype(np.int32)
        slots = np.stack([rng.choice(P, k, replace=False) for _ in range(B)]).astype(np.int32)
        slots[:, rep::4] = -1  # not copied
        lsa.lsa_fetch_chunks_staged(host_t, torch.from_numpy(ids), pool, *staging,
                                    host_slots=torch.from_numpy(slots), stream=side)
        side.synchronize()
        want = oracle_lib.fetch_chunks(host, ids, P, slots=slots, pool=want, skip_negative_slots=True)
        assert np.array_equal(pool.cpu().view(torch.int16).numpy().view(np.uint16), want), rep
    pool2 = torch.zeros((B, k, 2, Hkv, 64, d), dtype=torch.bfloat16, device="cuda")
    ev = torch.cuda.Event()
    ev.record(side)  # create the event before handing it to the library
    lsa.lsa_fetch_chunks_staged(host_t, torch.from_numpy(ids), pool2, *staging, stream=side, done=ev)
    ev.synchronize()
    assert np.array_equal(pool2.cpu().view(torch.int16).numpy().view(np.uint16), oracle_lib.fetch_chunks(host, ids, k))


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_fetch_staged_rejects(lsa):
    """Pageable staging memory and graph capture are refused before any copy
    (the call waits on the host for its copies)."""
    import torch
    host = torch.zeros((1, 4, 2, 1, 64, 64), dtype=torch.bfloat16).pin_memory()
    pool = torch.zeros((1, 2, 2, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    ids = torch.tensor([[0, 3]], dtype=torch.int32)
    host_stage, dev_stage = lsa.alloc_fetch_staging(host, 4)
    with pytest.raises(lsa.LsaError, match="pinned"):
        lsa.lsa_fetch_chunks_staged(host, ids, pool, torch.zeros(tuple(host_stage.shape), dtype=torch.bfloat16),
                                    dev_stage)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with pytest.raises(lsa.LsaError, match="capture"):
            with torch.cuda.graph(g, stream=s):
                lsa.lsa_fetch_chunks_staged(host, ids, pool, host_stage, dev_stage, stream=s)
    torch.cuda.synchronize()


def test_fetch_pull_byte_exact(lsa, oracle_lib, synth_lib):
    """The device-side gather: same pool bytes as the oracle's copy; entries
    with an id or slot out of range are skipped and leave their slot as it was."""
    import torch
    B, C, Hkv, d, k, P = 3, 40, 2, 128, 7, 9
    host = synth_lib.normal_bf16((B, C, 2, Hkv, 64, d), 19, synth_lib.stream(synth_lib.TAG_MISC, 960))
    host_t = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).pin_memory()
    ids = np.array([[0, 1, 2, 5, 17, 38, 39], [3, 4, 6, 8, 9, 10, 11], [1, 9, 12, 20, 25, 30, 33]], dtype=np.int32)
    slots = np.array([[8, 7, 6, 5, 4, 3, 2], [0, 1, 2, 3, 4, 5, 6], [2, 4, 6, 8, 1, 3, 5]], dtype=np.int32)
    pool = torch.zeros((B, P, 2, Hkv, 64, d), dtype=torch.bfloat16, device="cuda")
    for grid in (1, 5, 0):
        pool.zero_()
        lsa.lsa_fetch_chunks_pull(host_t, to_dev(ids), pool, slots=to_dev(slots), grid=grid)
        torch.cuda.synchronize()
        ref = oracle_lib.fetch_chunks(host, ids, P, slots=slots)
        assert np.array_equal(pool.cpu().view(torch.int16).numpy().view(np.uint16), ref), grid
    pool2 = torch.zeros((B, k, 2, Hkv, 64, d), dtype=torch.bfloat16, device="cuda")
    lsa.lsa_fetch_chunks_pull(host_t, to_dev(ids), pool2)
    torch.cuda.synchronize()
    assert np.array_equal(pool2.cpu().view(torch.int16).numpy().view(np.uint16), oracle_lib.fetch_chunks(host, ids, k))
    # out-of-range entries: skipped by the kernel's own bounds check
    bad_ids = ids.copy()
    bad_ids[0, 1] = C          # id past the store
    bad_ids[1, 2] = -1         # negative id
    bad_slots = slots.copy()
    bad_slots[2, 3] = P        # slot past the pool
    pool.fill_(1.0)
    lsa.lsa_fetch_chunks_pull(host_t, to_dev(bad_ids), pool, slots=to_dev(bad_slots))
    torch.cuda.synchronize()
    got = pool.cpu().view(torch.int16).numpy().view(np.uint16)
    one = np.uint16(0x3F80)  # bf16 1.0
    for b in range(B):
        for j in range(k):
            c, p = bad_ids[b, j], bad_slots[b, j]
            if 0 <= c < C and 0 <= p < P:
                assert np.array_equal(got[b, p], host[b, c])
            elif 0 <= p < P:
                assert (got[b, p] == one).all()


def test_fetch_pull_rejects_pageable(lsa):
    import torch
    host = torch.zeros((1, 4, 2, 1, 64, 64), dtype=torch.bfloat16)
    pool = torch.zeros((1, 2, 2, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lsa.LsaError, match="pinned"):
        lsa.lsa_fetch_chunks_pull(host, torch.tensor([[0, 1]], dtype=torch.int32, device="cuda"), pool)


@pytest.mark.parametrize("B,C,k", [(1, 30, 5), (3, 2048, 276), (4, 16384, 1638), (2, 100, 1)])
def test_pool_assign_parity(lsa, oracle_lib, synth_lib, B, C, k):
    """Delta-fetch slots: bit-exact with the oracle over a chain of selections
    (overlapping ones, disjoint ones, identical ones)."""
    P = 2 * k
    prev_ids = prev_slots = None
    prev_d = (None, None)
    for step in range(6):
        span = C if step % 2 else max(k, C // 3)  # alternate wide and narrow draws: overlaps vary
        ids = np.stack([np.sort(synth_lib.choose(k, span, 8, synth_lib.stream(synth_lib.TAG_MISC, 2000 + 16 * step + b)))
                        for b in range(B)]).astype(np.int32)
        if step == 3:
            ids = prev_ids.copy()  # the same selection again: nothing to fetch
        ns_ref, fs_ref = oracle_lib.pool_assign(prev_ids, prev_slots, ids, P)
        ids_d = to_dev(ids)
        ns, fs = lsa.lsa_pool_assign(prev_d[0], prev_d[1], ids_d, P)
        assert np.array_equal(ns.cpu().numpy(), ns_ref), step
        assert np.array_equal(fs.cpu().numpy(), fs_ref), step
        if step == 3:
            assert (fs_ref == -1).all()
        prev_ids, prev_slots = ids, ns_ref
        prev_d = (ids_d, ns)


def test_fetch_rejects_pageable(lsa):
    import torch
    host = torch.zeros((1, 4, 2, 1, 64, 64), dtype=torch.bfloat16)  # not pinned
    pool = torch.zeros((1, 2, 2, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lsa.LsaError, match="pinned"):
        lsa.lsa_fetch_chunks(host, torch.tensor([[0, 1]], dtype=torch.int32), pool)


def test_concurrent_streams_match_serial(lsa, synth_lib):
    """Calls on two HIP streams with their own workspaces, interleaved and
    running concurrently, give the bits of the same calls run one at a time
    (the library keeps no mutable state between calls)."""
    import torch
    B, Hq, Hkv, d, C, k = 4, 64, 8, 128, 40, 24
    probs = []
    for seed in (90, 91):
        q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=seed)
        ids = _ids(synth_lib, B, C, k, seed=seed + 10)
        probs.append((to_dev_bf16(q), to_dev_bf16(kv), to_dev(ids), to_dev(np.full(B, C * 64, dtype=np.int32))))
    serial = [lsa.lsa_gather_attend(*p, n_split=3).cpu().numpy() for p in probs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [lsa.alloc_workspace(B, Hq, Hkv, d, k, 3) for _ in streams]
    outs = [[torch.empty((B, Hq, d), dtype=torch.float32, device="cuda") for _ in range(6)] for _ in streams]
    torch.cuda.synchronize()
    for rep in range(6):
        for sidx, st in enumerate(streams):
            lsa.lsa_gather_attend(*probs[sidx], n_split=3, workspace=wss[sidx], out=outs[sidx][rep],
                                  stream=st)
    torch.cuda.synchronize()
    for sidx in range(2):
        for rep in range(6):
            assert np.array_equal(outs[sidx][rep].cpu().numpy(), serial[sidx]), (sidx, rep)
