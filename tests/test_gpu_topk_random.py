"""Randomised parity of the select kernels with the oracle: seeded draws of
row shapes, budgets and key distributions (ties, both-sign extremes, crowded
bands, signed zeros, infinities, subnormals, partial contexts, ragged entry
counts), every output compared bit for bit.  The draws are fixed by their
case number, so a failure names a reproducible case."""
import numpy as np
import pytest

from conftest import gpu_available
from helpers import to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def lsa():
    import lookahead_chunk_sparse_amd as m
    return m


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ chunk logits

def _logit_case(i):
    rng = np.random.default_rng(1000 + i)
    C = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 4000)), int(rng.integers(4000, 12000))]))
    R = int(rng.integers(1, 5))
    k = int(rng.choice([1, C, int(rng.integers(1, C + 1))]))
    kind = str(rng.choice(["wide", "narrow", "few", "crowded", "equal"]))
    thr = int(rng.choice([0, -3, 1, 2 ** 31 - 1, -(2 ** 31)]))
    return R, C, k, kind, thr


def _logit_rows(synth_lib, kind, R, C, case):
    s = synth_lib.stream(synth_lib.TAG_MISC, 5000 + case)
    if kind == "wide":
        return synth_lib.uniform_i32((R, C), case, s, -(2 ** 31), 2 ** 31 - 1)
    if kind == "narrow":
        return synth_lib.uniform_i32((R, C), case, s, -50, 50)
    if kind == "few":
        return synth_lib.uniform_i32((R, C), case, s, 0, 2)
    if kind == "crowded":  # a narrow band between outliers at both ends of the int32 range
        v = synth_lib.uniform_i32((R, C), case, s, 0, 4095)
        v[:, 0] = 2 ** 31 - 1
        v[:, -1] = -(2 ** 31)
        return v
    return np.full((R, C), -5, dtype=np.int32)


@pytest.mark.parametrize("case", range(100))
def test_topk_and_threshold_random(lsa, oracle_lib, synth_lib, case):
    R, C, k, kind, thr = _logit_case(case)
    say("random logits case", case, R, C, k, kind, thr)
    rows = _logit_rows(synth_lib, kind, R, C, case)
    dl = to_dev(rows)
    got = lsa.lsa_topk_chunks(dl, k).cpu().numpy()
    assert np.array_equal(got, oracle_lib.topk_chunks(rows.astype(np.int64), k)), (case, R, C, k, kind)
    ids, counts = lsa.lsa_threshold_chunks(dl, k, thr)
    ref_ids, ref_counts = oracle_lib.threshold_chunks(rows.astype(np.int64), k, thr)
    assert np.array_equal(counts.cpu().numpy(), ref_counts), (case, R, C, k, kind, thr)
    assert np.array_equal(ids.cpu().numpy(), ref_ids), (case, R, C, k, kind, thr)


# ------------------------------------------------------------------ token scores

def _token_case(i):
    rng = np.random.default_rng(2000 + i)
    k = int(rng.integers(1, 300))
    C = int(rng.integers(k, 4096))
    B = int(rng.integers(1, 5))
    k_tok = int(rng.choice([1, int(rng.integers(1, k * 64 + 1)), k * 64 + 50]))
    kind = str(rng.choice(["normal", "quarters", "band", "equal"]))
    split = bool(rng.integers(0, 2))
    return B, C, k, k_tok, kind, split, rng


def _token_scores(synth_lib, kind, B, n, case):
    s = synth_lib.stream(synth_lib.TAG_MISC, 6000 + case)
    if kind in ("normal", "quarters"):
        x = synth_lib.bf16_bits_to_f32(synth_lib.normal_bf16((B, n), case, s)).astype(np.float64)
        if kind == "quarters":
            x = np.round(x * 4) / 4
    elif kind == "band":  # 2^20 + 1 values spread over [1, 2]: the whole list shares its top key bits
        x = 1.0 + synth_lib.uniform_i32((B, n), case, s, 0, 2 ** 20).astype(np.float64) / 2 ** 20
    else:
        x = np.full((B, n), 0.5)
    x = x.astype(np.float32)
    if n > 8:  # special values at fixed places
        x[:, 1] = -0.0
        x[:, 2] = 0.0
        x[:, 3] = np.inf
        x[:, 4] = -np.inf
        x[:, 5] = np.float32(1e-40)
        x[:, 6] = np.float32(-1e-40)
    return np.ascontiguousarray(x)


@pytest.mark.parametrize("case", range(80))
def test_topk_tokens_random(lsa, oracle_lib, synth_lib, tune, case):
    B, C, k, k_tok, kind, split, rng = _token_case(case)
    say("random token case", case, B, C, k, k_tok, kind, split)
    if split:  # the slice + candidates path wherever the row can be split
        tune(topk_split_min_n=1)
    scores = _token_scores(synth_lib, kind, B, k * 64, case)
    ids = np.stack([np.sort(synth_lib.choose(k, C, case, synth_lib.stream(synth_lib.TAG_MISC, 6100 + b)))
                    for b in range(B)]).astype(np.int32)
    ctx = np.full(B, C * 64, dtype=np.int32)
    for b in range(B):
        r = int(rng.integers(0, 4))
        if r == 1:    # the context ends inside a listed chunk
            ctx[b] = int(ids[b, int(rng.integers(0, k))]) * 64 + int(rng.integers(0, 64))
        elif r == 2:  # no context at all
            ctx[b] = 0
    counts = rng.integers(0, k + 1, B).astype(np.int32) if rng.integers(0, 2) else None
    ref, rc = oracle_lib.topk_tokens(scores, ids, ctx, k_tok, counts=counts)
    tok, tc = lsa.lsa_topk_tokens(to_dev(scores), to_dev(ids), to_dev(ctx), k_tok,
                                  counts=None if counts is None else to_dev(counts), workspace="auto")
    assert np.array_equal(tc.cpu().numpy(), rc), (case, B, C, k, k_tok, kind, split)
    assert np.array_equal(tok.cpu().numpy(), ref), (case, B, C, k, k_tok, kind, split)


# ---- the token select's candidate path and its fallbacks -----------------

def _sample_positions(n_pos: int):
    """Positions whose keys form the token select's sample: for s = 0..127,
    token (29 s + 7) mod 64 of list entry s * n_list / 128."""
    n_list = n_pos // 64
    return np.array([64 * (s * n_list // 128) + (29 * s + 7) % 64 for s in range(128)])


@pytest.mark.parametrize("kind", ["normal", "quarters", "all_equal", "sample_high", "few_competing", "tiny_k",
                                  "k_near_n", "negative", "narrow", "cluster", "full_precision", "ascending",
                                  "band_at_boundary"])
@pytest.mark.parametrize("split", [False, True], ids=["one_workgroup", "slices"])
def test_topk_tokens_candidate_path(lsa, oracle_lib, synth_lib, tune, kind, split):
    """Rows that take the candidate path (a sample bound, then a select
    among the keys at or above it) and rows that miss it on purpose and run
    the full select: all keys equal (more candidates than LDS holds), the
    largest scores placed exactly on the sample (too few candidates), fewer
    competing positions than k_tok, and extreme k_tok.  Scores within a few
    thousand ulps of each other ("narrow") make the candidates' histogram
    exact at once; a dense cluster of values 4 ulps apart holding the k-th
    largest ("cluster") sends it through three histogram levels; unrounded
    fp32 normals ("full_precision") leave several values in the k-th key's
    bin, which one wave then finishes (by pairwise counts; 40 distinct
    keys in one bin at the boundary, "band_at_boundary", bit by bit); scores
    ascending along the row
    ("ascending") give some waves more candidates than their LDS region
    holds, so the full select runs.  With `split` the row is cut into two
    slices (the slice + candidates path, whose two kernels take the same
    fast select); bit-exact with the oracle either way."""
    B, C, k = 3, 2048, 276
    n = k * 64
    s = synth_lib.bf16_bits_to_f32(synth_lib.normal_bf16((B, n), 31, synth_lib.stream(synth_lib.TAG_MISC, 6500)))
    k_tok = 2048
    ids = np.stack([np.sort(synth_lib.choose(k, C, 5, synth_lib.stream(synth_lib.TAG_MISC, 6600 + b)))
                    for b in range(B)]).astype(np.int32)
    ctx = np.full(B, C * 64, dtype=np.int32)
    counts = None
    if kind == "quarters":
        s = np.round(s * 4) / 4
    elif kind == "all_equal":
        s[:] = 0.75
    elif kind == "sample_high":
        s = s - 10.0
        s[:, _sample_positions(n)] = 5.0 + s[:, _sample_positions(n)] / 100
    elif kind == "few_competing":
        counts = np.array([20, 40, k], dtype=np.int32)  # 1,280 and 2,560 positions compete
        ctx[2] = int(ids[2, 30]) * 64 + 7
    elif kind == "tiny_k":
        k_tok = 1
    elif kind == "k_near_n":
        k_tok = n - 5
    elif kind == "negative":
        s = -np.abs(s) - 1.0
    elif kind == "narrow":
        r = np.random.default_rng(65)
        s = (np.float32(1.0) + r.integers(0, 3000, s.shape) * np.float32(2.0 ** -23)).astype(np.float32)
    elif kind == "band_at_boundary":  # 2,038 large keys, then 40 distinct keys in [1, 1 + 2^-12): k-th in the band
        r = np.random.default_rng(68)
        for b in range(B):
            perm = r.permutation(n)
            s[b] = -50.0 + r.standard_normal(n)
            s[b, perm[:2038]] = 50.0 + r.standard_normal(2038)
            s[b, perm[2038:2078]] = 1.0 + r.random(40) * 2.0 ** -12
    elif kind == "ascending":  # the candidates crowd the last waves' ranges: more than a wave's LDS region holds
        s = np.sort(s, axis=1)
    elif kind == "full_precision":  # all 23 mantissa bits: the k-th largest key's bin holds several values
        s = np.random.default_rng(67).standard_normal(s.shape).astype(np.float32)
    elif kind == "cluster":
        r = np.random.default_rng(66)
        inside = r.random(s.shape) < 0.4
        s = np.where(inside, np.float32(2.0) + r.integers(0, 64, s.shape) * np.float32(2.0 ** -20), s)
    s = np.ascontiguousarray(s, dtype=np.float32)
    if split:
        tune(topk_split_min_n=1)
    ref, rc = oracle_lib.topk_tokens(s, ids, ctx, k_tok, counts=counts)
    tok, tc = lsa.lsa_topk_tokens(to_dev(s), to_dev(ids), to_dev(ctx), k_tok,
                                  counts=None if counts is None else to_dev(counts),
                                  workspace="auto" if split else None)
    assert np.array_equal(tc.cpu().numpy(), rc), (kind, split)
    assert np.array_equal(tok.cpu().numpy(), ref), (kind, split)
