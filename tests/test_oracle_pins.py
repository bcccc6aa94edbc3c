"""Pins of the CPU oracle against things other than itself: brute force on
tiny inputs, library routines (numpy integer matmul, scipy's expit, torch's
dense scaled-dot-product attention in float64), closed forms worked out by hand
(tests/golden/closed_forms.json) and invariants of the definitions."""
import itertools
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bf16(x):
    """float array -> bf16 bits (round to nearest even); test inputs only."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f32(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def make_store(K, V, Hkv=1, T=64):
    """Tokens [n][d] of one request/head -> kv store [1][C][2][Hkv][T][d]."""
    K = np.asarray(K, dtype=np.float32)
    V = np.asarray(V, dtype=np.float32)
    n, d = K.shape
    C = (n + T - 1) // T
    kv = np.zeros((1, C, 2, Hkv, T, d), dtype=np.uint16)
    for j in range(n):
        c, t = divmod(j, T)
        for g in range(Hkv):
            kv[0, c, 0, g, t] = bf16(K[j])
            kv[0, c, 1, g, t] = bf16(V[j])
    return kv


# ---------------------------------------------------------------- indexer

def test_logits_closed_form(oracle_lib):
    g = _golden("closed_forms.json")["indexer_logits"]
    q = np.array(g["q"], dtype=np.int8).reshape(1, 1, -1)
    K = np.array(g["keys"], dtype=np.int8).reshape(1, len(g["keys"]), -1)
    assert oracle_lib.index_logits(q, K)[0].tolist() == g["expected"]


def test_logits_extreme_fits_int32(oracle_lib):
    g = _golden("closed_forms.json")["indexer_logits_extreme"]
    q = np.full((1, 1, g["d_idx"]), g["q_value"], dtype=np.int8)
    K = np.full((1, 3, g["d_idx"]), g["key_value"], dtype=np.int8)
    K[0, 1] = 127
    out = oracle_lib.index_logits(q, K)[0]
    assert out[0] == g["expected"] == 2 ** 21
    assert out[1] == -128 * 127 * 128
    assert out[2] == g["expected"]


def test_logits_vs_numpy_integer_matmul(oracle_lib, synth_lib):
    q = synth_lib.uniform_i8((3, 2, 128), 11, synth_lib.stream(synth_lib.TAG_MISC, 1), -128, 127)
    K = synth_lib.uniform_i8((3, 50, 128), 11, synth_lib.stream(synth_lib.TAG_MISC, 2), -128, 127)
    ref = np.einsum("brd,bcd->brc", q.astype(np.int64), K.astype(np.int64)).reshape(6, 50)
    assert np.array_equal(oracle_lib.index_logits(q, K), ref)


def test_logits_golden_key_closed_form(oracle_lib, synth_lib):
    """A key equal to 8*sign(q) scores exactly 8*sum|q|."""
    q = synth_lib.uniform_i8((2, 1, 64), 5, synth_lib.stream(synth_lib.TAG_MISC, 3), -16, 15)
    K = (8 * np.sign(q.astype(np.int32))).astype(np.int8)  # [2][1][64] -> one chunk each
    out = oracle_lib.index_logits(q, K)
    assert out[:, 0].tolist() == [8 * int(np.abs(q[b, 0].astype(np.int64)).sum()) for b in range(2)]


def test_scores_closed_form_and_expit(oracle_lib):
    from scipy.special import expit
    g = _golden("closed_forms.json")["sigmoid"]
    logits = np.array([c["logit"] for c in g["cases"]], dtype=np.int64)
    s = oracle_lib.index_scores(logits, g["alpha"])
    assert s[0] == 0.5
    for got, c in zip(s, g["cases"]):
        assert abs(got - c["expected"]) <= 1e-15
    # against scipy's logistic on the same fp32 argument, over a wide range
    L = np.arange(-200000, 200001, 37, dtype=np.int64)
    alpha = 2.0 ** -11
    x = (np.float32(alpha) * L.astype(np.float32)).astype(np.float64)
    np.testing.assert_allclose(oracle_lib.index_scores(L, alpha), expit(x), rtol=1e-14, atol=0)
    # symmetry sigma(x) + sigma(-x) = 1
    np.testing.assert_allclose(oracle_lib.index_scores(L, alpha) + oracle_lib.index_scores(-L, alpha), 1.0,
                               rtol=0, atol=1e-15)


def test_scores_argument_is_fp32_product(oracle_lib):
    """A non-power-of-two alpha: the argument is rounded to fp32 before the sigmoid."""
    alpha = 0.1
    L = np.array([3, 7, 1234567], dtype=np.int64)
    x32 = (np.float32(alpha) * L.astype(np.float32)).astype(np.float64)
    want = 1.0 / (1.0 + np.exp(-x32))
    assert np.array_equal(oracle_lib.index_scores(L, alpha), want)


# ---------------------------------------------------------------- selection

def brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda c: (-row[c], c))
    return sorted(order[:k])


def test_topk_closed_form(oracle_lib):
    g = _golden("closed_forms.json")["topk"]
    L = np.array([g["logits"]], dtype=np.int64)
    for c in g["cases"]:
        assert oracle_lib.topk_chunks(L, c["k"])[0].tolist() == c["expected"]


@pytest.mark.parametrize("kind", ["random", "equal", "two_valued", "few_values", "descending"])
def test_topk_vs_brute_force(oracle_lib, synth_lib, kind):
    """T1: the rank-count selection equals a full sort on tiny inputs."""
    for C in (1, 2, 3, 7, 16, 33, 64):
        if kind == "random":
            row = synth_lib.uniform_i32((C,), 1, synth_lib.stream(synth_lib.TAG_MISC, 10 + C), -1000, 1000)
        elif kind == "equal":
            row = np.full(C, 42, dtype=np.int32)
        elif kind == "two_valued":
            row = synth_lib.uniform_i32((C,), 2, synth_lib.stream(synth_lib.TAG_MISC, 100 + C), 0, 1) * 5 - 2
        elif kind == "few_values":
            row = synth_lib.uniform_i32((C,), 3, synth_lib.stream(synth_lib.TAG_MISC, 200 + C), -2, 2)
        else:
            row = np.arange(C, 0, -1, dtype=np.int32)
        for k in sorted({1, C, max(1, C // 2), max(1, C - 1)}):
            got = oracle_lib.topk_chunks(row.reshape(1, -1).astype(np.int64), k)[0].tolist()
            assert got == brute_topk(row.tolist(), k), (kind, C, k)


def test_topk_rejects_bad_k(oracle_lib):
    L = np.zeros((1, 4), dtype=np.int64)
    for k in (0, 5, -1):
        with pytest.raises(ValueError):
            oracle_lib.topk_chunks(L, k)


def test_selection_by_score_equals_selection_by_logit(oracle_lib, synth_lib):
    """T4: sigmoid is monotone, so selecting on sigma(alpha*l) picks the same
    chunks as selecting on l; in the workloads' argument range distinct
    logits give distinct fp64 scores, so ties are the same ties."""
    from synth import workloads as W
    for name in ("tiny", "32k", "128k"):
        w = W.WORKLOADS[name]
        K = W.indexer_keys(w)
        for it in range(w.intervals if w.drift else 1):
            q = W.indexer_query(w, it)
            L = oracle_lib.index_logits(q, K)
            S = oracle_lib.index_scores(L, w.alpha)
            assert np.abs(L).max() * w.alpha <= 12.0
            ids_l = oracle_lib.topk_chunks(L, w.k)
            ids_s = oracle_lib.topk_chunks(S, w.k)
            assert np.array_equal(ids_l, ids_s), (name, it)
            for r in range(L.shape[0]):
                u_l = np.unique(L[r])
                u_s = np.unique(S[r])
                assert u_l.size == u_s.size  # distinct logits -> distinct scores


# ---------------------------------------------------------------- attention

def _attend_one(oracle_lib, case, Hkv=1):
    d = case["d"]
    kv = make_store(case["K"], case["V"], Hkv=Hkv)
    q = bf16(np.array(case["q"], dtype=np.float32)).reshape(1, 1, d)
    ids = np.array([[0]], dtype=np.int32)
    return oracle_lib.gather_attend(q, kv, ids, np.array([case["ctx_len"]]), Hkv, case["scale"])


def test_attention_closed_forms(oracle_lib):
    for case in _golden("closed_forms.json")["attention"]["cases"]:
        out = _attend_one(oracle_lib, case)
        np.testing.assert_allclose(out[0, 0], case["expected"], rtol=0, atol=1e-14, err_msg=case["name"])


def test_attention_masks_tokens_past_context(oracle_lib):
    """Tokens at or past ctx_len must not count, whatever they hold."""
    case = _golden("closed_forms.json")["attention"]["cases"][0]
    K = np.array(case["K"] + [[50.0, 0.0]] * 3, dtype=np.float32)
    V = np.array(case["V"] + [[1000.0, -1000.0]] * 3, dtype=np.float32)
    out = _attend_one(oracle_lib, dict(case, K=K.tolist(), V=V.tolist()))
    np.testing.assert_allclose(out[0, 0], case["expected"], rtol=0, atol=1e-14)


def _random_problem(synth_lib, B, Hq, Hkv, d, C, seed, T=64, qscale=1.0):
    s = synth_lib.stream
    q = synth_lib.normal_bf16((B, Hq, d), seed, s(synth_lib.TAG_MISC, 300), scale=qscale)
    kv = synth_lib.normal_bf16((B, C, 2, Hkv, T, d), seed, s(synth_lib.TAG_MISC, 301))
    return q, kv


def _sdpa_dense(q, kv, ctx, Hkv, scale, T=64):
    """Dense attention over the first ctx[b] tokens with torch's float64 SDPA."""
    import torch
    B, Hq, d = q.shape
    outs = []
    for b in range(B):
        C = kv.shape[1]
        K = f32(kv[b, :, 0]).transpose(1, 0, 2, 3).reshape(Hkv, C * T, d)[:, : ctx[b]]
        V = f32(kv[b, :, 1]).transpose(1, 0, 2, 3).reshape(Hkv, C * T, d)[:, : ctx[b]]
        Q = torch.from_numpy(f32(q[b]).astype(np.float64)).reshape(1, Hq, 1, d)
        Kt = torch.from_numpy(K.astype(np.float64)).reshape(1, Hkv, -1, d)
        Vt = torch.from_numpy(V.astype(np.float64)).reshape(1, Hkv, -1, d)
        o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, scale=scale, enable_gqa=True)
        outs.append(o.reshape(Hq, d).numpy())
    return np.stack(outs)


@pytest.mark.parametrize("B,Hq,Hkv,d,C,ctx", [
    (1, 8, 1, 64, 4, [256]),
    (2, 16, 2, 128, 3, [192, 150]),       # second request: partial last chunk
    (2, 64, 8, 128, 2, [128, 65]),        # DeepSeek-V4 GQA shape, one token in last chunk
    (1, 4, 4, 32, 3, [130]),              # MHA special case
])
def test_all_chunks_equals_dense_sdpa(oracle_lib, synth_lib, B, Hq, Hkv, d, C, ctx):
    """T2: with every chunk kept, sparse attention is dense attention."""
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=7)
    ctx = np.array(ctx, dtype=np.int32)
    ids = np.tile(np.arange(C, dtype=np.int32), (B, 1))
    scale = 1.0 / math.sqrt(d)
    out = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, scale)
    ref = _sdpa_dense(q, kv, ctx, Hkv, scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_sparse_equals_sdpa_over_selected_tokens(oracle_lib, synth_lib):
    """A strict subset of chunks: dense SDPA on the gathered tokens only."""
    import torch
    B, Hq, Hkv, d, C, T = 2, 16, 2, 64, 6, 64
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=8, qscale=4.0)
    ids = np.array([[1, 4, 5], [0, 2, 3]], dtype=np.int32)
    ctx = np.array([C * T - 10, C * T], dtype=np.int32)
    out = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / math.sqrt(d))
    for b in range(B):
        toks = [c * T + t for c in ids[b] for t in range(T) if c * T + t < ctx[b]]
        Kall = f32(kv[b, :, 0]).transpose(1, 0, 2, 3).reshape(Hkv, C * T, d)[:, toks]
        Vall = f32(kv[b, :, 1]).transpose(1, 0, 2, 3).reshape(Hkv, C * T, d)[:, toks]
        Q = torch.from_numpy(f32(q[b]).astype(np.float64)).reshape(1, Hq, 1, d)
        o = torch.nn.functional.scaled_dot_product_attention(
            Q, torch.from_numpy(Kall.astype(np.float64))[None], torch.from_numpy(Vall.astype(np.float64))[None],
            scale=1 / math.sqrt(d), enable_gqa=True)
        np.testing.assert_allclose(out[b], o.reshape(Hq, d).numpy(), rtol=1e-12, atol=1e-14)


def test_softmax_weights_sum_to_one(oracle_lib, synth_lib):
    """T3."""
    B, Hq, Hkv, d, C = 2, 16, 2, 128, 5
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=9, qscale=8.0)
    ids = np.array([[0, 2, 4], [1, 3, 4]], dtype=np.int32)
    ctx = np.array([C * 64 - 40, C * 64], dtype=np.int32)
    _, w = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / math.sqrt(d), want_weights=True)
    np.testing.assert_allclose(w.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    assert (w >= 0).all()
    # the masked tail of request 0 (chunk 4, tokens 24..63) has zero weight
    assert (w[0, :, 2 * 64 + 24:] == 0).all()


def test_single_token_returns_its_value(oracle_lib, synth_lib):
    B, Hq, Hkv, d, C = 1, 8, 1, 64, 3
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=10, qscale=3.0)
    ids = np.array([[2]], dtype=np.int32)
    ctx = np.array([2 * 64 + 1], dtype=np.int32)  # only token 128 (chunk 2, t = 0) is valid
    out = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 0.125)
    v = f32(kv[0, 2, 1, 0, 0]).astype(np.float64)
    assert np.array_equal(out[0], np.tile(v, (Hq, 1)))


def test_identical_keys_give_mean_of_values(oracle_lib, synth_lib):
    B, Hq, Hkv, d, C = 1, 8, 1, 64, 2
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=11)
    kv[:, :, 0] = kv[0, 0, 0, 0, 0]  # every key the same vector
    ids = np.array([[0, 1]], dtype=np.int32)
    out = oracle_lib.gather_attend(q, kv, ids, np.array([128]), Hkv, 0.125)
    V = f32(kv[0, :, 1, 0]).reshape(128, d).astype(np.float64)
    np.testing.assert_allclose(out[0], np.tile(V.mean(axis=0), (Hq, 1)), rtol=1e-13, atol=1e-15)


def test_convex_hull_and_gqa_as_mha(oracle_lib, synth_lib):
    B, Hq, Hkv, d, C = 2, 16, 2, 64, 4
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=12, qscale=5.0)
    ids = np.array([[0, 3], [1, 2]], dtype=np.int32)
    ctx = np.array([C * 64, C * 64 - 5], dtype=np.int32)
    out = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / 8)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            V = np.concatenate([f32(kv[b, c, 1, g]) for c in ids[b]])
            assert (out[b, h] >= V.min(axis=0) - 1e-12).all() and (out[b, h] <= V.max(axis=0) + 1e-12).all()
    # MHA with each KV head repeated Hq/Hkv times gives the same result
    kv_mha = np.repeat(kv, Hq // Hkv, axis=3)
    out_mha = oracle_lib.gather_attend(q, kv_mha, ids, ctx, Hq, 1 / 8)
    np.testing.assert_allclose(out, out_mha, rtol=0, atol=0)


def test_chunk_order_and_slots(oracle_lib, synth_lib):
    """Listing chunks in another order, or storing them at other slots, does
    not change the result beyond summation order."""
    B, Hq, Hkv, d, C = 1, 16, 2, 64, 6
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=13, qscale=2.0)
    ctx = np.array([C * 64 - 7], dtype=np.int32)
    ids = np.array([[0, 2, 5]], dtype=np.int32)
    base = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / 8)
    for perm in itertools.permutations(range(3)):
        p = ids[:, list(perm)]
        np.testing.assert_allclose(oracle_lib.gather_attend(q, kv, p, ctx, Hkv, 1 / 8), base, rtol=1e-12,
                                   atol=1e-14)
    pool = kv[:, [5, 0, 2]]  # compact pool holding chunks 5, 0, 2 in slots 0, 1, 2
    out = oracle_lib.gather_attend(q, pool, ids, ctx, Hkv, 1 / 8, slots=np.array([[1, 2, 0]], dtype=np.int32))
    np.testing.assert_allclose(out, base, rtol=0, atol=0)


def test_attention_vs_python_loops(oracle_lib, synth_lib):
    """Brute force with math.exp on a tiny case (independent of numpy/torch)."""
    B, Hq, Hkv, d, C, T = 1, 4, 2, 8, 2, 64
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=14, qscale=2.0)
    ids = np.array([[1, 0]], dtype=np.int32)
    ctx = np.array([100], dtype=np.int32)
    out = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 0.3)
    qf, kf = f32(q).astype(float), f32(kv).astype(float)
    for h in range(Hq):
        g = h // 2
        toks = [(c, t) for c in (1, 0) for t in range(T) if c * T + t < 100]
        z = [sum(qf[0, h, i] * kf[0, c, 0, g, t, i] for i in range(d)) * 0.3 for c, t in toks]
        m = max(z)
        w = [math.exp(x - m) for x in z]
        o = [sum(w[j] * kf[0, c, 1, g, t, i] for j, (c, t) in enumerate(toks)) / sum(w) for i in range(d)]
        np.testing.assert_allclose(out[0, h], o, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- fetch + schedule

def test_fetch_is_a_byte_copy(oracle_lib, synth_lib):
    host = synth_lib.normal_bf16((2, 9, 2, 2, 64, 16), 3, synth_lib.stream(synth_lib.TAG_MISC, 400))
    ids = np.array([[0, 4, 8], [3, 4, 5]], dtype=np.int32)
    slots = np.array([[2, 0, 1], [0, 1, 2]], dtype=np.int32)
    pool = oracle_lib.fetch_chunks(host, ids, P=4, slots=slots)
    for b in range(2):
        for j in range(3):
            assert np.array_equal(pool[b, slots[b, j]], host[b, ids[b, j]])
        assert (pool[b, 3] == 0).all()
    with pytest.raises(ValueError):
        oracle_lib.fetch_chunks(host, np.array([[9]], dtype=np.int32), P=1)


def test_schedule(oracle_lib):
    tau = _golden("pages_figures.json")["tau_steps"]["value"]
    assert [t for t in range(256) if oracle_lib.is_reselect_step(t, tau)] == [0, 64, 128, 192]
    assert [oracle_lib.selection_for_step(t, tau, 0) for t in (0, 63, 64, 255)] == [0, 0, 1, 3]
    assert [oracle_lib.selection_for_step(t, tau, 1) for t in (0, 63, 64, 127, 128, 255)] == [0, 0, 0, 0, 1, 2]


# ---------------------------------------------------------------- delta-fetch slots

def test_pool_assign_closed_form(oracle_lib):
    g = _golden("closed_forms.json")["pool_assign"]
    ns, fs = oracle_lib.pool_assign(np.array([g["prev_ids"]]), np.array([g["prev_slots"]]),
                                    np.array([g["new_ids"]]), g["P"])
    assert ns[0].tolist() == g["expected_new_slots"]
    assert fs[0].tolist() == g["expected_fetch_slots"]


def test_pool_assign_chain_keeps_pool_consistent(oracle_lib, synth_lib):
    """Over a chain of random selections, with only the new chunks fetched:
    kept chunks keep their slots, new chunks land in slots the previous
    selection does not hold (distinct, lowest first), and the pool always
    holds every selected chunk at its slot (checked against a full copy)."""
    B, C, k = 3, 40, 9
    P = 2 * k
    host = synth_lib.normal_bf16((B, C, 2, 1, 64, 8), 4, synth_lib.stream(synth_lib.TAG_MISC, 1700))
    pool = np.zeros((B, P, 2, 1, 64, 8), dtype=np.uint16)
    prev_ids = prev_slots = None
    for step in range(12):
        ids = np.stack([np.sort(synth_lib.choose(k, C if step % 3 else 12, 4,
                                                 synth_lib.stream(synth_lib.TAG_MISC, 1800 + 10 * step + b)))
                        for b in range(B)]).astype(np.int32)
        ns, fs = oracle_lib.pool_assign(prev_ids, prev_slots, ids, P)
        for b in range(B):
            assert len(set(ns[b].tolist())) == k and (ns[b] >= 0).all() and (ns[b] < P).all()
            prev_map = {} if prev_ids is None else dict(zip(prev_ids[b].tolist(), prev_slots[b].tolist()))
            held = set(prev_map.values())
            new_slots = []
            for j in range(k):
                c = int(ids[b, j])
                if c in prev_map:
                    assert ns[b, j] == prev_map[c] and fs[b, j] == -1
                else:
                    assert fs[b, j] == ns[b, j] and ns[b, j] not in held
                    new_slots.append(int(ns[b, j]))
            free = [s for s in range(P) if s not in held]
            assert new_slots == free[:len(new_slots)]  # lowest free slots, in id order
        oracle_lib.fetch_chunks(host, ids, P, slots=fs, pool=pool, skip_negative_slots=True)
        for b in range(B):
            for j in range(k):
                assert np.array_equal(pool[b, ns[b, j]], host[b, ids[b, j]]), (step, b, j)
        prev_ids, prev_slots = ids, ns


def test_pool_assign_variable_counts(oracle_lib, synth_lib):
    """Selections of varying size, padded with -1 past each count (as the
    threshold select writes them): padding in the previous list holds no
    slot, padding in the new list gets slot -1 and is not fetched, and the
    pool stays consistent across a chain of such selections."""
    B, C, k = 3, 40, 9
    P = 2 * k
    host = synth_lib.normal_bf16((B, C, 2, 1, 64, 8), 5, synth_lib.stream(synth_lib.TAG_MISC, 1750))
    pool = np.zeros((B, P, 2, 1, 64, 8), dtype=np.uint16)
    rng = np.random.default_rng(5)
    prev_ids = prev_slots = None
    for step in range(15):
        counts = rng.integers(0, k + 1, B)
        ids = np.full((B, k), -1, dtype=np.int32)
        for b in range(B):
            ids[b, :counts[b]] = np.sort(rng.choice(C if step % 3 else 14, counts[b], replace=False))
        ns, fs = oracle_lib.pool_assign(prev_ids, prev_slots, ids, P)
        for b in range(B):
            n = int(counts[b])
            assert (ns[b, n:] == -1).all() and (fs[b, n:] == -1).all()
            used = ns[b, :n]
            assert len(set(used.tolist())) == n and (used >= 0).all() and (used < P).all()
            prev_map = {}
            if prev_ids is not None:
                prev_map = {c: s for c, s in zip(prev_ids[b].tolist(), prev_slots[b].tolist()) if c >= 0}
            held = set(prev_map.values())
            fetched = []
            for j in range(n):
                c = int(ids[b, j])
                if c in prev_map:
                    assert ns[b, j] == prev_map[c] and fs[b, j] == -1
                else:
                    assert fs[b, j] == ns[b, j] and ns[b, j] not in held
                    fetched.append(int(ns[b, j]))
            free = [x for x in range(P) if x not in held]
            assert fetched == free[:len(fetched)]
        oracle_lib.fetch_chunks(host, np.maximum(ids, 0), P, slots=fs, pool=pool, skip_negative_slots=True)
        for b in range(B):
            for j in range(int(counts[b])):
                assert np.array_equal(pool[b, ns[b, j]], host[b, ids[b, j]]), (step, b, j)
        # the slots of entries not in use are not looked at: make them garbage
        prev_ids, prev_slots = ids, np.where(ids >= 0, ns, 10 ** 6).astype(np.int32)


# ---------------------------------------------------------------- threshold selection

def brute_threshold(row, thr, k_max):
    passing = [c for c in range(len(row)) if row[c] > thr]
    order = sorted(passing, key=lambda c: (-row[c], c))[:k_max]
    return sorted(order)


@pytest.mark.parametrize("kind", ["random", "few_values", "none_pass", "all_pass"])
def test_threshold_vs_brute_force(oracle_lib, synth_lib, kind):
    for C in (1, 5, 33, 64, 200):
        if kind == "random":
            row = synth_lib.uniform_i32((C,), 6, synth_lib.stream(synth_lib.TAG_MISC, 2100 + C), -50, 50)
        elif kind == "few_values":
            row = synth_lib.uniform_i32((C,), 7, synth_lib.stream(synth_lib.TAG_MISC, 2200 + C), -1, 1)
        elif kind == "none_pass":
            row = -np.abs(synth_lib.uniform_i32((C,), 8, synth_lib.stream(synth_lib.TAG_MISC, 2300 + C), 0, 9))
        else:
            row = 1 + np.abs(synth_lib.uniform_i32((C,), 9, synth_lib.stream(synth_lib.TAG_MISC, 2400 + C), 0, 9))
        for k_max in sorted({1, C, max(1, C // 3)}):
            for thr in (-1, 0, 3):
                ids, counts = oracle_lib.threshold_chunks(row.reshape(1, -1).astype(np.int64), k_max, thr)
                want = brute_threshold(row.tolist(), thr, k_max)
                assert counts[0] == len(want)
                assert ids[0, :len(want)].tolist() == want and (ids[0, len(want):] == -1).all()


def test_threshold_zero_is_sigmoid_half(oracle_lib, synth_lib):
    """sigma(alpha * logit) > 0.5 keeps the same chunks as logit > 0 (scipy's
    logistic on the fp32 argument decides the first)."""
    from scipy.special import expit
    row = synth_lib.uniform_i32((300,), 10, synth_lib.stream(synth_lib.TAG_MISC, 2500), -3000, 3000)
    row[:5] = [0, 1, -1, 2, -2]
    alpha = 2.0 ** -11
    x = (np.float32(alpha) * row.astype(np.float32)).astype(np.float64)
    passing = np.nonzero(expit(x) > 0.5)[0]
    ids, counts = oracle_lib.threshold_chunks(row.reshape(1, -1).astype(np.int64), 300, 0)
    assert np.array_equal(ids[0, :counts[0]], passing)


def test_attention_counts_truncate_lists(oracle_lib, synth_lib):
    """counts[b] limits request b to its first counts[b] entries."""
    B, Hq, Hkv, d, C = 3, 8, 2, 64, 6
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=15, qscale=2.0)
    ids = np.array([[0, 2, 4, 5], [1, 3, 5, -1], [4, -1, -1, -1]], dtype=np.int32)
    counts = np.array([4, 3, 1], dtype=np.int32)
    ctx = np.full(B, C * 64, dtype=np.int32)
    out = oracle_lib.gather_attend(q, kv, np.where(ids < 0, 0, ids), ctx, Hkv, 0.125, counts=counts)
    for b in range(B):
        ref = oracle_lib.gather_attend(q[b:b + 1], kv[b:b + 1], ids[b:b + 1, :counts[b]], ctx[b:b + 1], Hkv, 0.125)
        np.testing.assert_allclose(out[b], ref[0], rtol=0, atol=0)


# ---------------------------------------------------------------- resident segment (local window)

def test_segment_joins_chunks_in_one_softmax(oracle_lib, synth_lib):
    """Chunks plus a resident segment equal dense SDPA over the concatenated
    tokens; with no chunk in use (counts = 0) the segment alone is dense
    attention over it; the weights of both parts sum to 1."""
    import torch
    B, Hq, Hkv, d, C, S = 2, 16, 2, 64, 5, 128
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=16, qscale=3.0)
    seg = synth_lib.normal_bf16((B, 2, Hkv, S, d), 16, synth_lib.stream(synth_lib.TAG_MISC, 2600))
    seg_len = np.array([100, 1], dtype=np.int32)
    ids = np.array([[0, 3], [1, 4]], dtype=np.int32)
    ctx = np.array([C * 64 - 30, C * 64], dtype=np.int32)
    out, w = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 0.125, seg_kv=seg, seg_len=seg_len, want_weights=True)
    np.testing.assert_allclose(w.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    for b in range(B):
        toks = [c * 64 + t for c in ids[b] for t in range(64) if c * 64 + t < ctx[b]]
        K = np.concatenate([f32(kv[b, :, 0]).transpose(1, 0, 2, 3).reshape(Hkv, C * 64, d)[:, toks],
                            f32(seg[b, 0, :, :seg_len[b]])], axis=1)
        V = np.concatenate([f32(kv[b, :, 1]).transpose(1, 0, 2, 3).reshape(Hkv, C * 64, d)[:, toks],
                            f32(seg[b, 1, :, :seg_len[b]])], axis=1)
        Q = torch.from_numpy(f32(q[b]).astype(np.float64)).reshape(1, Hq, 1, d)
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, torch.from_numpy(K.astype(np.float64))[None], torch.from_numpy(V.astype(np.float64))[None],
            scale=0.125, enable_gqa=True).reshape(Hq, d).numpy()
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-14)
    # segment only
    only = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 0.125, counts=np.zeros(B, dtype=np.int32),
                                    seg_kv=seg, seg_len=seg_len)
    np.testing.assert_allclose(only[1], np.tile(f32(seg[1, 1, :, 0]).astype(np.float64).repeat(Hq // Hkv, 0)
                                                .reshape(Hq, d), 1), rtol=0, atol=0)


# ------------------------------------------------------------------ token selection inside recalled chunks

def brute_tokens(scores, ids, ctx, k_tok, counts=None, T=64):
    """Python's sorted() on (-score, position) over the usable positions."""
    B, n = scores.shape
    out = np.full((B, k_tok), -1, dtype=np.int32)
    cnt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        kb = ids.shape[1] if counts is None else min(max(int(counts[b]), 0), ids.shape[1])
        use = [p for p in range(n) if p // T < kb and int(ids[b, p // T]) * T + p % T < int(ctx[b])]
        keep = sorted(sorted(use, key=lambda p: (-float(scores[b, p]), p))[:k_tok])
        out[b, :len(keep)] = keep
        cnt[b] = len(keep)
    return out, cnt


def _token_scores(synth_lib, B, n, seed):
    """bf16-rounded normals (many exact ties) with signed zeros and infinities planted."""
    s = synth_lib.bf16_bits_to_f32(synth_lib.normal_bf16((B, n), seed, synth_lib.stream(synth_lib.TAG_MISC, 1400)))
    s = np.round(s * 4) / 4  # coarser still: long runs of equal scores
    s[:, 3::17] = 0.0
    s[:, 5::19] = -0.0
    s[:, 7::41] = np.inf
    s[:, 11::43] = -np.inf
    return s.astype(np.float32)


@pytest.mark.parametrize("T,k,k_tok", [(4, 5, 3), (4, 5, 7), (8, 6, 20), (64, 3, 50), (64, 3, 192), (4, 3, 100)])
def test_token_select_vs_brute_force(oracle_lib, synth_lib, T, k, k_tok):
    B, C = 4, 12
    scores = _token_scores(synth_lib, B, k * T, seed=T + k)
    ids = np.stack([np.sort(synth_lib.choose(k, C, 5, synth_lib.stream(synth_lib.TAG_MISC, 1410 + b)))
                    for b in range(B)]).astype(np.int32)
    ctx = np.array([C * T, ids[1, -1] * T + T // 2, ids[2, 1] * T + 1, 0], dtype=np.int32)  # full, partial, short, none
    counts = np.array([k, k, k - 1, k], dtype=np.int32)
    for cn in (None, counts):
        got, gc = oracle_lib.topk_tokens(scores, ids, ctx, k_tok, counts=cn, T=T)
        ref, rc = brute_tokens(scores, ids, ctx, k_tok, counts=cn, T=T)
        assert np.array_equal(gc, rc) and np.array_equal(got, ref), (T, k, k_tok, cn)


def test_token_select_special_cases(oracle_lib):
    """Equal scores keep the lowest positions; a budget above the usable
    count keeps every usable token; signed zeros are equal scores."""
    T, k = 4, 3
    ids = np.array([[2, 5, 9]], dtype=np.int32)
    ctx = np.array([9 * T + 2], dtype=np.int32)  # tokens 0, 1 of the last chunk are usable
    flat = np.zeros((1, k * T), dtype=np.float32)
    tok, tc = oracle_lib.topk_tokens(flat, ids, ctx, 5, T=T)
    assert tok.tolist() == [[0, 1, 2, 3, 4]] and tc.tolist() == [5]
    tok, tc = oracle_lib.topk_tokens(flat, ids, ctx, 40, T=T)
    assert tc.tolist() == [10] and tok[0, :10].tolist() == list(range(10)) and (tok[0, 10:] == -1).all()
    z = np.array([[0.0, -0.0, 0.0, -0.0] * 3], dtype=np.float32)
    tok, _ = oracle_lib.topk_tokens(z, ids, ctx, 3, T=T)
    assert tok.tolist() == [[0, 1, 2]]
    ranked = np.arange(k * T, dtype=np.float32)[None]  # later positions score higher
    tok, tc = oracle_lib.topk_tokens(ranked, ids, ctx, 3, T=T)
    assert tok.tolist() == [[7, 8, 9]] and tc.tolist() == [3]  # 10, 11 are past the context


def test_token_attention_equals_sdpa_over_listed_tokens(oracle_lib, synth_lib):
    """Attention over a token list is dense SDPA over exactly those tokens;
    listed positions of unused entries or past the context are dropped."""
    import torch
    B, Hq, Hkv, d, C, T, k = 2, 16, 2, 64, 6, 64, 3
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=21, qscale=4.0)
    ids = np.array([[1, 4, 5], [0, 2, 3]], dtype=np.int32)
    ctx = np.array([5 * T + 10, C * T], dtype=np.int32)
    counts = np.array([3, 2], dtype=np.int32)
    tok = np.array([[130, 5, 64, 140, 63, 129, 200, -1],      # 140 is position 5*64+12 >= ctx: dropped
                    [3, 70, 127, 128, 190, 0, 1, 2]], dtype=np.int32)  # 128, 190 name unused entry 2
    tok_counts = np.array([7, 8], dtype=np.int32)
    out = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / math.sqrt(d), counts=counts, tok=tok,
                                   tok_counts=tok_counts)
    for b in range(B):
        keep = [int(p) for p in tok[b, :tok_counts[b]]
                if 0 <= p < counts[b] * T and ids[b, p // T] * T + p % T < ctx[b]]
        pos = [int(ids[b, p // T]) * T + p % T for p in keep]
        Kall = f32(kv[b, :, 0]).transpose(1, 0, 2, 3).reshape(Hkv, C * T, d)[:, pos]
        Vall = f32(kv[b, :, 1]).transpose(1, 0, 2, 3).reshape(Hkv, C * T, d)[:, pos]
        Q = torch.from_numpy(f32(q[b]).astype(np.float64)).reshape(1, Hq, 1, d)
        o = torch.nn.functional.scaled_dot_product_attention(
            Q, torch.from_numpy(Kall.astype(np.float64))[None], torch.from_numpy(Vall.astype(np.float64))[None],
            scale=1 / math.sqrt(d), enable_gqa=True)
        np.testing.assert_allclose(out[b], o.reshape(Hq, d).numpy(), rtol=1e-12, atol=1e-14)


def test_token_attention_all_tokens_equals_chunk_attention(oracle_lib, synth_lib):
    """Listing every token of the used entries reduces to chunk attention,
    output and weights alike; the list order does not matter."""
    B, Hq, Hkv, d, C, T = 2, 8, 1, 64, 5, 64
    q, kv = _random_problem(synth_lib, B, Hq, Hkv, d, C, seed=22, qscale=2.0)
    ids = np.array([[0, 2, 4], [1, 3, 4]], dtype=np.int32)
    ctx = np.array([C * T - 30, C * T], dtype=np.int32)
    ref, wref = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 0.125, want_weights=True)
    perm = np.stack([np.random.default_rng(b).permutation(3 * T) for b in range(B)]).astype(np.int32)
    got, wgot = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 0.125, want_weights=True, tok=perm)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(wgot, wref, rtol=1e-12, atol=1e-15)


_THREADS_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np
import oracle
rng = np.random.default_rng(11)
keys = rng.integers(-3, 4, size=(3, 3000)).astype(np.int64)
sc = rng.integers(-2, 3, size=(2, 40 * 64)).astype(np.float32)
ids = np.stack([np.sort(rng.choice(200, 40, replace=False)) for _ in range(2)]).astype(np.int32)
ctx = np.array([200 * 64, int(ids[1, 30]) * 64 + 9], dtype=np.int32)
t_ids, t_cnt = oracle.threshold_chunks(keys, 700, 1)
tok, tc = oracle.topk_tokens(sc, ids, ctx, 900)
np.savez({out!r}, topk=oracle.topk_chunks(keys, 1000), t_ids=t_ids, t_cnt=t_cnt, tok=tok, tc=tc)
"""


@pytest.mark.parametrize("threads", [1, 3])
def test_selections_do_not_depend_on_thread_count(tmp_path, threads):
    """The selections count ranks in parallel iterations: one thread, three
    threads and the default give the same lists on tie-heavy rows."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = {}
    for name, env_threads in (("default", None), ("set", str(threads))):
        out = tmp_path / f"{name}.npz"
        env = dict(os.environ)
        env.pop("OMP_NUM_THREADS", None)
        if env_threads:
            env["OMP_NUM_THREADS"] = env_threads
        r = subprocess.run([sys.executable, "-c", _THREADS_CHILD.format(root=root, out=str(out))], env=env,
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        outs[name] = np.load(out)
    for key in ("topk", "t_ids", "t_cnt", "tok", "tc"):
        assert np.array_equal(outs["default"][key], outs["set"][key]), key
