"""Randomised parity of the gathered attention with the oracle: seeded draws
of GQA shapes (1 to 16 query heads per KV head, head dim 64 or 128), list
lengths, split counts, partial contexts, ragged entry counts, pool slots,
resident segments and token lists (with invalid entries), within the
attention tolerance of fp64.  Every request keeps one valid token (token 0
of chunk 0, listed first), since the oracle rejects a request with none."""
import math

import numpy as np
import pytest

from conftest import gpu_available
from helpers import check_attention, to_dev, to_dev_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def lsa():
    import lookahead_chunk_sparse_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def _case(i):
    rng = np.random.default_rng(3000 + i)
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([g for g in (1, 2, 3, 4, 8, 16) if Hkv * g <= 64]))
    B = int(rng.integers(1, 5))
    C = int(rng.integers(2, 120))
    k = int(rng.integers(1, min(C, 48) + 1))
    n_split = int(rng.choice([0, 1, 2, 3, 5, 8, 13]))
    qscale = float(rng.choice([1.0, 4.0, 8.0]))
    mode = str(rng.choice(["chunks", "tokens"]))
    return dict(d=d, Hkv=Hkv, Hq=Hkv * G, B=B, C=C, k=k, n_split=n_split, qscale=qscale, mode=mode), rng


@pytest.mark.parametrize("case", range(150))
def test_attend_random(lsa, oracle_lib, synth_lib, case):
    p, rng = _case(case)
    B, Hq, Hkv, d, C, k = p["B"], p["Hq"], p["Hkv"], p["d"], p["C"], p["k"]
    s = synth_lib.stream
    q = synth_lib.normal_bf16((B, Hq, d), case, s(synth_lib.TAG_MISC, 7000), scale=p["qscale"])
    kv = synth_lib.normal_bf16((B, C, 2, Hkv, 64, d), case, s(synth_lib.TAG_MISC, 7001))
    ids = np.stack([np.sort(synth_lib.choose(k, C, case, s(synth_lib.TAG_MISC, 7100 + b))) for b in range(B)])
    ids = ids.astype(np.int32)
    ids[:, 0] = 0  # the smallest of distinct ascending ids becomes chunk 0: still distinct
    ctx = np.array([C * 64 if rng.integers(0, 2) else int(rng.integers(1, C * 64 + 1)) for _ in range(B)],
                   dtype=np.int32)
    counts = rng.integers(1, k + 1, B).astype(np.int32) if rng.integers(0, 2) else None
    store, slots = kv, None
    if rng.integers(0, 2):  # a compact pool in permuted slot order
        slots = np.stack([rng.permutation(k) for _ in range(B)]).astype(np.int32)
        store = np.zeros((B, k, 2, Hkv, 64, d), dtype=np.uint16)
        for b in range(B):
            store[b, slots[b]] = kv[b, ids[b]]
    seg = seg_len = None
    S_max = int(rng.choice([0, 0, 64, 192, 256]))  # the ABI takes whole 64-token rows of storage
    if S_max:
        seg = synth_lib.normal_bf16((B, 2, Hkv, S_max, d), case, s(synth_lib.TAG_MISC, 7002))
        seg_len = rng.integers(0, S_max + 1, B).astype(np.int32)
    tok = tok_counts = None
    if p["mode"] == "tokens":
        n_pos = k * 64
        k_tok = int(rng.integers(1, n_pos + 20))
        tok = rng.integers(-1, n_pos + 3, (B, k_tok)).astype(np.int32)  # repeats and invalid entries allowed
        tok[:, 0] = 0
        tok_counts = rng.integers(1, k_tok + 1, B).astype(np.int32) if rng.integers(0, 2) else None
    say("random attend case", case, p, "slots" if slots is not None else "", "counts" if counts is not None else "",
        f"seg {S_max}" if S_max else "")
    kw = {}
    if seg is not None:
        kw.update(seg_kv=to_dev_bf16(seg), seg_len=to_dev(seg_len))
    if tok is not None:
        kw.update(tok=to_dev(tok), tok_counts=None if tok_counts is None else to_dev(tok_counts))
    scale = 1.0 / math.sqrt(d)
    out = lsa.lsa_gather_attend(to_dev_bf16(q), to_dev_bf16(store), to_dev(ids), to_dev(ctx), scale,
                                slots=None if slots is None else to_dev(slots), n_split=p["n_split"],
                                counts=None if counts is None else to_dev(counts), **kw)
    ref = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, scale, counts=counts, seg_kv=seg, seg_len=seg_len,
                                   tok=tok, tok_counts=tok_counts)
    say("  ", check_attention(out.cpu().numpy(), ref, f"random attend case {case}"))
