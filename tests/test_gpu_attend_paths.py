"""Parity of the attention kernel's less common internal paths with the fp64
oracle (bf16 inputs, fp32 accumulation: max-abs 1e-2, mean-abs 1e-3, and
max error within 1e-3 of the output RMS):

  * a workgroup whose chunk list is longer than the 512 entries its LDS
    holds at a time (several staging rounds, each restarting the register
    ring), from a single split over 600 or 1100 chunks, or from chunks plus
    resident-segment blocks;
  * token lists over more than 1024 recalled chunks, where the kernel looks
    chunk ids and store positions up in global memory instead of LDS;
    among them the call the 1M two-stage benchmark makes (K/V in HBM, the
    top 2048 tokens of 1638 recalled chunks);
  * register ring depths 3 and 4 (the attend_depth knob), which must give
    the same bits as the default depth 2, set in-process and through the
    environment in a fresh process.

The attention formula and the GQA grouping follow the sergiiob.dev handbook
(DeepSeek-V4), "Grouped Query Attention (GQA) vs. Multi-Head Attention
(MHA)"; the token-level stage the paperlayer.ai summary of FlashMemory-
DeepSeek-V4, 2.1 Architecture."""
import math
import os
import subprocess
import sys

import numpy as np
import pytest

from conftest import gpu_available
from helpers import ATT_MAX_REL_RMS_FULL, check_attention, to_dev, to_dev_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lsa():
    import lookahead_chunk_sparse_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def _problem(synth_lib, B, Hq, Hkv, d, C, seed, qscale=2.0):
    s = synth_lib.stream
    q = synth_lib.normal_bf16((B, Hq, d), seed, s(synth_lib.TAG_MISC, 7100), scale=qscale)
    kv = synth_lib.normal_bf16((B, C, 2, Hkv, 64, d), seed, s(synth_lib.TAG_MISC, 7101))
    return q, kv


def _ids(synth_lib, B, C, k, seed):
    """Ascending distinct chunk ids per request, chunk 0 always among them."""
    out = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        out[b] = np.sort(synth_lib.choose(k, C, seed, synth_lib.stream(synth_lib.TAG_MISC, 7200 + b)))
        out[b, 0] = 0
    return out


def _compact_pool(kv, ids, k):
    """The listed chunks stored in a compact pool of k slots, slot order
    permuted: (pool, slots)."""
    B = kv.shape[0]
    perm = np.array([[(j * 7 + 3) % k for j in range(k)]] * B, dtype=np.int32)
    if math.gcd(7, k) != 1:  # (7j + 3) mod k must be a permutation
        perm = np.array([[(j * 11 + 3) % k for j in range(k)]] * B, dtype=np.int32)
    assert all(len(set(r)) == k for r in perm)
    pool = np.zeros((B, k) + kv.shape[2:], dtype=np.uint16)
    for b in range(B):
        pool[b, perm[b]] = kv[b, ids[b]]
    return pool, perm


# ----------------------------------------------------- chunk lists beyond LDS

LONG_CASES = [
    # B, Hq, Hkv, d, C, k, n_split, slots, partial context
    (2, 8, 1, 128, 650, 600, 1, False, False),
    (2, 8, 1, 128, 1150, 1100, 1, True, True),
    (2, 8, 1, 128, 1150, 1100, 2, False, True),   # 550 entries per workgroup
    (1, 12, 4, 64, 1040, 1025, 1, False, False),  # one entry past two full rounds of 512
]


@pytest.mark.parametrize("B,Hq,Hkv,d,C,k,n_split,use_slots,partial", LONG_CASES)
def test_attend_long_chunk_list(lsa, oracle_lib, synth_lib, B, Hq, Hkv, d, C, k, n_split, use_slots, partial):
    say("long chunk list", B, Hq, Hkv, d, C, k, n_split, use_slots, partial)
    q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=k + n_split)
    ids = _ids(synth_lib, B, C, k, seed=k)
    ctx = np.full(B, C * 64, dtype=np.int32)
    if partial:  # the context ends inside a listed chunk of the second round
        ctx[0] = int(ids[0, 700 if k > 700 else k - 1]) * 64 + 21
    counts = None
    if B > 1:
        counts = np.full(B, k, dtype=np.int32)
        counts[1] = k - 7  # ragged: the last 7 entries of request 1 are not in use
    store, slots = kv, None
    if use_slots:
        store, slots = _compact_pool(kv, ids, k)
    out = lsa.lsa_gather_attend(to_dev_bf16(q), to_dev_bf16(store), to_dev(ids), to_dev(ctx), 1 / math.sqrt(d),
                                slots=None if slots is None else to_dev(slots), n_split=n_split,
                                counts=None if counts is None else to_dev(counts))
    ref = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / math.sqrt(d), counts=counts)
    say("  ", check_attention(out.cpu().numpy(), ref, "long chunk list"))


@pytest.mark.parametrize("k,seg_len", [(480, 3840), (480, 3801), (10, 64 * 600 - 5)])
def test_attend_long_list_with_segment(lsa, oracle_lib, synth_lib, k, seg_len):
    """Chunks plus resident-segment blocks beyond 512 entries in one
    workgroup: the staging round boundary falls among the segment's blocks."""
    B, Hq, Hkv, d = 2, 8, 1, 128
    C = k + 20
    say("long list with segment", k, seg_len)
    q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=seg_len)
    ids = _ids(synth_lib, B, C, k, seed=k + 1)
    ctx = np.full(B, C * 64, dtype=np.int32)
    S_max = (seg_len + 63) // 64 * 64 + 64
    seg = synth_lib.normal_bf16((B, 2, Hkv, S_max, d), 7, synth_lib.stream(synth_lib.TAG_MISC, 7300))
    sl = np.array([seg_len, 100], dtype=np.int32)
    out = lsa.lsa_gather_attend(to_dev_bf16(q), to_dev_bf16(kv), to_dev(ids), to_dev(ctx), 1 / math.sqrt(d),
                                n_split=1, seg_kv=to_dev_bf16(seg), seg_len=to_dev(sl))
    ref = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / math.sqrt(d), seg_kv=seg, seg_len=sl)
    say("  ", check_attention(out.cpu().numpy(), ref, "long list with segment"))


# ------------------------------------------ token lists over > 1024 chunks

def _random_token_list(rng, k, k_tok, B):
    """Unsorted positions with invalid entries: -1, a position of an entry
    not in use, and a repeated position."""
    tok = np.stack([rng.permutation(k * 64)[:k_tok] for _ in range(B)]).astype(np.int32)
    tok[:, 1] = -1
    tok[:, 2] = k * 64 + 3
    tok[:, 4] = tok[:, 3]
    return tok


@pytest.mark.parametrize("k,n_split,use_slots,ordered", [
    (1638, 1, False, True), (1638, 3, True, True), (1638, 3, False, False), (1100, 1, True, False),
    (1025, 2, False, True),
])
def test_attend_tokens_long_recall(lsa, oracle_lib, synth_lib, k, n_split, use_slots, ordered):
    """The 1M workload's recall size (1638 chunks) and others past 1024: the
    kernel reads chunk ids and store positions from global memory."""
    B, Hq, Hkv, d, k_tok = 2, 16, 2, 128, 2048
    C = k + 40
    say("token list over a long recall", k, n_split, use_slots, ordered)
    q, kv = _problem(synth_lib, B, Hq, Hkv, d, C, seed=k + 11, qscale=4.0)
    ids = _ids(synth_lib, B, C, k, seed=k + 12)
    ctx = np.full(B, C * 64, dtype=np.int32)
    ctx[1] = int(ids[1, k - 3]) * 64 + 9  # the last chunks of request 1 lie past its context
    counts = np.array([k, k - 5], dtype=np.int32)
    if ordered:  # as the token select writes it: the best k_tok by a score, ascending
        s = synth_lib.bf16_bits_to_f32(synth_lib.normal_bf16((B, k * 64), k, synth_lib.stream(synth_lib.TAG_MISC, 7400)))
        tok, tc = oracle_lib.topk_tokens(s, ids, ctx, k_tok, counts=counts)
    else:
        tok = _random_token_list(np.random.default_rng(k), k, k_tok, B)
        tc = np.array([k_tok, k_tok - 100], dtype=np.int32)
    store, slots = kv, None
    if use_slots:
        store, slots = _compact_pool(kv, ids, k)
    out = lsa.lsa_gather_attend_tokens(to_dev_bf16(q), to_dev_bf16(store), to_dev(ids), to_dev(ctx), to_dev(tok),
                                       to_dev(tc), sm_scale=1 / math.sqrt(d), n_split=n_split, counts=to_dev(counts),
                                       slots=None if slots is None else to_dev(slots))
    ref = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / math.sqrt(d), counts=counts, tok=tok, tok_counts=tc)
    say("  ", check_attention(out.cpu().numpy(), ref, "token list over a long recall"))


@pytest.mark.slow
def test_token_stage_1m_bench_call(oracle_lib):
    """`bench.py --workload 1m_host --token-topk 2048` at full size: the whole
    1M-token K/V of batch 4 in HBM, the top 1638 of 16,384 chunks re-selected,
    then the top 2048 of their 104,832 tokens by a per-step score, attended
    over in the launch configuration the benchmark times.  Every request's
    selections and outputs are checked."""
    import torch

    import synth
    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    w = W.WORKLOADS["1m_host"]
    k_tok, steps = 2048, (0, 1)
    dev = torch.device("cuda")
    say(f"1M token stage: B={w.B} C={w.C} k={w.k} k_tok={k_tok}, K/V in HBM")
    K = W.indexer_keys(w)
    dec = LsaDecoder(k_idx=to_dev(K), ctx_len=to_dev(W.ctx_lens(w)), Hq=w.Hq, k=w.k, alpha=w.alpha,
                     kv=W.device_kv_store(w, dev), token_topk=k_tok)
    say("  inputs placed")
    scores = {t: synth.bf16_bits_to_f32(synth.normal_bf16((w.B, w.k * 64), 8, synth.stream(synth.TAG_MISC, 7500 + t)))
              for t in steps}
    dec.reselect(to_dev(W.indexer_query(w, 0)), 0)
    outs, toks = {}, {}
    for t in steps:
        o = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
        dec.attend(to_dev_bf16(W.attn_query(w, t)), 0, o, token_scores=to_dev(scores[t]))
        toks[t] = (dec.tok.cpu().numpy().copy(), dec.tok_counts.cpu().numpy().copy())
        outs[t] = o.cpu().numpy()
    ids = dec.sel_ids[0].cpu().numpy()
    say("  GPU run done")
    _, _, ref_ids = oracle_lib.select(W.indexer_query(w, 0), K, w.k, w.alpha)
    assert np.array_equal(ids, ref_ids)
    ctx = W.ctx_lens(w)
    for t in steps:
        ref_tok, ref_tc = oracle_lib.topk_tokens(scores[t], ids, ctx, k_tok)
        assert np.array_equal(toks[t][0], ref_tok) and np.array_equal(toks[t][1], ref_tc), t
        for b in range(w.B):
            chunks = W.kv_chunks(w, b, ids[b])[None]
            ref = oracle_lib.gather_attend(W.attn_query(w, t)[b:b + 1], chunks, ids[b:b + 1], ctx[b:b + 1], w.Hkv,
                                           w.sm_scale, slots=np.arange(w.k, dtype=np.int32)[None],
                                           tok=ref_tok[b:b + 1], tok_counts=ref_tc[b:b + 1])
            st = check_attention(outs[t][b], ref[0], f"1M token stage step {t} request {b}",
                                 max_rel_rms=ATT_MAX_REL_RMS_FULL)
            say(f"  step {t} request {b}: max err / RMS {st['max_rel_rms']:.2e}")


# ------------------------------------------------------- ring depths 3 and 4

def _depth_cases(synth_lib):
    """(name, inputs, call kwargs, oracle kwargs) covering chunk mode with
    splits, d = 64, a long list, a segment, and token mode."""
    cases = []
    q, kv = _problem(synth_lib, 3, 64, 8, 128, 60, seed=1)
    ids = _ids(synth_lib, 3, 60, 33, seed=2)
    ctx = np.array([60 * 64, int(ids[1, 20]) * 64 + 5, 60 * 64], dtype=np.int32)
    cases.append(("chunks d128 split 3", (q, kv, ids, ctx, 8), dict(n_split=3), {}))
    q2, kv2 = _problem(synth_lib, 2, 12, 4, 64, 40, seed=3)
    ids2 = _ids(synth_lib, 2, 40, 17, seed=4)
    cases.append(("chunks d64 group 3", (q2, kv2, ids2, np.full(2, 40 * 64, np.int32), 4), dict(n_split=2), {}))
    q3, kv3 = _problem(synth_lib, 1, 8, 1, 128, 620, seed=5)
    ids3 = _ids(synth_lib, 1, 620, 601, seed=6)
    cases.append(("long list", (q3, kv3, ids3, np.full(1, 620 * 64, np.int32), 1), dict(n_split=1), {}))
    seg = synth_lib.normal_bf16((3, 2, 8, 256, 128), 9, synth_lib.stream(synth_lib.TAG_MISC, 7600))
    sl = np.array([256, 70, 1], dtype=np.int32)
    cases.append(("chunks + segment", (q, kv, ids, ctx, 8), dict(n_split=2, seg=(seg, sl)),
                  dict(seg_kv=seg, seg_len=sl)))
    tok = _random_token_list(np.random.default_rng(5), 33, 700, 3)
    tc = np.array([700, 650, 1], dtype=np.int32)
    cases.append(("token list", (q, kv, ids, ctx, 8), dict(n_split=3, tok=(tok, tc)), dict(tok=tok, tok_counts=tc)))
    return cases


def _run_case(lsa, inputs, kw):
    q, kv, ids, ctx, _ = inputs
    kw = dict(kw)
    extra = {}
    if "seg" in kw:
        seg, sl = kw.pop("seg")
        extra.update(seg_kv=to_dev_bf16(seg), seg_len=to_dev(sl))
    if "tok" in kw:
        tok, tc = kw.pop("tok")
        extra.update(tok=to_dev(tok), tok_counts=to_dev(tc))
    d = q.shape[2]
    return lsa.lsa_gather_attend(to_dev_bf16(q), to_dev_bf16(kv), to_dev(ids), to_dev(ctx), 1 / math.sqrt(d),
                                 **kw, **extra).cpu().numpy()


def test_attend_ring_depths_same_bits(lsa, oracle_lib, synth_lib, tune):
    """Depths 3 and 4 only change how many tiles are in flight, not the order
    of any arithmetic: outputs equal depth 2's bit for bit, and the oracle."""
    cases = _depth_cases(synth_lib)
    base = {name: _run_case(lsa, inputs, kw) for name, inputs, kw, _ in cases}
    for depth in (3, 4):
        tune(attend_depth=depth)
        assert lsa.lsa_get_tuning("attend_depth") == depth
        for name, inputs, kw, okw in cases:
            say(f"depth {depth}: {name}")
            got = _run_case(lsa, inputs, kw)
            q, kv, ids, ctx, Hkv = inputs
            ref = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, 1 / math.sqrt(q.shape[2]), **okw)
            check_attention(got, ref, f"depth {depth} {name}")
            assert np.array_equal(got.view(np.uint32), base[name].view(np.uint32)), f"depth {depth} {name}"


_CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import numpy as np
import synth
import lookahead_chunk_sparse_amd as lsa
import test_gpu_attend_paths as T
print("child: depth", lsa.lsa_get_tuning("attend_depth"), flush=True)
outs = {{name: T._run_case(lsa, inputs, kw) for name, inputs, kw, _ in T._depth_cases(synth)}}
np.savez({out!r}, depth=lsa.lsa_get_tuning("attend_depth"), **{{n.replace(" ", "_"): o for n, o in outs.items()}})
print("child: done", flush=True)
"""


@pytest.mark.parametrize("depth", [3, 4])
def test_attend_depth_from_environment(lsa, synth_lib, tmp_path, depth):
    """LSA_ATTEND_DEPTH set in the environment of a fresh process (read once
    there, before its first call) gives depth 2's bits too."""
    import synth
    out = tmp_path / f"depth{depth}.npz"
    code = _CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), out=str(out))
    env = dict(os.environ, LSA_ATTEND_DEPTH=str(depth))
    say(f"fresh process with LSA_ATTEND_DEPTH={depth}")
    r = subprocess.run([sys.executable, "-u", "-c", code], env=env, capture_output=True, text=True, timeout=240)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-3000:]
    got = np.load(out)
    assert int(got["depth"]) == depth
    for name, inputs, kw, _ in _depth_cases(synth):
        base = _run_case(lsa, inputs, kw)
        assert np.array_equal(got[name.replace(" ", "_")].view(np.uint32), base.view(np.uint32)), name
