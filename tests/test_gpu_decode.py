"""Whole-path parity: the decode schedule (re-selection every tau = 64 steps,
lag 0 for an HBM-resident store, lag 1 for the host tier) run through the
library at every workload's full size, in the launch configuration the
benchmark times (default split count), checked against the oracle on
sampled steps and requests.  The oracle regenerates just the chunks it needs
from the seeded generator."""
import numpy as np
import pytest

from conftest import gpu_available
from helpers import ATT_MAX_REL_RMS_FULL, check_attention, to_dev, to_dev_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SAMPLED = {
    "tiny": (list(range(64)), [0]),
    "32k": ([0, 1, 63, 64, 128, 192, 255], [0, 1, 2, 3]),
    "128k": ([0, 1, 63, 64, 128, 192, 255], [0, 5, 15]),
    "500k": ([0, 64, 127], [0, 7]),
    "1m_host": ([0, 63, 64, 127], [0, 3]),
}
# one sampled step per workload at which every request of the batch is
# compared, not only the sampled ones
EVERY_REQUEST = {"128k": 64, "500k": 127, "1m_host": 64, "128k_host": 192}


def say(*a):
    print(*a, flush=True)


def oracle_selections(oracle, W, w):
    """Per re-selection interval: the oracle's chunk ids int32 [B][k]."""
    K = W.indexer_keys(w)
    sels = []
    for i in range(w.intervals):
        _, _, ids = oracle.select(W.indexer_query(w, i), K, w.k, w.alpha)
        sels.append(ids)
    return sels


def oracle_output(oracle, W, w, t, b, ids_b):
    """fp64 [Hq][d]: attention of request b at step t over chunks ids_b."""
    chunks = W.kv_chunks(w, b, ids_b)[None]  # [1][k][2][Hkv][T][d]
    q = W.attn_query(w, t)[b:b + 1]
    slots = np.arange(len(ids_b), dtype=np.int32)[None]
    ctx = W.ctx_lens(w)[b:b + 1]
    return oracle.gather_attend(q, chunks, ids_b[None].astype(np.int32), ctx, w.Hkv, w.sm_scale, slots=slots)[0]


@pytest.mark.parametrize("name,fetch,delta", [("tiny", None, None), ("32k", None, None), ("128k", None, None),
                                              ("500k", None, None), ("1m_host", "pull", True),
                                              ("1m_host", "pull", False), ("1m_host", "memcpy", False),
                                              ("1m_host", "memcpy", True), ("128k_host", "pull", True),
                                              ("128k_host", "memcpy", True), ("32k_churn", "pull", True),
                                              ("32k_churn", "memcpy", True), ("32k_churn", "staged", True),
                                              ("1m_host", "staged", True), ("128k_host", "staged", False)])
def test_decode_workload(oracle_lib, name, fetch, delta):
    import torch

    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    if name == "128k_host":  # the drifting 128K workload on the host tier: selections change every interval
        w = W.WORKLOADS["128k"].replace(host_tier=True)
        steps, reqs = [0, 63, 64, 128, 191, 192, 255], [0, 9]
    elif name == "32k_churn":  # the ring indexer: a quarter of the chunks are new every interval
        w = W.WORKLOADS["32k"].replace(host_tier=True, churn=0.25)
        steps, reqs = [0, 64, 128, 192, 255], [0, 1, 2, 3]
    else:
        w = W.WORKLOADS[name]
        steps, reqs = SAMPLED[name]
    say(f"decode {name}: B={w.B} C={w.C} k={w.k} steps={w.steps} host_tier={w.host_tier}")
    dev = torch.device("cuda")
    K = to_dev(W.indexer_keys(w))
    ctx = to_dev(W.ctx_lens(w))
    if w.host_tier:
        dec = LsaDecoder(k_idx=K, ctx_len=ctx, Hq=w.Hq, k=w.k, alpha=w.alpha, host_kv=W.pinned_kv_store(w),
                         fetch=fetch, delta=delta)
    else:
        dec = LsaDecoder(k_idx=K, ctx_len=ctx, Hq=w.Hq, k=w.k, alpha=w.alpha, kv=W.device_kv_store(w, dev))
    say("  inputs placed")
    keep = {t: torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev) for t in steps}
    scratch = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    gpu_sel = {}
    for i in range(w.intervals):
        ts = range(i * w.tau, min((i + 1) * w.tau, w.steps))
        qs = [to_dev_bf16(W.attn_query(w, t)) for t in ts]
        dec.run_interval(i, to_dev(W.indexer_query(w, i)), qs, [keep.get(t, scratch) for t in ts])
        gpu_sel[i] = dec.sel_ids[i % 2].clone()
    dec.join()
    torch.cuda.synchronize()
    say("  GPU run done")

    sels = oracle_selections(oracle_lib, W, w)
    for i in range(w.intervals):
        assert np.array_equal(gpu_sel[i].cpu().numpy(), sels[i]), f"selection {i} differs"
    worst = 0.0
    for t in steps:
        src = oracle_lib.selection_for_step(t, w.tau, w.lag)
        out = keep[t].cpu().numpy()
        for b in (range(w.B) if EVERY_REQUEST.get(name) == t else reqs):
            ref = oracle_output(oracle_lib, W, w, t, b, sels[src][b])
            st = check_attention(out[b], ref, f"{name} step {t} request {b}",
                                 max_rel_rms=ATT_MAX_REL_RMS_FULL)
            worst = max(worst, st["max_rel_rms"])
    say(f"  parity ok; worst max-abs error / output RMS = {worst:.3e}")

    if w.host_tier:
        # the pool holds, byte for byte, the chunks of the last fetched selection at their slots
        last = w.intervals - 1
        pool = dec.pool[last % 2].cpu().view(torch.int16).numpy().view(np.uint16)
        slots = dec.sel_slots[last % 2].cpu().numpy() if dec.delta else np.tile(np.arange(w.k), (w.B, 1))
        for b in reqs:
            assert np.array_equal(pool[b][slots[b]], W.kv_chunks(w, b, sels[last][b])), f"pool of request {b}"


def test_decode_threshold_selection(oracle_lib):
    """The pages' gating rule end to end: sigma > 0.5 (logit > 0) with the pool
    size as cap.  A calibrated indexer is synthesised: background keys lean
    against the query (negative logits), each request plants its own number
    of relevant chunks, so the budget differs per request and per interval."""
    import torch

    import synth
    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    w = W.WORKLOADS["32k"].replace(B=4, k=64)
    dev = torch.device("cuda")
    s = synth.stream
    sets = {}
    q0 = W.indexer_query(w, 0)
    q_idx = [q0, q0]  # same query; the second interval adds a second relevant set
    noise = synth.uniform_i8((w.B, w.C, w.d_idx), 3, s(synth.TAG_MISC, 3001), -4, 4).astype(np.int32)
    K = (-np.sign(q_idx[0].astype(np.int32)) + noise).astype(np.int8)  # background: logit about -sum|q|
    for it, q in enumerate(q_idx):
        for b in range(w.B):
            n_rel = [5, 20, 90, 0][(b + it) % 4]  # 90 > k: the cap applies (sets may overlap)
            pos = synth.choose(n_rel, w.C, 3, s(synth.TAG_MISC, 3100 + 10 * it + b))
            sets[(it, b)] = pos
            K[b, pos] = (8 * np.sign(q[b, 0].astype(np.int32)) + noise[b, pos]).astype(np.int8)
    kv = W.device_kv_store(w, dev)
    ctx = to_dev(W.ctx_lens(w))
    dec = LsaDecoder(k_idx=to_dev(K), ctx_len=ctx, Hq=w.Hq, k=w.k, alpha=w.alpha, kv=kv, selection="threshold")
    outs = {}
    for it in range(2):
        qs = [to_dev_bf16(W.attn_query(w, 64 * it + t)) for t in range(3)]
        o = [torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev) for _ in range(3)]
        dec.run_interval(it, to_dev(q_idx[it]), qs, o)
        torch.cuda.synchronize()
        L = oracle_lib.index_logits(q_idx[it], K)
        ref_ids, ref_counts = oracle_lib.threshold_chunks(L, w.k, 0)
        got_counts = dec.sel_counts[it % 2].cpu().numpy()
        assert np.array_equal(got_counts, ref_counts), (it, got_counts, ref_counts)
        assert np.array_equal(dec.sel_ids[it % 2].cpu().numpy(), ref_ids)
        assert len(set(ref_counts.tolist())) >= 3  # the budget really varies
        for b in range(w.B):
            if ref_counts[b] == 0:
                assert (o[0][b].cpu().numpy() == 0).all()
                continue
            idsb = ref_ids[b, :ref_counts[b]]
            for t in range(3):
                chunks = W.kv_chunks(w, b, idsb)[None]
                ref = oracle_lib.gather_attend(W.attn_query(w, 64 * it + t)[b:b + 1], chunks, idsb[None],
                                               W.ctx_lens(w)[b:b + 1], w.Hkv, w.sm_scale,
                                               slots=np.arange(len(idsb), dtype=np.int32)[None])
                check_attention(o[t][b].cpu().numpy(), ref[0], f"threshold interval {it} request {b} step {t}")


def test_decode_with_local_window_and_decoded_tokens(oracle_lib):
    """Recalled history chunks + the resident local window, which grows by one
    freshly decoded token per step (the caller writes the token's K/V and
    bumps seg_len between steps); history chunks overlapping the window are
    excluded from the indexer's scan by construction (ctx_len = history)."""
    import torch

    import synth
    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    w = W.WORKLOADS["32k"]
    W_len, S_max, steps = 1024, 1024 + 128, 6
    hist = w.N - W_len                       # tokens of the offloadable history
    C_hist = hist // 64
    dev = torch.device("cuda")
    K = W.indexer_keys(w)[:, :C_hist].copy()  # only history chunks are scored
    kv = W.device_kv_store(w, dev)
    seg = synth.normal_bf16((w.B, 2, w.Hkv, S_max, w.d), 5, synth.stream(synth.TAG_MISC, 3200))
    seg_d = to_dev_bf16(seg)
    seg_len = torch.full((w.B,), W_len, dtype=torch.int32, device=dev)
    ctx = torch.full((w.B,), hist, dtype=torch.int32, device=dev)
    dec = LsaDecoder(k_idx=to_dev(K), ctx_len=ctx, Hq=w.Hq, k=w.k, alpha=w.alpha, kv=kv[:, :C_hist].contiguous(),
                     seg_kv=seg_d, seg_len=seg_len)
    q_idx = W.indexer_query(w, 0)
    _, _, ids_ref = oracle_lib.select(q_idx, K, w.k, w.alpha)
    kv_host = None
    for t in range(steps):
        q = W.attn_query(w, t)
        out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
        if t == 0:
            dec.reselect(to_dev(q_idx), 0)
        dec.attend(to_dev_bf16(q), 0, out)
        torch.cuda.synchronize()
        assert np.array_equal(dec.sel_ids[0].cpu().numpy(), ids_ref)
        n_seg = W_len + t
        for b in (0, w.B - 1):
            chunks = W.kv_chunks(w, b, ids_ref[b])[None]
            ref = oracle_lib.gather_attend(q[b:b + 1], chunks, ids_ref[b:b + 1], np.array([hist]), w.Hkv,
                                           w.sm_scale, slots=np.arange(w.k, dtype=np.int32)[None],
                                           seg_kv=seg[b:b + 1], seg_len=np.array([n_seg], dtype=np.int32))
            check_attention(out[b].cpu().numpy(), ref[0], f"window step {t} request {b}")
        seg_len += 1  # the token just decoded joins the window


def test_decode_layers_share_one_selection(oracle_lib):
    """Three layers, one indexer scan per interval: every layer attends over
    the chunks that scan selected, with its own K/V and its own query."""
    import torch

    import synth
    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    w = W.WORKLOADS["32k"]
    L, n_steps = 3, 70  # crosses one re-selection
    dev = torch.device("cuda")
    K = W.indexer_keys(w)
    layer_w = [w.replace(seed=w.seed + 1000 * l) for l in range(L)]
    stores = [W.device_kv_store(lw, dev) for lw in layer_w]
    dec = LsaDecoder(k_idx=to_dev(K), ctx_len=to_dev(W.ctx_lens(w)), Hq=w.Hq, k=w.k, alpha=w.alpha, kv=stores)
    check_t = (0, 63, 64, 69)
    qh = {(t, l): synth.normal_bf16((w.B, w.Hq, w.d), 5, synth.stream(synth.TAG_MISC, 3300 + 10 * t + l))
          for t in check_t for l in range(L)}
    keep = {key: torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev) for key in qh}
    scratch = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    filler = to_dev_bf16(W.attn_query(w, 1))
    sels = []
    for i in range(2):
        ts = range(i * w.tau, min((i + 1) * w.tau, n_steps))
        qs = [[to_dev_bf16(qh[(t, l)]) if (t, l) in qh else filler for l in range(L)] for t in ts]
        outs = [[keep.get((t, l), scratch) for l in range(L)] for t in ts]
        dec.run_interval(i, to_dev(W.indexer_query(w, i)), qs, outs)
        torch.cuda.synchronize()
        sels.append(dec.sel_ids[i % 2].cpu().numpy().copy())
    for i in range(2):
        _, _, ref_ids = oracle_lib.select(W.indexer_query(w, i), K, w.k, w.alpha)
        assert np.array_equal(sels[i], ref_ids), f"selection {i}"
    ctx = W.ctx_lens(w)
    for (t, l), o in keep.items():
        ids = sels[t // w.tau]
        for b in (0, w.B - 1):
            chunks = W.kv_chunks(layer_w[l], b, ids[b])[None]
            ref = oracle_lib.gather_attend(qh[(t, l)][b:b + 1], chunks, ids[b:b + 1], ctx[b:b + 1], w.Hkv,
                                           w.sm_scale, slots=np.arange(w.k, dtype=np.int32)[None])
            check_attention(o[b].cpu().numpy(), ref[0], f"layer {l} step {t} request {b}")


def test_decode_token_stage_128k(oracle_lib):
    """The two-stage selection at the 128K workload's full size: chunks by the
    memory indexer every 64 steps, then at every step the 2048 best tokens
    of the recalled chunks by a per-step token score, attended over in the
    benchmark's launch configuration."""
    import torch

    import synth
    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    w = W.WORKLOADS["128k"]
    k_tok, steps, reqs = 2048, (0, 1, 64, 65), [0, 9]
    dev = torch.device("cuda")
    say(f"token stage 128k: B={w.B} k={w.k} k_tok={k_tok}")
    K = W.indexer_keys(w)
    dec = LsaDecoder(k_idx=to_dev(K), ctx_len=to_dev(W.ctx_lens(w)), Hq=w.Hq, k=w.k, alpha=w.alpha,
                     kv=W.device_kv_store(w, dev), token_topk=k_tok)
    scores = {t: synth.bf16_bits_to_f32(synth.normal_bf16((w.B, w.k * 64), 5, synth.stream(synth.TAG_MISC, 4100 + t)))
              for t in steps}
    outs, toks, sels = {}, {}, {}
    for i in range(2):
        ts = [t for t in steps if t // w.tau == i]
        o = [torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev) for _ in ts]
        qs = [to_dev_bf16(W.attn_query(w, t)) for t in ts]
        dec.reselect(to_dev(W.indexer_query(w, i)), i)
        for t, q, oo in zip(ts, qs, o):
            dec.attend(q, i, oo, token_scores=to_dev(np.ascontiguousarray(scores[t], dtype=np.float32)))
            toks[t] = (dec.tok.cpu().numpy().copy(), dec.tok_counts.cpu().numpy().copy())
            outs[t] = oo
        torch.cuda.synchronize()
        sels[i] = dec.sel_ids[i % 2].cpu().numpy().copy()
    say("  GPU run done")
    ctx = W.ctx_lens(w)
    for t in steps:
        ids = sels[t // w.tau]
        _, _, ref_ids = oracle_lib.select(W.indexer_query(w, t // w.tau), K, w.k, w.alpha)
        assert np.array_equal(ids, ref_ids)
        ref_tok, ref_tc = oracle_lib.topk_tokens(scores[t][reqs], ids[reqs], ctx[reqs], k_tok)
        assert np.array_equal(toks[t][0][reqs], ref_tok) and np.array_equal(toks[t][1][reqs], ref_tc), t
        out = outs[t].cpu().numpy()
        for n, b in enumerate(reqs):
            chunks = W.kv_chunks(w, b, ids[b])[None]
            ref = oracle_lib.gather_attend(W.attn_query(w, t)[b:b + 1], chunks, ids[b:b + 1], ctx[b:b + 1], w.Hkv,
                                           w.sm_scale, slots=np.arange(w.k, dtype=np.int32)[None],
                                           tok=ref_tok[n:n + 1], tok_counts=ref_tc[n:n + 1])
            check_attention(out[b], ref[0], f"token stage step {t} request {b}", max_rel_rms=ATT_MAX_REL_RMS_FULL)


def test_decode_token_stage_on_host_tier(oracle_lib):
    """Token stage over the host tier's HBM pool: the listed positions name
    entries of the selection in use (lag 1), whose K/V sit at the delta
    fetch's pool slots; the third interval attends a delta-fetched selection."""
    import torch

    import synth
    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    w = W.WORKLOADS["32k"].replace(host_tier=True)
    k_tok = 500
    dev = torch.device("cuda")
    K = W.indexer_keys(w)
    dec = LsaDecoder(k_idx=to_dev(K), ctx_len=to_dev(W.ctx_lens(w)), Hq=w.Hq, k=w.k, alpha=w.alpha,
                     host_kv=W.pinned_kv_store(w), token_topk=k_tok)
    plan = {0: [0, 1], 1: [64], 2: [128, 129]}  # interval -> steps
    outs, toks = {}, {}
    for i, ts in plan.items():
        src = max(i - 1, 0)  # lag 1
        for n, t in enumerate(ts):
            q = to_dev_bf16(W.attn_query(w, t))
            sc = synth.bf16_bits_to_f32(synth.normal_bf16((w.B, w.k * 64), 6, synth.stream(synth.TAG_MISC, 4200 + t)))
            o = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
            if n == 0:  # the interval's re-selection, fetch and first step
                dec.run_interval(i, to_dev(W.indexer_query(w, i)), [q], [o], token_scores=[to_dev(sc)])
            else:       # a further step of the same interval
                dec.attend(q, src, o, token_scores=to_dev(sc))
            torch.cuda.synchronize()
            toks[t] = (src, sc, dec.tok.cpu().numpy().copy(), dec.tok_counts.cpu().numpy().copy())
            outs[t] = o
    dec.join()
    torch.cuda.synchronize()
    ctx = W.ctx_lens(w)
    for t, (src, scores, tok, tc) in toks.items():
        _, _, ids = oracle_lib.select(W.indexer_query(w, src), K, w.k, w.alpha)
        ref_tok, ref_tc = oracle_lib.topk_tokens(scores, ids, ctx, k_tok)
        assert np.array_equal(tok, ref_tok) and np.array_equal(tc, ref_tc), t
        out = outs[t].cpu().numpy()
        for b in range(w.B):
            chunks = W.kv_chunks(w, b, ids[b])[None]
            ref = oracle_lib.gather_attend(W.attn_query(w, t)[b:b + 1], chunks, ids[b:b + 1], ctx[b:b + 1], w.Hkv,
                                           w.sm_scale, slots=np.arange(w.k, dtype=np.int32)[None],
                                           tok=ref_tok[b:b + 1], tok_counts=ref_tc[b:b + 1])
            check_attention(out[b], ref[0], f"host-tier token stage step {t} request {b}")


def test_decode_128k_sharpened(oracle_lib):
    """A sharpened query (q x 8) at the 128K workload's full size: the softmax
    over 17,664 tokens concentrates on a few of them, so the output is far
    from the near-uniform average of the N(0,1) case and an error in any
    single token's weight or V row shows up in the comparison."""
    import torch

    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    w = W.WORKLOADS["128k"]
    reqs = [0, 7, 15]
    dev = torch.device("cuda")
    say(f"sharpened 128k: B={w.B} k={w.k}, q x 8")
    K = W.indexer_keys(w)
    dec = LsaDecoder(k_idx=to_dev(K), ctx_len=to_dev(W.ctx_lens(w)), Hq=w.Hq, k=w.k, alpha=w.alpha,
                     kv=W.device_kv_store(w, dev))
    dec.reselect(to_dev(W.indexer_query(w, 0)), 0)
    q = W.attn_query(w, 5, scale=8.0)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    dec.attend(to_dev_bf16(q), 0, out)
    ids = dec.sel_ids[0].cpu().numpy()
    out = out.cpu().numpy()
    _, _, ref_ids = oracle_lib.select(W.indexer_query(w, 0), K, w.k, w.alpha)
    assert np.array_equal(ids, ref_ids)
    ctx = W.ctx_lens(w)
    for b in reqs:
        chunks = W.kv_chunks(w, b, ids[b])[None]
        ref, wts = oracle_lib.gather_attend(q[b:b + 1], chunks, ids[b:b + 1], ctx[b:b + 1], w.Hkv, w.sm_scale,
                                            slots=np.arange(w.k, dtype=np.int32)[None], want_weights=True)
        # the weights are concentrated: the largest weight of every head is
        # hundreds of times the uniform 1/17,664, and the output RMS is O(1)
        assert wts.max(axis=-1).min() > 300.0 / (w.k * 64)
        st = check_attention(out[b], ref[0], f"sharpened request {b}", max_rel_rms=ATT_MAX_REL_RMS_FULL)
        assert st["ref_rms"] > 0.1
        say(f"  request {b}: {st}")
