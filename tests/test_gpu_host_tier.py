"""The host tier with the pages' own selection rule and with layers sharing a
selection, through the decode schedule (lag 1: interval i attends the
selection made at interval i-1 while interval i's chunks are fetched):

  * sigmoid gating, sigma > 0.5 (logit > 0) capped at the pool's k slots, so
    each request keeps its own number of chunks per interval (paperlayer.ai
    summary of FlashMemory-DeepSeek-V4, 2.1 Architecture: threshold
    selection; non-recalled entries are evicted to CPU memory), through the
    delta fetch (pool slots assigned on the GPU from -1-padded lists; pull and
    DMA copies) and the two-buffer pull fetch, at the 32K shape and at the
    full 1M size;
  * several layers sharing one selection, each with its own host store and
    HBM pool (the lightning-indexer listing's cross-layer index reuse).

Selections and counts are compared bit for bit with the oracle, the pool
bytes at their slots with the host store, and attention with the fp64 oracle
over exactly the chunks each request kept."""
import numpy as np
import pytest

from conftest import gpu_available
from helpers import ATT_MAX_REL_RMS_FULL, check_attention, to_dev, to_dev_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True)


def calibrated_indexer(synth, w, n_intervals, n_rel, seed):
    """Indexer queries and keys for threshold selection.  Every interval's
    query shares its first half with the others (q_common) and draws its
    second half afresh.  Background keys lean against q_common (logit about
    -2 sum|q_common|, far below 0); the chunks relevant to interval i also
    match that interval's second half (logit about +3000).  n_rel(i, b)
    chunks are planted per interval and request, so the kept count varies,
    and a chunk planted for one interval sometimes passes in another (the
    gating's leak).  Returns (q_idx per interval, int8 [B][1][d]; K)."""
    s = synth.stream
    h = w.d_idx // 2
    q_common = synth.uniform_i8((w.B, 1, h), seed, s(synth.TAG_MISC, 8000), -16, 15)
    qs = []
    for i in range(n_intervals):
        tail = synth.uniform_i8((w.B, 1, w.d_idx - h), seed, s(synth.TAG_MISC, 8001 + i), -16, 15)
        qs.append(np.concatenate([q_common, tail], axis=2))
    noise = synth.uniform_i8((w.B, w.C, w.d_idx), seed, s(synth.TAG_MISC, 8100), -1, 1).astype(np.int32)
    K = noise.copy()
    K[:, :, :h] += -2 * np.sign(q_common.astype(np.int32))
    for i in range(n_intervals):
        for b in range(w.B):
            n = n_rel(i, b)
            pos = synth.choose(n, w.C, seed, s(synth.TAG_MISC, 8200 + 16 * i + b))
            K[b, pos, h:] = 8 * np.sign(qs[i][b, 0, h:].astype(np.int32)) + noise[b, pos, h:]
    return qs, K.astype(np.int8)


def _run_threshold_host(oracle_lib, w, n_intervals, n_rel, steps_per_interval, check_reqs, delta, max_rel_rms,
                        fetch="pull"):
    import torch

    import synth
    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    dev = torch.device("cuda")
    qs, K = calibrated_indexer(synth, w, n_intervals, n_rel, seed=11)
    say(f"  host store: B={w.B} C={w.C} k={w.k}, delta={delta}, fetch={fetch}")
    dec = LsaDecoder(k_idx=to_dev(K), ctx_len=to_dev(W.ctx_lens(w)), Hq=w.Hq, k=w.k, alpha=w.alpha,
                     host_kv=W.pinned_kv_store(w), selection="threshold", fetch=fetch, delta=delta)
    outs, sels = {}, {}
    for i in range(n_intervals):
        ts = [i * w.tau + j for j in range(steps_per_interval)]
        o = [torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev) for _ in ts]
        dec.run_interval(i, to_dev(qs[i]), [to_dev_bf16(W.attn_query(w, t)) for t in ts], o)
        torch.cuda.synchronize()
        sels[i] = (dec.sel_ids[i % 2].cpu().numpy().copy(), dec.sel_counts[i % 2].cpu().numpy().copy())
        for t, oo in zip(ts, o):
            outs[t] = oo.cpu().numpy()
    dec.join()
    torch.cuda.synchronize()
    say("  GPU run done")
    ref = {}
    for i in range(n_intervals):
        ref[i] = oracle_lib.threshold_chunks(oracle_lib.index_logits(qs[i], K), w.k, 0)
        assert np.array_equal(sels[i][1], ref[i][1]), (i, sels[i][1], ref[i][1])
        assert np.array_equal(sels[i][0], ref[i][0]), i
    counts = np.stack([ref[i][1] for i in range(n_intervals)])
    say(f"  kept chunks per interval and request:\n{counts}")
    assert len(set(counts.ravel().tolist())) >= 4 and (counts == w.k).any() and (counts == 0).any()
    ctx = W.ctx_lens(w)
    for t, out in outs.items():
        src = oracle_lib.selection_for_step(t, w.tau, lag=1)
        ids, cnt = ref[src]
        for b in check_reqs:
            n = int(cnt[b])
            if n == 0:
                assert (out[b] == 0).all(), f"step {t} request {b}: no chunk kept, output must be 0"
                continue
            idsb = ids[b, :n]
            r = oracle_lib.gather_attend(W.attn_query(w, t)[b:b + 1], W.kv_chunks(w, b, idsb)[None], idsb[None],
                                         ctx[b:b + 1], w.Hkv, w.sm_scale, slots=np.arange(n, dtype=np.int32)[None])
            check_attention(out[b], r[0], f"threshold host tier step {t} request {b}", max_rel_rms=max_rel_rms)
    # the pool holds the last fetched selection's chunks at their slots
    last = n_intervals - 1
    pool = dec.pool[last % 2].cpu().view(torch.int16).numpy().view(np.uint16)
    slots = dec.sel_slots[last % 2].cpu().numpy() if dec.delta else np.tile(np.arange(w.k), (w.B, 1))
    ids, cnt = ref[last]
    for b in check_reqs:
        n = int(cnt[b])
        if dec.delta:
            assert (slots[b, n:] == -1).all()
        assert np.array_equal(pool[b][slots[b, :n]], W.kv_chunks(w, b, ids[b, :n])), f"pool of request {b}"


@pytest.mark.parametrize("delta,fetch", [(True, "pull"), (False, "pull"), (True, "memcpy"), (True, "staged")])
def test_threshold_selection_host_tier_32k(oracle_lib, delta, fetch):
    """With fetch='memcpy' the DMA copies skip the -1 padding through its
    slot (-1) and spread over the library's copy streams; with 'staged' the
    host gathers only the entries with a slot."""
    from synth import workloads as W
    w = W.WORKLOADS["32k"].replace(B=4, k=64, host_tier=True)
    table = [[5, 20, 90, 0], [0, 40, 3, 90], [64, 1, 0, 30], [12, 0, 70, 64]]  # 90 > k: capped
    say(f"threshold host tier 32k, delta={delta}, fetch={fetch}")
    _run_threshold_host(oracle_lib, w, 4, lambda i, b: table[i][b], 2, range(w.B), delta, 1e-3, fetch=fetch)


@pytest.mark.slow
def test_threshold_selection_host_tier_1m(oracle_lib):
    """The full 1M host-tier size: 16,384 chunks per request, at most 1,638
    (10%) kept, the K/V of batch 4 in pinned host memory."""
    from synth import workloads as W
    w = W.WORKLOADS["1m_host"]
    table = [[300, 1200, 2500, 0], [1638, 0, 900, 2000], [50, 1700, 0, 1000]]
    say("threshold host tier 1M")
    _run_threshold_host(oracle_lib, w, 3, lambda i, b: table[i][b], 1, range(w.B), True, ATT_MAX_REL_RMS_FULL)


def test_layers_share_one_selection_on_host_tier(oracle_lib):
    """Two layers on the host tier: one scan and selection per interval, each
    layer's chunks fetched from its own host store into its own pool at the
    same slots, each layer attending with its own query."""
    import torch

    import synth
    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    w = W.WORKLOADS["32k"].replace(host_tier=True, drift=True, n_golden=26)
    L, n_int = 2, 3
    dev = torch.device("cuda")
    K = W.indexer_keys(w)
    layer_w = [w.replace(seed=w.seed + 1000 * l) for l in range(L)]
    dec = LsaDecoder(k_idx=to_dev(K), ctx_len=to_dev(W.ctx_lens(w)), Hq=w.Hq, k=w.k, alpha=w.alpha,
                     host_kv=[W.pinned_kv_store(lw) for lw in layer_w])
    assert len(dec.pools) == L and dec.delta
    qh, outs = {}, {}
    for i in range(n_int):
        ts = [i * w.tau, i * w.tau + 1]
        for t in ts:
            for l in range(L):
                qh[(t, l)] = synth.normal_bf16((w.B, w.Hq, w.d), 6, synth.stream(synth.TAG_MISC, 8300 + 10 * t + l))
        o = [[torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev) for _ in range(L)] for _ in ts]
        dec.run_interval(i, to_dev(W.indexer_query(w, i)), [[to_dev_bf16(qh[(t, l)]) for l in range(L)] for t in ts],
                         o)
        torch.cuda.synchronize()
        for t, ol in zip(ts, o):
            for l in range(L):
                outs[(t, l)] = ol[l].cpu().numpy()
    dec.join()
    torch.cuda.synchronize()
    sels = [oracle_lib.select(W.indexer_query(w, i), K, w.k, w.alpha)[2] for i in range(n_int)]
    ctx = W.ctx_lens(w)
    for (t, l), out in outs.items():
        ids = sels[oracle_lib.selection_for_step(t, w.tau, lag=1)]
        for b in range(w.B):
            r = oracle_lib.gather_attend(qh[(t, l)][b:b + 1], W.kv_chunks(layer_w[l], b, ids[b])[None], ids[b:b + 1],
                                         ctx[b:b + 1], w.Hkv, w.sm_scale, slots=np.arange(w.k, dtype=np.int32)[None])
            check_attention(out[b], r[0], f"layer {l} step {t} request {b}", max_rel_rms=ATT_MAX_REL_RMS_FULL)
    # each layer's pool holds that layer's chunks at the shared slots
    slots = dec.sel_slots[(n_int - 1) % 2].cpu().numpy()
    for l in range(L):
        pool = dec.pools[l][0].cpu().view(torch.int16).numpy().view(np.uint16)
        for b in range(w.B):
            assert np.array_equal(pool[b][slots[b]], W.kv_chunks(layer_w[l], b, sels[-1][b])), (l, b)


def test_threshold_host_tier_memcpy_needs_delta():
    """The DMA fetch skips the -1 padding of a variable-size selection through
    its slot; without the delta fetch's slots there is none, and asking for
    that combination says so."""
    import torch

    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    host = torch.empty((1, 4, 2, 1, 64, 64), dtype=torch.bfloat16, pin_memory=True)
    with pytest.raises(NotImplementedError, match="delta=True"):
        LsaDecoder(k_idx=torch.zeros((1, 4, 64), dtype=torch.int8, device="cuda"),
                   ctx_len=torch.full((1,), 256, dtype=torch.int32, device="cuda"), Hq=8, k=2, alpha=0.01,
                   host_kv=host, selection="threshold", fetch="memcpy", delta=False)


@pytest.mark.parametrize("B,C,k", [(3, 40, 9), (4, 2048, 276), (4, 16384, 1638)])
def test_pool_assign_padded_lists_parity(oracle_lib, synth_lib, B, C, k):
    """Pool slots for variable-size selections (-1 padding past each count,
    as the threshold select writes them), over a chain of selections, bit
    for bit against the oracle."""
    import lookahead_chunk_sparse_amd as lsa
    rng = np.random.default_rng(k)
    P = 2 * k
    prev = prev_d = None
    for step in range(6):
        counts = rng.integers(0, k + 1, B)
        counts[0] = k if step % 2 else 0
        ids = np.full((B, k), -1, dtype=np.int32)
        for b in range(B):
            ids[b, :counts[b]] = np.sort(rng.choice(C, counts[b], replace=False))
        ns_ref, fs_ref = oracle_lib.pool_assign(prev[0] if prev else None, prev[1] if prev else None, ids, P)
        ids_d = to_dev(ids)
        ns, fs = lsa.lsa_pool_assign(prev_d[0] if prev_d else None, prev_d[1] if prev_d else None, ids_d, P)
        assert np.array_equal(ns.cpu().numpy(), ns_ref) and np.array_equal(fs.cpu().numpy(), fs_ref), (step, counts)
        # entries not in use carry garbage slots in the next call: they must not be read
        garbage = np.where(ids >= 0, ns_ref, 7 * P + 3).astype(np.int32)
        prev, prev_d = (ids, garbage), (ids_d, to_dev(garbage))
