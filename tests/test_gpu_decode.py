"""Whole-path parity: the decode schedule (re-selection every tau = 64 steps,
lag 0 for an HBM-resident store, lag 1 for the host tier) run through the
library at every workload's full size, in the launch configuration the
benchmark times (default split count), checked against the oracle on
sampled steps and requests.  The oracle regenerates just the chunks it needs
from the seeded generator."""
import numpy as np
import pytest

from conftest import gpu_available
from helpers import check_attention, to_dev, to_dev_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SAMPLED = {
    "tiny": (list(range(64)), [0]),
    "32k": ([0, 1, 63, 64, 128, 192, 255], [0, 1, 2, 3]),
    "128k": ([0, 1, 63, 64, 128, 192, 255], [0, 5, 15]),
    "500k": ([0, 64, 127], [0, 7]),
    "1m_host": ([0, 63, 64, 127], [0, 3]),
}


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
                                              ("128k_host", "pull", True)])
def test_decode_workload(oracle_lib, name, fetch, delta):
    import torch

    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    if name == "128k_host":  # the drifting 128K workload on the host tier: selections change every interval
        w = W.WORKLOADS["128k"].replace(host_tier=True)
        steps, reqs = [0, 63, 64, 128, 191, 192, 255], [0, 9]
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
        for b in reqs:
            ref = oracle_output(oracle_lib, W, w, t, b, sels[src][b])
            st = check_attention(out[b], ref, f"{name} step {t} request {b}")
            worst = max(worst, st["max_rel_rms"])
    say(f"  parity ok; worst max-abs error / output RMS = {worst:.3e}")

    if w.host_tier:
        # the pool holds, byte for byte, the chunks of the last fetched selection at their slots
        last = w.intervals - 1
        pool = dec.pool[last % 2].cpu().view(torch.int16).numpy().view(np.uint16)
        slots = dec.sel_slots[last % 2].cpu().numpy() if dec.delta else np.tile(np.arange(w.k), (w.B, 1))
        for b in reqs:
            assert np.array_equal(pool[b][slots[b]], W.kv_chunks(w, b, sels[last][b])), f"pool of request {b}"
