"""The decode interval captured as a HIP graph (the way the benchmark times
it) gives, on every replay, the bits of the same work launched eagerly --
with other eager work and synchronisations between replays."""
import numpy as np
import pytest

from conftest import gpu_available
from helpers import to_dev, to_dev_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("n_split", [0, 3])
def test_graph_replays_match_eager(n_split):
    import torch

    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    w = W.WORKLOADS["32k"]
    dev = torch.device("cuda")
    K = to_dev(W.indexer_keys(w))
    ctx = to_dev(W.ctx_lens(w))
    kv = W.device_kv_store(w, dev)
    dec = LsaDecoder(k_idx=K, ctx_len=ctx, Hq=w.Hq, k=w.k, alpha=w.alpha, kv=kv, n_split=n_split)
    steps = 8
    qs = [to_dev_bf16(W.attn_query(w, t)) for t in range(steps)]
    qidx = to_dev(W.indexer_query(w, 0))
    outs = [torch.zeros((w.B, w.Hq, w.d), dtype=torch.float32, device=dev) for _ in range(steps)]

    dec.run_interval(0, qidx, qs, outs)  # eager
    torch.cuda.synchronize()
    eager = [o.cpu().numpy().copy() for o in outs]
    ids_eager = dec.sel_ids[0].cpu().numpy().copy()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dec.run_interval(0, qidx, qs, outs)
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        dec.sel_ids[0].fill_(-1)
        junk.mul_(1.0001)            # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(dec.sel_ids[0].cpu().numpy(), ids_eager), f"replay {rep}: selection"
        for t in range(steps):
            assert np.array_equal(outs[t].cpu().numpy(), eager[t]), f"replay {rep}, step {t}"
    # and eager again after the replays
    dec.run_interval(0, qidx, qs, outs)
    torch.cuda.synchronize()
    for t in range(steps):
        assert np.array_equal(outs[t].cpu().numpy(), eager[t])


def test_host_tier_graph_replays_match_eager():
    """Host tier with the device-side fetch: two intervals (fetch, lag 1,
    both pool buffers) captured in one graph replay to the eager bits."""
    import torch

    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    w = W.WORKLOADS["32k"].replace(host_tier=True)
    dev = torch.device("cuda")
    K = to_dev(W.indexer_keys(w))
    ctx = to_dev(W.ctx_lens(w))
    dec = LsaDecoder(k_idx=K, ctx_len=ctx, Hq=w.Hq, k=w.k, alpha=w.alpha, host_kv=W.pinned_kv_store(w))
    per = 4
    qs = [[to_dev_bf16(W.attn_query(w, 64 * i + t)) for t in range(per)] for i in range(3)]
    qidx = [to_dev(W.indexer_query(w, i)) for i in range(3)]
    outs = [[torch.zeros((w.B, w.Hq, w.d), dtype=torch.float32, device=dev) for _ in range(per)] for _ in range(3)]

    def run():
        for i in range(3):
            dec.run_interval(i, qidx[i], qs[i], outs[i])
        dec.join()

    run()
    torch.cuda.synchronize()
    eager = [[o.cpu().numpy().copy() for o in row] for row in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    dec._attn_done_valid = False
    with torch.cuda.graph(g, stream=s):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for row in outs:
            for o in row:
                o.fill_(float("nan"))
        for p in dec.pool:
            p.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            for t in range(per):
                assert np.array_equal(outs[i][t].cpu().numpy(), eager[i][t]), f"replay {rep}, interval {i}, step {t}"


@pytest.mark.parametrize("split", [False, True])
def test_token_stage_graph_replays_match_eager(tune, split):
    """Chunk selection, then per step the token top-k and the token-list
    attention, captured in one graph: every replay gives the eager bits.
    split=True forces the slices + candidates select (two launches and a
    workspace per step), as long recalls take it."""
    import torch

    if split:  # consulted when the workspace is sized and at every call, so set before the decoder exists
        tune(topk_split_min_n=1, topk_split_slices=4)

    import synth
    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    w = W.WORKLOADS["32k"]
    dev = torch.device("cuda")
    dec = LsaDecoder(k_idx=to_dev(W.indexer_keys(w)), ctx_len=to_dev(W.ctx_lens(w)), Hq=w.Hq, k=w.k,
                     alpha=w.alpha, kv=W.device_kv_store(w, dev), token_topk=300)
    assert (dec.tok_workspace is not None) == split
    steps = 6
    qs = [to_dev_bf16(W.attn_query(w, t)) for t in range(steps)]
    sc = [to_dev(np.ascontiguousarray(synth.bf16_bits_to_f32(
        synth.normal_bf16((w.B, w.k * 64), 3, synth.stream(synth.TAG_MISC, 5100 + t))), dtype=np.float32))
        for t in range(steps)]
    qidx = to_dev(W.indexer_query(w, 0))
    outs = [torch.zeros((w.B, w.Hq, w.d), dtype=torch.float32, device=dev) for _ in range(steps)]
    dec.run_interval(0, qidx, qs, outs, token_scores=sc)
    torch.cuda.synchronize()
    eager = [o.cpu().numpy().copy() for o in outs]
    tok_eager = dec.tok.cpu().numpy().copy()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dec.run_interval(0, qidx, qs, outs, token_scores=sc)
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        dec.tok.fill_(-7)
        junk.mul_(1.0001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(dec.tok.cpu().numpy(), tok_eager), f"replay {rep}: token list"
        for t in range(steps):
            assert np.array_equal(outs[t].cpu().numpy(), eager[t]), f"replay {rep}, step {t}"
