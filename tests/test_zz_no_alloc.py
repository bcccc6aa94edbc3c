"""lsa_gather_attend_noalloc, the attention entry point for callers that
cannot allocate: its split partials live in the library's static device
buffer instead of a workspace.  Through the C ABI (ctypes binding), two calls
in a row, the second on smaller inputs, each compared with lsa_gather_attend
on the same inputs (the same kernels: bit for bit) and with the oracle.  The
rejection of sizes beyond the static buffer is checked on the CPU, before any
HIP call."""
import ctypes
import math

import numpy as np
import pytest

from conftest import gpu_available
from helpers import check_attention, to_dev, to_dev_bf16

BOGUS = 1 << 20  # a non-null, aligned address that is never dereferenced


@pytest.fixture(scope="module")
def lsa():
    import lookahead_chunk_sparse_amd as m
    return m


def test_noalloc_rejects_before_any_hip_call(lsa):
    """Sizes whose partials exceed LSA_NOALLOC_SCRATCH_BYTES give
    LSA_ERR_WORKSPACE, and invalid shapes lsa_gather_attend's own error,
    before any HIP call (so also on a machine without a GPU)."""
    L = lsa.load_library()
    B, Hq, Hkv, d, k, n_split = 64, 64, 8, 128, 64, 16
    need = lsa.lsa_gather_attend_workspace_size(B, Hq, Hkv, d, k, n_split)
    assert need > lsa.NOALLOC_SCRATCH_BYTES
    st = L.lsa_gather_attend_noalloc(BOGUS, BOGUS, 100, BOGUS, None, None, BOGUS, None, None, 0, B, Hq, Hkv, d, k,
                                     0.1, n_split, BOGUS, None)
    assert st == 3, L.lsa_last_error()  # LSA_ERR_WORKSPACE
    assert b"static scratch" in L.lsa_last_error()
    st = L.lsa_gather_attend_noalloc(BOGUS, BOGUS, 100, BOGUS, None, None, BOGUS, None, None, 0, 2, 64, 7, 128, 4,
                                     0.1, 0, BOGUS, None)
    assert st == 1, L.lsa_last_error()  # Hq not a multiple of Hkv
    # the largest size that fits is accepted by the size check
    assert lsa.lsa_gather_attend_workspace_size(16, 64, 8, 128, 276, 0) <= lsa.NOALLOC_SCRATCH_BYTES


def _case(synth_lib, B, Hq, Hkv, d, C, k, seed):
    s = synth_lib.stream
    q = synth_lib.normal_bf16((B, Hq, d), seed, s(synth_lib.TAG_MISC, 9100), scale=2.0)
    kv = synth_lib.normal_bf16((B, C, 2, Hkv, 64, d), seed, s(synth_lib.TAG_MISC, 9101))
    ids = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        ids[b] = np.sort(synth_lib.choose(k, C, seed, s(synth_lib.TAG_MISC, 9200 + b)))
        ids[b, 0] = 0
    return q, kv, ids


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU")
def test_noalloc_matches_gather_attend(lsa, oracle_lib, synth_lib):
    import torch

    # call 1: the DeepSeek-V4 GQA shape with the library's split count (8);
    # call 2: smaller, a group of 3 query heads at d = 64, ragged counts,
    # a partial context and a resident segment, 3 splits
    calls = [
        dict(shape=(4, 64, 8, 128, 40, 32), n_split=0, extras=False),
        dict(shape=(2, 12, 4, 64, 12, 6), n_split=3, extras=True),
    ]
    for n, c in enumerate(calls):
        B, Hq, Hkv, d, C, k = c["shape"]
        print(f"no-alloc call {n}: B={B} Hq={Hq} Hkv={Hkv} d={d} k={k} n_split={c['n_split']}", flush=True)
        q, kv, ids = _case(synth_lib, B, Hq, Hkv, d, C, k, seed=17 + n)
        ctx = np.full(B, C * 64, dtype=np.int32)
        kw, okw = {}, {}
        if c["extras"]:
            ctx[0] = int(ids[0, 3]) * 64 + 11
            counts = np.array([k, k - 2], dtype=np.int32)
            seg = synth_lib.normal_bf16((B, 2, Hkv, 128, d), 5, synth_lib.stream(synth_lib.TAG_MISC, 9300))
            sl = np.array([100, 128], dtype=np.int32)
            kw = dict(counts=to_dev(counts), seg_kv=to_dev_bf16(seg), seg_len=to_dev(sl))
            okw = dict(counts=counts, seg_kv=seg, seg_len=sl)
        args = (to_dev_bf16(q), to_dev_bf16(kv), to_dev(ids), to_dev(ctx))
        scale = 1.0 / math.sqrt(d)
        ref = lsa.lsa_gather_attend(*args, scale, n_split=c["n_split"], **kw)
        out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        lsa.lsa_gather_attend_noalloc(*args, out=out, sm_scale=scale, n_split=c["n_split"], **kw)
        torch.cuda.synchronize()
        # the call allocates nothing: device free memory is unchanged by a repeat
        free0 = torch.cuda.mem_get_info()[0]
        lsa.lsa_gather_attend_noalloc(*args, out=out, sm_scale=scale, n_split=c["n_split"], **kw)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        got, want = out.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"call {n} differs from lsa_gather_attend"
        oref = oracle_lib.gather_attend(q, kv, ids, ctx, Hkv, scale, **okw)
        print("  ", check_attention(got, oref, f"no-alloc call {n}"), flush=True)
