"""The library driven from plain C programs through include/lsa.h, with
HIP runtime memory and no PyTorch in the process that runs the kernels.

tests/c/decode_interval.c runs two re-selection intervals (a drifting
indexer query, so the second selection differs from the first) with delta
pool slots, the pull fetch from pinned host memory and the DMA fetch; every
output it writes is checked against the oracle.  Its workload is the 32K
shape (4 requests, 64/8 heads, d = 128, 32 kept chunks) over a ragged
8,229-token context, so the last chunk is partial.

tests/c/threaded_calls.c checks the threading promise of the header."""
import os
import subprocess

import numpy as np
import pytest

from conftest import gpu_available
from helpers import check_attention

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "lookahead_chunk_sparse_amd")


def say(*a):
    print(*a, flush=True)


def _compile(exe: str, source: str = "decode_interval.c") -> None:
    assert os.path.exists(os.path.join(LIBDIR, "liblsa.so")), "liblsa.so is not built"
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-pthread",
                           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                           os.path.join(ROOT, "tests", "c", source), "-o", exe,
                           "-L", LIBDIR, "-llsa", "-L", "/opt/rocm/lib", "-lamdhip64",
                           f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath,/opt/rocm/lib"])


def _load(d, name, dtype, shape):
    a = np.fromfile(os.path.join(d, name), dtype=dtype)
    assert a.size == int(np.prod(shape)), (name, a.size, shape)
    return a.reshape(shape)


def test_c_program_two_intervals(tmp_path, oracle_lib):
    from synth import workloads as W
    w = W.WORKLOADS["32k"].replace(name="c-client", N=8229, steps=128, drift=True)
    B, C, k, Hq, Hkv, d = w.B, w.C, w.k, w.Hq, w.Hkv, w.d
    P = 2 * k
    q_idx = np.stack([W.indexer_query(w, i) for i in range(2)])          # [2][B][1][d_idx]
    K = W.indexer_keys(w)
    q = np.stack([W.attn_query(w, i * w.tau) for i in range(2)])         # [2][B][Hq][d]
    kv = W.kv_store(w)
    ctx = W.ctx_lens(w)
    out_dir = str(tmp_path)
    q_idx.tofile(os.path.join(out_dir, "q_idx.bin"))
    K.tofile(os.path.join(out_dir, "k_idx.bin"))
    q.tofile(os.path.join(out_dir, "q.bin"))
    kv.tofile(os.path.join(out_dir, "kv.bin"))
    ctx.tofile(os.path.join(out_dir, "ctx.bin"))
    exe = os.path.join(out_dir, "decode_interval")
    _compile(exe)

    args = [exe, out_dir, B, C, w.d_idx, k, Hq, Hkv, d, repr(w.alpha), repr(w.sm_scale)]
    say("C client:", " ".join(str(a) for a in args[2:]))
    r = subprocess.run([str(a) for a in args], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip(), r.stderr.strip())
    assert r.returncode == 0, r.stdout + r.stderr

    prev_ids = prev_slots = None
    pool_ref = np.zeros((B, P, 2, Hkv, w.T, d), dtype=np.uint16)
    outs = []
    for i in range(2):
        L_ref, S_ref, ids_ref = oracle_lib.select(q_idx[i], K, k, w.alpha)
        logits = _load(out_dir, f"logits{i}.bin", np.int32, L_ref.shape)
        scores = _load(out_dir, f"scores{i}.bin", np.float32, S_ref.shape).astype(np.float64)
        ids = _load(out_dir, f"ids{i}.bin", np.int32, (B, k))
        assert np.array_equal(logits, L_ref), f"interval {i}: logits differ"
        assert (np.abs(scores - S_ref) <= 1e-6 * np.abs(S_ref) + 2.0 ** -126).all(), f"interval {i}: scores differ"
        assert np.array_equal(ids, ids_ref.reshape(B, k)), f"interval {i}: selection differs"

        slots_ref, fslots_ref = oracle_lib.pool_assign(prev_ids, prev_slots, ids_ref.reshape(B, k), P)
        assert np.array_equal(_load(out_dir, f"slots{i}.bin", np.int32, (B, k)), slots_ref), f"interval {i}: slots"
        assert np.array_equal(_load(out_dir, f"fslots{i}.bin", np.int32, (B, k)), fslots_ref), f"interval {i}: fetch"
        oracle_lib.fetch_chunks(kv, ids_ref.reshape(B, k), P, fslots_ref, pool=pool_ref, skip_negative_slots=True)

        ref = oracle_lib.gather_attend(q[i], kv, ids_ref.reshape(B, k), ctx, Hkv, w.sm_scale)
        out = _load(out_dir, f"out{i}.bin", np.float32, (B, Hq, d))
        say(f"interval {i}:", check_attention(out, ref, f"C client interval {i}"))
        outs.append(out)
        prev_ids, prev_slots = ids_ref.reshape(B, k), slots_ref
    assert not np.array_equal(_load(out_dir, "ids0.bin", np.int32, (B, k)),
                              _load(out_dir, "ids1.bin", np.int32, (B, k))), "the two selections should differ"

    # the DMA fetch feeds the same kernel the same values in the same list order
    assert np.array_equal(_load(out_dir, "out0_dma.bin", np.float32, (B, Hq, d)), outs[0]), "DMA-fetch attention"

    # every slot either interval wrote holds the chunk the oracle's fetch put there
    pool = _load(out_dir, "pool.bin", np.uint16, pool_ref.shape)
    s0 = _load(out_dir, "slots0.bin", np.int32, (B, k))
    s1 = _load(out_dir, "slots1.bin", np.int32, (B, k))
    for b in range(B):
        used = np.union1d(s0[b], s1[b])
        assert np.array_equal(pool[b, used], pool_ref[b, used]), f"pool of request {b}"


def test_c_program_threads(tmp_path):
    """tests/c/threaded_calls.c: four host threads, each on its own stream
    and workspace, repeat scan -> select -> attend and match a serial run bit
    for bit; a rejected call's message belongs to its own thread."""
    exe = str(tmp_path / "threaded_calls")
    _compile(exe, "threaded_calls.c")
    say("C threads: 4 threads x 12 repetitions")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip(), r.stderr.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "threaded_calls: ok" in r.stdout
