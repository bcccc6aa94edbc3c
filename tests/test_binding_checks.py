"""Host-side checks of the Python binding and the tuning knobs, on the CPU.

The binding passes raw pointers to kernels that write exactly the sizes the
arguments imply, so a caller-supplied output of the wrong dtype, shape or
device must be refused before the library is called.  Each case below
swaps the loaded library for a stub that fails the test if any entry point
is reached.  No GPU is used: every tensor is a CPU tensor, and a device
mismatch is shown with a second (meta) device."""
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lsa():
    import lookahead_chunk_sparse_amd as m
    return m


class _NoCalls:
    """Stands in for liblsa.so: any attribute access is a test failure."""

    def __getattr__(self, name):
        raise AssertionError(f"the library was called ({name}) although the arguments are invalid")


@pytest.fixture
def no_lib(lsa):
    import lookahead_chunk_sparse_amd._binding as b
    saved = b._lib
    b._lib = _NoCalls()
    try:
        yield b
    finally:
        b._lib = saved


def _i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def _bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _attend_inputs(B=2, Hq=16, Hkv=2, d=64, C=5, k=3):
    return dict(q=_bf16(B, Hq, d), kv=_bf16(B, C, 2, Hkv, 64, d), chunk_ids=_i32(B, k), ctx_len=_i32(B))


BAD_OUTPUTS = [
    ("float64 instead of float32", lambda: torch.zeros((2, 16, 64), dtype=torch.float64)),
    ("bf16 instead of float32", lambda: _bf16(2, 16, 64)),
    ("too short", lambda: torch.zeros((2, 16, 63), dtype=torch.float32)),
    ("too long", lambda: torch.zeros((3, 16, 64), dtype=torch.float32)),
    ("flattened", lambda: torch.zeros((2 * 16 * 64,), dtype=torch.float32)),
    ("not contiguous", lambda: torch.zeros((2, 64, 16), dtype=torch.float32).transpose(1, 2)),
    ("another device", lambda: torch.zeros((2, 16, 64), dtype=torch.float32, device="meta")),
    ("not a tensor", lambda: [0.0] * (2 * 16 * 64)),
]


@pytest.mark.parametrize("what,make", BAD_OUTPUTS, ids=[b[0] for b in BAD_OUTPUTS])
def test_attend_rejects_bad_out(lsa, no_lib, what, make):
    x = _attend_inputs()
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises((TypeError, ValueError)):
        lsa.lsa_gather_attend(x["q"], x["kv"], x["chunk_ids"], x["ctx_len"], workspace=ws, out=make())


@pytest.mark.parametrize("field,bad", [
    ("slots", lambda: _i32(2, 4)), ("slots", lambda: torch.zeros((2, 3), dtype=torch.int64)),
    ("counts", lambda: _i32(3)), ("seg_len", lambda: _i32(3)),
    ("tok_counts", lambda: _i32(1)), ("chunk_ids", lambda: _i32(2, 3).to("meta")),
    ("workspace", lambda: torch.zeros(64, dtype=torch.float32)),
])
def test_attend_rejects_bad_side_inputs(lsa, no_lib, field, bad):
    x = _attend_inputs()
    kw = dict(workspace=torch.zeros(1 << 16, dtype=torch.uint8))
    if field in ("slots", "counts", "workspace"):
        kw[field] = bad()
    elif field == "seg_len":
        kw.update(seg_kv=_bf16(2, 2, 2, 64, 64), seg_len=bad())
    elif field == "tok_counts":
        kw.update(tok=_i32(2, 10), tok_counts=bad())
    elif field == "chunk_ids":
        x["chunk_ids"] = bad()
    with pytest.raises((TypeError, ValueError)):
        lsa.lsa_gather_attend(x["q"], x["kv"], x["chunk_ids"], x["ctx_len"], **kw)


def test_attend_segment_needs_length(lsa, no_lib):
    x = _attend_inputs()
    with pytest.raises(ValueError, match="seg_len"):
        lsa.lsa_gather_attend(x["q"], x["kv"], x["chunk_ids"], x["ctx_len"], seg_kv=_bf16(2, 2, 2, 64, 64),
                              workspace=torch.zeros(64, dtype=torch.uint8))


def test_score_and_select_reject_bad_outputs(lsa, no_lib):
    q = torch.zeros((2, 1, 64), dtype=torch.int8)
    K = torch.zeros((2, 100, 64), dtype=torch.int8)
    with pytest.raises(ValueError):
        lsa.lsa_index_score(q, K, 0.01, logits=_i32(2, 1, 99))
    with pytest.raises(TypeError):
        lsa.lsa_index_score(q, K, 0.01, logits=_i32(2, 1, 100), scores=_i32(2, 1, 100))
    logits = _i32(2, 100)
    with pytest.raises(ValueError):
        lsa.lsa_topk_chunks(logits, 10, chunk_ids=_i32(2, 9))
    with pytest.raises(ValueError):
        lsa.lsa_threshold_chunks(logits, 10, chunk_ids=_i32(2, 10), counts=_i32(3))
    with pytest.raises(TypeError):
        lsa.lsa_threshold_chunks(logits, 10, chunk_ids=torch.zeros((2, 10), dtype=torch.int64))


def test_token_select_rejects_bad_outputs(lsa, no_lib):
    scores = torch.zeros((2, 3 * 64), dtype=torch.float32)
    ids, ctx = _i32(2, 3), _i32(2)
    with pytest.raises(ValueError):
        lsa.lsa_topk_tokens(scores, ids, ctx, 50, tok=_i32(2, 49), workspace=None)
    with pytest.raises(ValueError):
        lsa.lsa_topk_tokens(scores, ids, ctx, 50, tok_counts=_i32(1), workspace=None)
    with pytest.raises(ValueError):
        lsa.lsa_topk_tokens(scores, ids, _i32(3), 50, workspace=None)
    with pytest.raises(TypeError):
        lsa.lsa_topk_tokens(scores, ids, ctx, 50, workspace=torch.zeros(8, dtype=torch.int32))


def test_pool_assign_rejects_bad_outputs(lsa, no_lib):
    new = _i32(2, 5)
    with pytest.raises(ValueError):
        lsa.lsa_pool_assign(None, None, new, 10, new_slots=_i32(2, 4))
    with pytest.raises(TypeError):
        lsa.lsa_pool_assign(None, None, new, 10, fetch_slots=torch.zeros((2, 5), dtype=torch.int64))


@pytest.mark.parametrize("pool_shape", [(2, 6, 2, 3, 64, 64), (3, 6, 2, 2, 64, 64), (2, 6, 2, 2, 64, 128),
                                        (2, 6, 1, 2, 64, 64)])
def test_fetch_pool_must_match_host_store(lsa, no_lib, pool_shape):
    host = _bf16(2, 9, 2, 2, 64, 64)
    pool = _bf16(*pool_shape)
    with pytest.raises(ValueError, match="pool_kv shape"):
        lsa.lsa_fetch_chunks(host, _i32(2, 4), pool)
    with pytest.raises(ValueError):
        lsa.lsa_fetch_chunks_pull(host, _i32(2, 4), pool)


def test_fetch_staged_checks_staging(lsa, no_lib):
    """The staging buffers must hold chunks of the store's shape, the host one
    on the host and the device one on the device."""
    host, pool = _bf16(2, 9, 2, 2, 64, 64), _bf16(2, 6, 2, 2, 64, 64)
    with pytest.raises(ValueError, match="staging"):
        lsa.lsa_fetch_chunks_staged(host, _i32(2, 4), pool.to("meta"), _bf16(4, 2, 2, 64, 32), _bf16(4, 2, 2, 64, 32))
    with pytest.raises(ValueError):
        lsa.lsa_fetch_chunks_staged(host, _i32(2, 4), pool, _bf16(4, 2, 2, 64, 64), _bf16(4, 2, 2, 64, 64))
    with pytest.raises(TypeError):
        lsa.lsa_fetch_chunks_staged(host, _i32(2, 4), pool, _bf16(4, 2, 2, 64, 64), _i32(4, 2, 2, 64, 64))


# ---- tuning knobs ---------------------------------------------------------

def test_tuning_defaults_and_overrides(lsa):
    base = {k: lsa.lsa_get_tuning(k) for k in lsa.TUNE_KNOBS}
    if "LSA_ATTEND_DEPTH" not in os.environ:
        assert base["attend_depth"] == 2
    with lsa.tuning(attend_depth=3, topk_split_slices=5):
        assert lsa.lsa_get_tuning("attend_depth") == 3
        assert lsa.lsa_get_tuning("topk_split_slices") == 5
        with lsa.tuning(attend_depth=4):
            assert lsa.lsa_get_tuning("attend_depth") == 4
        assert lsa.lsa_get_tuning("attend_depth") == 3
    assert {k: lsa.lsa_get_tuning(k) for k in lsa.TUNE_KNOBS} == base


@pytest.mark.parametrize("knob,value", [("attend_depth", 1), ("attend_depth", 5), ("score_mfma_min_nq", -1),
                                        ("fetch_lanes", 17), (99, 1)])
def test_tuning_rejects_bad_values(lsa, knob, value):
    with pytest.raises(lsa.LsaError):
        lsa.lsa_set_tuning(knob, value)


def test_tuning_override_is_per_thread(lsa):
    import threading
    seen = {}
    with lsa.tuning(score_mfma_min_nq=77):
        t = threading.Thread(target=lambda: seen.setdefault("other", lsa.lsa_get_tuning("score_mfma_min_nq")))
        t.start()
        t.join()
        assert lsa.lsa_get_tuning("score_mfma_min_nq") == 77
    assert seen["other"] != 77


def test_tuning_environment_is_read_once():
    """The environment supplies the defaults, read at the first use; a later
    change of the variable is not seen (no getenv on the hot path)."""
    code = (
        "import os, sys; sys.path.insert(0, %r)\n"
        "import lookahead_chunk_sparse_amd as m\n"
        "a = m.lsa_get_tuning('attend_depth'); b = m.lsa_get_tuning('topk_stream_min_c')\n"
        "os.environ['LSA_ATTEND_DEPTH'] = '4'\n"
        "print(a, b, m.lsa_get_tuning('attend_depth'))\n" % ROOT)
    env = dict(os.environ, LSA_ATTEND_DEPTH="3", LSA_TOPK_STREAM_MIN_C="123")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["3", "123", "3"]
    env["LSA_ATTEND_DEPTH"] = "9"  # out of range: ignored, the default stays
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split()[0] == "2"


def test_check_ids_argument_validation(lsa):
    """lsa_check_ids rejects bad sizes before any HIP call (no GPU here)."""
    L = lsa.load_library()
    P = 1 << 20  # never dereferenced
    assert L.lsa_check_ids(None, None, None, 1, 1, 10, 10, P, None) == 1
    assert L.lsa_check_ids(P, None, None, 1, 16385, 20000, 20000, P, None) == 2  # beyond the LDS sort
    assert L.lsa_check_ids(P, None, None, 1 << 22, 1, 10, 10, P, None) == 2
    assert L.lsa_check_ids(P, None, None, 2, 3, 0, 10, P, None) == 1
    assert L.lsa_check_ids(P + 2, None, None, 2, 3, 10, 10, P, None) == 1  # misaligned
    with pytest.raises(ValueError):
        lsa.lsa_check_ids(torch.zeros((2, 3), dtype=torch.int32), 10, counts=torch.zeros(3, dtype=torch.int32))
