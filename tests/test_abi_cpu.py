"""The C-ABI library loads without a GPU, exports every symbol include/lsa.h
declares, and rejects bad arguments before any HIP call (no kernel is
launched by these tests: every call below fails validation first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")

BOGUS = 1 << 20  # a non-null, aligned, never dereferenced address


@pytest.fixture(scope="module")
def lsa():
    import lookahead_chunk_sparse_amd as m
    return m


@pytest.fixture(scope="module")
def lib(lsa):
    return lsa.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("lsa_index_score", "lsa_topk_chunks", "lsa_gather_attend", "lsa_fetch_chunks"):
        assert n in names


def test_every_declared_symbol_is_exported(lsa, lib):
    names = declared_functions()
    assert set(names) == set(lsa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    # and they are C symbols (no C++ mangling)
    out = os.popen(f"nm -D --defined-only {lsa.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_status_strings(lib):
    assert lib.lsa_status_string(0) == b"LSA_OK"
    assert lib.lsa_status_string(3) == b"LSA_ERR_WORKSPACE"
    assert lib.lsa_status_string(99) == b"LSA_ERR_UNKNOWN"


def _err(lib):
    return lib.lsa_last_error().decode()


def test_index_score_validation(lib):
    f = lib.lsa_index_score
    assert f(0, BOGUS, 1, 1, 4, 64, 1.0, BOGUS, 0, 0) == 1 and "required" in _err(lib)
    assert f(BOGUS, BOGUS, 0, 1, 4, 64, 1.0, BOGUS, 0, 0) == 1
    assert f(BOGUS, BOGUS, 1, 1, 0, 64, 1.0, BOGUS, 0, 0) == 1
    assert f(BOGUS, BOGUS, 1, 1, 4, 48, 1.0, BOGUS, 0, 0) == 2 and "d_idx=48" in _err(lib)
    assert f(BOGUS, BOGUS, 1, 1, 4, 64, float("inf"), BOGUS, 0, 0) == 1
    assert f(BOGUS + 1, BOGUS, 1, 1, 4, 64, 1.0, BOGUS, 0, 0) == 1 and "alignment" in _err(lib)
    assert f(BOGUS, BOGUS, 65536, 1, 65536, 64, 1.0, BOGUS, 0, 0) == 1  # B*nq*C overflows int32


def test_topk_validation(lib):
    f = lib.lsa_topk_chunks
    assert f(0, 1, 8, 2, BOGUS, 0) == 1
    assert f(BOGUS, 1, 8, 0, BOGUS, 0) == 1 and "k=0" in _err(lib)
    assert f(BOGUS, 1, 8, 9, BOGUS, 0) == 1
    assert f(BOGUS, 0, 8, 1, BOGUS, 0) == 1
    assert f(BOGUS, 1, (1 << 30) + 1, 1, BOGUS, 0) == 2


def test_threshold_validation(lib):
    f = lib.lsa_threshold_chunks
    assert f(0, 1, 8, 0, 2, BOGUS, BOGUS, 0) == 1
    assert f(BOGUS, 1, 8, 0, 2, BOGUS, 0, 0) == 1 and "counts" in _err(lib)
    assert f(BOGUS, 1, 8, 0, 0, BOGUS, BOGUS, 0) == 1 and "k_max=0" in _err(lib)
    assert f(BOGUS, 1, 8, 0, 9, BOGUS, BOGUS, 0) == 1
    assert f(BOGUS, 1, (1 << 30) + 1, 0, 1, BOGUS, BOGUS, 0) == 2


def test_attend_validation(lsa, lib):
    f = lib.lsa_gather_attend
    # q, kv, C_store, ids, slots, counts, ctx, B, Hq, Hkv, d, k, scale, ws, ws_bytes, n_split, out, stream
    ok = dict(q=BOGUS, kv=BOGUS, C=16, ids=BOGUS, slots=0, ctx=BOGUS, B=2, Hq=64, Hkv=8, d=128, k=4,
              scale=0.088, ws=0, wsb=0, ns=1, out=BOGUS)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["kv"], a["C"], a["ids"], a["slots"], 0, a["ctx"], a.get("seg", 0), a.get("seg_len", 0),
                 a.get("S_max", 0), a["B"], a["Hq"], a["Hkv"], a["d"], a["k"], a["scale"], a["ws"], a["wsb"],
                 a["ns"], a["out"], 0)

    assert call(q=0) == 1
    assert call(Hq=60) == 1 and "multiple" in _err(lib)
    assert call(Hq=136, Hkv=8) == 2 and "16 query heads" in _err(lib)
    assert call(d=96) == 2
    assert call(k=0) == 1
    assert call(C=0) == 1
    assert call(scale=float("nan")) == 1
    assert call(ns=-1) == 1
    assert call(out=BOGUS + 4) == 1 and "alignment" in _err(lib)
    assert call(seg=BOGUS) == 1 and "segment" in _err(lib)
    assert call(seg=BOGUS, seg_len=BOGUS, S_max=100) == 1 and "multiple of 64" in _err(lib)
    need = lsa.lsa_gather_attend_workspace_size(2, 64, 8, 128, 4, 2)
    assert need > 0
    assert call(ns=2) == 3 and "workspace" in _err(lib)
    assert call(ns=2, ws=BOGUS, wsb=need - 1) == 3
    assert call(ns=2, ws=BOGUS + 16, wsb=need) == 3 and "256-byte" in _err(lib)


def test_token_stage_validation(lib):
    f = lib.lsa_topk_tokens
    # scores, chunk_ids, counts, ctx_len, B, k, k_tok, tok, tok_counts, workspace, workspace_bytes, stream
    assert f(0, BOGUS, 0, BOGUS, 2, 4, 8, BOGUS, BOGUS, 0, 0, 0) == 1
    assert f(BOGUS, BOGUS, 0, BOGUS, 2, 4, 8, BOGUS, 0, 0, 0, 0) == 1 and "tok_counts" in _err(lib)
    assert f(BOGUS, BOGUS, 0, BOGUS, 2, 4, 0, BOGUS, BOGUS, 0, 0, 0) == 1 and "k_tok=0" in _err(lib)
    assert f(BOGUS, BOGUS, 0, BOGUS, 2, (1 << 24) + 1, 8, BOGUS, BOGUS, 0, 0, 0) == 2 and "k <= 16777216" in _err(lib)
    assert f(BOGUS + 2, BOGUS, 0, BOGUS, 2, 4, 8, BOGUS, BOGUS, 0, 0, 0) == 1 and "alignment" in _err(lib)
    assert lib.lsa_topk_tokens_workspace_size(16, 276, 2048) == 0  # 17,664 positions: no split
    need = lib.lsa_topk_tokens_workspace_size(4, 1638, 2048)      # the 1M recall: 16 slices
    assert need > 0
    assert f(BOGUS, BOGUS, 0, BOGUS, 4, 1638, 2048, BOGUS, BOGUS, BOGUS, need - 1, 0) == 3 and "workspace" in _err(lib)
    assert f(BOGUS, BOGUS, 0, BOGUS, 4, 1638, 2048, BOGUS, BOGUS, BOGUS + 16, need, 0) == 3 and "256-byte" in _err(lib)
    g = lib.lsa_gather_attend_tokens
    # q, kv, C, ids, slots, counts, ctx, tok, tok_counts, k_tok, seg, seg_len, S_max, B, Hq, Hkv, d, k, scale,
    # ws, ws_bytes, n_split, out, stream
    args = [BOGUS, BOGUS, 16, BOGUS, 0, 0, BOGUS, BOGUS, 0, 128, 0, 0, 0, 2, 64, 8, 128, 4, 0.088, 0, 0, 1, BOGUS, 0]
    a = list(args); a[7] = 0
    assert g(*a) == 1 and "tok is required" in _err(lib)
    a = list(args); a[9] = 0
    assert g(*a) == 1 and "k_tok=0" in _err(lib)
    a = list(args); a[2] = 1 << 22
    assert g(*a) == 2 and "C_store" in _err(lib)
    a = list(args); a[21] = 2  # two splits of the 2 token blocks need a workspace
    assert g(*a) == 3 and "workspace" in _err(lib)


def test_workspace_size_rules(lsa):
    # one split needs no workspace; the partials grow with the split count
    assert lsa.lsa_gather_attend_workspace_size(16, 64, 8, 128, 276, 1) == 0
    a = lsa.lsa_gather_attend_workspace_size(16, 64, 8, 128, 276, 4)
    b = lsa.lsa_gather_attend_workspace_size(16, 64, 8, 128, 276, 8)
    assert 0 < a < b
    # partial O (B*Hkv*splits*G*d fp32, rounded to 256 B), then the (m, l) pairs
    parts = 16 * 8 * 4 * 8
    assert a == (parts * 128 * 4 + 255) // 256 * 256 + parts * 2 * 4
    # splits are capped at k
    assert lsa.lsa_gather_attend_workspace_size(1, 8, 1, 64, 3, 50) == lsa.lsa_gather_attend_workspace_size(
        1, 8, 1, 64, 3, 3)
    for s in (lsa.lsa_gather_attend_default_splits(16, 8, 276), lsa.lsa_gather_attend_default_splits(1, 1, 8)):
        assert s >= 1
    assert lsa.lsa_gather_attend_default_splits(1, 1, 3) <= 3
    with pytest.raises(lsa.LsaError):
        lsa.lsa_gather_attend_workspace_size(1, 8, 3, 64, 3)


def test_fetch_validation(lib):
    import numpy as np
    f = lib.lsa_fetch_chunks
    ids = np.array([[0, 5]], dtype=np.int32)
    bad = np.array([[0, 9]], dtype=np.int32)
    slots_bad = np.array([[0, 3]], dtype=np.int32)
    # host_kv, C, ids, slots, pool, P, B, Hkv, d, k, stream, event
    assert f(0, 8, ids.ctypes.data, 0, BOGUS, 2, 1, 1, 64, 2, 0, 0) == 1
    assert f(BOGUS, 8, bad.ctypes.data, 0, BOGUS, 2, 1, 1, 64, 2, 0, 0) == 1 and "chunk id 9" in _err(lib)
    assert f(BOGUS, 8, ids.ctypes.data, slots_bad.ctypes.data, BOGUS, 2, 1, 1, 64, 2, 0, 0) == 1
    assert f(BOGUS, 8, ids.ctypes.data, 0, BOGUS, 1, 1, 1, 64, 2, 0, 0) == 1 and "k=2 > P=1" in _err(lib)


def test_fetch_staged_validation(lib):
    """Argument errors of the staged fetch are reported before any HIP call:
    missing buffers, a staging buffer of fewer than 2 chunks, ids and slots
    out of range (an entry with a negative slot is skipped, so its id is not
    checked), k above P with default slots, misaligned buffers."""
    import numpy as np
    f = lib.lsa_fetch_chunks_staged
    ids = np.array([[0, 5]], dtype=np.int32)
    bad = np.array([[0, 9]], dtype=np.int32)
    slots_bad = np.array([[0, 3]], dtype=np.int32)
    # host_kv, C, ids, slots, pool, P, B, Hkv, d, k, host_staging, dev_staging, stage_chunks, stream, event
    args = [BOGUS, 8, ids.ctypes.data, 0, BOGUS, 2, 1, 1, 64, 2, BOGUS, BOGUS, 4, 0, 0]

    def call(**over):
        a = list(args)
        for i, v in over.items():
            a[int(i[1:])] = v
        return f(*a)

    for i in (0, 2, 4, 10, 11):  # a required pointer missing
        assert call(**{f"a{i}": 0}) == 1 and "required" in _err(lib), i
    assert call(a12=1) == 1 and "stage_chunks=1" in _err(lib)
    assert call(a2=bad.ctypes.data) == 1 and "chunk id 9" in _err(lib)
    assert call(a3=slots_bad.ctypes.data) == 1 and "slot 3" in _err(lib)
    assert call(a5=1) == 1 and "k=2 > P=1" in _err(lib)
    assert call(a10=BOGUS + 8) == 1 and "alignment" in _err(lib)
    assert call(a7=0) == 1  # Hkv < 1
    # the id past C sits at an entry whose slot is negative: not read, so the
    # next check (pinned host memory) is the one that fails
    skip = np.array([[0, -1]], dtype=np.int32)
    assert call(a2=bad.ctypes.data, a3=skip.ctypes.data) == 1 and "chunk id" not in _err(lib)


def test_fetch_pull_validation(lib):
    """Argument errors of the pull fetch, reported before any HIP call."""
    import numpy as np
    f = lib.lsa_fetch_chunks_pull
    ids = np.array([[0, 5]], dtype=np.int32)
    # host_kv, C, ids, slots, pool, P, B, Hkv, d, k, grid, stream
    assert f(0, 8, BOGUS, 0, BOGUS, 2, 1, 1, 64, 2, 0, 0) == 1 and "required" in _err(lib)
    assert f(BOGUS, 8, BOGUS, 0, BOGUS, 2, 1, 1, 64, 2, -1, 0) == 1
    assert f(BOGUS, 8, BOGUS, 0, BOGUS, 2, 1, 1, 64, 2, 1 << 24, 0) == 1
    assert f(BOGUS, 8, BOGUS, 0, BOGUS, 2, 1, 1, 96, 2, 0, 0) == 2 and "d=96" in _err(lib)
    assert f(BOGUS, 8, BOGUS, 0, BOGUS, 1, 1, 1, 64, 2, 0, 0) == 1 and "k=2 > P=1" in _err(lib)
    assert f(BOGUS + 8, 8, BOGUS, 0, BOGUS, 2, 1, 1, 64, 2, 0, 0) == 1 and "alignment" in _err(lib)
    assert f(BOGUS, 8, BOGUS + 2, 0, BOGUS, 2, 1, 1, 64, 2, 0, 0) == 1 and "alignment" in _err(lib)
    del ids


def test_python_binding_checks_dtypes(lsa):
    import torch
    with pytest.raises(TypeError):
        lsa.lsa_topk_chunks(torch.zeros(4, dtype=torch.int64), 1)
    with pytest.raises(ValueError):
        lsa.lsa_index_score(torch.zeros((1, 1, 64), dtype=torch.int8), torch.zeros((1, 64), dtype=torch.int8), 1.0)
