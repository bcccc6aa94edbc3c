"""CPU oracle for the LSA decode path.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``lookahead_chunk_sparse_amd``) and does not import it.

The arithmetic lives in ``lsa_oracle.c`` (plain C, exact integers and IEEE
double); this module binds it with ctypes and adds the decode schedule:
re-selection at steps t = 0 (mod tau) with tau = 64 (paperlayer.ai summary of
"FlashMemory-DeepSeek-V4", 1 Introduction and 2.1 Architecture: the indexer
evaluates the current state every tau steps and predicts the entries the
upcoming tau-step window needs), and the lag between a selection and the
interval it serves (0 when every chunk is already in HBM; 1 for the host tier,
where the chunks of interval i are fetched while interval i-1 decodes --
the handbook page's "asynchronously prefetched").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblsa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile liblsa_oracle.so with gcc -O2 (no fast-math), OpenMP."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def configure(L):
    """Declare the C signatures on a loaded oracle library."""
    i64, vp, dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
    L.oracle_index_logits.argtypes = [vp, vp, i64, i64, i64, i64, vp]
    L.oracle_index_logits.restype = None
    L.oracle_index_scores.argtypes = [vp, i64, ctypes.c_float, vp]
    L.oracle_index_scores.restype = None
    L.oracle_topk_i64.argtypes = [vp, i64, i64, i64, vp]
    L.oracle_topk_i64.restype = ctypes.c_int
    L.oracle_topk_f64.argtypes = [vp, i64, i64, i64, vp]
    L.oracle_topk_f64.restype = ctypes.c_int
    L.oracle_gather_attend.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, dbl,
                                       vp, vp, vp, vp, i64]
    L.oracle_gather_attend.restype = ctypes.c_int
    L.oracle_topk_tokens.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp]
    L.oracle_topk_tokens.restype = ctypes.c_int
    L.oracle_fetch_chunks.argtypes = [vp, i64, vp, vp, vp, i64, i64, i64, i64, i64, i64]
    L.oracle_fetch_chunks.restype = ctypes.c_int
    L.oracle_pool_assign.argtypes = [vp, vp, i64, vp, i64, i64, i64, vp, vp]
    L.oracle_pool_assign.restype = ctypes.c_int
    L.oracle_threshold_i64.argtypes = [vp, i64, i64, i64, i64, vp, vp]
    L.oracle_threshold_i64.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = configure(ctypes.CDLL(_LIB_PATH))
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def index_logits(q_idx: np.ndarray, k_idx: np.ndarray) -> np.ndarray:
    """q_idx int8 [B][nq][d_idx], k_idx int8 [B][C][d_idx] -> int64 [B*nq][C]."""
    q_idx, k_idx = _c(q_idx, np.int8), _c(k_idx, np.int8)
    B, nq, d_idx = q_idx.shape
    Bk, C, dk = k_idx.shape
    assert Bk == B and dk == d_idx
    out = np.empty((B * nq, C), dtype=np.int64)
    lib().oracle_index_logits(q_idx.ctypes.data, k_idx.ctypes.data, B, nq, C, d_idx, out.ctypes.data)
    return out


def index_scores(logits: np.ndarray, alpha: float) -> np.ndarray:
    """sigmoid(alpha * logit), argument formed in fp32, sigmoid in fp64."""
    logits = _c(logits, np.int64)
    out = np.empty(logits.shape, dtype=np.float64)
    lib().oracle_index_scores(logits.ctypes.data, logits.size, ctypes.c_float(alpha), out.ctypes.data)
    return out


def topk_chunks(keys: np.ndarray, k: int) -> np.ndarray:
    """keys [R][C] (int or float) -> int32 [R][k], ascending chunk ids of the
    first k chunks in the order (key descending, index ascending)."""
    R, C = keys.shape
    out = np.empty((R, k), dtype=np.int32)
    if np.issubdtype(keys.dtype, np.integer):
        keys = _c(keys, np.int64)
        rc = lib().oracle_topk_i64(keys.ctypes.data, R, C, k, out.ctypes.data)
    else:
        keys = _c(keys, np.float64)
        rc = lib().oracle_topk_f64(keys.ctypes.data, R, C, k, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle top-k rejected its arguments (rc={rc}, k={k}, C={C})")
    return out


def gather_attend(q: np.ndarray, kv: np.ndarray, chunk_ids: np.ndarray, ctx_len: np.ndarray, Hkv: int,
                  sm_scale: float, slots: np.ndarray | None = None, T: int = 64,
                  want_weights: bool = False, counts: np.ndarray | None = None,
                  seg_kv: np.ndarray | None = None, seg_len: np.ndarray | None = None,
                  tok: np.ndarray | None = None, tok_counts: np.ndarray | None = None):
    """q uint16 (bf16 bits) [B][Hq][d]; kv uint16 [B][C_store][2][Hkv][T][d];
    chunk_ids int32 [B][k]; ctx_len int [B]; slots int32 [B][k] or None;
    counts int32 [B] (entries used per request) or None; seg_kv uint16
    [B][2][Hkv][S_max][d] with seg_len int [B] (resident tokens) or None;
    tok int32 [B][k_tok] (list positions j*T + t of the tokens to use) with
    tok_counts int32 [B] or None: None uses every token of the used entries.
    Returns out float64 [B][Hq][d] (and weights [B][Hq][k*T + S_max] if asked)."""
    q, kv = _c(q, np.uint16), _c(kv, np.uint16)
    chunk_ids = _c(chunk_ids, np.int32)
    ctx = _c(ctx_len, np.int32)
    B, Hq, d = q.shape
    assert kv.shape[0] == B and kv.shape[2] == 2 and kv.shape[3] == Hkv and kv.shape[4] == T and kv.shape[5] == d
    C_store = kv.shape[1]
    k = chunk_ids.shape[1]
    sl = 0
    if slots is not None:
        slots = _c(slots, np.int32)
        assert slots.shape == chunk_ids.shape
        sl = slots.ctypes.data
    cn = 0
    if counts is not None:
        counts = _c(counts, np.int32)
        cn = counts.ctypes.data
    sg, sgl, S_max = 0, 0, 0
    if seg_kv is not None:
        seg_kv = _c(seg_kv, np.uint16)
        seg_len = _c(seg_len, np.int32)
        assert seg_kv.shape[0] == B and seg_kv.shape[1] == 2 and seg_kv.shape[2] == Hkv and seg_kv.shape[4] == d
        sg, sgl, S_max = seg_kv.ctypes.data, seg_len.ctypes.data, seg_kv.shape[3]
    tk, tkc, k_tok = 0, 0, 0
    if tok is not None:
        tok = _c(tok, np.int32)
        assert tok.shape[0] == B
        tk, k_tok = tok.ctypes.data, tok.shape[1]
        if tok_counts is not None:
            tok_counts = _c(tok_counts, np.int32)
            tkc = tok_counts.ctypes.data
    out = np.empty((B, Hq, d), dtype=np.float64)
    wts = np.empty((B, Hq, k * T + S_max), dtype=np.float64) if want_weights else None
    rc = lib().oracle_gather_attend(q.ctypes.data, kv.ctypes.data, C_store, chunk_ids.ctypes.data, sl, cn,
                                    ctx.ctypes.data, sg, sgl, S_max, B, Hq, Hkv, d, k, T, float(sm_scale),
                                    out.ctypes.data,
                                    wts.ctypes.data if wts is not None else 0, tk, tkc, k_tok)
    if rc != 0:
        raise ValueError(f"oracle attention rejected its arguments (rc={rc})")
    return (out, wts) if want_weights else out


def topk_tokens(scores: np.ndarray, chunk_ids: np.ndarray, ctx_len: np.ndarray, k_tok: int,
                counts: np.ndarray | None = None, T: int = 64):
    """Token selection inside the recalled chunks: scores float32 [B][k*T]
    (list position j*T + t = token t of chunk_ids[b][j]) -> (tok int32
    [B][k_tok], ascending usable positions padded with -1; tok_counts int32
    [B])."""
    scores = _c(scores, np.float32)
    chunk_ids = _c(chunk_ids, np.int32)
    ctx = _c(ctx_len, np.int32)
    B, k = chunk_ids.shape
    assert scores.shape == (B, k * T)
    cn = 0
    if counts is not None:
        counts = _c(counts, np.int32)
        cn = counts.ctypes.data
    tok = np.empty((B, k_tok), dtype=np.int32)
    tc = np.empty(B, dtype=np.int32)
    rc = lib().oracle_topk_tokens(scores.ctypes.data, chunk_ids.ctypes.data, cn, ctx.ctypes.data, B, k, T, k_tok,
                                  tok.ctypes.data, tc.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle token selection rejected its arguments (rc={rc})")
    return tok, tc


def threshold_chunks(logits: np.ndarray, k_max: int, logit_threshold: int = 0):
    """Chunks with logit > logit_threshold, at most k_max (the first k_max of
    the order (logit descending, index ascending)): (ids int32 [R][k_max]
    padded with -1, counts int32 [R])."""
    logits = _c(logits, np.int64)
    R, C = logits.shape
    ids = np.empty((R, k_max), dtype=np.int32)
    counts = np.empty(R, dtype=np.int32)
    rc = lib().oracle_threshold_i64(logits.ctypes.data, R, C, int(logit_threshold), k_max, ids.ctypes.data,
                                    counts.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle threshold selection rejected its arguments (rc={rc})")
    return ids, counts


def fetch_chunks(host_kv: np.ndarray, chunk_ids: np.ndarray, P: int, slots: np.ndarray | None = None,
                 pool: np.ndarray | None = None, skip_negative_slots: bool = False) -> np.ndarray:
    """host_kv uint16 [B][C][2][Hkv][T][d] -> pool uint16 [B][P][2][Hkv][T][d]."""
    host_kv = _c(host_kv, np.uint16)
    B, C, _, Hkv, T, d = host_kv.shape
    chunk_ids = _c(chunk_ids, np.int32)
    k = chunk_ids.shape[1]
    if pool is None:
        pool = np.zeros((B, P, 2, Hkv, T, d), dtype=np.uint16)
    sl = 0
    if slots is not None:
        slots = _c(slots, np.int32)
        if skip_negative_slots:  # a delta fetch: entries with slot -1 copy nothing
            for b in range(B):
                keep = slots[b] >= 0
                if keep.any():
                    fetch_chunks(host_kv[b:b + 1], chunk_ids[b:b + 1, keep], P, slots[b:b + 1, keep],
                                 pool=pool[b:b + 1] if pool is not None else None)
            return pool
        sl = slots.ctypes.data
    rc = lib().oracle_fetch_chunks(host_kv.ctypes.data, C, chunk_ids.ctypes.data, sl, pool.ctypes.data, P, B,
                                   Hkv, d, k, T)
    if rc != 0:
        raise ValueError("oracle fetch: chunk id or slot out of range")
    return pool


def pool_assign(prev_ids, prev_slots, new_ids: np.ndarray, P: int):
    """Delta-fetch slots: (new_slots, fetch_slots) int32 [B][k]; prev_* may be
    None for the first selection."""
    new_ids = _c(new_ids, np.int32)
    B, k = new_ids.shape
    if prev_ids is None:
        n_prev, pi, ps = 0, 0, 0
    else:
        prev_ids, prev_slots = _c(prev_ids, np.int32), _c(prev_slots, np.int32)
        n_prev, pi, ps = prev_ids.shape[1], prev_ids.ctypes.data, prev_slots.ctypes.data
    new_slots = np.empty((B, k), dtype=np.int32)
    fetch_slots = np.empty((B, k), dtype=np.int32)
    rc = lib().oracle_pool_assign(pi, ps, n_prev, new_ids.ctypes.data, B, k, P, new_slots.ctypes.data,
                                  fetch_slots.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle pool assignment failed (rc={rc})")
    return new_slots, fetch_slots


# ---- decode schedule ----------------------------------------------------

def is_reselect_step(t: int, tau: int = 64) -> bool:
    """Re-selection happens at steps t = 0 (mod tau)."""
    return t % tau == 0


def selection_for_step(t: int, tau: int = 64, lag: int = 0) -> int:
    """Index of the re-selection whose chunks step t attends over:
    interval i = t // tau uses the selection made at step (i - lag) * tau,
    clamped at the first selection."""
    return max(t // tau - lag, 0)


def select(q_idx: np.ndarray, k_idx: np.ndarray, k: int, alpha: float):
    """One re-selection: logits, scores and the kept chunk ids per row."""
    logits = index_logits(q_idx, k_idx)
    scores = index_scores(logits, alpha)
    ids = topk_chunks(logits, k)
    return logits, scores, ids
