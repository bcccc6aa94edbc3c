"""ctypes binding of liblsa.so (the C ABI in include/lsa.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
the library.  PyTorch supplies device memory and streams; outputs that the
caller does not pass are allocated with ``torch.empty`` on the device of the
inputs.  There is no fallback: if the library is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblsa.so")
_lib = None

LSA_OK = 0
STATUS_NAMES = {0: "LSA_OK", 1: "LSA_ERR_INVALID_ARGUMENT", 2: "LSA_ERR_UNSUPPORTED", 3: "LSA_ERR_WORKSPACE",
                4: "LSA_ERR_HIP"}
CHUNK_TOKENS = 64

# Every symbol include/lsa.h declares.
EXPORTS = ("lsa_status_string", "lsa_last_error", "lsa_index_score", "lsa_topk_chunks", "lsa_threshold_chunks",
           "lsa_topk_tokens", "lsa_topk_tokens_workspace_size", "lsa_gather_attend_workspace_size", "lsa_gather_attend_default_splits",
           "lsa_gather_attend", "lsa_gather_attend_tokens", "lsa_fetch_chunks", "lsa_fetch_chunks_staged",
           "lsa_fetch_chunks_pull",
           "lsa_pool_assign", "lsa_set_tuning", "lsa_get_tuning", "lsa_gather_attend_noalloc", "lsa_check_ids")

# bytes of the static split-partials buffer of lsa_gather_attend_noalloc (LSA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 8 << 20

# lsa_tuning knobs (include/lsa.h)
TUNE_ATTEND_DEPTH = 0
TUNE_SCORE_MFMA_MIN_NQ = 1
TUNE_TOPK_STREAM_MIN_C = 2
TUNE_TOPK_SPLIT_MIN_N = 3
TUNE_TOPK_SPLIT_SLICES = 4
TUNE_FETCH_LANES = 5
TUNE_KNOBS = {"attend_depth": TUNE_ATTEND_DEPTH, "score_mfma_min_nq": TUNE_SCORE_MFMA_MIN_NQ,
              "topk_stream_min_c": TUNE_TOPK_STREAM_MIN_C, "topk_split_min_n": TUNE_TOPK_SPLIT_MIN_N,
              "topk_split_slices": TUNE_TOPK_SPLIT_SLICES, "fetch_lanes": TUNE_FETCH_LANES}


class LsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load liblsa.so (built by ``lookahead_chunk_sparse_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"HIP library {path} is not built; run __graft_entry__.build() "
                          "or python lookahead_chunk_sparse_amd/build.py")
    L = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.lsa_status_string.argtypes = [ctypes.c_int]
    L.lsa_status_string.restype = ctypes.c_char_p
    L.lsa_last_error.argtypes = []
    L.lsa_last_error.restype = ctypes.c_char_p
    L.lsa_index_score.argtypes = [vp, vp, i32, i32, i32, i32, f32, vp, vp, vp]
    L.lsa_index_score.restype = ctypes.c_int
    L.lsa_topk_chunks.argtypes = [vp, i32, i32, i32, vp, vp]
    L.lsa_topk_chunks.restype = ctypes.c_int
    L.lsa_gather_attend_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    L.lsa_gather_attend_workspace_size.restype = sz
    L.lsa_gather_attend_default_splits.argtypes = [i32, i32, i32]
    L.lsa_gather_attend_default_splits.restype = i32
    L.lsa_threshold_chunks.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    L.lsa_threshold_chunks.restype = ctypes.c_int
    L.lsa_gather_attend.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp, sz,
                                    i32, vp, vp]
    L.lsa_gather_attend.restype = ctypes.c_int
    L.lsa_gather_attend_noalloc.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                            i32, vp, vp]
    L.lsa_gather_attend_noalloc.restype = ctypes.c_int
    L.lsa_topk_tokens.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    L.lsa_topk_tokens.restype = ctypes.c_int
    L.lsa_topk_tokens_workspace_size.argtypes = [i32, i32, i32]
    L.lsa_topk_tokens_workspace_size.restype = sz
    L.lsa_gather_attend_tokens.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                           i32, f32, vp, sz, i32, vp, vp]
    L.lsa_gather_attend_tokens.restype = ctypes.c_int
    L.lsa_fetch_chunks.argtypes = [vp, i64, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp]
    L.lsa_fetch_chunks.restype = ctypes.c_int
    L.lsa_fetch_chunks_staged.argtypes = [vp, i64, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp, i64, vp, vp]
    L.lsa_fetch_chunks_staged.restype = ctypes.c_int
    L.lsa_fetch_chunks_pull.argtypes = [vp, i64, vp, vp, vp, i64, i32, i32, i32, i32, i32, vp]
    L.lsa_fetch_chunks_pull.restype = ctypes.c_int
    L.lsa_pool_assign.argtypes = [vp, vp, i32, vp, i32, i32, i64, vp, vp, vp]
    L.lsa_pool_assign.restype = ctypes.c_int
    L.lsa_check_ids.argtypes = [vp, vp, vp, i32, i32, i64, i64, vp, vp]
    L.lsa_check_ids.restype = ctypes.c_int
    L.lsa_set_tuning.argtypes = [ctypes.c_int, i32]
    L.lsa_set_tuning.restype = ctypes.c_int
    L.lsa_get_tuning.argtypes = [ctypes.c_int]
    L.lsa_get_tuning.restype = i32
    _lib = L
    return L


def _check(status: int):
    if status != LSA_OK:
        raise LsaError(status, load_library().lsa_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, name: str, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")


def _on(t: torch.Tensor, device: torch.device, name: str):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's tensors on {device}")


def _out(t, dtype, shape, device, name: str) -> torch.Tensor:
    """An output buffer: a new device tensor when t is None, else t checked
    for dtype, exact shape, device and contiguity (the kernels write exactly
    that many elements there)."""
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, dtype, name)
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    _on(t, device, name)
    return t


def lsa_set_tuning(knob, value: int):
    """Override a tuning knob (a name of TUNE_KNOBS or its number) for the
    calling thread; 0 drops the override."""
    _check(load_library().lsa_set_tuning(TUNE_KNOBS.get(knob, knob), int(value)))


def lsa_get_tuning(knob) -> int:
    """The value of a tuning knob in effect for the calling thread (0: chosen
    per call)."""
    v = int(load_library().lsa_get_tuning(TUNE_KNOBS.get(knob, knob)))
    if v < 0:
        raise LsaError(1, f"unknown tuning knob {knob!r}")
    return v


class tuning:
    """Context manager: tuning overrides for the calling thread, e.g.
    ``with tuning(attend_depth=3): ...``; the previous overrides (or their
    absence) come back on exit."""

    def __init__(self, **knobs):
        unknown = set(knobs) - set(TUNE_KNOBS)
        if unknown:
            raise ValueError(f"unknown tuning knobs {sorted(unknown)}")
        self.knobs = knobs
        self.saved = {}

    def __enter__(self):
        L = load_library()
        for name, v in self.knobs.items():
            # the thread's own override, if any, is what must come back: read
            # it by dropping the override and comparing with the value in effect
            knob = TUNE_KNOBS[name]
            before = int(L.lsa_get_tuning(knob))
            _check(L.lsa_set_tuning(knob, 0))
            base = int(L.lsa_get_tuning(knob))
            self.saved[name] = before if before != base else 0
            lsa_set_tuning(knob, v)
        return self

    def __exit__(self, *exc):
        for name, v in self.saved.items():
            lsa_set_tuning(TUNE_KNOBS[name], v)
        return False


def lsa_index_score(q_idx: torch.Tensor, k_idx: torch.Tensor, alpha: float, logits=None, scores=None,
                    want_scores: bool = True, stream=None):
    """q_idx int8 [B][nq][d_idx], k_idx int8 [B][C][d_idx] (device).
    Returns (logits int32 [B][nq][C], scores fp32 [B][nq][C] or None)."""
    _need(q_idx, torch.int8, "q_idx", 3)
    _need(k_idx, torch.int8, "k_idx", 3)
    B, nq, d_idx = q_idx.shape
    C = k_idx.shape[1]
    if k_idx.shape[0] != B or k_idx.shape[2] != d_idx:
        raise ValueError(f"k_idx shape {tuple(k_idx.shape)} does not match q_idx {tuple(q_idx.shape)}")
    dev = k_idx.device
    _on(q_idx, dev, "q_idx")
    logits = _out(logits, torch.int32, (B, nq, C), dev, "logits")
    if scores is not None or want_scores:
        scores = _out(scores, torch.float32, (B, nq, C), dev, "scores")
    _check(load_library().lsa_index_score(_ptr(q_idx), _ptr(k_idx), B, nq, C, d_idx, alpha, _ptr(logits),
                                          _ptr(scores), _stream(stream)))
    return logits, scores


def lsa_topk_chunks(logits: torch.Tensor, k: int, chunk_ids=None, stream=None) -> torch.Tensor:
    """logits int32 [..., C] (rows = all leading dims) -> int32 [..., k], ascending."""
    _need(logits, torch.int32, "logits")
    C = logits.shape[-1]
    R = logits.numel() // C
    chunk_ids = _out(chunk_ids, torch.int32, (*logits.shape[:-1], k), logits.device, "chunk_ids")
    _check(load_library().lsa_topk_chunks(_ptr(logits), R, C, k, _ptr(chunk_ids), _stream(stream)))
    return chunk_ids


def lsa_threshold_chunks(logits: torch.Tensor, k_max: int, logit_threshold: int = 0, chunk_ids=None, counts=None,
                         stream=None):
    """logits int32 [..., C] -> (chunk_ids int32 [..., k_max] padded with -1,
    counts int32 [...]): chunks with logit > logit_threshold, at most k_max."""
    _need(logits, torch.int32, "logits")
    C = logits.shape[-1]
    R = logits.numel() // C
    chunk_ids = _out(chunk_ids, torch.int32, (*logits.shape[:-1], k_max), logits.device, "chunk_ids")
    counts = _out(counts, torch.int32, logits.shape[:-1], logits.device, "counts")
    _check(load_library().lsa_threshold_chunks(_ptr(logits), R, C, int(logit_threshold), k_max, _ptr(chunk_ids),
                                               _ptr(counts), _stream(stream)))
    return chunk_ids, counts


def lsa_topk_tokens_workspace_size(B: int, k: int, k_tok: int) -> int:
    n = load_library().lsa_topk_tokens_workspace_size(B, k, k_tok)
    if n == ctypes.c_size_t(-1).value:
        raise LsaError(1, "invalid sizes for lsa_topk_tokens_workspace_size")
    return int(n)


def alloc_topk_tokens_workspace(B: int, k: int, k_tok: int, device="cuda"):
    """A workspace tensor for lsa_topk_tokens (None when none is used)."""
    n = lsa_topk_tokens_workspace_size(B, k, k_tok)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=device)


def lsa_topk_tokens(scores: torch.Tensor, chunk_ids: torch.Tensor, ctx_len: torch.Tensor, k_tok: int,
                    counts: torch.Tensor | None = None, tok=None, tok_counts=None, workspace="auto", stream=None):
    """scores fp32 [B][k*64] over the list positions of the recalled chunks
    chunk_ids int32 [B][k] -> (tok int32 [B][k_tok] ascending positions padded
    with -1, tok_counts int32 [B]).  workspace: a tensor from
    alloc_topk_tokens_workspace, None (one workgroup per request) or "auto"
    (allocated here when one is used)."""
    _need(scores, torch.float32, "scores", 2)
    _need(chunk_ids, torch.int32, "chunk_ids", 2)
    _need(ctx_len, torch.int32, "ctx_len", 1)
    B, k = chunk_ids.shape
    dev = scores.device
    if tuple(scores.shape) != (B, k * CHUNK_TOKENS):
        raise ValueError(f"scores shape {tuple(scores.shape)} is not [B][k*64] = [{B}][{k * CHUNK_TOKENS}]")
    if tuple(ctx_len.shape) != (B,):
        raise ValueError("ctx_len must have one entry per request")
    _on(chunk_ids, dev, "chunk_ids")
    _on(ctx_len, dev, "ctx_len")
    if counts is not None:
        _need(counts, torch.int32, "counts", 1)
        if tuple(counts.shape) != (B,):
            raise ValueError("counts must have one entry per request")
        _on(counts, dev, "counts")
    tok = _out(tok, torch.int32, (B, k_tok), dev, "tok")
    tok_counts = _out(tok_counts, torch.int32, (B,), dev, "tok_counts")
    if isinstance(workspace, str):
        workspace = alloc_topk_tokens_workspace(B, k, k_tok, device=dev)
    elif workspace is not None:
        _need(workspace, torch.uint8, "workspace", 1)
        _on(workspace, dev, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().lsa_topk_tokens(_ptr(scores), _ptr(chunk_ids), _ptr(counts), _ptr(ctx_len), B, k, k_tok,
                                          _ptr(tok), _ptr(tok_counts), _ptr(workspace), ws_bytes, _stream(stream)))
    return tok, tok_counts


def lsa_gather_attend_workspace_size(B: int, Hq: int, Hkv: int, d: int, k: int, n_split: int = 0) -> int:
    n = load_library().lsa_gather_attend_workspace_size(B, Hq, Hkv, d, k, n_split)
    if n == ctypes.c_size_t(-1).value:
        raise LsaError(1, load_library().lsa_last_error().decode())
    return int(n)


def lsa_gather_attend_default_splits(B: int, Hkv: int, k: int) -> int:
    return int(load_library().lsa_gather_attend_default_splits(B, Hkv, k))


def alloc_workspace(B: int, Hq: int, Hkv: int, d: int, k: int, n_split: int = 0, device="cuda"):
    """A workspace tensor for lsa_gather_attend (None when none is needed)."""
    n = lsa_gather_attend_workspace_size(B, Hq, Hkv, d, k, n_split)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def lsa_gather_attend(q: torch.Tensor, kv: torch.Tensor, chunk_ids: torch.Tensor, ctx_len: torch.Tensor,
                      sm_scale: float | None = None, slots: torch.Tensor | None = None, workspace=None,
                      n_split: int = 0, out=None, counts: torch.Tensor | None = None,
                      seg_kv: torch.Tensor | None = None, seg_len: torch.Tensor | None = None,
                      stream=None, tok: torch.Tensor | None = None,
                      tok_counts: torch.Tensor | None = None) -> torch.Tensor:
    """q bf16 [B][Hq][d]; kv bf16 [B][C_store][2][Hkv][64][d]; chunk_ids int32 [B][k];
    ctx_len int32 [B]; slots int32 [B][k] or None; counts int32 [B] or None;
    seg_kv bf16 [B][2][Hkv][S_max][d] (resident window) with seg_len int32 [B],
    or None.  With tok int32 [B][k_tok] (list positions, as lsa_topk_tokens
    writes them) and tok_counts int32 [B] or None, the call is
    lsa_gather_attend_tokens.  Returns fp32 [B][Hq][d]."""
    _need(q, torch.bfloat16, "q", 3)
    _need(kv, torch.bfloat16, "kv", 6)
    _need(chunk_ids, torch.int32, "chunk_ids", 2)
    _need(ctx_len, torch.int32, "ctx_len", 1)
    B, Hq, d = q.shape
    _, C_store, two, Hkv, T, dk = kv.shape
    k = chunk_ids.shape[1]
    dev = q.device
    if kv.shape[0] != B or two != 2 or T != CHUNK_TOKENS or dk != d:
        raise ValueError(f"kv shape {tuple(kv.shape)} does not match q {tuple(q.shape)}")
    if chunk_ids.shape[0] != B or tuple(ctx_len.shape) != (B,):
        raise ValueError("chunk_ids / ctx_len batch size mismatch")
    for t, name in ((kv, "kv"), (chunk_ids, "chunk_ids"), (ctx_len, "ctx_len")):
        _on(t, dev, name)
    if slots is not None:
        _need(slots, torch.int32, "slots", 2)
        if tuple(slots.shape) != tuple(chunk_ids.shape):
            raise ValueError("slots must have the shape of chunk_ids")
        _on(slots, dev, "slots")
    if counts is not None:
        _need(counts, torch.int32, "counts", 1)
        if tuple(counts.shape) != (B,):
            raise ValueError("counts must have one entry per request")
        _on(counts, dev, "counts")
    S_max = 0
    if seg_kv is not None:
        _need(seg_kv, torch.bfloat16, "seg_kv", 5)
        if seg_len is None:
            raise ValueError("seg_kv needs seg_len")
        _need(seg_len, torch.int32, "seg_len", 1)
        if seg_kv.shape[0] != B or seg_kv.shape[1] != 2 or seg_kv.shape[2] != Hkv or seg_kv.shape[4] != d:
            raise ValueError(f"seg_kv shape {tuple(seg_kv.shape)} does not match [B][2][Hkv][S_max][d]")
        if tuple(seg_len.shape) != (B,):
            raise ValueError("seg_len must have one entry per request")
        _on(seg_kv, dev, "seg_kv")
        _on(seg_len, dev, "seg_len")
        S_max = seg_kv.shape[3]
    k_tok = 0
    if tok is not None:
        _need(tok, torch.int32, "tok", 2)
        if tok.shape[0] != B:
            raise ValueError("tok batch size mismatch")
        _on(tok, dev, "tok")
        k_tok = tok.shape[1]
        if tok_counts is not None:
            _need(tok_counts, torch.int32, "tok_counts", 1)
            if tuple(tok_counts.shape) != (B,):
                raise ValueError("tok_counts must have one entry per request")
            _on(tok_counts, dev, "tok_counts")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if workspace is None:
        entries = k if tok is None else (k_tok + CHUNK_TOKENS - 1) // CHUNK_TOKENS
        workspace = alloc_workspace(B, Hq, Hkv, d, entries, n_split, device=dev)
    else:
        _need(workspace, torch.uint8, "workspace", 1)
        _on(workspace, dev, "workspace")
    out = _out(out, torch.float32, (B, Hq, d), dev, "out")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if tok is not None:
        _check(load_library().lsa_gather_attend_tokens(_ptr(q), _ptr(kv), C_store, _ptr(chunk_ids), _ptr(slots),
                                                       _ptr(counts), _ptr(ctx_len), _ptr(tok), _ptr(tok_counts),
                                                       k_tok, _ptr(seg_kv), _ptr(seg_len), S_max, B, Hq, Hkv, d, k,
                                                       sm_scale, _ptr(workspace), ws_bytes, n_split, _ptr(out),
                                                       _stream(stream)))
        return out
    _check(load_library().lsa_gather_attend(_ptr(q), _ptr(kv), C_store, _ptr(chunk_ids), _ptr(slots),
                                            _ptr(counts), _ptr(ctx_len), _ptr(seg_kv), _ptr(seg_len), S_max, B, Hq,
                                            Hkv, d, k, sm_scale,
                                            _ptr(workspace), ws_bytes,
                                            n_split, _ptr(out), _stream(stream)))
    return out


def lsa_gather_attend_noalloc(q: torch.Tensor, kv: torch.Tensor, chunk_ids: torch.Tensor, ctx_len: torch.Tensor,
                              out: torch.Tensor, sm_scale: float | None = None, slots: torch.Tensor | None = None,
                              n_split: int = 0, counts: torch.Tensor | None = None,
                              seg_kv: torch.Tensor | None = None, seg_len: torch.Tensor | None = None,
                              stream=None) -> torch.Tensor:
    """lsa_gather_attend with the split partials in the library's static
    device buffer: no workspace, and the caller passes `out` (fp32
    [B][Hq][d]), so nothing is allocated on the call's path."""
    _need(q, torch.bfloat16, "q", 3)
    _need(kv, torch.bfloat16, "kv", 6)
    _need(chunk_ids, torch.int32, "chunk_ids", 2)
    _need(ctx_len, torch.int32, "ctx_len", 1)
    B, Hq, d = q.shape
    _, C_store, two, Hkv, T, dk = kv.shape
    k = chunk_ids.shape[1]
    dev = q.device
    if kv.shape[0] != B or two != 2 or T != CHUNK_TOKENS or dk != d:
        raise ValueError(f"kv shape {tuple(kv.shape)} does not match q {tuple(q.shape)}")
    if chunk_ids.shape[0] != B or tuple(ctx_len.shape) != (B,):
        raise ValueError("chunk_ids / ctx_len batch size mismatch")
    for t, name in ((kv, "kv"), (chunk_ids, "chunk_ids"), (ctx_len, "ctx_len")):
        _on(t, dev, name)
    if slots is not None:
        _need(slots, torch.int32, "slots", 2)
        if tuple(slots.shape) != tuple(chunk_ids.shape):
            raise ValueError("slots must have the shape of chunk_ids")
        _on(slots, dev, "slots")
    if counts is not None:
        _need(counts, torch.int32, "counts", 1)
        if tuple(counts.shape) != (B,):
            raise ValueError("counts must have one entry per request")
        _on(counts, dev, "counts")
    S_max = 0
    if seg_kv is not None:
        _need(seg_kv, torch.bfloat16, "seg_kv", 5)
        if seg_len is None:
            raise ValueError("seg_kv needs seg_len")
        _need(seg_len, torch.int32, "seg_len", 1)
        if seg_kv.shape[0] != B or seg_kv.shape[1] != 2 or seg_kv.shape[2] != Hkv or seg_kv.shape[4] != d:
            raise ValueError(f"seg_kv shape {tuple(seg_kv.shape)} does not match [B][2][Hkv][S_max][d]")
        if tuple(seg_len.shape) != (B,):
            raise ValueError("seg_len must have one entry per request")
        _on(seg_kv, dev, "seg_kv")
        _on(seg_len, dev, "seg_len")
        S_max = seg_kv.shape[3]
    if out is None:
        raise ValueError("lsa_gather_attend_noalloc needs the caller's out buffer")
    out = _out(out, torch.float32, (B, Hq, d), dev, "out")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    _check(load_library().lsa_gather_attend_noalloc(_ptr(q), _ptr(kv), C_store, _ptr(chunk_ids), _ptr(slots),
                                                    _ptr(counts), _ptr(ctx_len), _ptr(seg_kv), _ptr(seg_len), S_max,
                                                    B, Hq, Hkv, d, k, sm_scale, n_split, _ptr(out),
                                                    _stream(stream)))
    return out


def lsa_gather_attend_tokens(q: torch.Tensor, kv: torch.Tensor, chunk_ids: torch.Tensor, ctx_len: torch.Tensor,
                             tok: torch.Tensor, tok_counts: torch.Tensor | None = None, **kw) -> torch.Tensor:
    """Attention over the listed tokens of the recalled chunks (tok int32
    [B][k_tok] list positions, tok_counts int32 [B] or None); the other
    arguments as for lsa_gather_attend.  Returns fp32 [B][Hq][d]."""
    return lsa_gather_attend(q, kv, chunk_ids, ctx_len, tok=tok, tok_counts=tok_counts, **kw)


def _check_pool(host_kv: torch.Tensor, pool_kv: torch.Tensor):
    """The pool must hold chunks of the host store's shape: [B][P][2][Hkv][64][d]
    with the host's B, Hkv and d, in device memory; the host store on the host."""
    B, C, two, Hkv, T, d = host_kv.shape
    if two != 2 or T != CHUNK_TOKENS:
        raise ValueError(f"host_kv shape {tuple(host_kv.shape)} is not [B][C][2][Hkv][64][d]")
    if host_kv.is_cuda:
        raise ValueError("host_kv must be pinned host memory")
    pb, P, ptwo, pH, pT, pd = pool_kv.shape
    if (pb, ptwo, pH, pT, pd) != (B, 2, Hkv, T, d):
        raise ValueError(f"pool_kv shape {tuple(pool_kv.shape)} does not match [B][P][2][Hkv][64][d] = "
                         f"[{B}][P][2][{Hkv}][64][{d}]")
    if not pool_kv.is_cuda:
        raise ValueError("pool_kv must be device memory")


def lsa_fetch_chunks(host_kv: torch.Tensor, host_chunk_ids: torch.Tensor, pool_kv: torch.Tensor,
                     host_slots: torch.Tensor | None = None, stream=None, done=None):
    """host_kv pinned bf16 [B][C][2][Hkv][64][d]; host ids int32 [B][k] (CPU);
    pool_kv device bf16 [B][P][2][Hkv][64][d].  `done`: torch.cuda.Event or None."""
    _need(host_kv, torch.bfloat16, "host_kv", 6)
    _need(pool_kv, torch.bfloat16, "pool_kv", 6)
    _need(host_chunk_ids, torch.int32, "host_chunk_ids", 2)
    if host_chunk_ids.is_cuda or (host_slots is not None and host_slots.is_cuda):
        raise ValueError("chunk ids and slots for the fetch must be host tensors")
    B, C, _, Hkv, T, d = host_kv.shape
    P = pool_kv.shape[1]
    k = host_chunk_ids.shape[1]
    _check_pool(host_kv, pool_kv)
    if host_chunk_ids.shape[0] != B:
        raise ValueError("host_chunk_ids batch size mismatch")
    if host_slots is not None:
        _need(host_slots, torch.int32, "host_slots", 2)
        if tuple(host_slots.shape) != tuple(host_chunk_ids.shape):
            raise ValueError("host_slots must have the shape of host_chunk_ids")
    ev = 0
    if done is not None:
        ev = done.cuda_event if hasattr(done, "cuda_event") else int(done)
    _check(load_library().lsa_fetch_chunks(_ptr(host_kv), C, _ptr(host_chunk_ids), _ptr(host_slots),
                                           _ptr(pool_kv), P, B, Hkv, d, k, _stream(stream), ev))


def alloc_fetch_staging(host_kv: torch.Tensor, stage_chunks: int, device="cuda"):
    """The two staging buffers of lsa_fetch_chunks_staged, each stage_chunks
    chunks of host_kv's shape: (pinned host bf16, device bf16)
    [stage_chunks][2][Hkv][64][d]."""
    _, _, two, Hkv, T, d = host_kv.shape
    shape = (int(stage_chunks), two, Hkv, T, d)
    return (torch.empty(shape, dtype=torch.bfloat16, pin_memory=True),
            torch.empty(shape, dtype=torch.bfloat16, device=device))


def lsa_fetch_chunks_staged(host_kv: torch.Tensor, host_chunk_ids: torch.Tensor, pool_kv: torch.Tensor,
                            host_staging: torch.Tensor, dev_staging: torch.Tensor,
                            host_slots: torch.Tensor | None = None, stream=None, done=None):
    """lsa_fetch_chunks through staging buffers (alloc_fetch_staging): the
    host gathers the chunks to copy, which cross the link in large copies and
    are scattered into the pool on the device.  Waits on the host for its
    copies (so not under graph capture)."""
    _need(host_kv, torch.bfloat16, "host_kv", 6)
    _need(pool_kv, torch.bfloat16, "pool_kv", 6)
    _need(host_chunk_ids, torch.int32, "host_chunk_ids", 2)
    _need(host_staging, torch.bfloat16, "host_staging", 5)
    _need(dev_staging, torch.bfloat16, "dev_staging", 5)
    if host_chunk_ids.is_cuda or (host_slots is not None and host_slots.is_cuda):
        raise ValueError("chunk ids and slots for the fetch must be host tensors")
    B, C, _, Hkv, T, d = host_kv.shape
    P = pool_kv.shape[1]
    k = host_chunk_ids.shape[1]
    n_stage = host_staging.shape[0]
    if tuple(host_staging.shape[1:]) != tuple(host_kv.shape[2:]) or tuple(dev_staging.shape) != tuple(host_staging.shape):
        raise ValueError("host_staging and dev_staging must both be [stage_chunks][2][Hkv][64][d] of host_kv's chunks")
    _check_pool(host_kv, pool_kv)
    if host_chunk_ids.shape[0] != B:
        raise ValueError("host_chunk_ids batch size mismatch")
    if host_slots is not None:
        _need(host_slots, torch.int32, "host_slots", 2)
        if tuple(host_slots.shape) != tuple(host_chunk_ids.shape):
            raise ValueError("host_slots must have the shape of host_chunk_ids")
    if host_staging.is_cuda or not dev_staging.is_cuda:
        raise ValueError("host_staging must be pinned host memory and dev_staging device memory")
    ev = 0
    if done is not None:
        ev = done.cuda_event if hasattr(done, "cuda_event") else int(done)
    _check(load_library().lsa_fetch_chunks_staged(_ptr(host_kv), C, _ptr(host_chunk_ids), _ptr(host_slots),
                                                  _ptr(pool_kv), P, B, Hkv, d, k, _ptr(host_staging),
                                                  _ptr(dev_staging), n_stage, _stream(stream), ev))


def lsa_fetch_chunks_pull(host_kv: torch.Tensor, chunk_ids: torch.Tensor, pool_kv: torch.Tensor,
                          slots: torch.Tensor | None = None, grid: int = 0, stream=None):
    """host_kv pinned bf16 [B][C][2][Hkv][64][d]; chunk_ids (and slots) device
    int32 [B][k]; pool_kv device bf16 [B][P][2][Hkv][64][d]."""
    _need(host_kv, torch.bfloat16, "host_kv", 6)
    _need(pool_kv, torch.bfloat16, "pool_kv", 6)
    _need(chunk_ids, torch.int32, "chunk_ids", 2)
    if not chunk_ids.is_cuda or (slots is not None and not slots.is_cuda):
        raise ValueError("chunk ids and slots for the pull fetch must be device tensors")
    B, C, _, Hkv, T, d = host_kv.shape
    P = pool_kv.shape[1]
    k = chunk_ids.shape[1]
    _check_pool(host_kv, pool_kv)
    if chunk_ids.shape[0] != B:
        raise ValueError("chunk_ids batch size mismatch")
    _on(chunk_ids, pool_kv.device, "chunk_ids")
    if slots is not None:
        _need(slots, torch.int32, "slots", 2)
        if tuple(slots.shape) != tuple(chunk_ids.shape):
            raise ValueError("slots must have the shape of chunk_ids")
        _on(slots, pool_kv.device, "slots")
    _check(load_library().lsa_fetch_chunks_pull(_ptr(host_kv), C, _ptr(chunk_ids), _ptr(slots), _ptr(pool_kv), P,
                                                B, Hkv, d, k, grid, _stream(stream)))


def lsa_check_ids(chunk_ids: torch.Tensor, C_ctx: int, C_store: int | None = None, slots=None, counts=None,
                  result=None, stream=None):
    """Check a chunk list (int32 [B][k], with slots [B][k] and counts [B] if
    given) before it is attended over: ids in [0, C_ctx), store positions in
    [0, C_store) (C_store defaults to C_ctx), nothing listed twice, counts in
    [0, k].  Waits for the stream; raises LsaError naming the first offending
    entry."""
    _need(chunk_ids, torch.int32, "chunk_ids", 2)
    B, k = chunk_ids.shape
    dev = chunk_ids.device
    if slots is not None:
        _need(slots, torch.int32, "slots", 2)
        if tuple(slots.shape) != (B, k):
            raise ValueError("slots must have the shape of chunk_ids")
        _on(slots, dev, "slots")
    if counts is not None:
        _need(counts, torch.int32, "counts", 1)
        if tuple(counts.shape) != (B,):
            raise ValueError("counts must have one entry per request")
        _on(counts, dev, "counts")
    result = _out(result, torch.int32, (4,), dev, "result")
    _check(load_library().lsa_check_ids(_ptr(chunk_ids), _ptr(slots), _ptr(counts), B, k, int(C_ctx),
                                        int(C_ctx if C_store is None else C_store), _ptr(result), _stream(stream)))


def lsa_pool_assign(prev_ids, prev_slots, new_ids: torch.Tensor, P: int, new_slots=None, fetch_slots=None,
                    stream=None):
    """Slots for S_new given S_prev (ids [B][n_prev] at slots [B][n_prev], or
    None for the first selection).  Returns (new_slots, fetch_slots), int32 [B][k]."""
    _need(new_ids, torch.int32, "new_ids", 2)
    B, k = new_ids.shape
    dev = new_ids.device
    n_prev = 0
    if prev_ids is not None:
        _need(prev_ids, torch.int32, "prev_ids", 2)
        _need(prev_slots, torch.int32, "prev_slots", 2)
        n_prev = prev_ids.shape[1]
        if prev_ids.shape[0] != B or tuple(prev_slots.shape) != tuple(prev_ids.shape):
            raise ValueError("prev_ids / prev_slots shapes do not match")
        _on(prev_ids, dev, "prev_ids")
        _on(prev_slots, dev, "prev_slots")
    new_slots = _out(new_slots, torch.int32, (B, k), dev, "new_slots")
    fetch_slots = _out(fetch_slots, torch.int32, (B, k), dev, "fetch_slots")
    _check(load_library().lsa_pool_assign(_ptr(prev_ids), _ptr(prev_slots), n_prev, _ptr(new_ids), B, k, P,
                                          _ptr(new_slots), _ptr(fetch_slots), _stream(stream)))
    return new_slots, fetch_slots
