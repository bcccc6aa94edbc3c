"""The product path computes only in liblsa.so: the Python package marshals
arguments and orders calls, imports nothing from the oracle, calls no torch
routine that could stand in for a kernel, and refuses to load without the
built library (no CPU fallback).  Static checks plus one load attempt; no
GPU needed."""
import ast
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "lookahead_chunk_sparse_amd")

# torch / numpy compute that would amount to doing a step of the path on the
# side: matmuls, reductions over scores, selection, activations, attention
FORBIDDEN_CALLS = {
    "matmul", "mm", "bmm", "baddbmm", "einsum", "softmax", "log_softmax", "sigmoid", "expit", "topk", "sort",
    "argsort", "kthvalue", "scaled_dot_product_attention", "dot", "tensordot", "exp", "logsumexp", "argmax",
}


def _package_modules():
    return [os.path.join(PKG, f) for f in sorted(os.listdir(PKG)) if f.endswith(".py")]


@pytest.mark.parametrize("path", _package_modules(), ids=os.path.basename)
def test_no_oracle_import(path):
    tree = ast.parse(open(path).read(), path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            assert not any(a.name.split(".")[0] == "oracle" for a in node.names), path
        elif isinstance(node, ast.ImportFrom):
            assert (node.module or "").split(".")[0] != "oracle", path


@pytest.mark.parametrize("path", _package_modules(), ids=os.path.basename)
def test_no_compute_fallback(path):
    tree = ast.parse(open(path).read(), path)
    bad = []
    for node in ast.walk(tree):
        if isinstance(node, ast.Call):
            f = node.func
            name = f.attr if isinstance(f, ast.Attribute) else f.id if isinstance(f, ast.Name) else None
            if name in FORBIDDEN_CALLS:
                bad.append(f"{os.path.basename(path)}:{node.lineno} {name}()")
    assert not bad, bad


def test_missing_library_fails_loudly(tmp_path):
    import lookahead_chunk_sparse_amd._binding as b
    saved = b._lib
    try:
        b._lib = None
        with pytest.raises(ImportError, match="not built"):
            b.load_library(str(tmp_path / "liblsa.so"))
    finally:
        b._lib = saved
