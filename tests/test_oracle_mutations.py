"""The pins have teeth: plausible mistakes planted in copies of the oracle's
source (a dropped term, a wrong sign, index or operand, a reversed tie-break,
an off-by-one mask, ...) each make at least one pin fail.  The oracle itself
is untouched; every mutant is compiled on the CPU into a temporary library."""
import ctypes
import importlib.util
import os
import subprocess

import pytest

import test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lsa_oracle.c")
INIT = os.path.join(ROOT, "oracle", "__init__.py")

# (name, text in lsa_oracle.c, replacement, pins expected to notice)
MUTATIONS = [
    ("logits drop last term", "for (int64_t i = 0; i < d_idx; ++i) acc +=", "for (int64_t i = 0; i < d_idx - 1; ++i) acc +=",
     ["test_logits_closed_form", "test_logits_vs_numpy_integer_matmul"]),
    ("logits reversed key", "acc += (int64_t)qv[i] * (int64_t)kv[i];", "acc += (int64_t)qv[i] * (int64_t)kv[d_idx - 1 - i];",
     ["test_logits_closed_form", "test_logits_vs_numpy_integer_matmul"]),
    ("sigmoid sign", "scores[j] = 1.0 / (1.0 + exp(-(double)x));", "scores[j] = 1.0 / (1.0 + exp((double)x));",
     ["test_scores_closed_form_and_expit"]),
    ("sigmoid argument not fp32", "volatile float x = alpha * xl; /* one single-precision product */",
     "volatile double x = (double)alpha * (double)logits[j];", ["test_scores_argument_is_fp32_product"]),
    ("top-k tie to higher index", "if (row[c2] > row[c] || (row[c2] == row[c] && c2 < c)) ++before;\n            keep[c] = before < k;",
     "if (row[c2] > row[c] || (row[c2] == row[c] && c2 > c)) ++before;\n            keep[c] = before < k;",
     ["test_topk_vs_brute_force", "test_topk_closed_form"]),
    ("top-k ascending order", "if (row[c2] > row[c] || (row[c2] == row[c] && c2 < c)) ++before;\n            keep[c] = before < k;",
     "if (row[c2] < row[c] || (row[c2] == row[c] && c2 < c)) ++before;\n            keep[c] = before < k;",
     ["test_topk_vs_brute_force", "test_topk_closed_form"]),
    ("GQA head mapping", "const int64_t g = h / group;", "const int64_t g = h % Hkv;",
     ["test_all_chunks_equals_dense_sdpa", "test_convex_hull_and_gqa_as_mha"]),
    ("softmax scale dropped", "z[e] = dot * sm_scale;", "z[e] = dot;",
     ["test_attention_closed_forms", "test_all_chunks_equals_dense_sdpa"]),
    ("context mask off by one", "if (c * T + t < (int64_t)ctx_len[b]) {", "if (c * T + t <= (int64_t)ctx_len[b]) {",
     ["test_all_chunks_equals_dense_sdpa", "test_single_token_returns_its_value"]),
    ("normalisation dropped", "for (int64_t i = 0; i < d; ++i) o[i] /= l;", "",
     ["test_attention_closed_forms", "test_all_chunks_equals_dense_sdpa"]),
    ("V read from K", "const uint16_t* V = kv + (b * C_store + p) * chunk + (1 * Hkv + g) * tile;",
     "const uint16_t* V = kv + (b * C_store + p) * chunk + (0 * Hkv + g) * tile;",
     ["test_attention_closed_forms", "test_all_chunks_equals_dense_sdpa"]),
    ("slots ignored", "const int64_t p = slots ? slots[b * k + j] : c;\n                const uint16_t* K = kv",
     "const int64_t p = c;\n                const uint16_t* K = kv", ["test_chunk_order_and_slots"]),
    ("counts ignored", "const int64_t kb = counts ? (counts[b] < k ? counts[b] : k) : k;", "const int64_t kb = k;",
     ["test_attention_counts_truncate_lists", "test_segment_joins_chunks_in_one_softmax"]),
    ("segment V from K", "const uint16_t* V = seg_kv + ((b * 2 + 1) * Hkv + g) * S_max * d;",
     "const uint16_t* V = seg_kv + ((b * 2 + 0) * Hkv + g) * S_max * d;", ["test_segment_joins_chunks_in_one_softmax"]),
    ("fetch wrong source", "memcpy(pool_kv + (b * P + p) * chunk, host_kv + (b * C + c) * chunk,",
     "memcpy(pool_kv + (b * P + p) * chunk, host_kv + (b * C + j) * chunk,", ["test_fetch_is_a_byte_copy"]),
    ("delta slots never kept", "if (found >= 0) {", "if (0) {",
     ["test_pool_assign_closed_form", "test_pool_assign_chain_keeps_pool_consistent"]),
    ("delta slots reuse held", "while (next < P && held[next]) ++next;", "",
     ["test_pool_assign_closed_form", "test_pool_assign_chain_keeps_pool_consistent"]),
    ("threshold inclusive", "for (int64_t c = 0; c < C; ++c) above += row[c] > thr;",
     "for (int64_t c = 0; c < C; ++c) above += row[c] >= thr;",
     ["test_threshold_vs_brute_force", "test_threshold_zero_is_sigmoid_half"]),
    ("token tie to higher position", "if (usable[p2] && (row[p2] > row[p] || (row[p2] == row[p] && p2 < p))) ++before;",
     "if (usable[p2] && (row[p2] > row[p] || (row[p2] == row[p] && p2 > p))) ++before;",
     ["test_token_select_vs_brute_force", "test_token_select_special_cases"]),
    ("token usable ignores context",
     "usable[p] = j < kb && (int64_t)chunk_ids[b * k + j] * T + t < (int64_t)ctx_len[b];", "usable[p] = j < kb;",
     ["test_token_select_vs_brute_force", "test_token_select_special_cases"]),
    ("token list keeps tokens past context", "if (c * T + t >= (int64_t)ctx_len[b]) continue;", "",
     ["test_token_attention_equals_sdpa_over_listed_tokens"]),
    ("token list ignores entry count", "if (pos < 0 || pos >= kb * T) continue;", "if (pos < 0 || pos >= k * T) continue;",
     ["test_token_attention_equals_sdpa_over_listed_tokens"]),
]


def _mutant_module(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation '{name}': pattern must occur exactly once"
    c_path = tmp_path / "mutant.c"
    c_path.write_text(src.replace(old, new))
    so_path = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-fno-fast-math",
                           "-ffp-contract=off", str(c_path), "-o", str(so_path), "-lm"])
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{abs(hash(name))}", INIT)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._lib = mod.configure(ctypes.CDLL(str(so_path)))
    return mod


def _run_pin(fn, mod, synth_lib):
    """Run one pin (all its parametrisations) against the mutant; True if it fails."""
    import inspect
    marks = getattr(fn, "pytestmark", [])
    params = [None]
    for m in marks:
        if m.name == "parametrize":
            argname, values = m.args[0], m.args[1]
            params = [(argname, v) for v in values]
    for p in params:
        kwargs = {}
        sig = inspect.signature(fn).parameters
        if "oracle_lib" in sig:
            kwargs["oracle_lib"] = mod
        if "synth_lib" in sig:
            kwargs["synth_lib"] = synth_lib
        if p is not None:
            names = [n.strip() for n in p[0].split(",")]
            vals = p[1] if len(names) > 1 else (p[1],)
            kwargs.update(dict(zip(names, vals)))
        try:
            fn(**kwargs)
        except (AssertionError, ValueError):
            return True
    return False


@pytest.mark.parametrize("name,old,new,pin_names", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, synth_lib, name, old, new, pin_names):
    mod = _mutant_module(tmp_path, name, old, new)
    caught = [p for p in pin_names if _run_pin(getattr(pins, p), mod, synth_lib)]
    assert caught, f"no pin noticed the planted mistake '{name}'"


def test_unmutated_oracle_passes_the_same_pins(tmp_path, synth_lib):
    """Control: the same harness on the unchanged source finds nothing."""
    mod = _mutant_module(tmp_path, "control", "/* 1. logits[b*nq + r][c]", "/* 1. logits[b*nq + r][c]")
    names = sorted({p for m in MUTATIONS for p in m[3]})
    assert [p for p in names if _run_pin(getattr(pins, p), mod, synth_lib)] == []
