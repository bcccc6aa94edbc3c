"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

  * The oracle and the seeded input generator (plain C, gcc), driven by
    tests/c/sanitize_oracle.c over every function and its edge cases, with
    leak detection on.
  * The host side of the C ABI (argument validation, size queries, tuning
    knobs, the DMA fetch's run coalescing), driven by tests/c/sanitize_abi.cpp
    and built from the library's own sources with the sanitizers on the host
    pass only (hipcc -Xarch_host); the device code is built as usual but not
    run: no GPU is used.

  * The staged fetch's host gather threads (fetch_staged.hip), driven by
    tests/c/sanitize_host_pool.cpp under ThreadSanitizer and, separately,
    AddressSanitizer with UndefinedBehaviorSanitizer.

Any sanitizer report aborts the program (-fno-sanitize-recover=all;
ThreadSanitizer: halt_on_error)."""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lookahead_chunk_sparse_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(exe, env_extra, timeout=300):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=timeout, env=env)
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_and_generator_under_sanitizers(tmp_path):
    exe = tmp_path / "sanitize_oracle"
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", *SAN, "-Wall", "-Wextra", "-Werror",
                           os.path.join(ROOT, "tests", "c", "sanitize_oracle.c"),
                           os.path.join(ROOT, "oracle", "lsa_oracle.c"), os.path.join(ROOT, "synth", "synth.c"),
                           "-o", str(exe), "-lm"])
    r = _run(exe, {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "OMP_NUM_THREADS": "4"})
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "sanitize_oracle: ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_host_side_under_sanitizers(tmp_path):
    import lookahead_chunk_sparse_amd.build as B  # the library's own source list and device flags

    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]
    flags = [*B.DEVICE_FLAGS, "-O1", "-g", *host_san]
    sources = [os.path.join(CSRC, s) for s in B.SOURCES] + [os.path.join(ROOT, "tests", "c", "sanitize_abi.cpp")]
    objs = [str(tmp_path / f"{i}.o") for i in range(len(sources))]

    def compile_one(src, obj):
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as pool:
        for f in [pool.submit(compile_one, s, o) for s, o in zip(sources, objs)]:
            f.result()
    exe = tmp_path / "sanitize_abi"
    r = subprocess.run([HIPCC, *flags, *objs, "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # the HIP runtime keeps allocations until exit; leaks are not this test's subject
    r = _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "sanitize_abi: ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
@pytest.mark.parametrize("kind", ["thread", "address"])
def test_staged_fetch_host_threads_under_sanitizers(tmp_path, kind):
    """The staged fetch's host gather threads (fetch_staged.hip: the worker
    pool and its non-temporal chunk copies), driven by
    tests/c/sanitize_host_pool.cpp: ThreadSanitizer for the pool's hand-off
    and its callers on several threads; AddressSanitizer and
    UndefinedBehaviorSanitizer for the copies.  No GPU is used."""
    import lookahead_chunk_sparse_amd.build as B

    san = ["-fsanitize=thread"] if kind == "thread" else SAN
    host_san = [f for flag in san for f in ("-Xarch_host", flag)]
    flags = [*B.DEVICE_FLAGS, "-O1", "-g", *host_san]
    sources = [os.path.join(CSRC, "fetch_staged.hip"), os.path.join(ROOT, "tests", "c", "sanitize_host_pool.cpp")]
    objs = [str(tmp_path / f"{i}.o") for i in range(len(sources))]
    for src, obj in zip(sources, objs):
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
    exe = tmp_path / f"sanitize_host_pool_{kind}"
    r = subprocess.run([HIPCC, *flags, *objs, "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = {"TSAN_OPTIONS": "halt_on_error=1:second_deadlock_stack=1"} if kind == "thread" else \
        {"ASAN_OPTIONS": "detect_leaks=0"}
    r = _run(exe, env)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "sanitize_host_pool: ok" in r.stdout
