"""Build the HIP library liblsa.so in-tree for gfx950 (hipcc, no torch), and
the measurement-only libtileread.so that bench.py uses to state the HBM read
ceiling of the attention's access pattern."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "liblsa.so")
SOURCES = ["lsa_abi.hip", "index_score.hip", "topk_chunks.hip", "gather_attend.hip", "fetch_pull.hip",
           "pool_assign.hip", "noalloc.hip", "check_ids.hip", "fetch_staged.hip"]
MEASURE_SOURCES = ["measure/tile_read.hip"]
MEASURE_LIB_PATH = os.path.join(HERE, "libtileread.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are kept out of the device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # MFMA results in VGPRs: the softmax rescale works on the accumulators
                # with VALU ops, which cannot read AGPRs directly
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _run(cmd, verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature and says so; drop that line.
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return msg


def _compile(sources, out_path: str, verbose: bool) -> str:
    """Compile every source to an object in parallel, then link the shared
    library; the objects live in a temporary directory."""
    srcs = [os.path.join(CSRC, s) for s in sources]
    with tempfile.TemporaryDirectory(prefix="lsa_build_") as tmpdir:
        objs = [os.path.join(tmpdir, f"{i}_{os.path.basename(s)}.o") for i, s in enumerate(srcs)]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as pool:
            futs = [pool.submit(_run, [HIPCC, *DEVICE_FLAGS, "-c", "-o", o, src], verbose)
                    for src, o in zip(srcs, objs)]
            for f in futs:
                f.result()
        tmp = out_path + ".tmp"
        _run([HIPCC, *DEVICE_FLAGS, "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, out_path)
    return out_path


def build(verbose: bool = False) -> str:
    _compile(MEASURE_SOURCES, MEASURE_LIB_PATH, verbose)
    return _compile(SOURCES, LIB_PATH, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
