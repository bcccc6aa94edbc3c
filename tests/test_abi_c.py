"""include/lsa.h compiles as plain C11, links against liblsa.so, and a C
program gets the documented status codes back (validation paths only: no
GPU needed)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_against_header(tmp_path):
    import lookahead_chunk_sparse_amd as lsa
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(lsa.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", str(exe),
                           "-L", libdir, "-llsa", f"-Wl,-rpath,{libdir}"])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check: ok" in r.stdout
