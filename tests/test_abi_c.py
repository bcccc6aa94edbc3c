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


def test_c_decode_driver_compiles(tmp_path):
    """tests/c/decode_interval.c, the plain-C client the GPU suite runs,
    compiles warning-free against the header and links against liblsa.so and
    the HIP runtime alone."""
    import lookahead_chunk_sparse_amd as lsa
    exe = tmp_path / "decode_interval"
    libdir = os.path.dirname(lsa.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                           os.path.join(ROOT, "tests", "c", "decode_interval.c"), "-o", str(exe),
                           "-L", libdir, "-llsa", "-L", "/opt/rocm/lib", "-lamdhip64",
                           f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage:" in r.stderr  # argument check only: no HIP call is made


def test_c_threaded_client_compiles(tmp_path):
    """tests/c/threaded_calls.c (run by the GPU suite) compiles warning-free
    with pthreads against the header; it is not run here, since every path
    of it calls the GPU."""
    import lookahead_chunk_sparse_amd as lsa
    libdir = os.path.dirname(lsa.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-pthread", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                           os.path.join(ROOT, "tests", "c", "threaded_calls.c"), "-o", str(tmp_path / "threaded_calls"),
                           "-L", libdir, "-llsa", "-L", "/opt/rocm/lib", "-lamdhip64",
                           f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"])
