"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU only).

* The C oracle is rebuilt with gcc's ASan + UBSan (no OpenMP: one thread) and the oracle pins and
  the benchmark's CPU-leg tests run against it in a child process with the ASan runtime preloaded.
  The NumPy brute-force comparisons of the largest pins are left out (they spend their time in
  NumPy, not in the oracle); every oracle entry point is still called.
* The library's C ABI (argument validation, workspace layouts and sizes, status strings: the
  host code of api.hip) is rebuilt with clang's host ASan + UBSan (-Xarch_host, so the device
  code is unchanged), linked with the normally built kernel objects, and the C-ABI tests run
  against it.  No kernel is launched (there is no GPU here).
A sanitizer report makes the child fail (UBSan halts on the first error, ASan on any).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

ORACLE_SRC = os.path.join(ROOT, "oracle", "spark_oracle.c")
API_SRC = os.path.join(ROOT, "block_sparse_attention_score_amd", "csrc", "api.hip")
CLANG_ASAN = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def run_child(args, extra_env):
    env = dict(os.environ, **SAN_ENV, **extra_env)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", *args],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = r.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libspark_oracle_san.so")
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
         "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
         "-fsanitize=address,undefined",
         ORACLE_SRC, "-o", lib, "-lm"])
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    out = run_child(["tests/test_oracle_pins.py", "tests/test_bench_cpu.py",
                     "-k", "not test_oracle_matches_brute_force"],
                    {"LD_PRELOAD": asan, "SPARK_ORACLE_LIB": lib})
    print(out.strip().splitlines()[-1])


@pytest.mark.skipif(not os.path.exists(CLANG_ASAN), reason="clang ASan runtime not found")
def test_c_abi_under_asan_ubsan(tmp_path):
    from block_sparse_attention_score_amd import build as b

    objs = [os.path.join(b.BUILD, s.replace(".hip", ".o")) for s in b.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        b.build()
    api_o, lib = str(tmp_path / "api_san.o"), str(tmp_path / "libspark_attn_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    subprocess.check_call(
        [HIPCC, f"--offload-arch={b.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", *san,
         "-Xarch_host", "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", b.INCLUDE, "-I", b.CSRC, "-c", API_SRC, "-o", api_o],
        stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    subprocess.check_call([HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *san, "-Xarch_host",
                           "-shared-libsan", api_o, *objs, "-o", lib],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    out = run_child(["tests/test_abi_cpu.py"], {"LD_PRELOAD": CLANG_ASAN, "SPARK_ATTN_LIB": lib})
    print(out.strip().splitlines()[-1])
