"""Host-side sanitizer builds, for the CPU tier.

- The oracle (oracle/msa_oracle.c) built with gcc's AddressSanitizer and
  UndefinedBehaviorSanitizer, with leak detection, and driven through every
  function on valid and rejected inputs by tests/sanitize/oracle_driver.c.
- libmsa.so with its host code (argument validation, workspace sizing, grid
  and launch set-up) built with clang's AddressSanitizer and
  UndefinedBehaviorSanitizer (device code is compiled as usual), and the
  C-ABI validation tests (tests/test_abi.py, no GPU needed) run against it.

Any sanitizer report fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    subprocess.run(["gcc", "-g", "-O1", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "msa_oracle.c"),
                    "-o", str(exe), "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "oracle_driver: ok" in res.stdout
    assert "Sanitizer" not in res.stderr, res.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC) or _asan_runtime() is None, reason="hipcc or clang's ASan runtime absent")
def test_host_layer_under_address_and_undefined_sanitizers(tmp_path):
    srcs = sorted(glob.glob(os.path.join(ROOT, "block_sparse_long_score_amd", "csrc", "*.hip")))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "block_sparse_long_score_amd", "csrc")]
    procs, objs = [], []
    for src in srcs:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", src, "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT, text=True))
    for p, src in zip(procs, srcs):
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, f"{os.path.basename(src)}:\n{out}"
    lib = str(tmp_path / "libmsa_sanitized.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib], check=True)
    preload = " ".join(x for x in (_asan_runtime(), os.environ.get("LD_PRELOAD", "")) if x)
    env = dict(os.environ, MSA_LIBRARY=lib, LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "passed" in res.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
