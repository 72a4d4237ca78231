"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code,
on the CPU only.

- The C oracle (oracle/kda_oracle.c), built by gcc with -fsanitize=address,
  undefined, runs its pins and planted-mistake tests.
- The C ABI's host side (kda_api.hip: argument validation, size queries, the
  state handle, error strings), with the host pass of hipcc sanitized and the
  kernels' objects linked in unchanged, runs the ABI tests (every call there
  returns before touching a GPU).

Each runs in a child process with the matching runtime preloaded (gcc's
libasan + libubsan, or clang's ASan runtime, which carries the UBSan
handlers), and every sanitizer report is fatal (-fno-sanitize-recover=all).
Leak checking is off: the interpreter itself keeps its allocations to exit.
No GPU code is built with a sanitizer.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _child(mode, lib, preload, tmp):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitized_run.py"), mode,
                          lib], cwd=str(tmp), env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "passed" in out and "failed" not in out, out[-4000:]
    for marker in ("AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in out, out[-4000:]
    return out


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc has no {name}")
    return path


def test_oracle_under_asan_ubsan(tmp_path):
    from oracle.build import build

    lib = build(out=str(tmp_path / "libkda_oracle_san.so"), extra_flags=("-g", *SAN))
    preload = _gcc_runtime("libasan.so") + ":" + _gcc_runtime("libubsan.so")
    out = _child("oracle", lib, preload, tmp_path)
    print(out.strip().splitlines()[-1])


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("no clang ASan runtime under /opt/rocm/llvm")
    return hits[-1]


def test_abi_host_code_under_asan_ubsan(tmp_path):
    from gated_delta_rule_83_amd import build as B

    objs = [os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES
            if s != "kda_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api_obj = str(tmp_path / "kda_api_san.o")
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]  # host pass only
    cmd = [B.HIPCC, *B.CFLAGS, "-O1", "-g", *host_san, "-c",
           os.path.join(B.CSRC, "kda_api.hip"), "-o", api_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    lib = str(tmp_path / "libkda_san.so")
    # the sanitizer symbols resolve against the preloaded runtime at load time
    res = subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", api_obj, *objs,
                          "-o", lib], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    out = _child("abi", lib, _clang_asan_runtime(), tmp_path)
    print(out.strip().splitlines()[-1])
