"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two builds, each run in a subprocess with the sanitizer runtime preloaded
(the Python interpreter itself is not instrumented) and failing on the first
report:
  * the fp64 oracle (oracle.c, gcc -fsanitize=address,undefined), running
    every pin of test_oracle_pins that the mutation check uses;
  * the library's host half -- swa_abi.cpp's argument checks, block-mask and
    workspace sizing -- compiled by hipcc with the sanitizers on the host pass
    only (each -fsanitize= after -Xarch_host; the device code is the normal
    build), linked with the library's other objects, running the ABI host
    tests (tests/test_abi_host.py) against it.
No GPU is used: the ABI host tests stop at the host checks.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
PKG = os.path.join(ROOT, "sparse_masked_transformer_amd")
ENV = dict(ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")


def _runtime(pattern):
    found = sorted(glob.glob(pattern))
    if not found:
        pytest.skip(f"no sanitizer runtime matching {pattern}")
    return found[-1]


def _run(cmd, preload, extra_env=None):
    env = dict(os.environ, **ENV, LD_PRELOAD=preload, **(extra_env or {}))
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_and_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-shared", "-fPIC", os.path.join(ROOT, "oracle", "oracle.c"), "-o", so, "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    code = (f"import sys; sys.path[:0] = [{ROOT!r}, {TESTS!r}]\n"
            "import oracle, test_oracle_mutations as mu\n"
            f"with oracle.using_library({so!r}):\n"
            "    for name, pin in mu.all_pins():\n"
            "        pin()\n"
            "print('pins passed')\n")
    out = _run([sys.executable, "-c", code], asan)
    assert "pins passed" in out


def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, PKG)
    try:
        import build
    finally:
        sys.path.pop(0)
    if not glob.glob(os.path.join(build.BUILD, "*.o")):
        build.build()
    src = os.path.join(build.CSRC, "swa_abi.cpp")
    obj = str(tmp_path / "swa_abi_san.o")
    san = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([build.HIPCC] + build.COMMON + san + ["-c", src, "-o", obj], check=True,
                   capture_output=True)
    # (the library's objects: one per compiled source, named <source>.o)
    others = [o for o in glob.glob(os.path.join(build.BUILD, "*.o"))
              if o.endswith((".hip.o", ".cpp.o")) and not o.endswith("swa_abi.cpp.o")]
    so = str(tmp_path / "libswa_san.so")
    subprocess.run([build.HIPCC, f"--offload-arch={build.ARCH}", "-shared", "-fPIC", "-o", so, obj] + others,
                   check=True, capture_output=True)
    asan = _runtime("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    out = _run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                os.path.join(TESTS, "test_abi_host.py")], asan, {"SWA_ABI_LIBRARY": so})
    assert " passed" in out and " failed" not in out
