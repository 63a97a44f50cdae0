"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

* The oracle (oracle/oracle.c), built with gcc and -fsanitize=address,
  undefined, driven through every entry point on small heads and edge-case
  masks by tests/native/sanitize_oracle.c.
* The C-ABI layer (csrc/api.hip) compiled with the same sanitizers on its
  host side (hipcc, host flags only), linked with tests/native/
  sanitize_abi.cpp, which stubs the kernel launchers, the HIP queries and
  the registration of api.hip's one device array, and calls every entry
  point with refused and accepted arguments.

Either run fails on the first sanitizer report (no recovery) or on a wrong
return code.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd, r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_oracle")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-fast-math",
          "-ffp-contract=off", "-fexcess-precision=standard",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(NATIVE, "sanitize_oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV)
    assert "0 failures" in r.stdout, r.stdout
    assert "Sanitizer" not in r.stderr, r.stderr[-4000:]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="needs hipcc and the ROCm clang++")
def test_c_abi_host_layer_under_address_and_undefined_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROOT, "reduced_vocab_nvfp4_amd", "csrc")]
    flags = ["-x", "hip", "-O1", "-g", "-std=c++17",
             "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]
    objs = []
    # api.hip declares a device array, so it is built with its device code
    # (the sanitizers apply to the host side only); the driver is host code
    for src, target in (
            (os.path.join(ROOT, "reduced_vocab_nvfp4_amd", "csrc", "api.hip"),
             ["--offload-arch=gfx950"]),
            (os.path.join(NATIVE, "sanitize_abi.cpp"),
             ["--offload-host-only"])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *target, *flags, *inc, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "sanitize_abi")
    _run([CLANGXX, "-fsanitize=address,undefined", *objs, "-o", exe])
    r = _run([exe], env=ENV)
    assert "0 failures" in r.stdout, r.stdout
    assert "Sanitizer" not in r.stderr, r.stderr[-4000:]
