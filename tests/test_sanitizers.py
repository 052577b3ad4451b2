"""Sanitizer builds on the CPU (no GPU needed):

- the fp64 oracle (gcc, AddressSanitizer + UndefinedBehaviorSanitizer) driven
  over small shapes: ragged chunks, masks, an empty sequence, a single step,
  GQA, both backward storage modes, the per-key-channel gate, the conv update;
- the C ABI's host code (gdn_api.hip: validation, route choice, workspace and
  saved-record layouts, the no-allocation entry point's size check) built by
  hipcc with the sanitizers on the host side only, its kernel launchers
  replaced by stubs that read both ends of every workspace / checkpoint region
  they are handed, driven over a grid of shapes, dtypes, kernel families and
  the saved record with the buffers allocated at exactly the queried sizes.

Either program exits non-zero on the first failed expectation or sanitizer
report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "gdn_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1"), timeout=300)
    assert "ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    flags = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I" + os.path.join(ROOT, "include")]
    srcs = [(os.path.join(ROOT, "linear_attention_recurrence_fwd_amd", "csrc", "gdn_api.hip"), []),
            (os.path.join(SAN, "host_stubs.cpp"), ["-x", "hip"]),
            (os.path.join(SAN, "abi_driver.cpp"), ["-x", "hip"])]
    procs, objs = [], []
    for src, extra in srcs:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, *extra, "-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, err[-4000:]
    exe = str(tmp_path / "abi_san")
    # host link with the sanitizer runtimes (no device code is sanitized)
    _run([HIPCC, "-fsanitize=address,undefined", "-fno-gpu-sanitize", "--offload-arch=gfx950", *objs, "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.startswith("ok:")
