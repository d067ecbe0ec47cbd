"""Address and undefined-behaviour sanitizers on host code (no GPU).

* The C ABI's host paths: tests/abi_sanitize.cpp drives the planner over a
  grid of shapes, dtypes, depths and options, the argument validation of both
  entry points, the models, the variant table and the status strings.  The
  translation units holding that host code (pgemm_abi.cpp, hazard_demo.hip)
  and the driver are rebuilt with the sanitizers on the host side only (each
  flag behind -Xarch_host: no device code is instrumented); the kernel
  translation units are the library's own objects.
* The oracle's C code: tests/oracle_sanitize.c runs every entry point on
  exact-size buffers under gcc's sanitizers.

A report from either sanitizer aborts the program and fails the test.
"""
import os
import shutil
import subprocess

import pytest

from software_pipelined_tiled_loop_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SAN = []
for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
    HOST_SAN += ["-Xarch_host", flag]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), r.stdout[-4000:])
    return r.stdout


def test_abi_host_paths_under_sanitizers(tmp_path):
    try:
        hipcc = build._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    csrc = build.CSRC
    build.generate_tables()
    flags = [f for f in build.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g", "-I" + build.GEN_DIR]
    objs = []
    for name in ("kern_f32.hip", "kern_f16.hip", "kern_bf16.hip", "kern_i8.hip"):
        built = os.path.join(build.BUILD_DIR, name + ".o")
        if os.path.exists(built) and os.path.getmtime(built) >= os.path.getmtime(os.path.join(csrc, name)):
            objs.append(built)  # the library's object of this kernel file
        else:
            objs.append(build._compile(os.path.join(csrc, name)))
    for src in (os.path.join(csrc, "pgemm_abi.cpp"), os.path.join(csrc, "hazard_demo.hip"),
                os.path.join(ROOT, "tests", "abi_sanitize.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([hipcc] + flags + HOST_SAN + ["-x", "hip", "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_sanitize")
    _run([hipcc, "--offload-arch=" + build.ARCH] + HOST_SAN + objs + ["-o", exe])
    out = _run([exe], env=ENV, timeout=600)
    assert out.strip().splitlines()[-1].startswith("OK"), out[-2000:]


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    _run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "tests", "oracle_sanitize.c"), "-o", exe, "-lm"])
    out = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1"), timeout=600)
    assert out.strip().splitlines()[-1].startswith("OK"), out[-2000:]
