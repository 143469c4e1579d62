"""The host-only C-ABI validation (config checks, weight specification, device check, the
kernel-level entry points' argument checks) built with AddressSanitizer and run on the CPU:
tests/asan/host_validation.cpp drives it over the presets and a seeded sweep of malformed
configs. The library source that holds the validation is compiled with host-side ASan (the
device code is compiled as usual); the other objects are those of the normal build."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    noise = "is not a recognized feature for this target"
    out = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    return r.returncode, out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not installed")
def test_host_validation_under_asan():
    import sys
    sys.path.insert(0, os.path.join(ROOT, "flow_matching_vla_amd"))
    import build as B
    os.makedirs(OUT, exist_ok=True)
    os.makedirs(B.BUILD, exist_ok=True)
    # the kernels' objects of the normal build (compiled here when absent or older than a source)
    objs = []
    for src in B.SOURCES:
        if src == "fm_api.cpp":
            continue
        o = os.path.join(B.BUILD, os.path.splitext(src)[0] + ".o")
        deps = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)]
        if not os.path.exists(o) or os.path.getmtime(o) < max(os.path.getmtime(d) for d in deps):
            o = B._compile(src)
        objs.append(o)
    api = os.path.join(OUT, "fm_api_asan.o")
    rc, out = _run([HIPCC, *B.FLAGS, "-O1", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-c", os.path.join(B.CSRC, "fm_api.cpp"), "-o", api])
    assert rc == 0, out
    lib = os.path.join(OUT, "libfmvla_asan.so")
    rc, out = _run([CLANGXX, "-shared", "-fsanitize=address", "-shared-libsan", api, *objs, "-L/opt/rocm/lib",
                    "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    assert rc == 0, out
    drv = os.path.join(OUT, "libhost_validation.so")
    rc, out = _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address", "-shared-libsan",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "asan", "host_validation.cpp"), lib, "-Wl,-rpath," + OUT, "-o", drv])
    assert rc == 0, out
    rt = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(rt):
        import glob
        rt = (glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so") or [""])[0]
    assert os.path.exists(rt), "ASan runtime not found"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:exitcode=23")
    code = ("import ctypes, sys; ctypes.CDLL(%r, mode=ctypes.RTLD_GLOBAL); "
            "sys.exit(ctypes.CDLL(%r).fm_host_validation())" % (lib, drv))
    rc, out = _run([sys.executable, "-c", code], env=env, timeout=300)
    assert "AddressSanitizer" not in out, out[-4000:]
    assert rc == 0, out[-4000:]
    assert "0 with an undefined status" in out, out[-2000:]
