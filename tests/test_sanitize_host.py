"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The HIP sources are compiled again into a temporary directory with the sanitizers on the
host side only (each -fsanitize= behind -Xarch_host; device code is unchanged), then:
  1. tests/c_abi/host_checks.c, a plain C driver built with the same sanitizers, runs every
     host-side path that needs no GPU (argument checks of every entry point, workspace sizes,
     the split rule, the RoPE frequency tables, status strings);
  2. tests/test_abi.py runs in a copy of the package whose libgqa.so is that build, with the
     sanitizer runtime preloaded into Python.
Any report of either sanitizer fails the test."""
import concurrent.futures as cf
import glob
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _build_module():
    path = os.path.join(ROOT, "attention_head_qk_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_gqa_build_san", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    b = _build_module()
    try:
        hipcc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = _runtime()
    clang = "/opt/rocm/llvm/bin/clang"
    if rt is None or not os.path.exists(clang):
        pytest.skip("no sanitizer runtime")
    out = tmp_path_factory.mktemp("san")
    flags = [f for f in b.common_flags() if f != "-O3"] + ["-O1", "-g"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = str(out / (os.path.splitext(src)[0] + ".o"))
        r = subprocess.run([hipcc, *flags, *san, "-c", os.path.join(b.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(len(b.SOURCES)) as ex:
        objs = list(ex.map(compile_one, b.SOURCES))
    lib = out / "libgqa.so"
    # the sanitizer symbols stay undefined in the library: the executable (or the preloaded
    # runtime) provides them
    r = subprocess.run([hipcc, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *objs, "-o", str(lib)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return out, lib, rt, clang


def test_c_driver_host_paths_clean(san_lib):
    out, lib, rt, clang = san_lib
    exe = out / "host_checks"
    r = subprocess.run([clang, "-g", "-fsanitize=address,undefined", "-shared-libasan",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c_abi", "host_checks.c"), "-o", str(exe),
                        "-L", str(out), "-lgqa", "-L", "/opt/rocm/lib", "-lamdhip64", "-lm",
                        f"-Wl,-rpath,{out}", "-Wl,-rpath,/opt/rocm/lib",
                        f"-Wl,-rpath,{os.path.dirname(rt)}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, **SAN_ENV))
    assert r.returncode == 0 and "host checks: OK" in r.stdout, r.stdout + r.stderr[-5000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-5000:]


def test_abi_suite_under_sanitizers(san_lib, tmp_path):
    out, lib, rt, clang = san_lib
    for sub in ("include", "oracle", "tests"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub,
                        ignore=shutil.ignore_patterns("__pycache__"))
    for f in ("workloads.py", "pytest.ini"):
        shutil.copy(os.path.join(ROOT, f), tmp_path / f)
    pkg = tmp_path / "attention_head_qk_amd"
    pkg.mkdir()
    for f in glob.glob(os.path.join(ROOT, "attention_head_qk_amd", "*.py")):
        shutil.copy(f, pkg)
    shutil.copy(lib, pkg / "libgqa.so")
    env = dict(os.environ, **SAN_ENV, PYTHONDONTWRITEBYTECODE="1")
    # the sanitizer runtime must come first; anything already preloaded stays after it
    env["LD_PRELOAD"] = rt + (":" + os.environ["LD_PRELOAD"] if os.environ.get("LD_PRELOAD") else "")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_abi_sweep.py", "-k", "not c_client"],
                       cwd=tmp_path, capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-5000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-5000:]
