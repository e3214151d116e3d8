"""The library's host layer (argument validation, planners, cache metadata,
page lists: dflash_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU.  The host pass of dflash_api.cpp is rebuilt with both sanitizers
(the device code and the kernels' objects are the product build's), linked
into a library of the same name in a scratch copy of the package, and the
host-only test modules (test_abi.py, test_cache_model.py) run against it in a
child process with the sanitizer runtime preloaded.  Any report fails."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_diffusion_draft_fc_amd")


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.timeout(900)
def test_host_layer_under_asan_and_ubsan(tmp_path):
    rt = _runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc or sanitizer runtime")
    sys.path.insert(0, ROOT)
    from block_diffusion_draft_fc_amd import build as B

    objs = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    # the scratch copy: package sources, headers, oracle, workloads and the host-only tests
    for d in ("block_diffusion_draft_fc_amd", "include", "oracle", "workloads"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "test_abi.py", "test_cache_model.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    san_obj = str(tmp_path / "dflash_api_san.o")
    src = os.path.join(PKG, "csrc", "dflash_api.cpp")
    cmd = [B.HIPCC, *B.FLAGS, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-x", "hip", "-c", src, "-o", san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    others = [o for o in objs if not o.endswith("dflash_api.o")]
    lib = str(tmp_path / "block_diffusion_draft_fc_amd" / "libdflash.so")
    r = subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", san_obj, *others,
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-shared-libsan", "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the host layer is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = subprocess.run([sys.executable, "-c", "import block_diffusion_draft_fc_amd._lib as L; print(L.LIB_PATH)"],
                           cwd=tmp_path, env=env, capture_output=True, text=True)
    assert probe.stdout.strip() == lib, probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_cache_model.py"], cwd=tmp_path, env=env,
                       capture_output=True, text=True, timeout=800)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
