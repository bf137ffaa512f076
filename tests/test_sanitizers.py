"""Host-side sanitizer runs (no GPU): the oracle's C entry points on small
inputs, and the library's argument validation and workspace sizing, each built
with AddressSanitizer and UndefinedBehaviorSanitizer.  The GPU code is built
as usual; only host code is instrumented."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "block_scaled_fp4_amd", "csrc")
SOURCES = ["api.cpp", "quantize.hip", "topk.hip", "attn_fwd.hip", "attn_decode.hip", "kvcache.hip",
           "attn_train.hip", "attn_mx.hip"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])}...: rc {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off", os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "fp4_oracle.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="4")
    r = _run([exe], env=env, timeout=300)
    assert "oracle driver ok" in r.stdout


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
def test_library_host_side_under_asan_ubsan(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        _run(["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SAN,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result",
              "-I", os.path.join(ROOT, "include"), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    exe = str(tmp_path / "abi_asan")
    _run(["hipcc", "--offload-arch=gfx950", "-g", *HOST_SAN[:4], "-I", os.path.join(ROOT, "include"), *objs,
          "-x", "c++", os.path.join(HERE, "abi_driver.cpp"), "-o", exe])
    # the HIP runtime keeps allocations until exit: leak reports are off, every other check is on
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = _run([exe], env=env, timeout=300)
    assert "abi driver ok" in r.stdout
