"""Address sanitizer on the host code (CPU): the oracle's C sources built with gcc
-fsanitize=address run every CPU pin, and the library's host code (argument validation,
size queries, dispatch up to the launch) built with hipcc -Xarch_host -fsanitize=address
runs the boundary and wrapper tests, which launch nothing. Each runs in a child process
with the sanitizer runtime preloaded; any report fails the child. Device code is not
instrumented (there is no GPU address sanitizer here)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/lib/llvm/bin/clang"


def _child(code, preload, timeout):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    assert r.returncode == 0 and "AddressSanitizer" not in r.stderr, (r.stdout[-3000:] + r.stderr[-6000:])
    return r.stdout


def test_oracle_pins_under_asan(tmp_path):
    src = [os.path.join(ROOT, "oracle", n) for n in ("attn_oracle.c", "fp8_quant_oracle.c", "attn_bwd_oracle.c")]
    so = str(tmp_path / "liboracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-fopenmp", "-shared",
                    "-fPIC", "-std=c99", "-ffp-contract=off", "-o", so, *src, "-lm"], check=True)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    out = _child(f"""
import sys
sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
import oracle
oracle._LIB = oracle.load({so!r})
from tests import pins
for p in pins.ALL_PINS:
    p()
print("pins", len(pins.ALL_PINS))
""", libasan, 600)
    assert "pins" in out


@pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists(CLANG), reason="needs hipcc")
def test_library_host_code_under_asan(tmp_path):
    so = str(tmp_path / "libfa_asan.so")
    srcs = [os.path.join(ROOT, "exact_tiled_attention_03_amd", "csrc", n)
            for n in ("fa_fwd.hip", "fa_quant.hip", "fa_bwd.hip", "fa_splitkv.hip")]
    # device code at -O1: it is only loaded, never run here
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-shared", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-o", so, *srcs],
                   check=True, capture_output=True)
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True,
                        check=True).stdout.strip()
    out = _child(f"""
import sys
sys.path.insert(0, {ROOT!r})
import exact_tiled_attention_03_amd.fa as F
F.LIB_PATH = {so!r}
import pytest
rc = pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu", "tests/test_boundary.py", "tests/test_wrappers.py"])
print("pytest rc", int(rc))
sys.exit(int(rc))
""", rt, 600)
    assert "pytest rc 0" in out
