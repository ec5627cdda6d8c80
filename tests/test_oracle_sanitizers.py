"""Sanitizer builds on the CPU (no GPU): the oracle (oracle/qmv_oracle.c) with
AddressSanitizer and UndefinedBehaviorSanitizer, driven through every entry
point on exactly sized buffers (oracle/sanitize_driver.c), and the C ABI's
host layer (qmv_api.cpp: argument checks, segment tables, dispatch) with the
same sanitizers on the host side, its launch functions replaced by
recording stubs (tests/abi_sanitize_driver.cpp).  Each build must run clean:
exit status 0 and no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def run(cmd, cwd, env=None):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=env, timeout=600)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_san")
    rc, out = run(["gcc", "-std=c11", "-g", "-O1", "-fno-omit-frame-pointer", *SAN,
                   os.path.join(ROOT, "oracle", "qmv_oracle.c"),
                   os.path.join(ROOT, "oracle", "sanitize_driver.c"), "-lm", "-o", exe], ROOT)
    assert rc == 0, out
    rc, out = run([exe], ROOT)
    assert rc == 0 and "ok" in out and "runtime error" not in out and "Sanitizer" not in out, out


def test_abi_host_layer_under_asan_ubsan(tmp_path):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    # host-side sanitizers only: each -fsanitize= goes to the host compile
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    inc = ["-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "gguf_dequant_matvec_amd", "csrc")]
    common = ["-x", "hip", "-std=c++17", "-O1", "-g", "--offload-arch=gfx950", *inc, *host_san]
    objs = []
    for src in (os.path.join(ROOT, "gguf_dequant_matvec_amd", "csrc", "qmv_api.cpp"),
                os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        rc, out = run([hipcc, *common, "-c", src, "-o", obj], ROOT)
        assert rc == 0, out
        objs.append(obj)
    exe = str(tmp_path / "abi_san")
    rc, out = run([hipcc, "--offload-arch=gfx950", *host_san, *objs, "-o", exe], ROOT)
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    rc, out = run([exe], ROOT, env=env)
    assert rc == 0 and "ok" in out and "runtime error" not in out and "Sanitizer" not in out, out
