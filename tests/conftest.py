import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity against the oracle")


@pytest.fixture(scope="session")
def checked_build(tmp_path_factory):
    """One compile of the library for the static checks: host code under
    AddressSanitizer and UndefinedBehaviorSanitizer (-Xarch_host: no GPU code is
    built with a sanitizer), device code with the library's own flags, its AMD
    GPU assembly kept (-save-temps). Returns (library path, assembly path)."""
    hipcc = next((c for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                              shutil.which("hipcc")) if c and os.path.exists(c)), None)
    if hipcc is None:
        pytest.skip("hipcc is not installed")
    out = tmp_path_factory.mktemp("checked_build")
    csrc = os.path.join(ROOT, "paged_kv_gqa_decode_amd", "csrc")
    lib = out / "libpaged_attn_san.so"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-save-temps", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(csrc, "paged_attn.hip"), "-o", str(lib)]
    res = subprocess.run(cmd, cwd=out, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    asm = glob.glob(str(out / "paged_attn-hip-amdgcn-amd-amdhsa-gfx950.s"))
    assert asm, os.listdir(out)
    return str(lib), asm[0]
