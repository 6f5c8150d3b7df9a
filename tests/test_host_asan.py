"""Host-side AddressSanitizer run of the C ABI's validation code (CPU only).

The library is rebuilt into a temporary directory with AddressSanitizer on the
host code only (device code is compiled as usual; hipcc's -Xarch_host puts the
flag on the host compile), and tests/abi_check.c -- every entry point's
argument validation, status strings and width factorisation, none of which
launches a kernel -- runs against it.  Any heap, stack or global overflow,
use-after-free or double free in that host code aborts the program."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "hadamard_rotation_int4_amd" / "csrc"
HIPCC = Path("/opt/rocm/bin/hipcc")
CLANG = Path("/opt/rocm/llvm/bin/clang")
CLANGXX = Path("/opt/rocm/llvm/bin/clang++")


def _asan_runtime_dir():
    for base in (Path("/opt/rocm/lib/llvm/lib/clang"), Path("/opt/rocm/llvm/lib/clang")):
        if base.is_dir():
            for p in sorted(base.glob("*/lib/linux/libclang_rt.asan-x86_64.so")):
                return p.parent
    return None


RT = _asan_runtime_dir()
pytestmark = pytest.mark.skipif(
    not (HIPCC.exists() and CLANG.exists() and CLANGXX.exists() and RT is not None),
    reason="hipcc, clang or the clang AddressSanitizer runtime is not installed")


def _compile(src: Path, out: Path):
    extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"] if src.name == "kv_decode.hip" else []
    cmd = [str(HIPCC), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-ffp-contract=off", "-fconstexpr-steps=50000000", "-Wno-unused-result",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *extra,
           f"-I{ROOT / 'include'}", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fno-omit-frame-pointer", "-c", str(src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


def test_abi_validation_clean_under_host_asan(tmp_path):
    srcs = sorted(list(CSRC.glob("*.hip")) + list(CSRC.glob("*.cpp")))
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, tmp_path / (s.name + ".o")), srcs))
    lib = tmp_path / "libquarot_hip_asan.so"
    r = subprocess.run([str(CLANGXX), "-shared", "-fPIC", "-fsanitize=address", "-shared-libsan",
                        "-o", str(lib), *map(str, objs), "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = tmp_path / "abi_check_asan"
    r = subprocess.run([str(CLANG), "-std=c99", "-g", "-fsanitize=address", "-shared-libsan",
                        "-fno-omit-frame-pointer", f"-I{ROOT / 'include'}", "-I/opt/rocm/include",
                        "-D__HIP_PLATFORM_AMD__", str(ROOT / "tests" / "abi_check.c"),
                        f"-L{tmp_path}", "-lquarot_hip_asan", f"-Wl,-rpath,{tmp_path}",
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = f"{RT}:" + env.get("LD_LIBRARY_PATH", "")
    # the HIP runtime's own allocations at exit are not this library's
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "abi_check: ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
