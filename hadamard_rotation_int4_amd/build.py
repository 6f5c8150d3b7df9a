"""Build libquarot_hip.so in-tree for gfx950 with hipcc.

    python -m hadamard_rotation_int4_amd.build [--jobs N] [--verbose]

Every source under ``csrc/`` is compiled to an object in ``_build/`` (in
parallel) and linked into ``hadamard_rotation_int4_amd/lib/libquarot_hip.so``.
Flags: ``-O3``, no fast-math, ``-ffp-contract=off`` (the quantization recipe
rounds every step explicitly), and packed-fp32 VALU instructions disabled.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIBDIR = PKG / "lib"
LIB = LIBDIR / "libquarot_hip.so"
BUILD = ROOT / "_build"
ARCH = os.environ.get("QR_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fconstexpr-steps=50000000",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    f"-I{ROOT / 'include'}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def sources() -> list[Path]:
    return sorted(list(CSRC.glob("*.hip")) + list(CSRC.glob("*.cpp")))


# Per-source extra flags.  The decode-attention kernel keeps its matrix-core
# results in ordinary VGPRs: it has few accumulators and feeds most MFMA
# results straight into VALU work, which AGPR results would first have to be
# copied out of.
EXTRA_FLAGS = {"kv_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: Path, verbose: bool) -> Path:
    obj = BUILD / (src.name + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src.name, []), "-c", str(src), "-o", str(obj)]
    if src.suffix == ".cpp":
        cmd = [hipcc(), *[f for f in COMMON_FLAGS if not f.startswith("--offload")], "-x", "hip",
               "--offload-arch=" + ARCH, "-c", str(src), "-o", str(obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(ln for ln in res.stderr.splitlines()
                     if "packed-fp32-ops" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{errs}")
    if verbose and errs.strip():
        print(errs)
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    LIBDIR.mkdir(exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    lib = build(args.jobs, args.verbose)
    print(f"built {lib}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
