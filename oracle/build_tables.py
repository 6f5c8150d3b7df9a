"""Regenerate oracle/data/williamson43.txt (test infrastructure only).

Compiles oracle/williamson_search.c with the host C compiler and runs it with
multiplier-subgroup generator 7.  The search is deterministic (it keeps the
lexicographically smallest solution), so rerunning reproduces the committed
file byte for byte.

    python oracle/build_tables.py [--check]
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
import tempfile
from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "williamson_search.c"
OUT = HERE / "data" / "williamson43.txt"
HEADER = (
    "# Williamson sequences of order 43 (first rows of four symmetric circulant\n"
    "# +-1 matrices A, B, C, D with A^2+B^2+C^2+D^2 = 172 I), one per line.\n"
    "# Written by oracle/build_tables.py, which compiles and runs\n"
    "# oracle/williamson_search.c with multiplier-subgroup generator 7.\n"
)


def compile_search(dst: Path) -> None:
    cc = os.environ.get("CC", "gcc")
    subprocess.run([cc, "-O2", "-fopenmp", "-o", str(dst), str(SRC), "-lm"], check=True)


def generate() -> str:
    with tempfile.TemporaryDirectory() as td:
        exe = Path(td) / "williamson_search"
        compile_search(exe)
        res = subprocess.run([str(exe), "7"], check=True, capture_output=True, text=True)
    return HEADER + res.stdout


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--check", action="store_true", help="compare with the committed file")
    args = ap.parse_args()
    text = generate()
    if args.check:
        same = OUT.read_text() == text
        print("williamson43.txt reproduced" if same else "williamson43.txt DIFFERS")
        return 0 if same else 1
    OUT.write_text(text)
    print(f"wrote {OUT}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
