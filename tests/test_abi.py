"""The C-ABI library loads, exports every symbol include/qr.h declares, and its
host-side validation rejects bad arguments before any launch (no GPU needed:
every call here returns before touching the device)."""
import ctypes
import re
import subprocess
from pathlib import Path

import pytest

import hadamard_rotation_int4_amd as qr

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "qr.h"

QR_OK, QR_ERR_NULL, QR_ERR_SHAPE, QR_ERR_UNSUPPORTED, QR_ERR_ALIGN, QR_ERR_LAUNCH, QR_ERR_ARG, \
    QR_ERR_SCRATCH = range(8)


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qr_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not qr.LIB_PATH.exists():
        pytest.fail(f"{qr.LIB_PATH} not built: run `python -m hadamard_rotation_int4_amd.build`")
    return qr._load()


def test_header_declares_the_path():
    names = declared_functions()
    for must in ("qr_hadamard_quant", "qr_hadamard", "qr_w4a4_gemm", "qr_kv_rotate_quant",
                 "qr_kv_decode_attention", "qr_kv_decode_workspace_bytes",
                 "qr_kv_decode_attention_noalloc",
                 "qr_rmsnorm_quant", "qr_hadamard_heads_quant", "qr_hadamard_quant_i8",
                 "qr_rmsnorm_quant_i8", "qr_hadamard_heads_quant_i8", "qr_w8a8_gemm",
                 "qr_kv_rotate_quant_bits", "qr_hadamard_quant_groups", "qr_w4a4_gemm_groups",
                 "qr_hadamard_factor", "qr_status_str", "qr_abi_version"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", str(qr.LIB_PATH)], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(lib, n)


def test_version_and_status_strings(lib):
    assert qr.abi_version() == 1
    for code in range(8):
        assert qr.status_str(code).startswith("QR_")
    assert "unknown" in qr.status_str(99)


@pytest.mark.parametrize("d,expect", [(4096, (12, 1)), (8192, (13, 1)), (128, (7, 1)),
                                      (11008, (6, 172)), (28672, (10, 28)), (56, (1, 28)),
                                      (344, (1, 172))])
def test_factor(lib, d, expect):
    assert qr.hadamard_factor(d) == expect


@pytest.mark.parametrize("d", [0, 4, 43, 100, 16384, 172 * 128, 28 * 2048, 4097])
def test_factor_rejects(lib, d):
    n, m = ctypes.c_int32(-1), ctypes.c_int32(-1)
    assert lib.qr_hadamard_factor(d, ctypes.byref(n), ctypes.byref(m)) == QR_ERR_UNSUPPORTED
    assert n.value == -1 and m.value == -1
    assert lib.qr_hadamard_factor(4096, None, None) == QR_ERR_NULL


A16 = 1 << 20  # a fake, 16-byte-aligned non-null address (never dereferenced on the host)


def hq(lib, x=A16, T=4, d=4096, ld=4096, rot=1, signs=None, clip=1.0, q=A16, sc=A16, z=None):
    return lib.qr_hadamard_quant(x, T, d, ld, rot, signs, clip, q, sc, z, None)


def test_hadamard_quant_validation(lib):
    assert hq(lib, T=0) == QR_OK                       # empty: no launch
    assert hq(lib, T=-1) == QR_ERR_SHAPE
    assert hq(lib, ld=4000) == QR_ERR_SHAPE            # ld < d
    assert hq(lib, d=4100, ld=4104) == QR_ERR_UNSUPPORTED
    assert hq(lib, d=43, ld=48) == QR_ERR_UNSUPPORTED
    assert hq(lib, rot=7) == QR_ERR_ARG
    assert hq(lib, rot=3) == QR_ERR_ARG
    assert hq(lib, rot=2) == QR_ERR_UNSUPPORTED        # fp16 transform: d = 28672, 11008
    assert hq(lib, T=0, d=28672, ld=28672, rot=2) == QR_OK
    assert hq(lib, T=0, d=11008, ld=11008, rot=2) == QR_OK
    assert hq(lib, T=0, d=5504, ld=5504, rot=2) == QR_ERR_UNSUPPORTED
    assert hq(lib, clip=0.0) == QR_ERR_ARG
    assert hq(lib, clip=1.5) == QR_ERR_ARG
    assert hq(lib, clip=1e-4) == QR_ERR_ARG
    assert hq(lib, x=None) == QR_ERR_NULL
    assert hq(lib, q=None) == QR_ERR_NULL
    assert hq(lib, sc=None) == QR_ERR_NULL
    assert hq(lib, x=A16 + 8) == QR_ERR_ALIGN
    assert hq(lib, ld=4100) == QR_ERR_ALIGN
    assert hq(lib, q=A16 + 2) == QR_ERR_ALIGN
    assert hq(lib, z=A16 + 4) == QR_ERR_ALIGN
    # quantization without rotation accepts any width that is a multiple of 8
    assert hq(lib, T=0, d=4000, ld=4000, rot=0) == QR_OK
    assert hq(lib, d=4004, ld=4008, rot=0) == QR_ERR_UNSUPPORTED


def test_hadamard_validation(lib):
    assert lib.qr_hadamard(A16, 0, 128, 128, None, A16, 1, None) == QR_OK
    assert lib.qr_hadamard(A16, 3, 100, 100, None, A16, 1, None) == QR_ERR_UNSUPPORTED
    assert lib.qr_hadamard(None, 3, 128, 128, None, A16, 1, None) == QR_ERR_NULL
    assert lib.qr_hadamard(A16, 3, 128, 128, None, A16 + 4, 1, None) == QR_ERR_ALIGN


def gemm(lib, a=A16, asc=A16, T=16, w=A16, wsc=A16, N=16, K=4096, y=A16, acc=None):
    return lib.qr_w4a4_gemm(a, asc, T, w, wsc, N, K, y, acc, None)


def test_gemm_validation(lib):
    assert gemm(lib, T=0) == QR_OK
    assert gemm(lib, N=0) == QR_OK
    assert gemm(lib, T=-2) == QR_ERR_SHAPE
    assert gemm(lib, K=0) == QR_ERR_SHAPE
    assert gemm(lib, K=4100) == QR_ERR_UNSUPPORTED
    assert gemm(lib, K=131072) == QR_ERR_UNSUPPORTED
    assert gemm(lib, a=None) == QR_ERR_NULL
    assert gemm(lib, y=None) == QR_ERR_NULL
    assert gemm(lib, a=A16 + 4) == QR_ERR_ALIGN
    assert gemm(lib, y=A16 + 2) == QR_ERR_ALIGN


def kvq(lib, B=2, S_new=3, H=8, Dh=128, ld=1024, rot=1, group=128, clip=0.95, cq=A16, meta=A16,
        S_max=10, start=0, kv=A16):
    return lib.qr_kv_rotate_quant(kv, B, S_new, H, Dh, ld, rot, None, group, clip, cq, meta, S_max,
                                  start, None, None)


def test_kv_validation(lib):
    assert kvq(lib, S_new=0) == QR_OK
    assert kvq(lib, start=8) == QR_ERR_SHAPE          # 8 + 3 > 10: cache overflow
    assert kvq(lib, start=-1) == QR_ERR_SHAPE
    assert kvq(lib, B=0) == QR_ERR_SHAPE
    assert kvq(lib, Dh=96, ld=768) == QR_ERR_UNSUPPORTED
    assert kvq(lib, group=48) == QR_ERR_UNSUPPORTED
    assert kvq(lib, group=256) == QR_ERR_UNSUPPORTED
    assert kvq(lib, ld=1000) == QR_ERR_SHAPE
    assert kvq(lib, clip=2.0) == QR_ERR_ARG
    assert kvq(lib, rot=3) == QR_ERR_ARG
    assert kvq(lib, kv=None) == QR_ERR_NULL
    assert kvq(lib, cq=A16 + 2) == QR_ERR_ALIGN
    assert kvq(lib, ld=1028) == QR_ERR_ALIGN


def test_kv_bits_validation(lib):
    def kb(bits, S_new=3, start=0):
        return lib.qr_kv_rotate_quant_bits(A16, 2, S_new, 8, 128, 1024, 1, None, 128, 0.95, bits,
                                           A16, A16, 10, start, None, None)
    assert kb(3, S_new=0) == QR_OK
    assert kb(2, S_new=0) == QR_OK
    assert kb(1) == QR_ERR_ARG
    assert kb(5) == QR_ERR_ARG
    assert kb(3, start=8) == QR_ERR_SHAPE


def kvd(lib, q=A16, B=2, Hq=16, Hkv=2, Dh=128, kq=A16, km=A16, vq=A16, vm=A16, S_max=300, L=260,
        group=128, scale=0.088, out=A16, ws=A16, wsb=1 << 30):
    return lib.qr_kv_decode_attention(q, B, Hq, Hkv, Dh, kq, km, vq, vm, S_max, L, group, scale,
                                      out, ws, wsb, None)


def test_kv_decode_validation(lib):
    assert lib.qr_kv_decode_workspace_bytes(2, 16, 2, 128, 260) > 0
    assert lib.qr_kv_decode_workspace_bytes(0, 16, 2, 128, 260) == 0
    assert kvd(lib, B=0) == QR_OK
    assert kvd(lib, L=0) == QR_ERR_SHAPE
    assert kvd(lib, L=301) == QR_ERR_SHAPE              # past the cache
    assert kvd(lib, Hq=15) == QR_ERR_SHAPE              # not a multiple of Hkv
    assert kvd(lib, Dh=64) == QR_ERR_UNSUPPORTED
    assert kvd(lib, group=64) == QR_ERR_UNSUPPORTED
    assert kvd(lib, Hq=64, Hkv=2) == QR_ERR_UNSUPPORTED  # 32 query heads per KV head
    assert kvd(lib, scale=0.0) == QR_ERR_ARG
    assert kvd(lib, scale=float("nan")) == QR_ERR_ARG
    assert kvd(lib, q=None) == QR_ERR_NULL
    assert kvd(lib, ws=None) == QR_ERR_NULL
    need = lib.qr_kv_decode_workspace_bytes(2, 16, 2, 128, 260)
    assert kvd(lib, wsb=need - 4) == QR_ERR_SHAPE
    assert kvd(lib, kq=A16 + 4) == QR_ERR_ALIGN
    assert kvd(lib, km=A16 + 2) == QR_ERR_ALIGN


def rq(lib, x=A16, T=4, d=8192, ld=8192, eps=1e-5, clip=1.0, q=A16, sc=A16, r=None):
    return lib.qr_rmsnorm_quant(x, T, d, ld, eps, clip, q, sc, r, None)


def test_rmsnorm_quant_validation(lib):
    assert rq(lib, T=0) == QR_OK
    assert rq(lib, T=0, d=16384, ld=16384) == QR_OK
    assert rq(lib, T=-1) == QR_ERR_SHAPE
    assert rq(lib, ld=8184) == QR_ERR_SHAPE
    assert rq(lib, d=8196, ld=8200) == QR_ERR_UNSUPPORTED   # not a multiple of 8
    assert rq(lib, d=16392, ld=16392) == QR_ERR_UNSUPPORTED  # wider than 16384
    assert rq(lib, eps=-1e-6) == QR_ERR_ARG
    assert rq(lib, eps=float("nan")) == QR_ERR_ARG
    assert rq(lib, eps=2.0) == QR_ERR_ARG
    assert rq(lib, clip=0.0) == QR_ERR_ARG
    assert rq(lib, x=None) == QR_ERR_NULL
    assert rq(lib, sc=None) == QR_ERR_NULL
    assert rq(lib, x=A16 + 8) == QR_ERR_ALIGN
    assert rq(lib, ld=8196) == QR_ERR_ALIGN
    assert rq(lib, q=A16 + 2) == QR_ERR_ALIGN
    assert rq(lib, r=A16 + 2) == QR_ERR_ALIGN


def hh(lib, x=A16, T=4, nh=64, dh=128, ld=8192, clip=1.0, q=A16, sc=A16, z=None):
    return lib.qr_hadamard_heads_quant(x, T, nh, dh, ld, clip, q, sc, z, None)


def test_hadamard_heads_quant_validation(lib):
    assert hh(lib, T=0) == QR_OK
    for nh, dh in ((64, 128), (32, 128), (32, 256), (16, 512), (8, 64), (2, 32), (64, 8)):
        assert hh(lib, T=0, nh=nh, dh=dh, ld=nh * dh) == QR_OK, (nh, dh)
    assert hh(lib, T=-1) == QR_ERR_SHAPE
    assert hh(lib, nh=0) == QR_ERR_SHAPE
    assert hh(lib, ld=4096) == QR_ERR_SHAPE
    assert hh(lib, nh=48, ld=6144) == QR_ERR_UNSUPPORTED      # not a power of two
    assert hh(lib, nh=128, dh=64) == QR_ERR_UNSUPPORTED       # more than 64 heads
    assert hh(lib, nh=1, dh=128, ld=128) == QR_ERR_UNSUPPORTED
    assert hh(lib, nh=64, dh=256, ld=16384) == QR_ERR_UNSUPPORTED
    assert hh(lib, nh=32, dh=96, ld=3072) == QR_ERR_UNSUPPORTED
    assert hh(lib, nh=16, dh=16, ld=256) == QR_ERR_UNSUPPORTED
    assert hh(lib, clip=1.5) == QR_ERR_ARG
    assert hh(lib, q=None) == QR_ERR_NULL
    assert hh(lib, x=A16 + 2) == QR_ERR_ALIGN
    assert hh(lib, ld=8196) == QR_ERR_ALIGN
    assert hh(lib, z=A16 + 4) == QR_ERR_ALIGN


def test_i8_quantizers_validation(lib):
    A8 = A16 + 8  # 8-byte but not 16-byte aligned: fine for int8 codes, not for x
    f = lib.qr_hadamard_quant_i8
    assert f(A16, 0, 8192, 8192, 1, None, 1.0, 8, A16, A16, None, None) == QR_OK
    assert f(A16, 0, 28672, 28672, 1, None, 1.0, 6, A16, A16, None, None) == QR_OK
    assert f(A16, 4, 8192, 8192, 2, None, 1.0, 8, A16, A16, None, None) == QR_ERR_ARG  # no fp16 transform
    assert f(A16, 4, 8192, 8192, 1, None, 1.0, 9, A16, A16, None, None) == QR_ERR_ARG
    assert f(A16, 4, 8192, 8192, 1, None, 1.0, 1, A16, A16, None, None) == QR_ERR_ARG
    assert f(A16, 4, 4100, 4104, 1, None, 1.0, 8, A16, A16, None, None) == QR_ERR_UNSUPPORTED
    assert f(A16, 4, 8192, 8192, 1, None, 1.0, 8, A16 + 4, A16, None, None) == QR_ERR_ALIGN
    assert f(None, 4, 8192, 8192, 1, None, 1.0, 8, A16, A16, None, None) == QR_ERR_NULL
    g = lib.qr_rmsnorm_quant_i8
    assert g(A16, 0, 8192, 8192, 1e-5, 1.0, 8, A8, A16, None, None) == QR_OK
    assert g(A16, 4, 8192, 8192, 1e-5, 1.0, 0, A8, A16, None, None) == QR_ERR_ARG
    assert g(A16, 4, 8192, 8192, 1e-5, 1.0, 8, A16 + 4, A16, None, None) == QR_ERR_ALIGN
    h = lib.qr_hadamard_heads_quant_i8
    assert h(A16, 0, 64, 128, 8192, 1.0, 6, A8, A16, None, None) == QR_OK
    assert h(A16, 4, 64, 128, 8192, 1.0, 12, A8, A16, None, None) == QR_ERR_ARG
    assert h(A16, 4, 48, 128, 6144, 1.0, 8, A8, A16, None, None) == QR_ERR_UNSUPPORTED


def test_groups_quantizer_validation(lib):
    f = lib.qr_hadamard_quant_groups
    assert f(A16, 0, 8192, 8192, 1, None, 1.0, 128, A16, A16, None, None) == QR_OK
    assert f(A16, 0, 28672, 28672, 1, None, 1.0, 512, A16, A16, None, None) == QR_OK
    assert f(A16, 4, 8192, 8192, 1, None, 1.0, 96, A16, A16, None, None) == QR_ERR_UNSUPPORTED
    assert f(A16, 4, 8192, 8192, 1, None, 1.0, 1024, A16, A16, None, None) == QR_ERR_UNSUPPORTED
    assert f(A16, 4, 8192, 8192, 1, None, 1.0, 4, A16, A16, None, None) == QR_ERR_UNSUPPORTED
    assert f(A16, 4, 11008, 11008, 1, None, 1.0, 512, A16, A16, None, None) == QR_ERR_UNSUPPORTED
    assert f(A16, 4, 8192, 8192, 2, None, 1.0, 128, A16, A16, None, None) == QR_ERR_ARG
    assert f(None, 4, 8192, 8192, 1, None, 1.0, 128, A16, A16, None, None) == QR_ERR_NULL


def test_groups_gemm_validation(lib):
    f = lib.qr_w4a4_gemm_groups
    assert f(A16, A16, 0, A16, A16, 16, 4096, 128, A16, None) == QR_OK
    assert f(A16, A16, 16, A16, A16, 16, 4096, 96, A16, None) == QR_ERR_UNSUPPORTED
    assert f(A16, A16, 16, A16, A16, 16, 4096, 32, A16, None) == QR_ERR_UNSUPPORTED
    assert f(A16, A16, 16, A16, A16, 16, 4096, 1024, A16, None) == QR_ERR_UNSUPPORTED
    assert f(A16, A16, 16, A16, A16, 16, 4160, 128, A16, None) == QR_ERR_UNSUPPORTED  # 128 !| K
    assert f(None, A16, 16, A16, A16, 16, 4096, 128, A16, None) == QR_ERR_NULL
    assert f(A16, A16, -1, A16, A16, 16, 4096, 128, A16, None) == QR_ERR_SHAPE


def test_w8a8_gemm_validation(lib):
    f = lib.qr_w8a8_gemm
    assert f(A16, A16, 0, A16, A16, 16, 4096, A16, None, None) == QR_OK
    assert f(A16, A16, 16, A16, A16, 0, 4112, A16, None, None) == QR_OK
    assert f(A16, A16, 16, A16, A16, 16, 4100, A16, None, None) == QR_ERR_UNSUPPORTED  # K % 16
    assert f(A16, A16, 16, A16, A16, 16, 131024, A16, None, None) == QR_ERR_UNSUPPORTED
    assert f(A16, A16, -1, A16, A16, 16, 4096, A16, None, None) == QR_ERR_SHAPE
    assert f(None, A16, 16, A16, A16, 16, 4096, A16, None, None) == QR_ERR_NULL
    assert f(A16 + 8, A16, 16, A16, A16, 16, 4096, A16, None, None) == QR_ERR_ALIGN


def test_c_program_against_the_header(tmp_path):
    # the header is plain C: a C99 program compiled with gcc links every entry
    # point and gets the documented host-side answers
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None or not Path("/opt/rocm/include/hip/hip_runtime_api.h").exists():
        pytest.skip("gcc or the HIP headers are not available")
    if not qr.LIB_PATH.exists():
        pytest.fail(f"{qr.LIB_PATH} not built")
    exe = tmp_path / "abi_check"
    libdir = str(qr.LIB_PATH.parent)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    f"-I{ROOT / 'include'}", "-I/opt/rocm/include",
                    str(ROOT / "tests" / "abi_check.c"), "-o", str(exe), f"-L{libdir}",
                    "-lquarot_hip", f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    assert "abi_check: ok" in out.stdout


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((4, 128), dtype=torch.float16)
    with pytest.raises(ValueError):
        qr.hadamard_quant(x)
    with pytest.raises(TypeError):
        qr.hadamard_quant(x.float())
    with pytest.raises(ValueError):
        qr.rmsnorm_quant(x)
    with pytest.raises(ValueError):
        qr.hadamard_heads_quant(x, 4)


def test_noalloc_decode_rejects_calls_beyond_its_static_scratch(lib):
    # 255 sequences x 1 KV head x 16 query heads over 512 positions need 4.2 MB of
    # split records, more than the library's 4 MiB static buffer: QR_ERR_SCRATCH
    # before any pointer is looked at or anything runs.
    assert lib.qr_kv_decode_workspace_bytes(255, 16, 1, 128, 512) > 4 << 20
    code = lib.qr_kv_decode_attention_noalloc(None, 255, 16, 1, 128, None, None, None, None, 512,
                                              512, 128, 0.088, None, None)
    assert code == QR_ERR_SCRATCH, qr.status_str(code)
    assert "scratch" in qr.status_str(QR_ERR_SCRATCH)
    # the same shape fits the entry point that takes a workspace (its pointers are
    # checked next: NULL here)
    assert lib.qr_kv_decode_attention(None, 255, 16, 1, 128, None, None, None, None, 512, 512, 128,
                                      0.088, None, None, 0, None) == QR_ERR_NULL
    assert lib.qr_kv_decode_attention_noalloc(None, 2, 16, 2, 128, None, None, None, None, 512,
                                              512, 128, 0.088, None, None) == QR_ERR_NULL
