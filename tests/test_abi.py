"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host with the documented
status codes.  Every call below fails a host-side check, so nothing is ever
launched (the fake pointers are never dereferenced)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, LAUNCH = 0, 1, 2, 3, 4
BF16, FP32 = 0, 1
P = 0x10000        # a 256-byte-aligned fake device address, never dereferenced
MIS = 0x10008      # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    fa = pytest.importorskip("exact_io_aware_36_amd")
    return fa._lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("fa_fwd", "fa_fwd_ex", "fa_bwd", "fa_bwd_workspace_bytes",
                 "fa_fwd_blocksparse", "fa_status_str"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    import exact_io_aware_36_amd as fa

    raw = ctypes.CDLL(fa.library_path)
    for name in declared_functions():
        assert hasattr(raw, name), name
        # and the Python binding has a function of the same name
        assert callable(getattr(fa, name)), name


def test_status_strings(lib):
    import exact_io_aware_36_amd as fa

    assert fa.fa_status_str(OK) == "FA_OK"
    assert fa.fa_status_str(INVALID) == "FA_ERR_INVALID_ARG"
    assert fa.fa_status_str(UNSUPPORTED) == "FA_ERR_UNSUPPORTED"
    assert fa.fa_status_str(WORKSPACE) == "FA_ERR_WORKSPACE"
    assert fa.fa_status_str(LAUNCH) == "FA_ERR_LAUNCH"
    assert fa.fa_status_str(99) == "FA_ERR_UNKNOWN"


def test_workspace_bytes(lib):
    # two fp32 [B, H, N] row vectors, each rounded up to 256 bytes
    assert lib.fa_bwd_workspace_bytes(1, 16, 16384, 128) == 2 * 16 * 16384 * 4
    assert lib.fa_bwd_workspace_bytes(1, 1, 3, 64) == 2 * 256
    assert lib.fa_bwd_workspace_bytes(16, 16, 512, 64) == 2 * 16 * 16 * 512 * 4
    assert lib.fa_bwd_workspace_bytes(0, 1, 1, 64) == 0
    assert lib.fa_bwd_workspace_bytes(1, 1, 1, 96) == 0
    assert lib.fa_bwd_workspace_bytes(2, 16, 8192, 256) == 2 * 2 * 16 * 8192 * 4


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=64, causal=0, scale=0.125,
        lens=None, dtype=BF16, tile=None):
    if tile is None:
        return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, lens, dtype, None)
    return lib.fa_fwd_ex(q, k, v, o, lse, B, H, N, d, causal, scale, lens, dtype, tile, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(o=None), INVALID), (dict(lse=None), INVALID),
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(N=0), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256, dtype=FP32), UNSUPPORTED), (dict(d=0), UNSUPPORTED),
    (dict(d=512), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
    (dict(B=1 << 14, H=16, N=1 << 14, d=64), INVALID),      # B*H*N*d >= 2^31
    (dict(q=MIS), INVALID), (dict(o=MIS), INVALID), (dict(lse=P + 2), INVALID),
    (dict(lens=P + 1), INVALID),
])
def test_fwd_rejects(lib, kw, want):
    assert fwd(lib, **kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(tile=48), UNSUPPORTED), (dict(tile=512), UNSUPPORTED), (dict(tile=-1), UNSUPPORTED),
    (dict(tile=256, d=256), UNSUPPORTED), (dict(tile=256, dtype=FP32), UNSUPPORTED),
    (dict(tile=64, dtype=FP32), UNSUPPORTED), (dict(tile=16, dtype=FP32), UNSUPPORTED),
    (dict(tile=64, d=80), UNSUPPORTED), (dict(tile=64, q=None), INVALID),
    (dict(tile=128, d=256), UNSUPPORTED), (dict(tile=16, d=128), UNSUPPORTED),
])
def test_fwd_ex_rejects(lib, kw, want):
    assert fwd(lib, **kw) == want


def bwd(lib, q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, H=2, N=256, d=64, causal=0,
        scale=0.125, lens=None, dtype=BF16, ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(B, H, N, d)
    return lib.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, causal, scale, lens, dtype,
                      ws, ws_bytes, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(do=None), INVALID),
    (dict(lse=None), INVALID), (dict(dq=None), INVALID), (dict(dk=None), INVALID),
    (dict(dv=None), INVALID), (dict(N=0), INVALID), (dict(scale=0.0), INVALID),
    (dict(d=32), UNSUPPORTED), (dict(d=512), UNSUPPORTED), (dict(dtype=FP32), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=100), WORKSPACE),
    (dict(ws=P + 16), WORKSPACE), (dict(dq=MIS), INVALID),
])
def test_bwd_rejects(lib, kw, want):
    assert bwd(lib, **kw) == want


def sparse(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=256, d=64, scale=0.125, mask=P,
           mb=128, dtype=BF16):
    return lib.fa_fwd_blocksparse(q, k, v, o, lse, B, H, N, d, scale, mask, mb, dtype, None)


@pytest.mark.parametrize("kw,want", [
    (dict(mask=None), INVALID), (dict(mb=64), INVALID), (dict(mb=0), INVALID),
    (dict(N=200), INVALID), (dict(N=131072), UNSUPPORTED), (dict(dtype=FP32), UNSUPPORTED),
    (dict(d=96), UNSUPPORTED), (dict(o=None), INVALID), (dict(scale=-0.5), INVALID),
])
def test_sparse_rejects(lib, kw, want):
    assert sparse(lib, **kw) == want


def test_python_binding_checks_shapes():
    torch = pytest.importorskip("torch")
    fa = pytest.importorskip("exact_io_aware_36_amd")
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(q, q, torch.zeros(1, 1, 9, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fa.fwd(q.view(8, 64), q.view(8, 64), q.view(8, 64))
    with pytest.raises(ValueError):
        fa.fwd(q.half(), q.half(), q.half())


def test_library_has_no_unresolved_kernels():
    """Every kernel the launchers reference must be defined in libfa.so (a
    missing host-side kernel handle only shows as an undefined symbol)."""
    import shutil
    import subprocess

    fa = pytest.importorskip("exact_io_aware_36_amd")
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-u", fa.library_path], capture_output=True, text=True).stdout
    bad = [ln for ln in out.splitlines() if "_ZN2fa" in ln]
    assert not bad, bad


def bwd_sparse(lib, q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, H=1, N=256, d=64,
               scale=0.125, mask=P, mb=128, dtype=BF16, ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(B, H, N, d)
    return lib.fa_bwd_blocksparse(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, scale, mask, mb,
                                  dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,want", [
    (dict(mask=None), INVALID), (dict(mb=64), INVALID), (dict(N=200), INVALID),
    (dict(N=131072), UNSUPPORTED), (dict(dtype=FP32), UNSUPPORTED), (dict(d=96), UNSUPPORTED),
    (dict(dq=None), INVALID), (dict(lse=None), INVALID), (dict(ws=None), WORKSPACE),
    (dict(ws_bytes=8), WORKSPACE), (dict(scale=0.0), INVALID),
])
def test_bwd_sparse_rejects(lib, kw, want):
    assert bwd_sparse(lib, **kw) == want


def test_splitkv_plan(lib):
    # default: about 512 workgroups, at least 256 keys per split
    assert lib.fa_splitkv_splits(8, 16, 16384, 0) == 4
    assert lib.fa_splitkv_splits(1, 16, 16384, 0) == 32
    assert lib.fa_splitkv_splits(1, 1, 100, 0) == 1
    assert lib.fa_splitkv_splits(2, 2, 5000, 0) == 20
    # requested counts are lowered so that each split has >= 32 keys
    assert lib.fa_splitkv_splits(1, 1, 100, 5) == 4
    assert lib.fa_splitkv_splits(1, 1, 300, 1000) == 10
    assert lib.fa_splitkv_splits(1, 1, 1, 0) == 1
    assert lib.fa_splitkv_splits(0, 1, 1, 0) == 0
    assert lib.fa_splitkv_splits(1, 1, 100, -1) == 0
    # workspace: fp32 partial O [S][R][d] and LSE [S][R], each rounded to 256 B
    assert lib.fa_fwd_splitkv_workspace_bytes(8, 16, 1, 16384, 128, 0) == 4 * 128 * 128 * 4 + 4 * 128 * 4
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 1, 3, 100, 64, 0) == 0        # one split
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 1, 3, 100, 64, 4) == 4 * 3 * 64 * 4 + 256
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 1, 1, 100, 96, 0) == 0


def splitkv(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=1, Nk=100000, d=128, causal=0,
            scale=0.125, lens=None, ns=0, dtype=BF16, ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, ns)
    return lib.fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, lens, ns, dtype,
                              ws, ws_bytes, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(o=None), INVALID),
    (dict(lse=None), INVALID), (dict(B=0), INVALID), (dict(Nq=0), INVALID), (dict(Nk=0), INVALID),
    (dict(ns=-1), INVALID), (dict(scale=0.0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=512), UNSUPPORTED), (dict(Nq=9), UNSUPPORTED),
    (dict(dtype=FP32), UNSUPPORTED),
    (dict(B=64, H=64, Nk=8192), INVALID),                    # B*H*Nk*d >= 2^31
    (dict(q=MIS), INVALID), (dict(v=MIS), INVALID), (dict(lse=P + 2), INVALID),
    (dict(lens=P + 1), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws=P + 64), WORKSPACE), (dict(ws_bytes=1024), WORKSPACE),
])
def test_splitkv_rejects(lib, kw, want):
    assert splitkv(lib, **kw) == want


def merge(lib, op=P, lp=P, S=4, R=10, d=128, o=P, lse=P, dtype=BF16):
    return lib.fa_merge(op, lp, S, R, d, o, lse, dtype, None)


@pytest.mark.parametrize("kw,want", [
    (dict(op=None), INVALID), (dict(lp=None), INVALID), (dict(o=None), INVALID),
    (dict(lse=None), INVALID), (dict(S=0), INVALID), (dict(R=0), INVALID), (dict(d=0), INVALID),
    (dict(d=2048), INVALID), (dict(R=1 << 22, d=1024), INVALID), (dict(dtype=7), UNSUPPORTED),
    (dict(op=P + 2), INVALID), (dict(lse=P + 1), INVALID), (dict(o=P + 1), INVALID),
    (dict(o=P + 2, dtype=FP32), INVALID),
])
def test_merge_rejects(lib, kw, want):
    assert merge(lib, **kw) == want


def quant(lib, x=P, x8=P, ds=P, B=1, H=1, N=256, d=128, br=128, signs=None, tr=0, ws=None,
          ws_bytes=0):
    return lib.fa_quantize_fp8(x, x8, ds, B, H, N, d, br, signs, tr, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), INVALID), (dict(x8=None), INVALID), (dict(ds=None), INVALID),
    (dict(N=0), INVALID), (dict(br=64), INVALID), (dict(d=96), UNSUPPORTED),
    (dict(d=256), UNSUPPORTED), (dict(tr=1, N=200), INVALID), (dict(x=MIS), INVALID),
    (dict(ds=P + 2), INVALID), (dict(signs=P + 2), INVALID),
    (dict(br=0), WORKSPACE), (dict(br=0, ws=P, ws_bytes=16), WORKSPACE),
])
def test_quantize_fp8_rejects(lib, kw, want):
    assert quant(lib, **kw) == want


def test_quantize_fp8_workspace(lib):
    assert lib.fa_quantize_fp8_workspace_bytes(2, 3, 300, 128, 0) == 256      # 18 floats -> 256 B
    assert lib.fa_quantize_fp8_workspace_bytes(1, 16, 16384, 128, 0) == 16 * 128 * 4
    assert lib.fa_quantize_fp8_workspace_bytes(1, 16, 16384, 128, 128) == 0


def fwd8(lib, q=P, k=P, v=P, qs=P, ks=P, vs=P, o=P, lse=P, B=1, H=1, N=256, d=128, causal=0,
         scale=0.125, lens=None):
    return lib.fa_fwd_fp8(q, k, v, qs, ks, vs, o, lse, B, H, N, d, causal, scale, lens, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(vs=None), INVALID), (dict(lse=None), INVALID),
    (dict(N=200), INVALID), (dict(N=0), INVALID), (dict(scale=0.0), INVALID),
    (dict(d=256), UNSUPPORTED), (dict(d=32), UNSUPPORTED), (dict(v=MIS), INVALID),
    (dict(ks=P + 1), INVALID), (dict(lens=P + 2), INVALID), (dict(B=1 << 12, H=64, N=4096), INVALID),
])
def test_fwd_fp8_rejects(lib, kw, want):
    assert fwd8(lib, **kw) == want


def test_kvouter_workspace(lib):
    # fp32 O accumulator, then two fp32 [B, H, N] statistics, each rounded up to 256 bytes
    assert lib.fa_fwd_kvouter_workspace_bytes(1, 16, 8192, 128) == 16 * 8192 * 128 * 4 + 2 * 16 * 8192 * 4
    assert lib.fa_fwd_kvouter_workspace_bytes(1, 1, 3, 64) == 768 + 2 * 256
    assert lib.fa_fwd_kvouter_workspace_bytes(1, 1, 1, 256) == 0
    assert lib.fa_fwd_kvouter_workspace_bytes(0, 1, 1, 64) == 0
    assert lib.fa_fwd_kvouter_workspace_bytes(1, 1, 1 << 24, 128) == 0   # B*H*N*d >= 2^31


def kvouter(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=64, causal=0, scale=0.125,
            ws=P, wsb=1 << 30):
    return lib.fa_fwd_kvouter(q, k, v, o, lse, B, H, N, d, causal, scale, ws, wsb, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(lse=None), INVALID),
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(scale=0.0), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(q=MIS), INVALID), (dict(o=MIS), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(wsb=100), WORKSPACE), (dict(ws=MIS), WORKSPACE),
])
def test_kvouter_rejects(lib, kw, want):
    assert kvouter(lib, **kw) == want


def noalloc(lib, q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, H=2, N=256, d=64,
            causal=0, scale=0.125, lens=None, dtype=BF16):
    return lib.fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, causal, scale, lens,
                              dtype, None)


def test_bwd_noalloc_limit(lib):
    assert lib.fa_bwd_noalloc_max_rows() == 1 << 20


@pytest.mark.parametrize("kw,want", [
    (dict(N=(1 << 20) + 1, H=1), WORKSPACE), (dict(B=2, H=8, N=65537), WORKSPACE),
    (dict(q=None), INVALID), (dict(dq=None), INVALID), (dict(N=0), INVALID),
    (dict(scale=0.0), INVALID), (dict(d=80), UNSUPPORTED), (dict(dtype=FP32), UNSUPPORTED),
    (dict(dk=MIS), INVALID),
])
def test_bwd_noalloc_rejects(lib, kw, want):
    assert noalloc(lib, **kw) == want


def bwd_ex(lib, tile, q=P, B=1, H=2, N=256, d=64, dtype=BF16, ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(B, H, N, d)
    return lib.fa_bwd_ex(q, P, P, P, P, P, P, P, P, B, H, N, d, 0, 0.125, None, dtype, tile, ws,
                         ws_bytes, None)


@pytest.mark.parametrize("kw,want", [
    (dict(tile=32), UNSUPPORTED), (dict(tile=256), UNSUPPORTED), (dict(tile=-1), UNSUPPORTED),
    (dict(tile=128, d=256), UNSUPPORTED), (dict(tile=64, dtype=FP32), UNSUPPORTED),
    (dict(tile=128, q=None), INVALID), (dict(tile=128, ws=None), WORKSPACE),
    (dict(tile=64, ws_bytes=16), WORKSPACE),
])
def test_bwd_ex_rejects(lib, kw, want):
    assert bwd_ex(lib, **kw) == want

