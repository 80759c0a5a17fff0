"""fp64 CPU oracle for exact attention (forward and backward).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It shares
no code with the GPU library.

The arithmetic lives in ``fa_oracle.c`` (plain C, OpenMP over query rows or
heads); this module only marshals numpy arrays.  Inputs of any float dtype are
upcast losslessly to float64 before the call.  What is computed is the plain
definition O = softmax(scale * Q K^T) V of "FlashAttention: Mathematical
Foundations, IO-Aware Tiling, Online Softmax, and Recomputation Dynamics"
(section "The GPU Memory Hierarchy and the Attention Memory Wall"), with the
readings for causal masking, key padding and block masks stated in
``fa_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(force: bool = True) -> str:
    """Compile fa_oracle.c into liboracle.so next to it (gcc, -fopenmp)."""
    from .build import build_oracle

    return build_oracle(force=force)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.fa_oracle_threads.restype = ctypes.c_int
    lib.fa_oracle_fwd.restype = ctypes.c_int
    lib.fa_oracle_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                  _i32p, _u8p, ctypes.c_int]
    lib.fa_oracle_fwd_rows.restype = ctypes.c_int
    lib.fa_oracle_fwd_rows.argtypes = lib.fa_oracle_fwd.argtypes + [_i64p, ctypes.c_int64]
    lib.fa_oracle_bwd.restype = ctypes.c_int
    lib.fa_oracle_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_double, _i32p, _u8p, ctypes.c_int]
    lib.fa_oracle_bwd_sample.restype = ctypes.c_int
    lib.fa_oracle_bwd_sample.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_double, ctypes.c_int, _u8p,
                                         ctypes.c_int, _i64p, ctypes.c_int64, _dp, _i64p,
                                         ctypes.c_int64, _dp, _dp]
    lib.fa_oracle_decode.restype = ctypes.c_int
    lib.fa_oracle_decode.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_double, _i32p]
    lib.fa_oracle_merge.restype = ctypes.c_int
    lib.fa_oracle_merge.argtypes = [_dp, _dp, ctypes.c_int, ctypes.c_int64, ctypes.c_int, _dp, _dp]
    _lib = lib
    return lib


def threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().fa_oracle_threads())


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, typ):
    return a.ctypes.data_as(typ) if a is not None else None


def _prep(q, k, v, kv_lens, block_mask, mask_block):
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    lens = None
    if kv_lens is not None:
        lens = np.ascontiguousarray(np.asarray(kv_lens), dtype=np.int32)
        if lens.shape != (B,):
            raise ValueError("kv_lens must have shape [B]")
    mask = None
    if block_mask is not None:
        mask = np.ascontiguousarray(np.asarray(block_mask), dtype=np.uint8)
        nb = -(-N // mask_block)
        if mask.shape != (nb, nb):
            raise ValueError(f"block_mask must have shape [{nb}, {nb}]")
    return q, k, v, lens, mask, (B, H, N, d)


def fwd(q, k, v, causal: bool = False, scale: float | None = None, kv_lens=None,
        block_mask=None, mask_block: int = 128):
    """Return (O [B,H,N,d], LSE [B,H,N]) in float64."""
    q, k, v, lens, mask, (B, H, N, d) = _prep(q, k, v, kv_lens, block_mask, mask_block)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((B, H, N, d), np.float64)
    lse = np.empty((B, H, N), np.float64)
    rc = _load().fa_oracle_fwd(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(o, _dp),
                               _ptr(lse, _dp), B, H, N, d, int(bool(causal)), float(scale),
                               _ptr(lens, _i32p), _ptr(mask, _u8p), int(mask_block))
    if rc:
        raise RuntimeError(f"fa_oracle_fwd failed ({rc})")
    return o, lse


def fwd_rows(q, k, v, rows, causal: bool = False, scale: float | None = None, kv_lens=None,
             block_mask=None, mask_block: int = 128):
    """Forward for sampled rows only.  rows are flat indices (b*H + h)*N + i.
    Returns (O [len(rows), d], LSE [len(rows)])."""
    q, k, v, lens, mask, (B, H, N, d) = _prep(q, k, v, kv_lens, block_mask, mask_block)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.ascontiguousarray(np.asarray(rows), dtype=np.int64)
    o = np.empty((rows.size, d), np.float64)
    lse = np.empty((rows.size,), np.float64)
    rc = _load().fa_oracle_fwd_rows(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(o, _dp),
                                    _ptr(lse, _dp), B, H, N, d, int(bool(causal)), float(scale),
                                    _ptr(lens, _i32p), _ptr(mask, _u8p), int(mask_block),
                                    _ptr(rows, _i64p), rows.size)
    if rc:
        raise RuntimeError(f"fa_oracle_fwd_rows failed ({rc})")
    return o, lse


def bwd(q, k, v, dout, causal: bool = False, scale: float | None = None, kv_lens=None,
        block_mask=None, mask_block: int = 128):
    """Return (dQ, dK, dV [B,H,N,d], D [B,H,N]) in float64 for L = sum(O * dO)."""
    q, k, v, lens, mask, (B, H, N, d) = _prep(q, k, v, kv_lens, block_mask, mask_block)
    dout = _f64(dout)
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.empty_like(q)
    dk = np.empty_like(q)
    dv = np.empty_like(q)
    dvec = np.empty((B, H, N), np.float64)
    rc = _load().fa_oracle_bwd(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(dout, _dp),
                               _ptr(dq, _dp), _ptr(dk, _dp), _ptr(dv, _dp), _ptr(dvec, _dp),
                               B, H, N, d, int(bool(causal)), float(scale), _ptr(lens, _i32p),
                               _ptr(mask, _u8p), int(mask_block))
    if rc:
        raise RuntimeError(f"fa_oracle_bwd failed ({rc})")
    return dq, dk, dv, dvec


def bwd_sample(q, k, v, dout, qrows, krows, causal: bool = False, scale: float | None = None,
               kv_len: int | None = None, block_mask=None, mask_block: int = 128):
    """Backward of ONE head ([N, d] operands) for sampled rows.

    Returns (dQ[qrows], dK[krows], dV[krows]) in float64."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if q.ndim != 2 or not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("bwd_sample takes one head: q, k, v, dout of shape [N, d]")
    N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    mask = None
    if block_mask is not None:
        mask = np.ascontiguousarray(np.asarray(block_mask), dtype=np.uint8)
    qrows = np.ascontiguousarray(np.asarray(qrows), dtype=np.int64)
    krows = np.ascontiguousarray(np.asarray(krows), dtype=np.int64)
    dq = np.empty((qrows.size, d), np.float64)
    dk = np.empty((krows.size, d), np.float64)
    dv = np.empty((krows.size, d), np.float64)
    rc = _load().fa_oracle_bwd_sample(
        _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(dout, _dp), N, d, int(bool(causal)),
        float(scale), int(N if kv_len is None else kv_len), _ptr(mask, _u8p), int(mask_block),
        _ptr(qrows, _i64p), qrows.size, _ptr(dq, _dp), _ptr(krows, _i64p), krows.size,
        _ptr(dk, _dp), _ptr(dv, _dp))
    if rc:
        raise RuntimeError(f"fa_oracle_bwd_sample failed ({rc})")
    return dq, dk, dv


def decode(q, k, v, causal: bool = False, scale: float | None = None, kv_lens=None):
    """Decode-shaped forward: q [B,H,Nq,d] against k, v [B,H,Nk,d] whose first
    kv_lens[b] rows are filled.  The Nq queries are the newest positions
    (kv_len - Nq + t); with causal, query t sees keys j <= kv_len - Nq + t.
    Returns (O [B,H,Nq,d], LSE [B,H,Nq]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B,H,Nq,d] and k, v [B,H,Nk,d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lens = None
    if kv_lens is not None:
        lens = np.ascontiguousarray(np.asarray(kv_lens), dtype=np.int32)
        if lens.shape != (B,):
            raise ValueError("kv_lens must have shape [B]")
    o = np.empty((B, H, Nq, d), np.float64)
    lse = np.empty((B, H, Nq), np.float64)
    rc = _load().fa_oracle_decode(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(o, _dp),
                                  _ptr(lse, _dp), B, H, Nq, Nk, d, int(bool(causal)),
                                  float(scale), _ptr(lens, _i32p))
    if rc:
        raise RuntimeError(f"fa_oracle_decode failed ({rc})")
    return o, lse


def merge(o_parts, lse_parts):
    """Fold S partial (O, LSE) results over disjoint key sets: o_parts [S, R, d],
    lse_parts [S, R] (natural log, -inf = empty part).  Returns (O [R, d],
    LSE [R]) in float64."""
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    if o_parts.ndim != 3 or lse_parts.shape != o_parts.shape[:2]:
        raise ValueError("o_parts must be [S, R, d] and lse_parts [S, R]")
    S, R, d = o_parts.shape
    o = np.empty((R, d), np.float64)
    lse = np.empty((R,), np.float64)
    rc = _load().fa_oracle_merge(_ptr(o_parts, _dp), _ptr(lse_parts, _dp), S, R, d,
                                 _ptr(o, _dp), _ptr(lse, _dp))
    if rc:
        raise RuntimeError(f"fa_oracle_merge failed ({rc})")
    return o, lse
