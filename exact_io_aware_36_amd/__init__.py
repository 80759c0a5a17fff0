"""Python binding of libfa.so, the gfx950 exact-attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/fa.h.  The functions named like
the C entry points (fa_fwd, fa_fwd_ex, fa_bwd, fa_bwd_ex, fa_bwd_workspace_bytes,
fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq, fa_fwd_blocksparse, fa_bwd_blocksparse,
fa_status_str)
take torch device tensors, read their shapes and pointers and call the C
function of the same name on the current torch stream (or the stream given).  fwd, bwd, fwd_blocksparse and
bwd_blocksparse are the same calls with the outputs (and the backward
workspace) allocated by torch.

There is no fallback: importing this package raises if libfa.so has not been
built, and every call raises FAError on a non-zero status.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

import torch  # loads torch's HIP runtime first, so libfa.so binds to the same one

__all__ = [
    "FAError", "fa_status_str", "fa_fwd", "fa_fwd_ex", "fa_bwd", "fa_bwd_workspace_bytes",
    "fa_bwd_ex", "fa_bwd_noalloc", "fa_bwd_noalloc_max_rows",
    "fa_fwd_blocksparse", "fa_bwd_blocksparse", "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq",
    "fwd", "bwd", "fwd_blocksparse", "bwd_blocksparse", "library_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libfa.so")

if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is missing: build it first (python -m exact_io_aware_36_amd.build)")

_lib = ctypes.CDLL(library_path)


def _check_single_hip_runtime():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        return
    if len(paths) > 1:
        raise ImportError(f"two HIP runtimes are loaded ({sorted(paths)}); import torch first")


_check_single_hip_runtime()

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_lib.fa_status_str.restype = ctypes.c_char_p
_lib.fa_status_str.argtypes = [_i]
_lib.fa_fwd.restype = _i
_lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _i, _vp]
_lib.fa_fwd_ex.restype = _i
_lib.fa_fwd_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _i, _i, _vp]
_lib.fa_bwd_workspace_bytes.restype = _sz
_lib.fa_bwd_workspace_bytes.argtypes = [_i, _i, _i, _i]
_lib.fa_bwd.restype = _i
_lib.fa_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                        _vp, _i, _vp, _sz, _vp]
_lib.fa_bwd_ex.restype = _i
_lib.fa_bwd_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                           _vp, _i, _i, _vp, _sz, _vp]
_lib.fa_bwd_noalloc.restype = _i
_lib.fa_bwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                _f, _vp, _i, _vp]
_lib.fa_bwd_noalloc_max_rows.restype = _i
_lib.fa_bwd_noalloc_max_rows.argtypes = []
_lib.fa_bwd_preprocess.restype = _i
_lib.fa_bwd_preprocess.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp]
_lib.fa_bwd_dkdv.restype = _i
_lib.fa_bwd_dkdv.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _i,
                             _vp, _sz, _vp]
_lib.fa_bwd_dq.restype = _i
_lib.fa_bwd_dq.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _i, _vp, _sz,
                           _vp]
_lib.fa_bwd_blocksparse.restype = _i
_lib.fa_bwd_blocksparse.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f,
                                    _vp, _i, _i, _vp, _sz, _vp]
_lib.fa_fwd_blocksparse.restype = _i
_lib.fa_fwd_blocksparse.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _vp, _i, _i, _vp]
_lib.fa_splitkv_splits.restype = _i
_lib.fa_splitkv_splits.argtypes = [_i, _i, _i, _i]
_lib.fa_fwd_splitkv_workspace_bytes.restype = _sz
_lib.fa_fwd_splitkv_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.fa_fwd_splitkv.restype = _i
_lib.fa_fwd_splitkv.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _i, _i,
                                _vp, _sz, _vp]
_lib.fa_quantize_fp8_workspace_bytes.restype = _sz
_lib.fa_quantize_fp8_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
_lib.fa_quantize_fp8.restype = _i
_lib.fa_quantize_fp8.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _vp, _sz, _vp]
_lib.fa_fwd_fp8.restype = _i
_lib.fa_fwd_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp]
_lib.fa_fwd_kvouter_workspace_bytes.restype = _sz
_lib.fa_fwd_kvouter_workspace_bytes.argtypes = [_i, _i, _i, _i]
_lib.fa_fwd_kvouter.restype = _i
_lib.fa_fwd_kvouter.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]
_lib.fa_merge.restype = _i
_lib.fa_merge.argtypes = [_vp, _vp, _i, _i, _i, _vp, _vp, _i, _vp]

FA_DTYPE_BF16 = 0
FA_DTYPE_FP32 = 1
_DTYPES = {torch.bfloat16: FA_DTYPE_BF16, torch.float32: FA_DTYPE_FP32}


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_str(status)}")


def fa_status_str(status: int) -> str:
    return _lib.fa_status_str(int(status)).decode()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor, stream):
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _shape(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    return tuple(int(x) for x in q.shape)


def _dtype(q: torch.Tensor) -> int:
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    return _DTYPES[q.dtype]


def _require(ok: bool, msg: str):
    if not ok:
        raise ValueError(msg)


def _same(q, *ts):
    for t in ts:
        _require(t.shape == q.shape and t.dtype == q.dtype and t.device == q.device,
                 "tensors must share shape, dtype and device")
        _require(t.is_contiguous(), "tensors must be contiguous")
    _require(q.is_contiguous(), "tensors must be contiguous")


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _check_rc(rc: int, where: str):
    if rc != 0:
        raise FAError(rc, where)


def fa_fwd_ex(q, k, v, o, lse, causal=False, scale=None, kv_lens=None, tile_n=0, stream=None):
    B, H, N, d = _shape(q)
    _same(q, k, v, o)
    _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * H * N,
             "lse must be contiguous fp32 [B, H, N]")
    if kv_lens is not None:
        _require(kv_lens.dtype == torch.int32 and kv_lens.numel() == B, "kv_lens must be int32 [B]")
    rc = _lib.fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)),
                        _scale(scale, d), _ptr(kv_lens), _dtype(q), int(tile_n), _stream(q, stream))
    _check_rc(rc, "fa_fwd_ex")


def fa_fwd(q, k, v, o, lse, causal=False, scale=None, kv_lens=None, stream=None):
    B, H, N, d = _shape(q)
    _same(q, k, v, o)
    _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * H * N,
             "lse must be contiguous fp32 [B, H, N]")
    if kv_lens is not None:
        _require(kv_lens.dtype == torch.int32 and kv_lens.numel() == B, "kv_lens must be int32 [B]")
    rc = _lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)),
                     _scale(scale, d), _ptr(kv_lens), _dtype(q), _stream(q, stream))
    _check_rc(rc, "fa_fwd")


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.fa_bwd_workspace_bytes(B, H, N, d))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal=False, scale=None, kv_lens=None,
           stream=None):
    B, H, N, d = _shape(q)
    _same(q, k, v, o, dout, dq, dk, dv)
    _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * H * N,
             "lse must be contiguous fp32 [B, H, N]")
    if kv_lens is not None:
        _require(kv_lens.dtype == torch.int32 and kv_lens.numel() == B, "kv_lens must be int32 [B]")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = _lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                     _ptr(dv), B, H, N, d, int(bool(causal)), _scale(scale, d), _ptr(kv_lens),
                     _dtype(q), _ptr(workspace), ws_bytes, _stream(q, stream))
    _check_rc(rc, "fa_bwd")


def fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal=False, scale=None,
              kv_lens=None, tile_n=0, stream=None):
    B, H, N, d = _shape(q)
    _same(q, k, v, o, dout, dq, dk, dv)
    _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * H * N,
             "lse must be contiguous fp32 [B, H, N]")
    if kv_lens is not None:
        _require(kv_lens.dtype == torch.int32 and kv_lens.numel() == B, "kv_lens must be int32 [B]")
    rc = _lib.fa_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                        _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)), _scale(scale, d),
                        _ptr(kv_lens), _dtype(q), int(tile_n), _ptr(workspace),
                        _ws_bytes(workspace), _stream(q, stream))
    _check_rc(rc, "fa_bwd_ex")


def fa_bwd_noalloc_max_rows() -> int:
    return int(_lib.fa_bwd_noalloc_max_rows())


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal=False, scale=None, kv_lens=None,
                   stream=None):
    B, H, N, d = _shape(q)
    _same(q, k, v, o, dout, dq, dk, dv)
    _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * H * N,
             "lse must be contiguous fp32 [B, H, N]")
    if kv_lens is not None:
        _require(kv_lens.dtype == torch.int32 and kv_lens.numel() == B, "kv_lens must be int32 [B]")
    rc = _lib.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                             _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)), _scale(scale, d),
                             _ptr(kv_lens), _dtype(q), _stream(q, stream))
    _check_rc(rc, "fa_bwd_noalloc")


def _ws_bytes(workspace):
    return workspace.numel() * workspace.element_size() if workspace is not None else 0


def fa_bwd_preprocess(o, dout, lse, workspace, stream=None):
    B, H, N, d = _shape(o)
    _same(o, dout)
    rc = _lib.fa_bwd_preprocess(_ptr(o), _ptr(dout), _ptr(lse), B, H, N, d, _dtype(o),
                                _ptr(workspace), _ws_bytes(workspace), _stream(o, stream))
    _check_rc(rc, "fa_bwd_preprocess")


def fa_bwd_dkdv(q, k, v, dout, lse, dk, dv, workspace, causal=False, scale=None, kv_lens=None,
                stream=None):
    B, H, N, d = _shape(q)
    _same(q, k, v, dout, dk, dv)
    rc = _lib.fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(dk), _ptr(dv), B, H,
                          N, d, int(bool(causal)), _scale(scale, d), _ptr(kv_lens), _dtype(q),
                          _ptr(workspace), _ws_bytes(workspace), _stream(q, stream))
    _check_rc(rc, "fa_bwd_dkdv")


def fa_bwd_dq(q, k, v, dout, lse, dq, workspace, causal=False, scale=None, kv_lens=None,
              stream=None):
    B, H, N, d = _shape(q)
    _same(q, k, v, dout, dq)
    rc = _lib.fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(dq), B, H, N, d,
                        int(bool(causal)), _scale(scale, d), _ptr(kv_lens), _dtype(q),
                        _ptr(workspace), _ws_bytes(workspace), _stream(q, stream))
    _check_rc(rc, "fa_bwd_dq")


def fa_fwd_blocksparse(q, k, v, o, lse, block_mask, mask_block=128, scale=None, stream=None):
    B, H, N, d = _shape(q)
    _same(q, k, v, o)
    _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * H * N,
             "lse must be contiguous fp32 [B, H, N]")
    _require(block_mask.dtype == torch.uint8 and block_mask.is_contiguous(),
             "block_mask must be contiguous uint8")
    nb = N // mask_block if mask_block > 0 else 0
    _require(block_mask.numel() == nb * nb, "block_mask must be [N/mask_block, N/mask_block]")
    rc = _lib.fa_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                 _scale(scale, d), _ptr(block_mask), int(mask_block), _dtype(q),
                                 _stream(q, stream))
    _check_rc(rc, "fa_fwd_blocksparse")


def fa_bwd_blocksparse(q, k, v, o, dout, lse, dq, dk, dv, workspace, block_mask, mask_block=128,
                       scale=None, stream=None):
    B, H, N, d = _shape(q)
    _same(q, k, v, o, dout, dq, dk, dv)
    _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * H * N,
             "lse must be contiguous fp32 [B, H, N]")
    _require(block_mask.dtype == torch.uint8 and block_mask.is_contiguous(),
             "block_mask must be contiguous uint8")
    nb = N // mask_block if mask_block > 0 else 0
    _require(block_mask.numel() == nb * nb, "block_mask must be [N/mask_block, N/mask_block]")
    rc = _lib.fa_bwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                 _ptr(dk), _ptr(dv), B, H, N, d, _scale(scale, d), _ptr(block_mask),
                                 int(mask_block), _dtype(q), _ptr(workspace), _ws_bytes(workspace),
                                 _stream(q, stream))
    _check_rc(rc, "fa_bwd_blocksparse")


def fa_splitkv_splits(B: int, H: int, Nk: int, num_splits: int = 0) -> int:
    return int(_lib.fa_splitkv_splits(B, H, Nk, num_splits))


def fa_fwd_splitkv_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int,
                                   num_splits: int = 0) -> int:
    return int(_lib.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits))


def fa_fwd_splitkv(q, k, v, o, lse, workspace, causal=False, scale=None, kv_lens=None,
                   num_splits=0, stream=None):
    B, H, Nq, d = _shape(q)
    Bk, Hk, Nk, dk = _shape(k)
    _require((Bk, Hk, dk) == (B, H, d), "k must be [B, H, Nk, d] with q's B, H, d")
    _same(k, v)
    _same(q, o)
    _require(k.dtype == q.dtype and k.device == q.device, "q and k must share dtype and device")
    _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * H * Nq,
             "lse must be contiguous fp32 [B, H, Nq]")
    if kv_lens is not None:
        _require(kv_lens.dtype == torch.int32 and kv_lens.numel() == B, "kv_lens must be int32 [B]")
    rc = _lib.fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                             int(bool(causal)), _scale(scale, d), _ptr(kv_lens), int(num_splits),
                             _dtype(q), _ptr(workspace), _ws_bytes(workspace), _stream(q, stream))
    _check_rc(rc, "fa_fwd_splitkv")


def fa_merge(o_parts, lse_parts, o, lse, stream=None):
    _require(o_parts.dim() == 3 and o_parts.dtype == torch.float32 and o_parts.is_contiguous(),
             "o_parts must be contiguous fp32 [S, R, d]")
    S, R, d = (int(x) for x in o_parts.shape)
    _require(lse_parts.dtype == torch.float32 and lse_parts.is_contiguous()
             and tuple(lse_parts.shape) == (S, R), "lse_parts must be contiguous fp32 [S, R]")
    _require(o.is_contiguous() and o.numel() == R * d, "o must be contiguous [R, d]")
    _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == R,
             "lse must be contiguous fp32 [R]")
    rc = _lib.fa_merge(_ptr(o_parts), _ptr(lse_parts), S, R, d, _ptr(o), _ptr(lse), _dtype(o),
                       _stream(o_parts, stream))
    _check_rc(rc, "fa_merge")


def fa_quantize_fp8_workspace_bytes(B: int, H: int, N: int, d: int, block_rows: int = 128) -> int:
    return int(_lib.fa_quantize_fp8_workspace_bytes(B, H, N, d, block_rows))


def fa_quantize_fp8(x, x8, descale, block_rows=128, signs=None, transpose=False, workspace=None,
                    stream=None):
    B, H, N, d = _shape(x)
    _require(x.dtype == torch.bfloat16 and x.is_contiguous(), "x must be contiguous bf16")
    _require(x8.dtype == torch.uint8 and x8.is_contiguous() and x8.numel() == x.numel(),
             "x8 must be contiguous uint8 with x's element count")
    nblk = (N + 127) // 128 if block_rows else 1
    _require(descale.dtype == torch.float32 and descale.is_contiguous()
             and descale.numel() == B * H * nblk, "descale has the wrong size")
    if signs is not None:
        _require(signs.dtype == torch.float32 and signs.numel() == d, "signs must be fp32 [d]")
    rc = _lib.fa_quantize_fp8(_ptr(x), _ptr(x8), _ptr(descale), B, H, N, d, int(block_rows),
                              _ptr(signs), int(bool(transpose)), _ptr(workspace),
                              _ws_bytes(workspace), _stream(x, stream))
    _check_rc(rc, "fa_quantize_fp8")


def fa_fwd_fp8(q8, k8, v8t, q_descale, k_descale, v_descale, o, lse, causal=False, scale=None,
               kv_lens=None, stream=None):
    B, H, N, d = _shape(o)
    for t in (q8, k8, v8t):
        _require(t.dtype == torch.uint8 and t.is_contiguous() and t.numel() == B * H * N * d,
                 "q8, k8, v8t must be contiguous uint8 with o's element count")
    _require(o.dtype == torch.bfloat16 and o.is_contiguous(), "o must be contiguous bf16")
    _require(lse.dtype == torch.float32 and lse.numel() == B * H * N, "lse must be fp32 [B, H, N]")
    rc = _lib.fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8t), _ptr(q_descale), _ptr(k_descale),
                         _ptr(v_descale), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)),
                         _scale(scale, d), _ptr(kv_lens), _stream(o, stream))
    _check_rc(rc, "fa_fwd_fp8")


# -- the same calls with torch-allocated outputs ------------------------------
#
# Outputs and workspaces are allocated on the stream the kernels run on, so
# that torch's caching allocator does not hand a workspace freed on return to
# another stream's allocation while the kernels still use it.

def _on_stream(t: torch.Tensor, stream):
    if stream is None:
        return contextlib.nullcontext()
    if isinstance(stream, torch.cuda.Stream):
        return torch.cuda.stream(stream)
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.stream(torch.cuda.ExternalStream(s, device=t.device))


def fwd(q, k, v, causal=False, scale=None, kv_lens=None, tile_n=0, stream=None):
    """Return (O, LSE)."""
    B, H, N, d = _shape(q)
    with _on_stream(q, stream):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        fa_fwd_ex(q, k, v, o, lse, causal=causal, scale=scale, kv_lens=kv_lens, tile_n=tile_n,
                  stream=stream)
    return o, lse


def bwd(q, k, v, o, dout, lse, causal=False, scale=None, kv_lens=None, tile_n=0, stream=None):
    """Return (dQ, dK, dV)."""
    B, H, N, d = _shape(q)
    with _on_stream(q, stream):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
        fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, ws, causal=causal, scale=scale,
                  kv_lens=kv_lens, tile_n=tile_n, stream=stream)
    return dq, dk, dv


def bwd_blocksparse(q, k, v, o, dout, lse, block_mask, mask_block=128, scale=None, stream=None):
    """Return (dQ, dK, dV) of the block-sparse forward."""
    B, H, N, d = _shape(q)
    with _on_stream(q, stream):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
        fa_bwd_blocksparse(q, k, v, o, dout, lse, dq, dk, dv, ws, block_mask,
                           mask_block=mask_block, scale=scale, stream=stream)
    return dq, dk, dv


def fwd_blocksparse(q, k, v, block_mask, mask_block=128, scale=None, stream=None):
    """Return (O, LSE)."""
    B, H, N, d = _shape(q)
    with _on_stream(q, stream):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        fa_fwd_blocksparse(q, k, v, o, lse, block_mask, mask_block=mask_block, scale=scale,
                           stream=stream)
    return o, lse


def fwd_splitkv(q, k, v, causal=False, scale=None, kv_lens=None, num_splits=0, stream=None):
    """Decode-shaped forward of q [B, H, Nq, d] against the cache k, v
    [B, H, Nk, d]; return (O [B, H, Nq, d], LSE [B, H, Nq])."""
    B, H, Nq, d = _shape(q)
    Nk = int(k.shape[2]) if k.dim() == 4 else 0
    with _on_stream(q, stream):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
        nbytes = fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
        fa_fwd_splitkv(q, k, v, o, lse, ws, causal=causal, scale=scale, kv_lens=kv_lens,
                       num_splits=num_splits, stream=stream)
    return o, lse


def merge(o_parts, lse_parts, out_dtype=torch.bfloat16, stream=None):
    """Combine partial results o_parts [S, R, d], lse_parts [S, R]; return
    (O [R, d] in out_dtype, LSE [R])."""
    S, R, d = (int(x) for x in o_parts.shape)
    with _on_stream(o_parts, stream):
        o = torch.empty((R, d), dtype=out_dtype, device=o_parts.device)
        lse = torch.empty((R,), dtype=torch.float32, device=o_parts.device)
        fa_merge(o_parts, lse_parts, o, lse, stream=stream)
    return o, lse


def quantize_fp8(x, block_rows=128, signs=None, transpose=False, stream=None):
    """Return (codes uint8, descale fp32) of bf16 x [B, H, N, d]."""
    B, H, N, d = _shape(x)
    shape = (B, H, d, N) if transpose else (B, H, N, d)
    with _on_stream(x, stream):
        x8 = torch.empty(shape, dtype=torch.uint8, device=x.device)
        nblk = (N + 127) // 128 if block_rows else 1
        descale = torch.empty((B, H, nblk) if block_rows else (B, H), dtype=torch.float32,
                              device=x.device)
        nbytes = fa_quantize_fp8_workspace_bytes(B, H, N, d, block_rows)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device) if nbytes else None
        fa_quantize_fp8(x, x8, descale, block_rows=block_rows, signs=signs, transpose=transpose,
                        workspace=ws, stream=stream)
    return x8, descale


def fa_fwd_kvouter_workspace_bytes(B, H, N, d):
    return int(_lib.fa_fwd_kvouter_workspace_bytes(int(B), int(H), int(N), int(d)))


def fa_fwd_kvouter(q, k, v, o, lse, workspace, causal=False, scale=None, stream=None):
    """The key/value-outer loop order (IO ablation): same outputs as fa_fwd."""
    B, H, N, d = _shape(q)
    _same(q, k, v, o)
    _require(q.dtype == torch.bfloat16, "the key/value-outer forward is bf16 only")
    _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * H * N,
             "lse must be contiguous fp32 [B, H, N]")
    rc = _lib.fa_fwd_kvouter(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                             int(bool(causal)), _scale(scale, d), _ptr(workspace),
                             _ws_bytes(workspace), _stream(q, stream))
    _check_rc(rc, "fa_fwd_kvouter")


def fwd_kvouter(q, k, v, causal=False, scale=None, stream=None):
    """Key/value-outer forward with its own workspace; return (O, LSE)."""
    B, H, N, d = _shape(q)
    nbytes = fa_fwd_kvouter_workspace_bytes(B, H, N, d)
    _require(nbytes > 0, "unsupported size for the key/value-outer forward")
    with _on_stream(q, stream):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        fa_fwd_kvouter(q, k, v, o, lse, ws, causal=causal, scale=scale, stream=stream)
    return o, lse
def fwd_fp8(q8, k8, v8t, q_descale, k_descale, v_descale, causal=False, scale=None, kv_lens=None,
            stream=None):
    """FP8 forward on quantised inputs; return (O bf16 [B, H, N, d], LSE)."""
    B, H, N, d = (int(x) for x in q8.shape)
    with _on_stream(q8, stream):
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
        fa_fwd_fp8(q8, k8, v8t, q_descale, k_descale, v_descale, o, lse, causal=causal,
                   scale=scale, kv_lens=kv_lens, stream=stream)
    return o, lse
