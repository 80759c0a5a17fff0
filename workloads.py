"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: only shapes, seeds and random draws.
Both the oracle side and the GPU side take their inputs from here.

Recipe (every workload): one CPU ``torch.Generator`` seeded with the workload's
seed draws, in this order, Q, K, V (and dO when the workload has a backward)
as float32 ``randn`` of shape [B, H, N, d] (Q of a decode workload is
[B, H, nq, d] against an N-row cache), each multiplied by the workload's
input scale; then the key-padding lengths; then the block mask.  bf16
workloads cast the float32 draws to bf16 with round-to-nearest-even (torch's
``.to(torch.bfloat16)``).  The pages measure on GPT-2, BERT-large, Long Range
Arena and long-context training; these workloads stand in for them by shape
only, with no dataset.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "bf16" or "fp32"
    causal: bool
    seed: int
    input_scale: float = 1.0
    backward: bool = False
    kv_len_range: tuple | None = None   # inclusive (lo, hi) for key padding
    sparse_frac: float | None = None    # nonzero block fraction for block-sparse
    mask_block: int = 128
    nq: int | None = None                # decode: query rows per (b, h); N is then the cache length
    fp8: bool = False                    # run through the block-quantised FP8 forward
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)


# The five workloads of the measurement plan (shapes from the pages' workloads).
WORKLOADS = {
    "single_head_fp32": Workload("single_head_fp32", 1, 1, 256, 64, "fp32", False, 1001,
                                 note="single head, fp32, forward only"),
    "gpt2_medium_causal": Workload("gpt2_medium_causal", 8, 16, 1024, 64, "bf16", True, 1002,
                                   note="GPT-2-medium-shaped causal forward"),
    "bert_large_padded": Workload("bert_large_padded", 16, 16, 512, 64, "bf16", False, 1003,
                                  backward=True, kv_len_range=(384, 512),
                                  note="BERT-large-shaped fwd+bwd with key padding"),
    "long_context_causal": Workload("long_context_causal", 1, 16, 16384, 128, "bf16", True, 1004,
                                    input_scale=0.5, backward=True,
                                    note="long-context causal fwd+bwd, d=128"),
    "block_sparse": Workload("block_sparse", 4, 16, 4096, 64, "bf16", False, 1005,
                             sparse_frac=0.25,
                             note="block-sparse forward, 128x128 blocks, s=0.25"),
    # the same block-sparse shape with a backward pass (training-side use)
    "block_sparse_fwdbwd": Workload("block_sparse_fwdbwd", 4, 16, 4096, 64, "bf16", False, 1005,
                                    sparse_frac=0.25, backward=True,
                                    note="block-sparse forward + backward, s=0.25"),
    # the large head dimension at which the pages say the tiling loosens
    "d256_causal": Workload("d256_causal", 2, 16, 8192, 256, "bf16", True, 1007, input_scale=0.5,
                            note="causal forward at head dim 256"),
    # the same inputs with dO drawn after them, through forward and backward
    "d256_fwdbwd": Workload("d256_fwdbwd", 2, 16, 8192, 256, "bf16", True, 1007, input_scale=0.5,
                            backward=True, note="causal forward + backward at head dim 256"),
    # the long-context causal shape through the block-quantised FP8 forward
    # (Q, K rotated with random signs drawn after the mask, seed 1008)
    "long_context_fp8": Workload("long_context_fp8", 1, 16, 16384, 128, "bf16", True, 1008,
                                 input_scale=0.5, fp8=True,
                                 note="long-context causal forward, FP8 E4M3"),
    # one decode step: one new query row per (b, h) against a 16K-row cache
    # filled to a per-sequence length (the decoding case of the pages)
    "decode_splitkv": Workload("decode_splitkv", 8, 16, 16384, 128, "bf16", False, 1006,
                               kv_len_range=(8192, 16384), nq=1,
                               note="decode step, 1 query row vs a 16K cache, d=128"),
}


def torch_dtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def block_mask(nb: int, frac: float, gen: torch.Generator) -> torch.Tensor:
    """uint8 [nb, nb] mask: every diagonal block on, plus off-diagonal blocks
    drawn without replacement (one seeded permutation) until round(frac*nb*nb)
    blocks are on in total."""
    total = int(round(frac * nb * nb))
    if total < nb:
        raise ValueError("fraction too small to keep the diagonal")
    mask = torch.eye(nb, dtype=torch.uint8)
    off = [(i, j) for i in range(nb) for j in range(nb) if i != j]
    perm = torch.randperm(len(off), generator=gen)
    for t in perm[: total - nb].tolist():
        i, j = off[t]
        mask[i, j] = 1
    return mask


def make_inputs(w: Workload, *, B: int | None = None, H: int | None = None,
                N: int | None = None, seed: int | None = None) -> dict:
    """CPU tensors for workload ``w`` (optionally at a reduced B, H or N).

    Returns a dict with q, k, v (and dout), kv_lens (int32 [B] or None),
    block_mask (uint8 [N/mb, N/mb] or None), all on the CPU, in the workload
    dtype, plus the shape and flags."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    dt = torch_dtype(w)
    shape = (B, H, N, w.d)

    def draw(shp=shape):
        return (torch.randn(shp, generator=gen, dtype=torch.float32) * w.input_scale).to(dt)

    qshape = shape if w.nq is None else (B, H, w.nq, w.d)
    out = {"q": draw(qshape), "k": draw(), "v": draw()}
    out["dout"] = torch.randn(shape, generator=gen, dtype=torch.float32).to(dt) if w.backward else None
    kv_lens = None
    if w.kv_len_range is not None:
        lo, hi = w.kv_len_range
        lo, hi = min(lo, N), min(hi, N)
        kv_lens = torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int32)
    out["kv_lens"] = kv_lens
    mask = None
    if w.sparse_frac is not None:
        nb = N // w.mask_block
        mask = block_mask(nb, w.sparse_frac, gen)
    out["block_mask"] = mask
    out.update(B=B, H=H, N=N, d=w.d, causal=w.causal, scale=w.scale, dtype=w.dtype,
               mask_block=w.mask_block, nq=w.nq)
    return out


def random_qkv(B: int, H: int, N: int, d: int, seed: int, dtype=torch.bfloat16,
               input_scale: float = 1.0, with_dout: bool = True) -> dict:
    """Generic seeded q, k, v, dout (same recipe) for edge-case shapes."""
    gen = torch.Generator().manual_seed(seed)
    shape = (B, H, N, d)

    def draw():
        return (torch.randn(shape, generator=gen, dtype=torch.float32) * input_scale).to(dtype)

    out = {"q": draw(), "k": draw(), "v": draw()}
    out["dout"] = torch.randn(shape, generator=gen, dtype=torch.float32).to(dtype) if with_dout else None
    return out


def random_lengths(B: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    gen = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int32)


def random_signs(d: int, seed: int) -> torch.Tensor:
    """float32 [d] of +1/-1, each sign an independent fair draw (the random
    signs of the FP8 path's incoherent processing)."""
    gen = torch.Generator().manual_seed(seed)
    return (torch.randint(0, 2, (d,), generator=gen, dtype=torch.int32) * 2 - 1).to(torch.float32)


def random_block_mask(nb: int, frac: float, seed: int) -> torch.Tensor:
    return block_mask(nb, frac, torch.Generator().manual_seed(seed))
