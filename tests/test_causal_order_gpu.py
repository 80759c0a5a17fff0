"""GPU parity of the causal grids under each work order they can take.

A causal grid hands its (head, row block) items to workgroups in one of three
orders: heads of one XCD interleaved in groups sized to the XCD's L2 (the
last group of an XCD may hold fewer heads), head by head when a head has
fewer than four row blocks, and the plain XCD remap (or the identity) when
the heads do not split evenly over the 8 XCDs.  Each shape below reaches one
of them.  Every output element is prefilled with NaN, so an item that no
workgroup took shows up as a non-finite output; sampled rows of every head
(and the backward on three heads) are compared with the fp64 oracle at the
bf16 bars of the parity tests.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from test_parity_gpu import check_bf16, check_lse, f64, host, say

pytestmark = pytest.mark.gpu

CASES = [
    # (label, B, H, N, d)
    ("groups of 2 heads, last group of 1 (24 heads)", 1, 24, 8192, 64),
    ("one group of 2 heads", 2, 8, 2048, 128),
    ("groups at head dim 256", 1, 16, 1024, 256),
    ("three row blocks per head: head by head", 2, 8, 384, 64),
    ("6 heads: plain XCD remap", 1, 6, 1024, 128),
    ("5 heads x 5 blocks: identity order", 1, 5, 640, 64),
]


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import exact_io_aware_36_amd as fa

    return fa


def nan_like(t, dtype=None):
    return torch.full(t.shape, float("nan"), dtype=dtype or t.dtype, device=t.device)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_causal_grid_order(fa, case):
    label, B, H, N, d = case
    say(f"  causal order: {label}: B={B} H={H} N={N} d={d}")
    inp = workloads.random_qkv(B, H, N, d, seed=5000 + H * 7 + N + d)
    q, k, v, do = (inp[n].contiguous().cuda() for n in ("q", "k", "v", "dout"))
    scale = 1.0 / math.sqrt(d)
    o = nan_like(q)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_fwd(q, k, v, o, lse, causal=True, scale=scale)
    dq, dk, dv = nan_like(q), nan_like(q), nan_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=True, scale=scale)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert torch.isfinite(t).all(), f"{name}: elements left unwritten (NaN) or non-finite"

    # every head: its first and last rows (the shortest and the longest
    # block) and a few random rows
    rng = np.random.default_rng(B * 1000 + H * 10 + N + d)
    rows = []
    for bh in range(B * H):
        pick = np.concatenate([[0, N - 1, N // 2], rng.choice(N, 3, replace=False)])
        rows.append(bh * N + np.unique(pick))
    rows = np.concatenate(rows)
    qf, kf, vf, dof = (f64(inp[n]) for n in ("q", "k", "v", "dout"))
    Or, Lr = oracle.fwd_rows(qf, kf, vf, rows, causal=True, scale=scale)
    check_bf16("O[rows]", host(o).reshape(-1, d)[rows], Or)
    check_lse("LSE[rows]", host(lse).reshape(-1)[rows], Lr)

    # backward on the first head, a middle one and the last
    for bh in sorted({0, (B * H) // 2, B * H - 1}):
        b, h = divmod(bh, H)
        qr = np.unique(np.concatenate([[0, 1, N - 1], rng.choice(N, 13, replace=False)]))
        kr = np.unique(np.concatenate([[0, 1, N - 1], rng.choice(N, 13, replace=False)]))
        sq, sk, sv = oracle.bwd_sample(qf[b, h], kf[b, h], vf[b, h], dof[b, h], qr, kr,
                                       causal=True, scale=scale)
        check_bf16(f"dQ[{bh}]", host(dq)[b, h, qr], sq)
        check_bf16(f"dK[{bh}]", host(dk)[b, h, kr], sk)
        check_bf16(f"dV[{bh}]", host(dv)[b, h, kr], sv)
