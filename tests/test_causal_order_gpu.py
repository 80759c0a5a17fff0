"""GPU parity of the causal grids under each work order they can take.

A causal grid hands its (head, row block) items to workgroups in one of three
orders: heads of one XCD interleaved in groups sized to the XCD's L2 (the
last group of an XCD may hold fewer heads), head by head when a head has
fewer than four row blocks, and the plain XCD remap (or the identity) when
the heads do not split evenly over the 8 XCDs.  In the forward, when one
group holds all of an XCD's heads and its items overflow one round of
resident workgroups, the ranks that would start last are started first.
Each shape below reaches one of them.  Every output element is prefilled with NaN, so an item that no
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
    ("one group per XCD, ranks past the first round started first", 8, 16, 1024, 64),
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


def test_causal_grid_order_fp8(fa):
    """The FP8 forward's causal grid in groups of 2 heads with a last group of
    1 (24 heads at N = 8192, d = 128): every output written, sampled rows of
    every head within the quantisation bound of the FP8 parity tests."""
    import oracle.fp8 as ofp8
    from test_fp8_gpu import check_bound, oracle_inputs, qkv

    B, H, N, d = 1, 24, 8192, 128
    say(f"  causal order, fp8: B={B} H={H} N={N} d={d}")
    inp = qkv(B, H, N, d, 6100)
    q8, qs, k8, ks, v8, vs = oracle_inputs(inp, rot_seed=6101)
    cuda = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    fa.fa_fwd_fp8(cuda(q8), cuda(k8), cuda(v8.transpose(0, 1, 3, 2)), cuda(qs), cuda(ks),
                  cuda(vs.reshape(B, H)), o, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), "elements left unwritten"
    o, lse = host(o), host(lse)
    Q = ofp8.dequantize(q8, qs)
    K = ofp8.dequantize(k8, ks)
    V = ofp8.dequantize(v8, vs, 0)
    rng = np.random.default_rng(6102)
    for h in range(H):
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 6, replace=False)]))
        Or, Lr = oracle.fwd_rows(Q[:, h:h + 1], K[:, h:h + 1], V[:, h:h + 1], rows, causal=True,
                                 scale=scale)
        bound = ofp8.p_quant_bound_rows(Q[0, h, rows], rows, K[0, h], V[0, h], Lr, causal=True,
                                        scale=scale)
        check_bound(f"O[h={h}]", o[0, h, rows], Or, bound)
        check_lse(f"LSE[h={h}]", lse[0, h, rows], Lr)


@pytest.mark.parametrize("case", [c for c in CASES if c[4] <= 128][:3] + [c for c in CASES if c[4] == 256],
                         ids=lambda c: c[0])
def test_causal_grid_order_other_tiles(fa, case):
    """The forward's other key tiles (128 at d <= 128, 32 at d = 256) are
    separate kernel instances taking the same work orders."""
    label, B, H, N, d = case
    tile = 32 if d == 256 else 128
    say(f"  causal order, key tile {tile}: {label}: B={B} H={H} N={N} d={d}")
    inp = workloads.random_qkv(B, H, N, d, seed=7000 + H * 7 + N + d)
    q, k, v = (inp[n].contiguous().cuda() for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    o = nan_like(q)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_fwd_ex(q, k, v, o, lse, causal=True, scale=scale, tile_n=tile)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), "elements left unwritten"
    rng = np.random.default_rng(7001 + N + d)
    rows = np.concatenate([bh * N + np.unique(np.concatenate([[0, N - 1], rng.choice(N, 4, replace=False)]))
                           for bh in range(B * H)])
    qf, kf, vf = (f64(inp[n]) for n in ("q", "k", "v"))
    Or, Lr = oracle.fwd_rows(qf, kf, vf, rows, causal=True, scale=scale)
    check_bf16("O[rows]", host(o).reshape(-1, d)[rows], Or)
    check_lse("LSE[rows]", host(lse).reshape(-1)[rows], Lr)
