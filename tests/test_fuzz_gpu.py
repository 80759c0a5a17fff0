"""Seeded random configurations of every entry point against the fp64
oracle, through the C ABI: shapes, head dimensions, masks, key lengths, key
tiles, backward query tiles, softmax scales and split counts drawn from one
fixed seed per case, so a run is reproducible and names its case.  Same bars
as the parity tests (bf16 O, dQ, dK, dV; LSE; every fourth dense case also
runs the fp32 forward on the same inputs at the fp32 bar); the FP8 forward
against the oracle's probability-rounding bound.  Sizes stay small enough
for the oracle to finish in seconds.

The dense draws include key lengths as short as one key: then every query
row of that batch puts its whole softmax on a handful of keys, and those
keys' dV and dK rows are sums of hundreds of order-one terms (|dV| near 10
at N = 511 with 5 keys).  A fixed absolute bar there measures the size of
the gradient, not the kernel, so each gradient element may also be off by
its first-order bf16 rounding bound (the larger of the two applies); the
relative L2 bar is unchanged."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as ofp8
import workloads
from test_fp8_gpu import check_bound, check_lse_bound, run_fp8
from test_parity_gpu import (BF16_MAX_ABS, BF16_REL_L2, FP32_MAX_ABS, check_bf16, check_lse, f64,
                              half_ulp_bf16, host, say)
from test_rescale_gpu import rounding_bounds

pytestmark = pytest.mark.gpu

N_CASES = 48


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import exact_io_aware_36_amd as fa

    return fa


def check_grad(name, gpu, ref, bound):
    """Per element: error beyond half an ulp of the bf16 output within the
    larger of the absolute bar and the first-order rounding bound; overall:
    the relative L2 bar."""
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == ref.shape, name
    assert np.isfinite(gpu).all(), f"{name}: non-finite output"
    diff = np.abs(gpu - ref)
    allowed = np.maximum(BF16_MAX_ABS, bound)
    excess = float((diff - half_ulp_bf16(ref) - allowed).max()) if diff.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(gpu - ref) / nrm) if nrm > 0 else float(np.linalg.norm(gpu))
    say(f"    {name}: max_abs={diff.max() if diff.size else 0:.3e} max_bound={float(bound.max()) if bound.size else 0:.3e} "
        f"excess={excess:.3e} rel_l2={rel:.3e}")
    assert excess <= 0.0, f"{name}: error beyond max(abs bar, rounding bound) by {excess}"
    assert rel <= BF16_REL_L2, f"{name}: relative L2 {rel} > {BF16_REL_L2}"


def draw(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128, 256]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    N = int(rng.integers(1, 700))
    return rng, B, H, N, d


@pytest.mark.parametrize("case", range(N_CASES))
def test_fuzz_dense_fwd_bwd(fa, case):
    rng, B, H, N, d = draw(7000 + case)
    causal = bool(rng.integers(0, 2))
    padded = bool(rng.integers(0, 2))
    tile = int(rng.choice([0, 32, 64] if d == 256 else [0, 32, 64, 128, 256]))
    scale = float(rng.uniform(0.5, 1.5)) / math.sqrt(d)
    say(f"  dense case {case}: B={B} H={H} N={N} d={d} causal={causal} padded={padded} tile={tile} scale={scale:.4f}")
    inp = workloads.random_qkv(B, H, N, d, seed=7100 + case, input_scale=float(rng.uniform(0.3, 1.0)))
    lens = workloads.random_lengths(B, 1, N, 7200 + case) if padded else None
    btile = int(rng.choice([0, 64, 128])) if d != 256 else 0
    say(f"    backward query tile {btile}")
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "dout"))
    dl = None if lens is None else lens.cuda()
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale, kv_lens=dl, tile_n=tile)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=causal, scale=scale, kv_lens=dl, tile_n=btile)
    torch.cuda.synchronize()
    ln = None if lens is None else lens.numpy()
    Q, K, V, dO = f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dout"])
    O, L = oracle.fwd(Q, K, V, causal=causal, scale=scale, kv_lens=ln)
    dQ, dK, dV, _ = oracle.bwd(Q, K, V, dO, causal=causal, scale=scale, kv_lens=ln)
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)
    bq, bk, bv = rounding_bounds(Q, K, V, dO, O, L, causal, scale, kv_lens=ln)
    check_grad("dQ", host(dq), dQ, bq)
    check_grad("dK", host(dk), dK, bk)
    check_grad("dV", host(dv), dV, bv)
    if d != 256 and case % 4 == 0:
        # the fp32 forward on the same (exactly representable) inputs and scale
        o32, lse32 = fa.fwd(q.float(), k.float(), v.float(), causal=causal, scale=scale, kv_lens=dl)
        torch.cuda.synchronize()
        d_o = float(np.abs(host(o32) - O).max())
        say(f"    fp32 forward: O max_abs={d_o:.3e}")
        assert d_o <= FP32_MAX_ABS
        check_lse("LSE fp32", host(lse32), L, tol=FP32_MAX_ABS)


@pytest.mark.parametrize("case", range(N_CASES // 2))
def test_fuzz_blocksparse(fa, case):
    rng = np.random.default_rng(7300 + case)
    d = int(rng.choice([64, 128, 256]))
    B, H = 1, int(rng.integers(1, 3))
    N = 128 * int(rng.integers(1, 6))        # the block-sparse entry points take N % 128 == 0
    nb = N // 128
    mask = (rng.random((nb, nb)) < rng.uniform(0.2, 0.9)).astype(np.uint8)
    scale = float(rng.uniform(0.5, 1.5)) / math.sqrt(d)
    say(f"  sparse case {case}: H={H} N={N} d={d} scale={scale:.4f} mask rows {mask.sum(axis=1).tolist()}")
    inp = workloads.random_qkv(B, H, N, d, seed=7400 + case)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "dout"))
    tm = torch.from_numpy(mask).cuda()
    o, lse = fa.fwd_blocksparse(q, k, v, tm, scale=scale)
    dq, dk, dv = fa.bwd_blocksparse(q, k, v, o, do, lse, tm, scale=scale)
    torch.cuda.synchronize()
    Q, K, V, dO = f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dout"])
    O, L = oracle.fwd(Q, K, V, block_mask=mask, scale=scale)
    dQ, dK, dV, _ = oracle.bwd(Q, K, V, dO, block_mask=mask, scale=scale)
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)
    check_bf16("dQ", host(dq), dQ)
    check_bf16("dK", host(dk), dK)
    check_bf16("dV", host(dv), dV)


@pytest.mark.parametrize("case", range(N_CASES // 2))
def test_fuzz_splitkv(fa, case):
    rng = np.random.default_rng(7500 + case)
    d = int(rng.choice([64, 128, 256]))
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    Nq, Nk = int(rng.integers(1, 9)), int(rng.integers(1, 6000))
    causal = bool(rng.integers(0, 2))
    ns = int(rng.choice([0, 0, 1, int(rng.integers(2, 50))]))
    gen = torch.Generator().manual_seed(7600 + case)
    q = torch.randn((B, H, Nq, d), generator=gen).to(torch.bfloat16)
    k = torch.randn((B, H, Nk, d), generator=gen).to(torch.bfloat16)
    v = torch.randn((B, H, Nk, d), generator=gen).to(torch.bfloat16)
    lens = workloads.random_lengths(B, 0, Nk, 7700 + case) if rng.integers(0, 2) else None
    scale = float(rng.uniform(0.5, 1.5)) / math.sqrt(d)
    say(f"  decode case {case}: B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} splits={ns} "
        f"scale={scale:.4f} lens={None if lens is None else lens.tolist()}")
    o, lse = fa.fwd_splitkv(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale,
                            kv_lens=None if lens is None else lens.cuda(), num_splits=ns)
    torch.cuda.synchronize()
    O, L = oracle.decode(f64(q), f64(k), f64(v), causal=causal, scale=scale,
                         kv_lens=None if lens is None else lens.numpy())
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)


@pytest.mark.parametrize("case", range(N_CASES // 3))
def test_fuzz_fp8_and_kvouter(fa, case):
    rng = np.random.default_rng(7800 + case)
    d = int(rng.choice([64, 128]))
    B, H = 1, int(rng.integers(1, 3))
    N = 16 * int(rng.integers(1, 40))
    causal = bool(rng.integers(0, 2))
    scale = float(rng.uniform(0.5, 1.5)) / math.sqrt(d)
    say(f"  fp8 / keys-outer case {case}: H={H} N={N} d={d} causal={causal} scale={scale:.4f}")
    inp = workloads.random_qkv(B, H, N, d, seed=7900 + case)
    signs = workloads.random_signs(d, 8000 + case).numpy()
    q8, qs = ofp8.quantize(inp["q"].float().numpy(), 128, signs)
    k8, ks = ofp8.quantize(inp["k"].float().numpy(), 128, signs)
    v8, vs = ofp8.quantize(inp["v"].float().numpy(), 0)
    o8, l8 = run_fp8(fa, q8, qs, k8, ks, v8, vs, causal, None, scale=scale)
    O8, L8, (Q8, K8, V8) = ofp8.reference(q8, k8, v8, qs, ks, vs, causal=causal, scale=scale,
                                          kv_lens=None)
    check_bound("O fp8", o8, O8, ofp8.p_quant_bound(Q8, K8, V8, L8, causal=causal, scale=scale,
                                                    kv_lens=None))
    check_lse_bound("LSE fp8", l8, L8, ofp8.lse_bound(q8, qs, k8, ks, L8, causal=causal, scale=scale))
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o, lse = fa.fwd_kvouter(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal=causal, scale=scale)
    check_bf16("O keys-outer", host(o), O)
    check_lse("LSE keys-outer", host(lse), L)
