"""GPU parity of the block-quantised FP8 path, through the C ABI.

  * fa_quantize_fp8 is byte work: its codes and descales must equal the
    oracle quantiser's bit for bit (per block and per head, with and without
    the Hadamard rotation, plain and transposed layouts, ragged N).
  * fa_fwd_fp8 runs on codes made by the oracle's quantiser on the CPU; its
    output is compared with exact attention of the dequantised inputs.  The
    bar, derived from the arithmetic (oracle.fp8.p_quant_bound): element by
    element, |O_gpu - O_ref| minus half a bf16 ulp of O_ref must not exceed
    the bound on what rounding the probabilities to E4M3 can change; LSE
    (taken before that rounding) within 1e-3.
  * incoherent processing: on inputs with outlier coordinates, the rotated
    FP8 result is closer to exact attention of the original inputs than the
    unrotated one (the pages report 2.6x lower error for their setup).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import fp8 as ofp8
from test_parity_gpu import half_ulp_bf16, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import exact_io_aware_36_amd as fa

    return fa


def check_bound(name, gpu, ref, bound):
    gpu = np.asarray(gpu, np.float64)
    assert np.isfinite(gpu).all(), f"{name}: non-finite output"
    excess = np.abs(gpu - ref) - half_ulp_bf16(ref) - bound
    err = np.abs(gpu - ref)
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"    {name}: max_abs={err.max():.3e} max(err/bound)={float((err / np.maximum(bound + half_ulp_bf16(ref), 1e-30)).max()):.3f} rel_l2={rel:.3e}")
    assert excess.max() <= 0.0, f"{name}: error exceeds the E4M3 probability bound by {excess.max()}"


def check_lse_bound(name, gpu, ref, bound):
    """FP8 LSE against the bound derived from the E4M3 product sums' measured
    truncation and the fp32 work after them (oracle.fp8.lse_bound_rows)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert (np.isneginf(gpu) == np.isneginf(ref)).all(), f"{name}: -inf rows differ"
    fin = np.isfinite(ref)
    err = np.abs(np.where(fin, gpu - ref, 0.0))
    ratio = float((err / np.maximum(bound, 1e-30))[fin].max()) if fin.any() else 0.0
    say(f"    {name}: max_abs={err.max():.3e} max(err/bound)={ratio:.3f} max bound={bound.max():.3e}")
    assert np.all(err[fin] <= bound[fin]), f"{name}: LSE error exceeds its bound ({ratio:.3f} of it)"


def qkv(B, H, N, d, seed, outliers=False):
    inp = workloads.random_qkv(B, H, N, d, seed)
    if outliers:   # a few large coordinates in Q and K (what rotation spreads out)
        for t in ("q", "k"):
            x = inp[t].float()
            x[..., :3] *= 20.0
            inp[t] = x.to(torch.bfloat16)
    return inp


QUANT_CASES = [
    # (B, H, N, d, block_rows, rotate, transpose)
    (2, 2, 300, 64, 128, False, False), (1, 3, 256, 128, 128, True, False),
    (2, 1, 200, 128, 128, True, False), (1, 2, 272, 64, 0, False, True),
    (2, 2, 512, 128, 0, False, True), (1, 1, 130, 128, 0, True, False), (1, 2, 16, 64, 128, False, True),
]


@pytest.mark.parametrize("case", range(len(QUANT_CASES)))
def test_quantize_bit_exact(fa, case):
    B, H, N, d, br, rot, tr = QUANT_CASES[case]
    say(f"  quantize B={B} H={H} N={N} d={d} block_rows={br} rotate={rot} transpose={tr}")
    x = qkv(B, H, N, d, 500 + case, outliers=case % 2 == 1)["q"]
    signs = workloads.random_signs(d, 600 + case) if rot else None
    x8, ds = fa.quantize_fp8(x.cuda(), block_rows=br, signs=None if signs is None else signs.cuda(),
                             transpose=tr)
    torch.cuda.synchronize()
    codes, dref = ofp8.quantize(x.float().numpy(), block_rows=br,
                                signs=None if signs is None else signs.numpy())
    got = x8.cpu().numpy()
    if tr:
        got = got.transpose(0, 1, 3, 2)
    nbad = int((got != codes).sum())
    say(f"    codes differing: {nbad} of {codes.size}")
    assert nbad == 0
    assert np.array_equal(ds.cpu().numpy().reshape(dref.shape), dref)


def oracle_inputs(inp, rot_seed=None):
    """Codes and descales from the oracle quantiser (CPU)."""
    d = inp["q"].shape[-1]
    signs = None if rot_seed is None else workloads.random_signs(d, rot_seed).numpy()
    q8, qs = ofp8.quantize(inp["q"].float().numpy(), 128, signs)
    k8, ks = ofp8.quantize(inp["k"].float().numpy(), 128, signs)
    v8, vs = ofp8.quantize(inp["v"].float().numpy(), 0)
    return q8, qs, k8, ks, v8, vs


def run_fp8(fa, q8, qs, k8, ks, v8, vs, causal, lens, scale=None):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o, lse = fa.fwd_fp8(dev(q8), dev(k8), dev(v8.transpose(0, 1, 3, 2)), dev(qs), dev(ks),
                        dev(vs.reshape(vs.shape[0], vs.shape[1])), causal=causal, scale=scale,
                        kv_lens=None if lens is None else lens.cuda())
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("shape", [(2, 2, 256, 64), (1, 2, 320, 128), (1, 1, 16, 128), (2, 1, 400, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_fwd_fp8_small(fa, shape, causal, padded):
    B, H, N, d = shape
    say(f"  fwd fp8 B={B} H={H} N={N} d={d} causal={causal} padded={padded}")
    inp = qkv(B, H, N, d, 700 + N + d + 2 * causal + padded)
    lens = workloads.random_lengths(B, 1, N, 800 + N) if padded else None
    q8, qs, k8, ks, v8, vs = oracle_inputs(inp, rot_seed=900 + N)
    o, lse = run_fp8(fa, q8, qs, k8, ks, v8, vs, causal, lens)
    O, L, (Q, K, V) = ofp8.reference(q8, k8, v8, qs, ks, vs, causal=causal,
                                     kv_lens=None if lens is None else lens.numpy())
    kvl = None if lens is None else lens.numpy()
    bound = ofp8.p_quant_bound(Q, K, V, L, causal=causal, kv_lens=kvl)
    check_bound("O", o, O, bound)
    check_lse_bound("LSE", lse, L, ofp8.lse_bound(q8, qs, k8, ks, L, causal=causal, kv_lens=kvl))


def test_fwd_fp8_deterministic(fa):
    inp = qkv(1, 2, 512, 128, 31)
    args = oracle_inputs(inp, rot_seed=32)
    o1, l1 = run_fp8(fa, *args, True, None)
    o2, l2 = run_fp8(fa, *args, True, None)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_incoherent_processing_lowers_error(fa):
    """Outlier coordinates in Q and K: quantising after the random-sign
    Hadamard rotation gives a result closer to exact attention of the
    original bf16 inputs than quantising the raw operands."""
    B, H, N, d = 1, 4, 512, 128
    inp = qkv(B, H, N, d, 41, outliers=True)
    O_exact, _ = oracle.fwd(inp["q"].double().numpy(), inp["k"].double().numpy(),
                            inp["v"].double().numpy(), causal=True)
    errs = {}
    for name, seed in (("plain", None), ("rotated", 42)):
        o, _ = run_fp8(fa, *oracle_inputs(inp, rot_seed=seed), True, None)
        errs[name] = float(np.linalg.norm(o - O_exact) / np.linalg.norm(O_exact))
    say(f"    rel-L2 vs exact attention of the bf16 inputs: plain {errs['plain']:.3e}, "
        f"rotated {errs['rotated']:.3e} ({errs['plain'] / errs['rotated']:.2f}x lower)")
    assert errs["rotated"] < errs["plain"]


def test_workload_long_context_fp8(fa):
    """The long-context causal shape (B1 H16 N16384 d128) in FP8: codes from
    the oracle quantiser (rotated Q, K), the bound checked on 256 sampled rows
    over every head."""
    w = workloads.WORKLOADS["long_context_fp8"]
    inp = workloads.make_inputs(w)
    say(f"  {w.name}")
    q8, qs, k8, ks, v8, vs = oracle_inputs(inp, rot_seed=w.seed)
    o, lse = run_fp8(fa, q8, qs, k8, ks, v8, vs, True, None)
    N, d = w.N, w.d
    Q = ofp8.dequantize(q8, qs)
    K = ofp8.dequantize(k8, ks)
    V = ofp8.dequantize(v8, vs, 0)
    rng = np.random.default_rng(3)
    for h in range(w.H):
        rows = np.concatenate([[0, N - 1], rng.choice(N, 14, replace=False)])
        Or, Lr = oracle.fwd_rows(Q[:, h:h + 1], K[:, h:h + 1], V[:, h:h + 1], rows, causal=True,
                                 scale=w.scale)
        bound = ofp8.p_quant_bound_rows(Q[0, h, rows], rows, K[0, h], V[0, h], Lr, causal=True,
                                        scale=w.scale)
        check_bound(f"O[h={h}]", o[0, h, rows], Or, bound)
        lb = ofp8.lse_bound_rows(q8[0, h, rows], rows, qs[0, h, rows // 128], k8[0, h],
                                 ks[0, h, np.arange(N) // 128], Lr, causal=True, scale=w.scale)
        check_lse_bound(f"LSE[h={h}]", lse[0, h, rows], Lr, lb)
