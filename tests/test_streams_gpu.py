"""The allocating wrappers of the binding on a side stream: outputs and the
backward workspace are allocated on the launch stream, so allocations the
current stream makes (and overwrites) while the side stream still runs
cannot take a block the kernels are using.  The result is compared bit for
bit with the same calls on the current stream, and with the fp64 oracle on
sampled rows."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def half_ulp_bf16(x):
    ax = np.abs(x)
    return np.where(ax > 0, np.exp2(np.floor(np.log2(np.where(ax > 0, ax, 1.0))) - 8), 0.0)


def test_fwd_bwd_on_side_stream():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import exact_io_aware_36_amd as fa

    B, H, N, d = 4, 16, 2048, 128
    say(f"  side stream fwd+bwd B={B} H={H} N={N} d={d} causal")
    inp = workloads.random_qkv(B, H, N, d, seed=9301, input_scale=0.5)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "dout"))
    o_ref, lse_ref = fa.fwd(q, k, v, causal=True)
    dq_ref, dk_ref, dv_ref = fa.bwd(q, k, v, o_ref, do, lse_ref, causal=True)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ws_bytes = fa.fa_bwd_workspace_bytes(B, H, N, d)
    outs = []
    for rep in range(3):
        o, lse = fa.fwd(q, k, v, causal=True, stream=side)
        dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=True, stream=side)
        # the current stream allocates blocks of the workspace's and outputs'
        # sizes and overwrites them while the side stream is still busy
        junk = [torch.full((ws_bytes // 4,), float("nan"), device="cuda") for _ in range(8)]
        junk += [torch.full_like(q, float("nan")) for _ in range(4)]
        del junk
        outs.append((o, lse, dq, dk, dv))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for o, lse, dq, dk, dv in outs:
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        assert torch.equal(dq, dq_ref) and torch.equal(dk, dk_ref) and torch.equal(dv, dv_ref)

    # and the reference itself against the oracle on sampled rows of two heads
    rng = np.random.default_rng(3)
    qf, kf, vf, dof = (inp[n].double().numpy() for n in ("q", "k", "v", "dout"))
    for b, h in ((0, 0), (B - 1, H - 1)):
        qr = np.concatenate([[0, N - 1], rng.choice(N, 30, replace=False)])
        kr = np.concatenate([[0, N - 1], rng.choice(N, 30, replace=False)])
        sq, sk, sv = oracle.bwd_sample(qf[b, h], kf[b, h], vf[b, h], dof[b, h], qr, kr,
                                       causal=True, scale=1.0 / np.sqrt(d))
        for name, got, ref in (("dQ", dq_ref[b, h, qr], sq), ("dK", dk_ref[b, h, kr], sk),
                               ("dV", dv_ref[b, h, kr], sv)):
            got = got.float().cpu().numpy().astype(np.float64)
            excess = float((np.abs(got - ref) - half_ulp_bf16(ref)).max())
            rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
            say(f"    {name}[{b},{h}]: beyond-half-ulp={excess:.3e} rel_l2={rel:.3e}")
            assert excess <= 1e-2 and rel <= 5e-3, name
