"""GPU parity of the head-dimension-256 forward (dense, causal, padded,
block-sparse; key tiles 32 and 64) against the fp64 oracle, through the C
ABI.  Same bars as the other parity tests."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from test_parity_gpu import check_bf16, check_lse, dev, f64, host, run_fwd, say, small_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import exact_io_aware_36_amd as fa

    return fa


@pytest.mark.parametrize("shape", [(1, 2, 300, 256), (2, 1, 257, 256), (1, 1, 1, 256), (1, 2, 128, 256)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("tile_n", [32, 64])
def test_fwd_d256_small(fa, shape, causal, padded, tile_n):
    B, H, N, d = shape
    say(f"  fwd d256 B={B} H={H} N={N} causal={causal} padded={padded} tile={tile_n}")
    inp = small_case(B, H, N, d, causal, padded, seed=(N * 7 + causal * 3 + padded) % 10000)
    o, lse = run_fwd(fa, inp, tile_n)
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal=causal,
                      scale=inp["scale"], kv_lens=f64(inp["kv_lens"]))
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)


def test_blocksparse_d256(fa):
    N, d = 512, 256
    inp = workloads.random_qkv(2, 2, N, d, seed=256)
    mask = workloads.random_block_mask(N // 128, 0.5, seed=257)
    o, lse = fa.fwd_blocksparse(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(mask))
    torch.cuda.synchronize()
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), block_mask=mask.numpy(),
                      mask_block=128)
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)


def test_fwd_d256_deterministic(fa):
    inp = small_case(1, 2, 520, 256, True, True, seed=21)
    o1, l1 = run_fwd(fa, inp)
    o2, l2 = run_fwd(fa, inp)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("tile_n", [32, 64])
def test_workload_d256(fa, tile_n):
    """The head-dim-256 causal workload at full size; the oracle checks 512
    sampled rows spread over every head."""
    w = workloads.WORKLOADS["d256_causal"]
    inp = workloads.make_inputs(w)
    say(f"  {w.name} tile={tile_n}")
    o, lse = run_fwd(fa, inp, tile_n)
    B, H, N, d = w.B, w.H, w.N, w.d
    rng = np.random.default_rng(8)
    rows = np.concatenate([rng.choice(B * H * N, 500, replace=False),
                           [0, N - 1, N, B * H * N - 1] + [h * N + 127 for h in range(8)]])
    Or, Lr = oracle.fwd_rows(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), rows, causal=True,
                             scale=w.scale)
    check_bf16("O[rows]", host(o).reshape(-1, d)[rows], Or)
    check_lse("LSE[rows]", host(lse).reshape(-1)[rows], Lr)


# ---------------------------------------------------------------------------
# backward at head dim 256 (dV and dK in two launches)

@pytest.mark.parametrize("shape", [(1, 2, 300, 256), (2, 1, 257, 256), (1, 1, 1, 256)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_bwd_d256_small(fa, shape, causal, padded):
    B, H, N, d = shape
    say(f"  bwd d256 B={B} H={H} N={N} causal={causal} padded={padded}")
    inp = small_case(B, H, N, d, causal, padded, seed=(N * 11 + causal * 5 + padded) % 10000)
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    lens = dev(inp["kv_lens"])
    o, lse = fa.fwd(q, k, v, causal=causal, kv_lens=lens)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=causal, kv_lens=lens)
    torch.cuda.synchronize()
    dQ, dK, dV, _ = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dout"]),
                               causal=causal, kv_lens=f64(inp["kv_lens"]))
    check_bf16("dQ", host(dq), dQ)
    check_bf16("dK", host(dk), dK)
    check_bf16("dV", host(dv), dV)
    if padded:
        lens_h = inp["kv_lens"].numpy()
        for b in range(B):
            assert (host(dk)[b, :, lens_h[b]:] == 0).all()
            assert (host(dv)[b, :, lens_h[b]:] == 0).all()


def test_bwd_blocksparse_d256(fa):
    N, d = 384, 256
    inp = workloads.random_qkv(1, 2, N, d, seed=258)
    mask = torch.tensor([[1, 0, 1], [0, 1, 0], [1, 1, 1]], dtype=torch.uint8)
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    o, lse = fa.fwd_blocksparse(q, k, v, dev(mask))
    dq, dk, dv = fa.bwd_blocksparse(q, k, v, o, do, lse, dev(mask))
    torch.cuda.synchronize()
    dQ, dK, dV, _ = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dout"]),
                               block_mask=mask.numpy(), mask_block=128)
    check_bf16("dQ", host(dq), dQ)
    check_bf16("dK", host(dk), dK)
    check_bf16("dV", host(dv), dV)


def test_bwd_d256_deterministic(fa):
    inp = small_case(1, 2, 400, 256, True, False, seed=23)
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    o, lse = fa.fwd(q, k, v, causal=True)
    r1 = fa.bwd(q, k, v, o, do, lse, causal=True)
    r2 = fa.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_workload_d256_backward(fa):
    """The head-dim-256 causal workload with dO: dQ on 64 query rows and dK,
    dV on 64 key rows of two heads (oracle.bwd_sample)."""
    w = workloads.WORKLOADS["d256_fwdbwd"]
    inp = workloads.make_inputs(w)
    say(f"  {w.name}")
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    B, H, N, d = w.B, w.H, w.N, w.d
    rng = np.random.default_rng(9)
    qf, kf, vf, dof = (f64(inp[n]) for n in ("q", "k", "v", "dout"))
    for b, h in ((0, 0), (B - 1, H - 1)):
        qr = np.concatenate([[0, N - 1], rng.choice(N, 62, replace=False)])
        kr = np.concatenate([[0, N - 1], rng.choice(N, 62, replace=False)])
        sq, sk, sv = oracle.bwd_sample(qf[b, h], kf[b, h], vf[b, h], dof[b, h], qr, kr, causal=True,
                                       scale=w.scale)
        check_bf16(f"dQ[{b},{h}]", host(dq)[b, h, qr], sq)
        check_bf16(f"dK[{b},{h}]", host(dk)[b, h, kr], sk)
        check_bf16(f"dV[{b},{h}]", host(dv)[b, h, kr], sv)
