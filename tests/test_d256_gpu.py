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
