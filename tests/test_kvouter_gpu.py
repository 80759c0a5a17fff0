"""GPU parity of the key/value-outer forward (the IO ablation of the loop
order, fa_fwd_kvouter) against the fp64 oracle, through the C ABI, with the
forward's bars: bf16 O max abs <= 1e-2 beyond half a bf16 ulp and relative
L2 <= 5e-3, LSE max abs <= 1e-3."""
from __future__ import annotations

import pytest
import torch

import oracle
import workloads
from test_parity_gpu import check_bf16, check_lse, f64, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import exact_io_aware_36_amd as fa

    return fa


@pytest.mark.parametrize("shape", [(1, 1, 1, 64), (2, 3, 45, 128), (1, 2, 64, 64), (1, 2, 129, 128),
                                   (2, 2, 300, 64), (1, 2, 1000, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_kvouter_small(fa, shape, causal):
    B, H, N, d = shape
    say(f"  kv-outer B={B} H={H} N={N} d={d} causal={causal}")
    inp = workloads.random_qkv(B, H, N, d, seed=5000 + N + d + causal)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o, lse = fa.fwd_kvouter(q, k, v, causal=causal)
    torch.cuda.synchronize()
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal=causal)
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)


def test_kvouter_workspace_contents_do_not_matter(fa):
    """A workspace full of garbage (NaN bytes) gives the same output as a fresh one."""
    B, H, N, d = 1, 2, 200, 64
    inp = workloads.random_qkv(B, H, N, d, seed=5100)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    nbytes = fa.fa_fwd_kvouter_workspace_bytes(B, H, N, d)
    o1, l1 = torch.empty_like(q), torch.empty((B, H, N), device="cuda")
    o2, l2 = torch.empty_like(q), torch.empty((B, H, N), device="cuda")
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    fa.fa_fwd_kvouter(q, k, v, o1, l1, ws, causal=True)
    ws.fill_(0xFF)
    fa.fa_fwd_kvouter(q, k, v, o2, l2, ws, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
