"""GPU parity of the split-KV decode forward and of the (O, LSE) merge kernel
against the fp64 oracle, through the C ABI.  Same bars as the other parity
tests: bf16 O relative L2 <= 5e-3 and max abs <= 1e-2 beyond half a bf16 ulp;
LSE max abs <= 1e-3; fp32 merge output max abs <= 1e-5."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from test_parity_gpu import FP32_MAX_ABS, check_bf16, check_lse, dev, f64, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import exact_io_aware_36_amd as fa

    return fa


def decode_case(B, H, Nq, Nk, d, seed):
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, Nq, d), generator=gen).to(torch.bfloat16)
    k = torch.randn((B, H, Nk, d), generator=gen).to(torch.bfloat16)
    v = torch.randn((B, H, Nk, d), generator=gen).to(torch.bfloat16)
    return q, k, v


CASES = [
    # (B, H, Nq, Nk, d, causal, lens, num_splits)
    (2, 3, 1, 300, 128, False, None, 0),
    (2, 3, 1, 300, 64, False, "rand", 0),
    (3, 2, 1, 1000, 128, False, "rand", 7),
    (2, 2, 3, 257, 128, True, "rand", 0),
    (2, 2, 5, 513, 64, True, None, 3),
    (1, 4, 8, 4097, 128, False, "rand", 0),
    (1, 3, 6, 700, 64, True, "rand", 0),
    (1, 2, 2, 1, 64, False, None, 0),
    (2, 1, 4, 40, 128, True, [40, 2], 1),        # batch 1: early queries see no key
    (2, 2, 1, 2048, 128, False, [0, 2048], 0),   # batch 0: empty cache
    (1, 2, 1, 300, 128, False, None, 1000),      # more splits asked than 32-key chunks
    (1, 1, 1, 20000, 64, False, None, 0),        # one (b, h): many splits
    (2, 2, 1, 1000, 256, False, "rand", 0),      # head dim 256 (32 lanes per key row)
    (1, 2, 5, 700, 256, True, "rand", 3),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_splitkv_small(fa, case):
    B, H, Nq, Nk, d, causal, lens, ns = CASES[case]
    say(f"  splitkv case {case}: B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} lens={lens} splits={ns}"
        f" -> S={fa.fa_splitkv_splits(B, H, Nk, ns)}")
    q, k, v = decode_case(B, H, Nq, Nk, d, 4000 + case)
    if lens == "rand":
        lens = workloads.random_lengths(B, 1, Nk, 4100 + case)
    elif lens is not None:
        lens = torch.tensor(lens, dtype=torch.int32)
    o, lse = fa.fwd_splitkv(dev(q), dev(k), dev(v), causal=causal, kv_lens=dev(lens), num_splits=ns)
    torch.cuda.synchronize()
    O, L = oracle.decode(f64(q), f64(k), f64(v), causal=causal, scale=1.0 / math.sqrt(d),
                         kv_lens=None if lens is None else lens.numpy())
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)


def test_splitkv_split_counts_and_determinism(fa):
    """Every split count gives the oracle's answer, and a repeated call is
    bitwise identical."""
    B, H, Nq, Nk, d = 2, 4, 2, 3000, 128
    q, k, v = decode_case(B, H, Nq, Nk, d, 4200)
    lens = workloads.random_lengths(B, 1000, Nk, 4201)
    O, L = oracle.decode(f64(q), f64(k), f64(v), kv_lens=lens.numpy())
    qd, kd, vd, ld = dev(q), dev(k), dev(v), dev(lens)
    for ns in (1, 2, 5, 16, 94, 0):
        o, lse = fa.fwd_splitkv(qd, kd, vd, kv_lens=ld, num_splits=ns)
        torch.cuda.synchronize()
        say(f"  num_splits={ns} -> S={fa.fa_splitkv_splits(B, H, Nk, ns)}")
        check_bf16("O", host(o), O)
        check_lse("LSE", host(lse), L)
    o1, l1 = fa.fwd_splitkv(qd, kd, vd, kv_lens=ld)
    o2, l2 = fa.fwd_splitkv(qd, kd, vd, kv_lens=ld)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def random_parts(S, R, d, seed):
    rng = np.random.default_rng(seed)
    po = rng.standard_normal((S, R, d)).astype(np.float32)
    pl = (rng.standard_normal((S, R)) * 4.0 + 10.0).astype(np.float32)
    empty = rng.random((S, R)) < 0.2
    pl[empty] = -np.inf
    pl[:, R // 2] = -np.inf          # one row with every part empty
    po[empty] = 1e30                 # an empty part's rows must be ignored
    return po, pl


@pytest.mark.parametrize("S,R,d", [(1, 5, 64), (3, 37, 128), (70, 300, 128), (2, 9, 100), (5, 2, 1024)])
def test_merge_kernel(fa, S, R, d):
    po, pl = random_parts(S, R, d, 4300 + S + d)
    O, L = oracle.merge(po, pl)
    tpo, tpl = torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda()
    o32, l32 = fa.merge(tpo, tpl, out_dtype=torch.float32)
    o16, l16 = fa.merge(tpo, tpl, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    err = float(np.abs(host(o32) - O).max())
    say(f"  merge S={S} R={R} d={d}: fp32 max_abs={err:.3e}")
    assert err <= FP32_MAX_ABS
    check_lse("LSE fp32 out", host(l32), L, tol=FP32_MAX_ABS * 10)
    check_bf16("O bf16", host(o16), O)
    assert np.all(host(o32)[R // 2] == 0.0) and np.isneginf(host(l32)[R // 2])


def test_workload_decode(fa):
    w = workloads.WORKLOADS["decode_splitkv"]
    inp = workloads.make_inputs(w)
    say(f"  {w.name}: S={fa.fa_splitkv_splits(w.B, w.H, w.N, 0)}")
    q, k, v, lens = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["kv_lens"])
    o, lse = fa.fwd_splitkv(q, k, v, kv_lens=lens)
    torch.cuda.synchronize()
    O, L = oracle.decode(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale=w.scale,
                         kv_lens=inp["kv_lens"].numpy())
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)
