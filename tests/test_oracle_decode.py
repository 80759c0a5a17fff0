"""Pins for the oracle's decode-shaped forward and its partial-result merge (no GPU).

The decode oracle is checked against a 40-digit decimal brute force written
from the definition (no max shift), the Q = 0 closed form, torch's fp64 CPU
attention with an explicit boolean mask, and the square causal oracle where the
two readings coincide.  The merge oracle is checked against the definition
itself: partial results over any partition of the keys, merged, must equal one
softmax over all of them ("FlashAttention: Mathematical Foundations ...",
section "Incremental Online Updates").  A plausible slip (the causal limit off
by one, the query position taken from the top instead of the bottom, a merge
weight exp(LSE_s) without the new normaliser, an empty part treated as
weight 1) fails at least one of these.
"""
from __future__ import annotations

import decimal
import itertools

import numpy as np
import pytest
import torch

import oracle

D = decimal.Decimal


def visible_keys(len_b, Nq, t, causal):
    """How many leading keys query t sees (a description of the input mask)."""
    n = len_b - Nq + t + 1 if causal else len_b
    return max(0, n)


def brute_decode(q, k, v, causal, scale, lens):
    decimal.getcontext().prec = 40
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    O = np.zeros((B, H, Nq, d))
    L = np.full((B, H, Nq), -np.inf)
    for b, h, t in itertools.product(range(B), range(H), range(Nq)):
        len_b = Nk if lens is None else min(lens[b], Nk)
        n = visible_keys(len_b, Nq, t, causal)
        if n == 0:
            continue
        ex = [(D(float(scale)) * sum(D(float(q[b, h, t, e])) * D(float(k[b, h, j, e]))
                                     for e in range(d))).exp() for j in range(n)]
        tot = sum(ex)
        for e in range(d):
            O[b, h, t, e] = float(sum(ex[j] * D(float(v[b, h, j, e])) for j in range(n)) / tot)
        L[b, h, t] = float(tot.ln())
    return O, L


CASES = [
    dict(Nq=1, Nk=5, causal=False, lens=None),
    dict(Nq=1, Nk=6, causal=True, lens=[6, 3]),
    dict(Nq=3, Nk=6, causal=True, lens=None),
    dict(Nq=3, Nk=6, causal=True, lens=[5, 2]),      # query 0 of batch 1 sees nothing
    dict(Nq=2, Nk=4, causal=False, lens=[4, 1]),
    dict(Nq=4, Nk=3, causal=True, lens=[3, 0]),      # more queries than keys, an empty cache
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_decode_brute_force_decimal(case):
    c = CASES[case]
    rng = np.random.default_rng(700 + case)
    B, H, d = 2, 2, 3
    q = rng.standard_normal((B, H, c["Nq"], d)) * 2.0
    k = rng.standard_normal((B, H, c["Nk"], d)) * 2.0
    v = rng.standard_normal((B, H, c["Nk"], d))
    scale = 0.7
    o, lse = oracle.decode(q, k, v, causal=c["causal"], scale=scale, kv_lens=c["lens"])
    bo, bl = brute_decode(q, k, v, c["causal"], scale, c["lens"])
    assert np.max(np.abs(o - bo)) < 1e-13
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(lse[~fin] == -np.inf)
    assert np.max(np.abs(lse[fin] - bl[fin])) < 1e-13


def test_decode_zero_query_closed_form():
    rng = np.random.default_rng(11)
    B, H, Nq, Nk, d = 3, 2, 4, 37, 8
    lens = [37, 20, 5]
    q = np.zeros((B, H, Nq, d))
    k = rng.standard_normal((B, H, Nk, d))
    v = rng.standard_normal((B, H, Nk, d))
    o, lse = oracle.decode(q, k, v, causal=True, kv_lens=lens)
    for b, h, t in itertools.product(range(B), range(H), range(Nq)):
        n = visible_keys(lens[b], Nq, t, True)
        assert np.allclose(o[b, h, t], v[b, h, :n].mean(axis=0), atol=1e-14)
        assert abs(lse[b, h, t] - np.log(n)) < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_decode_against_torch_fp64(causal):
    rng = np.random.default_rng(12 + causal)
    B, H, Nq, Nk, d = 2, 3, 5, 50, 16
    lens = [50, 33]
    q = rng.standard_normal((B, H, Nq, d))
    k = rng.standard_normal((B, H, Nk, d))
    v = rng.standard_normal((B, H, Nk, d))
    o, lse = oracle.decode(q, k, v, causal=causal, kv_lens=lens)
    mask = torch.zeros(B, 1, Nq, Nk, dtype=torch.bool)
    for b, t in itertools.product(range(B), range(Nq)):
        mask[b, 0, t, :visible_keys(lens[b], Nq, t, causal)] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask)
    assert np.max(np.abs(o - ref.numpy())) < 1e-12
    s = torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2) / np.sqrt(d)
    ref_lse = torch.logsumexp(s.masked_fill(~mask, -float("inf")), dim=-1)
    assert np.max(np.abs(lse - ref_lse.numpy())) < 1e-12


def test_decode_square_causal_matches_forward():
    """With Nq = Nk and a full cache, the bottom-right causal mask is the
    square causal mask of the forward oracle (pinned on its own)."""
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((2, 2, 9, 4)) for _ in range(3))
    o1, l1 = oracle.decode(q, k, v, causal=True)
    o2, l2 = oracle.fwd(q, k, v, causal=True)
    assert np.max(np.abs(o1 - o2)) < 1e-14 and np.max(np.abs(l1 - l2)) < 1e-14


def test_decode_query_position_is_bottom_aligned():
    """One query with causal on sees the whole filled cache (the newest
    position), not only key 0."""
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 1, 1, 4))
    k = rng.standard_normal((1, 1, 8, 4))
    v = rng.standard_normal((1, 1, 8, 4))
    o1, _ = oracle.decode(q, k, v, causal=True, kv_lens=[6])
    o2, _ = oracle.decode(q, k[:, :, :6], v[:, :, :6], causal=False)
    assert np.max(np.abs(o1 - o2)) < 1e-15


# ---------------------------------------------------------------- merge

def parts_over(q, k, v, bounds):
    """Oracle results of each key range [a, b) (non-causal), as [S, R, d], [S, R]."""
    B, H, Nq, d = q.shape
    os, ls = [], []
    for a, b in bounds:
        if a == b:
            os.append(np.zeros((B * H * Nq, d)))
            ls.append(np.full((B * H * Nq,), -np.inf))
            continue
        o, lse = oracle.decode(q, k[:, :, a:b], v[:, :, a:b])
        os.append(o.reshape(-1, d))
        ls.append(lse.reshape(-1))
    return np.stack(os), np.stack(ls)


@pytest.mark.parametrize("cuts", [[0, 40], [0, 1, 40], [0, 13, 14, 30, 40], [0, 0, 20, 20, 40],
                                  list(range(41))])
def test_merge_of_partitions_equals_one_softmax(cuts):
    rng = np.random.default_rng(20 + len(cuts))
    q = rng.standard_normal((2, 2, 3, 8)) * 1.5
    k = rng.standard_normal((2, 2, 40, 8)) * 1.5
    v = rng.standard_normal((2, 2, 40, 8))
    po, pl = parts_over(q, k, v, list(zip(cuts[:-1], cuts[1:])))
    o, lse = oracle.merge(po, pl)
    ro, rl = oracle.decode(q, k, v)
    assert np.max(np.abs(o - ro.reshape(-1, 8))) < 1e-13
    assert np.max(np.abs(lse - rl.reshape(-1))) < 1e-13


def test_merge_is_order_free_and_handles_large_lse():
    rng = np.random.default_rng(30)
    S, R, d = 6, 10, 5
    po = rng.standard_normal((S, R, d))
    pl = rng.standard_normal((S, R)) * 300.0      # e^LSE overflows fp64 without the shift
    o1, l1 = oracle.merge(po, pl)
    perm = rng.permutation(S)
    o2, l2 = oracle.merge(po[perm], pl[perm])
    assert np.all(np.isfinite(o1)) and np.all(np.isfinite(l1))
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12
    # against the direct closed form with the max taken out
    mx = pl.max(axis=0)
    w = np.exp(pl - mx)
    ref_l = mx + np.log(w.sum(axis=0))
    ref_o = np.einsum("sr,srd->rd", w, po) / w.sum(axis=0)[:, None]
    assert np.max(np.abs(o1 - ref_o)) < 1e-12 and np.max(np.abs(l1 - ref_l)) < 1e-12


def test_merge_special_cases():
    rng = np.random.default_rng(31)
    po = rng.standard_normal((3, 4, 2))
    pl = rng.standard_normal((3, 4))
    # one part is the identity
    o, l = oracle.merge(po[:1], pl[:1])
    assert np.array_equal(o, po[0]) and np.array_equal(l, pl[0])
    # two equal parts: same O, LSE + ln 2
    o, l = oracle.merge(np.stack([po[0], po[0]]), np.stack([pl[0], pl[0]]))
    assert np.max(np.abs(o - po[0])) < 1e-15 and np.max(np.abs(l - pl[0] - np.log(2))) < 1e-15
    # empty parts contribute nothing; all-empty rows give O = 0, LSE = -inf
    pl2 = pl.copy()
    pl2[1, :] = -np.inf
    pl2[:, 3] = -np.inf
    po2 = po.copy()
    po2[1] = 1e300          # an empty part's O must be ignored, whatever it holds
    o, l = oracle.merge(po2, pl2)
    o_ref, l_ref = oracle.merge(po[[0, 2]][:, :3], pl[[0, 2]][:, :3])
    assert np.max(np.abs(o[:3] - o_ref)) < 1e-15 and np.max(np.abs(l[:3] - l_ref)) < 1e-15
    assert np.all(o[3] == 0.0) and l[3] == -np.inf


def test_decode_bad_arguments_raise():
    q = np.zeros((1, 1, 2, 4))
    with pytest.raises(ValueError):
        oracle.decode(q, np.zeros((1, 1, 5, 3)), np.zeros((1, 1, 5, 3)))
    with pytest.raises(ValueError):
        oracle.merge(np.zeros((2, 3, 4)), np.zeros((3, 2)))
