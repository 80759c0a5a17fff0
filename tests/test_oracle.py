"""Pins for the fp64 CPU oracle (no GPU).

Each check ties the oracle to something other than itself: a 40-digit decimal
brute force that computes softmax without the max shift, closed forms, the
two-block merge identity of "FlashAttention: Mathematical Foundations ..."
(section "Incremental Online Updates"), the running-statistics recurrence of
"The Attention Matrix You Never Write Down" (section "The running-statistics
trick"), invariances, finite differences of the oracle's own forward, and
torch's fp64 CPU attention with autograd.  A plausible slip in the oracle (a
dropped max shift, j < i instead of j <= i, a transposed score, a block mask
read as [j][i], a missing D term or scale in the backward) fails at least one
of these.
"""
from __future__ import annotations

import decimal
import itertools
import math

import numpy as np
import pytest
import torch

import oracle

D = decimal.Decimal


# --------------------------------------------------------------------------
# helpers that describe the inputs (masks), not the oracle's arithmetic

def allowed_matrix(N, causal, kv_len, mask, mb):
    A = np.ones((N, N), bool)
    if causal:
        A &= np.tril(np.ones((N, N), bool))
    A[:, kv_len:] = False
    if mask is not None:
        rb = np.arange(N) // mb
        A &= np.asarray(mask, bool)[rb[:, None], rb[None, :]]
    return A


def rand_case(rng, B, H, N, d, scale_in=1.0):
    q = rng.standard_normal((B, H, N, d)) * scale_in
    k = rng.standard_normal((B, H, N, d)) * scale_in
    v = rng.standard_normal((B, H, N, d))
    do = rng.standard_normal((B, H, N, d))
    return q, k, v, do


MODES = [
    dict(causal=False, lens=None, mask=None),
    dict(causal=True, lens=None, mask=None),
    dict(causal=False, lens=[3, 5], mask=None),
    dict(causal=True, lens=[4, 2], mask=None),
    # asymmetric block mask (mb=2 on N=6: 3x3 blocks), diagonal on
    dict(causal=False, lens=None, mask=[[1, 0, 1], [1, 1, 0], [0, 0, 1]]),
    dict(causal=False, lens=[6, 5], mask=[[1, 1, 0], [0, 1, 0], [1, 0, 1]]),
]


# --------------------------------------------------------------------------
# 1. brute force in 40-digit decimal, softmax as exp(s)/sum(exp(s)) with no
#    max shift (decimal's exponent range cannot overflow here)

def brute_fwd(q, k, v, causal, scale, lens, mask, mb):
    decimal.getcontext().prec = 40
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    L = np.full((B, H, N), -np.inf)
    sc = D(float(scale))
    for b, h, i in itertools.product(range(B), range(H), range(N)):
        kvl = N if lens is None else lens[b]
        A = allowed_matrix(N, causal, kvl, mask, mb)
        ex = {}
        for j in range(N):
            if A[i, j]:
                s = sc * sum(D(float(q[b, h, i, t])) * D(float(k[b, h, j, t])) for t in range(d))
                ex[j] = s.exp()
        if not ex:
            continue
        Z = sum(ex.values())
        for t in range(d):
            O[b, h, i, t] = float(sum(ex[j] / Z * D(float(v[b, h, j, t])) for j in ex))
        L[b, h, i] = float(Z.ln())
    return O, L


@pytest.mark.parametrize("mode", range(len(MODES)))
def test_brute_force_decimal(mode):
    m = MODES[mode]
    rng = np.random.default_rng(100 + mode)
    B, H, N, d = 2, 1, 6, 3
    q, k, v, _ = rand_case(rng, B, H, N, d)
    scale = 0.7
    O, L = oracle.fwd(q, k, v, causal=m["causal"], scale=scale, kv_lens=m["lens"],
                      block_mask=m["mask"], mask_block=2)
    Ob, Lb = brute_fwd(q, k, v, m["causal"], scale, m["lens"], m["mask"], 2)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-13)


def test_brute_force_large_scores():
    """Scores near 2000: exp without the max shift overflows fp64, so an
    oracle that dropped the shift returns inf/nan here."""
    rng = np.random.default_rng(7)
    q, k, v, _ = rand_case(rng, 1, 1, 5, 3, scale_in=25.0)
    O, L = oracle.fwd(q, k, v, causal=False, scale=1.0)
    Ob, Lb = brute_fwd(q, k, v, False, 1.0, None, None, 1)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    assert np.abs(Lb).max() > 710  # exp(Lb) would overflow a double
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=1e-14, atol=0)


def test_nonsquare_scores_not_transposed():
    """q and k with different content and a causal mask: the score for (i, j)
    must be q_i . k_j, not q_j . k_i (caught by the brute force too, this is
    a small explicit case with d = 1)."""
    q = np.array([1.0, 2.0, 3.0]).reshape(1, 1, 3, 1)
    k = np.array([0.5, -1.0, 0.25]).reshape(1, 1, 3, 1)
    v = np.array([1.0, 10.0, 100.0]).reshape(1, 1, 3, 1)
    O, L = oracle.fwd(q, k, v, causal=True, scale=1.0)
    # row 1 sees keys 0, 1: scores 2*0.5 = 1 and 2*(-1) = -2
    w0, w1 = math.exp(1.0), math.exp(-2.0)
    assert abs(O[0, 0, 1, 0] - (w0 * 1 + w1 * 10) / (w0 + w1)) < 1e-14
    assert abs(L[0, 0, 1] - math.log(w0 + w1)) < 1e-14
    # row 0 sees key 0 only
    assert abs(O[0, 0, 0, 0] - 1.0) < 1e-15 and abs(L[0, 0, 0] - 0.5) < 1e-15


def test_hand_worked_example():
    """d = 1, scale 1: scores 0 and ln 3 give weights 1/4 and 3/4, so
    O = 4/4 + 3*8/4 = 7 and LSE = ln(1 + 3) = ln 4."""
    q = np.array([1.0]).reshape(1, 1, 1, 1)
    q = np.concatenate([q, q], axis=2)
    k = np.array([0.0, math.log(3.0)]).reshape(1, 1, 2, 1)
    v = np.array([4.0, 8.0]).reshape(1, 1, 2, 1)
    O, L = oracle.fwd(q, k, v, causal=False, scale=1.0)
    assert abs(O[0, 0, 0, 0] - 7.0) < 1e-14
    assert abs(L[0, 0, 0] - math.log(4.0)) < 1e-14
    O, L = oracle.fwd(q, k, v, causal=True, scale=1.0)
    assert abs(O[0, 0, 0, 0] - 4.0) < 1e-15 and abs(L[0, 0, 0]) < 1e-15
    assert abs(O[0, 0, 1, 0] - 7.0) < 1e-14


# --------------------------------------------------------------------------
# 2. normalisation: rows of P sum to 1 ("01 · FlashAttention", step 2 of 5)

@pytest.mark.parametrize("mode", range(len(MODES)))
def test_rows_sum_to_one(mode):
    m = MODES[mode]
    rng = np.random.default_rng(200 + mode)
    q, k, v, _ = rand_case(rng, 2, 2, 6, 4)
    ones = np.ones_like(v)
    O, _ = oracle.fwd(q, k, ones, causal=m["causal"], kv_lens=m["lens"],
                      block_mask=m["mask"], mask_block=2)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-12)
    # convex combination: every output lies between the min and max of the
    # allowed values
    O, _ = oracle.fwd(q, k, v, causal=m["causal"], kv_lens=m["lens"],
                      block_mask=m["mask"], mask_block=2)
    for b, h in itertools.product(range(2), range(2)):
        kvl = 6 if m["lens"] is None else m["lens"][b]
        A = allowed_matrix(6, m["causal"], kvl, m["mask"], 2)
        for i in range(6):
            vs = v[b, h][A[i]]
            assert (O[b, h, i] >= vs.min(0) - 1e-12).all()
            assert (O[b, h, i] <= vs.max(0) + 1e-12).all()


# --------------------------------------------------------------------------
# 3. closed forms

@pytest.mark.parametrize("mode", range(len(MODES)))
def test_closed_form_zero_queries(mode):
    """Q = 0: every allowed score is 0, so O_i is the mean of the allowed
    v_j and LSE_i = ln |A_i|."""
    m = MODES[mode]
    rng = np.random.default_rng(300 + mode)
    _, k, v, _ = rand_case(rng, 2, 1, 6, 3)
    q = np.zeros_like(k)
    O, L = oracle.fwd(q, k, v, causal=m["causal"], kv_lens=m["lens"],
                      block_mask=m["mask"], mask_block=2)
    for b in range(2):
        kvl = 6 if m["lens"] is None else m["lens"][b]
        A = allowed_matrix(6, m["causal"], kvl, m["mask"], 2)
        for i in range(6):
            n = A[i].sum()
            np.testing.assert_allclose(O[b, 0, i], v[b, 0][A[i]].mean(0), atol=1e-14, rtol=0)
            assert abs(L[b, 0, i] - math.log(n)) < 1e-14


@pytest.mark.parametrize("mode", range(len(MODES)))
def test_closed_form_identical_keys(mode):
    """All keys equal to one vector kappa: every allowed score of row i is
    scale * q_i . kappa, so O_i is the mean of the allowed v_j and
    LSE_i = scale * q_i . kappa + ln |A_i|."""
    m = MODES[mode]
    rng = np.random.default_rng(400 + mode)
    q, _, v, _ = rand_case(rng, 2, 1, 6, 3)
    kappa = rng.standard_normal(3)
    k = np.broadcast_to(kappa, q.shape).copy()
    scale = 0.9
    O, L = oracle.fwd(q, k, v, causal=m["causal"], scale=scale, kv_lens=m["lens"],
                      block_mask=m["mask"], mask_block=2)
    for b in range(2):
        kvl = 6 if m["lens"] is None else m["lens"][b]
        A = allowed_matrix(6, m["causal"], kvl, m["mask"], 2)
        for i in range(6):
            n = A[i].sum()
            np.testing.assert_allclose(O[b, 0, i], v[b, 0][A[i]].mean(0), atol=1e-13, rtol=0)
            want = scale * float(q[b, 0, i] @ kappa) + math.log(n)
            assert abs(L[b, 0, i] - want) < 1e-13


def test_fully_masked_row_reading():
    """A row with no allowed key (reachable only through a block mask with an
    empty row): O = 0, LSE = -inf, zero gradients."""
    rng = np.random.default_rng(5)
    q, k, v, do = rand_case(rng, 1, 1, 4, 2)
    mask = [[0, 0], [1, 1]]
    O, L = oracle.fwd(q, k, v, block_mask=mask, mask_block=2)
    assert (O[0, 0, :2] == 0).all() and np.isneginf(L[0, 0, :2]).all()
    assert np.isfinite(L[0, 0, 2:]).all()
    dq, dk, dv, _ = oracle.bwd(q, k, v, do, block_mask=mask, mask_block=2)
    assert (dq[0, 0, :2] == 0).all()


def test_lse_bounds():
    """max_j s_ij <= LSE_i <= max_j s_ij + ln |A_i|."""
    rng = np.random.default_rng(11)
    q, k, v, _ = rand_case(rng, 1, 2, 9, 4)
    for causal in (False, True):
        O, L = oracle.fwd(q, k, v, causal=causal, scale=0.5)
        for h in range(2):
            S = 0.5 * q[0, h] @ k[0, h].T
            A = allowed_matrix(9, causal, 9, None, 1)
            for i in range(9):
                mx = S[i][A[i]].max()
                assert mx - 1e-12 <= L[0, h, i] <= mx + math.log(A[i].sum()) + 1e-12


def test_key_permutation_invariance():
    """Non-causal, no padding: permuting the rows of K and V by one
    permutation leaves O and LSE unchanged; dQ is unchanged and dK, dV are
    permuted the same way."""
    rng = np.random.default_rng(12)
    q, k, v, do = rand_case(rng, 2, 2, 7, 3)
    perm = rng.permutation(7)
    O1, L1 = oracle.fwd(q, k, v)
    O2, L2 = oracle.fwd(q, k[:, :, perm], v[:, :, perm])
    np.testing.assert_allclose(O1, O2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(L1, L2, atol=1e-13, rtol=0)
    dq1, dk1, dv1, _ = oracle.bwd(q, k, v, do)
    dq2, dk2, dv2, _ = oracle.bwd(q, k[:, :, perm], v[:, :, perm], do)
    np.testing.assert_allclose(dq1, dq2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(dk1[:, :, perm], dk2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(dv1[:, :, perm], dv2, atol=1e-13, rtol=0)


# --------------------------------------------------------------------------
# 4. the two-block merge and the running-statistics recurrence, checked
#    against the oracle's one-shot softmax

def _block_stats(s, vv):
    m = s.max()
    e = np.exp(s - m)
    return m, e.sum(), e @ vv  # (m, l, unnormalised output)


def test_two_block_merge_equals_one_shot():
    """Split each row's keys into [0, c) and [c, N) at every c, take each
    block's (m, l, O) and merge with m_new = max(m1, m2),
    l_new = l1 e^(m1 - m_new) + l2 e^(m2 - m_new) and the output update in its
    overflow-safe form (block 2's exponentials taken against m_new).  The
    result must equal the oracle's one-shot softmax."""
    rng = np.random.default_rng(13)
    N, d, scale = 9, 4, 0.8
    q, k, v, _ = rand_case(rng, 1, 1, N, d, scale_in=2.0)
    O, L = oracle.fwd(q, k, v, scale=scale)
    for i in range(N):
        s = scale * (k[0, 0] @ q[0, 0, i])
        for c in range(1, N):
            m1, l1, o1 = _block_stats(s[:c], v[0, 0, :c])
            m2, l2, o2 = _block_stats(s[c:], v[0, 0, c:])
            mn = max(m1, m2)
            ln = l1 * math.exp(m1 - mn) + l2 * math.exp(m2 - mn)
            # the page's normalised form: O1 normalised by l1, block-2 sum
            # of exp(x_j - m_new) v_j, everything divided by l_new
            O1n = o1 / l1
            On = (l1 * math.exp(m1 - mn) / ln) * O1n + np.exp(s[c:] - mn) @ v[0, 0, c:] / ln
            np.testing.assert_allclose(On, O[0, 0, i], atol=1e-13, rtol=0)
            assert abs(mn + math.log(ln) - L[0, 0, i]) < 1e-13


def test_printed_merge_form_overflows():
    """The page prints block 2's term as exp(-m_new) * sum exp(x_j) v_j.  That
    is algebraically the same but overflows for large scores, which is why
    the safe form (exp(x_j - m_new)) is the one read and used."""
    s2 = np.array([800.0, 801.0])
    with np.errstate(over="ignore", invalid="ignore"):
        literal = math.exp(-801.0) * np.exp(s2).sum()
    safe = np.exp(s2 - 801.0).sum()
    assert not np.isfinite(literal) or literal == 0.0
    assert np.isfinite(safe) and safe > 1.0


@pytest.mark.parametrize("bc", [1, 2, 3, 4, 7])
def test_running_recurrence_equals_one_shot(bc):
    """The four steps of the running-statistics trick over key blocks of
    size bc: new max m' = max(m, block max), rescale l and the output by
    e^(m - m'), add the block's exponentials taken against m', divide by l at
    the end.  Equal to the oracle for every block size, with causal and
    padded keys."""
    rng = np.random.default_rng(14 + bc)
    N, d, scale = 11, 3, 0.6
    q, k, v, _ = rand_case(rng, 1, 1, N, d, scale_in=1.5)
    for causal, kvl in [(False, N), (True, N), (False, 8), (True, 6)]:
        O, L = oracle.fwd(q, k, v, causal=causal, scale=scale, kv_lens=[kvl])
        A = allowed_matrix(N, causal, kvl, None, 1)
        for i in range(N):
            m, l, acc = -np.inf, 0.0, np.zeros(d)
            for j0 in range(0, N, bc):
                js = [j for j in range(j0, min(j0 + bc, N)) if A[i, j]]
                if not js:
                    continue
                s = scale * (k[0, 0, js] @ q[0, 0, i])
                mp = max(m, s.max())
                alpha = math.exp(m - mp) if np.isfinite(m) else 0.0
                p = np.exp(s - mp)
                l = alpha * l + p.sum()
                acc = alpha * acc + p @ v[0, 0, js]
                m = mp
            np.testing.assert_allclose(acc / l, O[0, 0, i], atol=1e-13, rtol=0)
            assert abs(m + math.log(l) - L[0, 0, i]) < 1e-13


def test_garbled_update_reading_is_wrong():
    """The page's Algorithm-1 output update prints the rescale factor with an
    inverse (multiply by e^(m_new - m)).  Run that way the recurrence
    disagrees with the one-shot softmax whenever the max grows, while the
    reading without the inverse agrees (previous test)."""
    rng = np.random.default_rng(21)
    N, d = 6, 2
    q, k, v, _ = rand_case(rng, 1, 1, N, d, scale_in=2.0)
    O, _ = oracle.fwd(q, k, v, scale=1.0)
    worst = 0.0
    for i in range(N):
        m, l, acc = -np.inf, 0.0, np.zeros(d)
        for j in range(N):
            s = float(k[0, 0, j] @ q[0, 0, i])
            mp = max(m, s)
            fac = math.exp(mp - m) if np.isfinite(m) else 0.0  # the inverse
            l = (math.exp(m - mp) if np.isfinite(m) else 0.0) * l + math.exp(s - mp)
            acc = fac * acc + math.exp(s - mp) * v[0, 0, j]
            m = mp
        worst = max(worst, np.abs(acc / l - O[0, 0, i]).max())
    assert worst > 1e-3


# --------------------------------------------------------------------------
# 5. backward: finite differences of the oracle's forward, invariances

def _loss(q, k, v, do, **kw):
    O, _ = oracle.fwd(q, k, v, **kw)
    return float((O * do).sum())


@pytest.mark.parametrize("case", [
    dict(causal=False), dict(causal=True), dict(kv_lens=[5]),
    dict(causal=True, kv_lens=[6]), dict(block_mask=[[1, 0], [1, 1]], mask_block=4),
])
def test_backward_finite_differences(case):
    rng = np.random.default_rng(31)
    q, k, v, do = rand_case(rng, 1, 1, 8, 4)
    kw = dict(scale=0.55, **case)
    dq, dk, dv, _ = oracle.bwd(q, k, v, do, **kw)
    h = 1e-6
    for name, X, G in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(X)
        for idx in itertools.product(*[range(s) for s in X.shape]):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = dict(q=q, k=k, v=v)
            args_m = dict(q=q, k=k, v=v)
            args_p[name], args_m[name] = Xp, Xm
            fd[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, **kw)
                       - _loss(args_m["q"], args_m["k"], args_m["v"], do, **kw)) / (2 * h)
        err = np.abs(fd - G).max() / max(1.0, np.abs(G).max())
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("mode", range(len(MODES)))
def test_backward_invariants(mode):
    """sum_j dS_ij = 0 for every row, so sum_j dK_j = 0 per head; rows of P
    sum to 1, so sum_j dV_j = sum of dO_i over rows with an allowed key;
    D_i = dO_i . O_i."""
    m = MODES[mode]
    rng = np.random.default_rng(500 + mode)
    q, k, v, do = rand_case(rng, 2, 2, 6, 3)
    kw = dict(causal=m["causal"], kv_lens=m["lens"], block_mask=m["mask"], mask_block=2)
    O, L = oracle.fwd(q, k, v, **kw)
    dq, dk, dv, Dv = oracle.bwd(q, k, v, do, **kw)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12, rtol=0)
    live = np.isfinite(L)[..., None]
    np.testing.assert_allclose(dv.sum(axis=2), (do * live).sum(axis=2), atol=1e-12, rtol=0)
    np.testing.assert_allclose(Dv, (do * O).sum(-1), atol=1e-12, rtol=0)


def test_padded_keys_get_zero_gradient():
    rng = np.random.default_rng(41)
    q, k, v, do = rand_case(rng, 2, 1, 7, 3)
    dq, dk, dv, _ = oracle.bwd(q, k, v, do, kv_lens=[4, 7])
    assert (dk[0, 0, 4:] == 0).all() and (dv[0, 0, 4:] == 0).all()
    assert np.abs(dk[1, 0, 4:]).max() > 0


# --------------------------------------------------------------------------
# 6. torch's fp64 CPU attention and autograd (a library route that shares
#    nothing with the oracle's C code)

@pytest.mark.parametrize("mode", range(len(MODES)))
def test_against_torch_fp64(mode):
    m = MODES[mode]
    rng = np.random.default_rng(600 + mode)
    B, H, N, d = 2, 3, 6, 5
    q, k, v, do = rand_case(rng, B, H, N, d)
    scale = 0.45
    kw = dict(causal=m["causal"], scale=scale, kv_lens=m["lens"], block_mask=m["mask"],
              mask_block=2)
    O, L = oracle.fwd(q, k, v, **kw)
    dq, dk, dv, _ = oracle.bwd(q, k, v, do, **kw)
    masks = np.stack([allowed_matrix(N, m["causal"], N if m["lens"] is None else m["lens"][b],
                                     m["mask"], 2) for b in range(B)])
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    am = torch.tensor(masks)[:, None]
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=scale)
    out.backward(torch.tensor(do))
    np.testing.assert_allclose(O, out.detach().numpy(), atol=1e-13, rtol=0)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12, rtol=0)
    # LSE against torch's logsumexp over allowed scores
    S = torch.tensor(q) @ torch.tensor(k).transpose(-1, -2) * scale
    S = S.masked_fill(~am, float("-inf"))
    np.testing.assert_allclose(L, torch.logsumexp(S, -1).numpy(), atol=1e-13, rtol=0)


# --------------------------------------------------------------------------
# 7. sampled entry points agree with the full ones

def test_sampled_rows_match_full():
    rng = np.random.default_rng(51)
    B, H, N, d = 2, 2, 10, 3
    q, k, v, do = rand_case(rng, B, H, N, d)
    lens = [7, 10]
    mask = [[1, 0, 1, 1, 0], [1, 1, 0, 0, 1], [0, 1, 1, 0, 0], [1, 1, 1, 1, 0], [0, 0, 1, 0, 1]]
    for kw in (dict(causal=True, kv_lens=lens), dict(block_mask=mask, mask_block=2)):
        O, L = oracle.fwd(q, k, v, **kw)
        rows = np.array([0, 5, 13, 27, 39])
        Or, Lr = oracle.fwd_rows(q, k, v, rows, **kw)
        np.testing.assert_array_equal(Or, O.reshape(-1, d)[rows])
        np.testing.assert_array_equal(Lr, L.reshape(-1)[rows])
        dq, dk, dv, _ = oracle.bwd(q, k, v, do, **kw)
        b, h = 1, 0
        kvl = None if "kv_lens" not in kw else kw["kv_lens"][b]
        qr, kr = np.array([0, 3, 9]), np.array([1, 6, 8])
        sq, sk, sv = oracle.bwd_sample(q[b, h], k[b, h], v[b, h], do[b, h], qr, kr,
                                       causal=kw.get("causal", False), kv_len=kvl,
                                       block_mask=kw.get("block_mask"), mask_block=2)
        np.testing.assert_allclose(sq, dq[b, h, qr], atol=1e-14, rtol=0)
        np.testing.assert_allclose(sk, dk[b, h, kr], atol=1e-14, rtol=0)
        np.testing.assert_allclose(sv, dv[b, h, kr], atol=1e-14, rtol=0)


def test_bad_arguments_raise():
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        oracle.fwd(q, q, np.zeros((1, 1, 5, 2)))
    with pytest.raises(ValueError):
        oracle.fwd(q, q, q, kv_lens=[1, 2])
    with pytest.raises(RuntimeError):
        oracle.fwd_rows(q, q, q, [4])
