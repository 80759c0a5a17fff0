"""Pins for the FP8 part of the oracle (no GPU): the E4M3FN encoder against a
brute-force nearest-code search and the constants of the OCP 8-bit floating
point specification, the fp32 Walsh-Hadamard rotation against scipy's
Hadamard matrix in fp64, the block quantiser's error and scale rules, and the
probability-rounding error bound against a direct simulation."""
from __future__ import annotations

import numpy as np
import pytest
import scipy.linalg

from oracle import fp8

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def brute_nearest(x):
    """Nearest finite E4M3 code by exhaustive search; ties to the even code;
    magnitudes beyond the 448/480 midpoint are NaN codes."""
    vals = fp8.e4m3_decode(FINITE)
    out = np.empty(x.shape, np.uint8)
    for i, xv in enumerate(np.asarray(x, np.float64).ravel()):
        if abs(xv) > 464.0:
            out.flat[i] = 0xFF if xv < 0 else 0x7F
            continue
        d = np.abs(vals - xv)
        best = np.flatnonzero(d == d.min())
        cand = FINITE[best]
        if cand.size > 1:        # a tie: the code with the even mantissa
            cand = cand[(cand & 1) == 0]
        # +-0: keep the sign of x
        c = int(cand[0])
        if vals[best[0]] == 0.0:
            c = 0x80 if np.signbit(xv) else 0x00
        out.flat[i] = c
    return out


def test_spec_constants():
    # OCP 8-bit floating point, E4M3: bias 7, max finite 448, min normal 2^-6,
    # min subnormal 2^-9, S.1111.111 NaN, no infinities
    d = fp8.e4m3_decode
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9 and d(0x38) == 1.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert not np.isinf(d(np.arange(256, dtype=np.uint8))).any()


def test_round_trip_every_finite_code():
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(FINITE).astype(np.float32)), FINITE)


def test_positive_values_are_monotone():
    v = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_ties_go_to_even():
    pos = FINITE[FINITE < 0x7E]
    lo, hi = fp8.e4m3_decode(pos), fp8.e4m3_decode(pos + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)     # exact in fp32
    want = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    assert np.array_equal(fp8.e4m3_encode(mid), want)
    assert np.array_equal(fp8.e4m3_encode(-mid), want | 0x80)


def test_encoder_equals_brute_force_nearest():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-470, 470, 3000), np.exp(rng.uniform(np.log(1e-5), np.log(460), 4000)) *
        rng.choice([-1, 1], 4000), rng.uniform(-0.03, 0.03, 2000), [0.0, -0.0, 464.0, -464.0, 465.0]]
    ).astype(np.float32)
    assert np.array_equal(fp8.e4m3_encode(x), brute_nearest(x))


def test_overflow_and_signed_zero_readings():
    e = fp8.e4m3_encode
    assert e(np.float32(464.0)) == 0x7E and e(np.float32(465.0)) == 0x7F and e(np.float32(-1e6)) == 0xFF
    assert e(np.float32(-0.0)) == 0x80 and e(np.float32(-1e-4)) == 0x80 and e(np.float32(1e-4)) == 0x00


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_matches_hadamard_matrix(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, d)).astype(np.float32)
    s = rng.choice([-1.0, 1.0], d).astype(np.float32)
    R = np.diag(s.astype(np.float64)) @ scipy.linalg.hadamard(d).astype(np.float64) / np.sqrt(d)
    want = x.astype(np.float64) @ R
    got = fp8.rotate_fp32(x, s)
    assert got.dtype == np.float32
    assert np.max(np.abs(got - want)) < 1e-5 * np.abs(x).sum(axis=1).max()
    # orthogonal: norms and dot products survive
    assert np.allclose(np.linalg.norm(got, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)
    y = rng.standard_normal((7, d)).astype(np.float32)
    assert np.allclose(got.astype(np.float64) @ fp8.rotate_fp32(y, s).T.astype(np.float64),
                       x.astype(np.float64) @ y.T.astype(np.float64), atol=1e-4)


def test_quantize_error_and_scale_rules():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((2, 3, 300, 64)) * rng.uniform(0.1, 10, (2, 3, 1, 1))).astype(np.float32)
    x[1, 2, 128:256] = 0.0                                   # an all-zero block
    codes, ds = fp8.quantize(x)
    assert codes.shape == x.shape and ds.shape == (2, 3, 3)
    assert ds[1, 2, 1] == 1.0 and np.all(codes[1, 2, 128:256] == 0)
    deq = fp8.dequantize(codes, ds)
    rows = np.arange(300) // 128
    dsr = ds[:, :, rows][..., None].astype(np.float64)
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * dsr) * (1 + 1e-6))
    # every non-zero block's largest element lands on +-448
    for b, h, i in [(0, 0, 0), (1, 1, 2), (0, 2, 1)]:
        blk = x[b, h, i * 128:(i + 1) * 128]
        r, c = np.unravel_index(np.abs(blk).argmax(), blk.shape)
        assert codes[b, h, i * 128 + r, c] & 0x7F == 0x7E
    # one block per head
    c0, d0 = fp8.quantize(x, block_rows=0)
    assert d0.shape == (2, 3, 1)
    assert np.allclose(d0[:, :, 0], np.abs(x).max(axis=(2, 3)) / 448, rtol=1e-6)


def test_p_rounding_bound_holds_for_a_direct_simulation():
    """Quantise the probabilities of one-shot softmax (reference max exact) and
    of a lowered reference (as the lazy rescale allows) to E4M3 and check the
    change of O against the bound."""
    rng = np.random.default_rng(2)
    B, H, N, d = 1, 2, 200, 16
    Q = rng.standard_normal((B, H, N, d)) * 2
    K = rng.standard_normal((B, H, N, d)) * 2
    V = rng.standard_normal((B, H, N, d))
    import oracle

    for causal in (False, True):
        O, L = oracle.fwd(Q, K, V, causal=causal)
        bound = fp8.p_quant_bound(Q, K, V, L, causal=causal)
        for shift in (0.0, 5.0):
            s = (Q[0] @ K[0].transpose(0, 2, 1)) / np.sqrt(d)
            if causal:
                s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
            m = s.max(axis=-1, keepdims=True) - shift * np.log(2)    # lowered reference
            pt = np.exp(s - m).astype(np.float32)
            pq = fp8.e4m3_decode(fp8.e4m3_encode(pt))
            Osim = (pq @ V[0]) / pt.astype(np.float64).sum(axis=-1, keepdims=True)
            assert np.all(np.abs(Osim - O[0]) <= bound[0]), (causal, shift)


def test_p_rounding_bound_is_nearly_attained():
    """Two equal scores with the reference lowered so that both p~ equal
    1.0624 (just below the 1.0 / 1.125 midpoint): both round to 1.0 and O
    shrinks by 1 - 1/1.0624 ~ 0.94 * 2^-4 -- a bound any smaller than
    2^-4 sum P|v| would be violated."""
    import oracle

    Q = np.ones((1, 1, 2, 1))
    K = np.ones((1, 1, 2, 1))
    V = np.ones((1, 1, 2, 1))
    O, L = oracle.fwd(Q, K, V, scale=1.0)
    bound = fp8.p_quant_bound(Q, K, V, L, scale=1.0, n_slack=0)
    pt = np.full((2,), 1.0624, np.float32)
    pq = fp8.e4m3_decode(fp8.e4m3_encode(pt))
    assert np.all(pq == 1.0)
    Osim = pq.sum() / pt.astype(np.float64).sum()
    err = abs(Osim - O[0, 0, 1, 0])
    assert err <= bound[0, 0, 1, 0] and err >= 0.9 * bound[0, 0, 1, 0]


def simulate_scores(q8, k8, window=14):
    """The measured arithmetic of the E4M3 product sum, written directly: per
    64-product block every product truncated toward zero to a multiple of
    2^(E - window) (E = binade of the block's largest |product|), the
    block's sum added to an fp32 accumulator."""
    a = fp8.e4m3_decode(q8).astype(np.float64)
    b = fp8.e4m3_decode(k8).astype(np.float64)
    n, d = a.shape
    acc = np.zeros((n, b.shape[0]), dtype=np.float32)
    for c in range(0, d, 64):
        p = a[:, None, c:c + 64] * b[None, :, c:c + 64]
        mx = np.abs(p).max(axis=-1, keepdims=True)
        e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
        lsb = np.exp2(e - window)
        t = np.trunc(p / lsb) * lsb
        acc = (acc.astype(np.float64) + t.sum(axis=-1)).astype(np.float32)
    return acc.astype(np.float64)


def lse_of(s):
    m = s.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]


@pytest.mark.parametrize("kind", ["random", "aligned", "spread"])
def test_lse_bound_holds_for_a_direct_simulation(kind):
    """Scores from the simulated E4M3 product sums against exact ones: the LSE
    difference stays within lse_bound_rows (for random codes; for queries and
    keys along one direction, with scores ramping up to ~80 nats; and with
    every key near 80 nats, so that the probability -- and the error LSE
    inherits from every score -- is spread over all keys)."""
    rng = np.random.default_rng(5)
    n, N, d = 48, 96, 128
    if kind == "random":
        q = rng.standard_normal((n, d)) * 3
        k = rng.standard_normal((N, d)) * 3
    else:
        u = rng.standard_normal(d)
        u /= np.linalg.norm(u)
        q = 4 * u + 0.05 * rng.standard_normal((n, d)) / np.sqrt(d)
        top = np.linspace(0, 120, N) if kind == "aligned" else np.full(N, 115.0)
        k = (top / (4 / np.sqrt(d) * 1.4426950408889634))[:, None] * u \
            + 0.05 * rng.standard_normal((N, d)) / np.sqrt(d)
    q8, qs = fp8.quantize(q[None, None], 0)
    k8, ks = fp8.quantize(k[None, None], 0)
    q8, k8 = q8[0, 0], k8[0, 0]
    craw = (1 / np.sqrt(d)) * float(qs[0, 0, 0]) * float(ks[0, 0, 0])
    exact = craw * (fp8.e4m3_decode(q8) @ fp8.e4m3_decode(k8).T)
    sim = craw * simulate_scores(q8, k8)
    L = lse_of(exact)
    bound = fp8.lse_bound_rows(q8, np.arange(n), np.full(n, qs[0, 0, 0]), k8, np.full(N, ks[0, 0, 0]), L)
    err = np.abs(lse_of(sim) - L)
    assert np.all(err <= bound), (kind, float((err / bound).max()))
    print(kind, float(np.abs(exact).max()), float(err.max()), float((err / bound).max()))
    if kind != "random":
        assert float(np.abs(exact).max()) > 70          # the large-score regime
        assert float((err / bound).max()) > 0.05        # not vacuous there


def test_score_bound_is_nearly_attained():
    """One product 2^7 and 63 products whose lowest bit lies one place below
    the 14-bit window: each loses exactly that bit, 63 * 2^(E - 15) in all,
    a quarter of the bound's 63 * 2^(E - 13); one bit more of window in the
    bound (2^(E - 14)) would leave only twice the truncation."""
    a = np.zeros((1, 64), np.float32)
    b = np.zeros((1, 64), np.float32)
    a[0, 0], b[0, 0] = 16.0, 8.0                                     # 2^7, exact
    a[0, 1:], b[0, 1:] = 1.875 * 2.0 ** -4, 1.875 * 2.0 ** -4         # 3.515625 * 2^-8 each
    q8, k8 = fp8.e4m3_encode(a), fp8.e4m3_encode(b)
    exact = float((fp8.e4m3_decode(q8) @ fp8.e4m3_decode(k8).T)[0, 0])
    sim = float(simulate_scores(q8, k8)[0, 0])
    err = exact - sim
    bound = float(fp8.score_error_bound(q8, k8)[0, 0])
    assert err > 0 and err <= bound
    assert err >= 0.2 * bound, (err, bound)

