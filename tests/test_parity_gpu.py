"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Bars (written here, applied per output tensor):
  bf16 O, dQ, dK, dV: relative L2 <= 5e-3 and max abs error <= 1e-2, where the
      max abs error of an element is taken beyond half a bf16 ulp of the
      oracle value (the rounding every bf16 output carries by format: above
      |x| = 4 half an ulp is already 0.0156);
  LSE (fp32): max abs <= 1e-3;
  fp32 path: O and LSE max abs <= 1e-5.
Small cases span several tiles and a ragged tail; the five measured workloads
run at full size, every element compared (the long-context case also has a
faster check on sampled rows, used for its tile variants).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

BF16_MAX_ABS, BF16_REL_L2, LSE_MAX_ABS, FP32_MAX_ABS = 1e-2, 5e-3, 1e-3, 1e-5


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import exact_io_aware_36_amd as fa

    return fa


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def check_bf16(name, gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, name
    assert np.isfinite(gpu).all(), f"{name}: non-finite output"
    diff = np.abs(gpu - ref)
    excess = float((diff - half_ulp_bf16(ref)).max()) if diff.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(gpu - ref) / nrm) if nrm > 0 else float(np.linalg.norm(gpu))
    # the literal bar, for the record: elements whose raw error passes 1e-2
    # (all of them carry a bf16 half ulp above 1e-2 only when |ref| >= 2)
    over = diff > BF16_MAX_ABS
    n_over = int(over.sum())
    over_txt = (f" literal>1e-2: {n_over} of {diff.size} (max {diff[over].max():.3e} at "
                f"|ref|={np.abs(ref[over]).max():.3g})") if n_over else " literal>1e-2: 0"
    say(f"    {name}: max_abs={diff.max() if diff.size else 0:.3e} beyond-half-ulp={excess:.3e} "
        f"rel_l2={rel:.3e}{over_txt}")
    assert excess <= BF16_MAX_ABS, f"{name}: max abs error {excess} > {BF16_MAX_ABS}"
    assert rel <= BF16_REL_L2, f"{name}: relative L2 {rel} > {BF16_REL_L2}"


def check_lse(name, gpu, ref, tol=LSE_MAX_ABS):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    both_inf = np.isneginf(gpu) & np.isneginf(ref)
    assert (np.isneginf(gpu) == np.isneginf(ref)).all(), f"{name}: -inf rows differ"
    with np.errstate(invalid="ignore"):      # -inf - -inf where both rows saw no key
        d = np.abs(np.where(both_inf, 0.0, gpu - ref))
    say(f"    {name}: max_abs={d.max() if d.size else 0:.3e}")
    assert d.max() <= tol, f"{name}: {d.max()} > {tol}"


def dev(t):
    return None if t is None else t.contiguous().cuda()


def host(t):
    return t.detach().float().cpu().numpy()


def f64(t):
    return None if t is None else t.detach().double().cpu().numpy()


def run_fwd(fa, inp, tile_n=0):
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    lens = dev(inp.get("kv_lens"))
    o, lse = fa.fwd(q, k, v, causal=inp["causal"], scale=inp["scale"], kv_lens=lens, tile_n=tile_n)
    torch.cuda.synchronize()
    return o, lse


def small_case(B, H, N, d, causal, padded, seed, dtype=torch.bfloat16):
    inp = workloads.random_qkv(B, H, N, d, seed, dtype=dtype)
    inp.update(causal=causal, scale=1.0 / math.sqrt(d))
    inp["kv_lens"] = workloads.random_lengths(B, 1, N, seed + 7) if padded else None
    return inp


# ---------------------------------------------------------------------------
# forward, small shapes: several tiles, ragged tails, every mask mode

SMALL = [
    # (B, H, N, d)
    (2, 3, 300, 64), (1, 2, 300, 128), (1, 1, 64, 64), (1, 1, 1, 64), (2, 2, 257, 128),
    (1, 2, 128, 128), (3, 1, 45, 64),
]


@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("tile_n", [32, 64, 128, 256])
def test_fwd_small(fa, shape, causal, padded, tile_n):
    B, H, N, d = shape
    say(f"  fwd bf16 B={B} H={H} N={N} d={d} causal={causal} padded={padded} tile={tile_n}")
    inp = small_case(B, H, N, d, causal, padded, seed=hash((shape, causal, padded)) % 10000)
    o, lse = run_fwd(fa, inp, tile_n)
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal=causal,
                      scale=inp["scale"], kv_lens=f64(inp["kv_lens"]))
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)


@pytest.mark.parametrize("shape", [(2, 3, 300, 64), (1, 2, 257, 128), (1, 1, 1, 64)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_fwd_fp32_small(fa, shape, causal, padded):
    B, H, N, d = shape
    say(f"  fwd fp32 B={B} H={H} N={N} d={d} causal={causal} padded={padded}")
    inp = small_case(B, H, N, d, causal, padded, seed=77, dtype=torch.float32)
    o, lse = run_fwd(fa, inp)
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal=causal,
                      scale=inp["scale"], kv_lens=f64(inp["kv_lens"]))
    d_o = np.abs(host(o) - O).max()
    say(f"    O max_abs={d_o:.3e}")
    assert d_o <= FP32_MAX_ABS
    check_lse("LSE", host(lse), L, tol=FP32_MAX_ABS)


def test_fwd_deterministic(fa):
    inp = small_case(2, 4, 640, 128, True, True, seed=5)
    o1, l1 = run_fwd(fa, inp)
    o2, l2 = run_fwd(fa, inp)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_zero_length_rows(fa):
    """kv_len = 0 leaves no allowed key: O = 0 and LSE = -inf."""
    inp = small_case(2, 1, 130, 64, False, False, seed=3)
    inp["kv_lens"] = torch.tensor([0, 130], dtype=torch.int32)
    o, lse = run_fwd(fa, inp)
    assert (host(o)[0] == 0).all() and np.isneginf(host(lse)[0]).all()
    O, L = oracle.fwd(f64(inp["q"])[1:], f64(inp["k"])[1:], f64(inp["v"])[1:], scale=inp["scale"])
    check_bf16("O[b=1]", host(o)[1:], O)


# ---------------------------------------------------------------------------
# block-sparse forward

@pytest.mark.parametrize("N,d,frac", [(512, 64, 0.25), (384, 128, 0.5), (1024, 64, 0.125)])
def test_blocksparse_small(fa, N, d, frac):
    say(f"  sparse N={N} d={d} frac={frac}")
    inp = workloads.random_qkv(2, 2, N, d, seed=N + d)
    mask = workloads.random_block_mask(N // 128, frac, seed=N)
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    o, lse = fa.fwd_blocksparse(q, k, v, dev(mask))
    torch.cuda.synchronize()
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), block_mask=mask.numpy(),
                      mask_block=128)
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)


def test_blocksparse_empty_row_and_full_mask(fa):
    N, d = 384, 64
    inp = workloads.random_qkv(1, 2, N, d, seed=9)
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    mask = torch.tensor([[1, 0, 1], [0, 0, 0], [1, 1, 1]], dtype=torch.uint8)
    o, lse = fa.fwd_blocksparse(q, k, v, dev(mask))
    torch.cuda.synchronize()
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), block_mask=mask.numpy(),
                      mask_block=128)
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)
    # an all-ones mask equals the dense forward
    ones = torch.ones(3, 3, dtype=torch.uint8)
    o1, l1 = fa.fwd_blocksparse(q, k, v, dev(ones))
    o2, l2 = fa.fwd(q, k, v)
    torch.cuda.synchronize()
    check_bf16("O(all-ones vs dense)", host(o1), host(o2).astype(np.float64))


# ---------------------------------------------------------------------------
# block-sparse backward

@pytest.mark.parametrize("N,d,mask", [
    (512, 64, "random25"), (384, 128, "random50"), (384, 64, "holes"), (256, 128, "ones")])
def test_blocksparse_bwd_small(fa, N, d, mask):
    say(f"  sparse bwd N={N} d={d} mask={mask}")
    inp = workloads.random_qkv(2, 2, N, d, seed=N + d + 7)
    nb = N // 128
    if mask == "random25":
        m = workloads.random_block_mask(nb, 0.25, seed=1)
    elif mask == "random50":
        m = workloads.random_block_mask(nb, 0.5, seed=2)
    elif mask == "holes":
        # row 1 empty (its queries see nothing), column 2 empty (its keys get no gradient)
        m = torch.tensor([[1, 0, 0], [0, 0, 0], [1, 1, 0]], dtype=torch.uint8)
    else:
        m = torch.ones(nb, nb, dtype=torch.uint8)
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    dm = dev(m)
    o, lse = fa.fwd_blocksparse(q, k, v, dm)
    dq, dk, dv = fa.bwd_blocksparse(q, k, v, o, do, lse, dm)
    torch.cuda.synchronize()
    dQ, dK, dV, _ = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dout"]),
                               block_mask=m.numpy(), mask_block=128)
    check_bf16("dQ", host(dq), dQ)
    check_bf16("dK", host(dk), dK)
    check_bf16("dV", host(dv), dV)
    if mask == "holes":
        assert (host(dq)[:, :, 128:256] == 0).all()
        assert (host(dk)[:, :, 256:] == 0).all() and (host(dv)[:, :, 256:] == 0).all()
    if mask == "ones":
        r = fa.bwd(q, k, v, o, do, lse)
        torch.cuda.synchronize()
        for a, b in zip((dq, dk, dv), r):
            assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# backward, small shapes

@pytest.mark.parametrize("shape", [(2, 2, 300, 64), (1, 2, 257, 128), (1, 1, 64, 64),
                                   (2, 1, 130, 128), (1, 1, 1, 64), (1, 2, 520, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("tile_n", [64, 128])
def test_bwd_small(fa, shape, causal, padded, tile_n):
    B, H, N, d = shape
    say(f"  bwd B={B} H={H} N={N} d={d} causal={causal} padded={padded} tile={tile_n}")
    inp = small_case(B, H, N, d, causal, padded, seed=hash((shape, causal, padded, 1)) % 10000)
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    lens = dev(inp["kv_lens"])
    o, lse = fa.fwd(q, k, v, causal=causal, kv_lens=lens)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=causal, kv_lens=lens, tile_n=tile_n)
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


def test_bwd_deterministic(fa):
    inp = small_case(1, 4, 520, 128, True, False, seed=11)
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    o, lse = fa.fwd(q, k, v, causal=True)
    r1 = fa.bwd(q, k, v, o, do, lse, causal=True)
    r2 = fa.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# the five measured workloads at full size

def test_workload_single_head_fp32(fa):
    w = workloads.WORKLOADS["single_head_fp32"]
    inp = workloads.make_inputs(w)
    say(f"  {w.name}")
    o, lse = run_fwd(fa, inp)
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale=w.scale)
    d_o = np.abs(host(o) - O).max()
    say(f"    O max_abs={d_o:.3e}")
    assert d_o <= FP32_MAX_ABS
    check_lse("LSE", host(lse), L, tol=FP32_MAX_ABS)


def test_workload_gpt2_medium_causal(fa):
    w = workloads.WORKLOADS["gpt2_medium_causal"]
    inp = workloads.make_inputs(w)
    say(f"  {w.name}")
    o, lse = run_fwd(fa, inp)
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal=True, scale=w.scale)
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)


def test_workload_bert_large_padded(fa):
    w = workloads.WORKLOADS["bert_large_padded"]
    inp = workloads.make_inputs(w)
    say(f"  {w.name}")
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    lens = dev(inp["kv_lens"])
    o, lse = fa.fwd(q, k, v, kv_lens=lens)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, kv_lens=lens)
    torch.cuda.synchronize()
    lens_h = inp["kv_lens"].numpy()
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale=w.scale, kv_lens=lens_h)
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)
    dQ, dK, dV, _ = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dout"]),
                               scale=w.scale, kv_lens=lens_h)
    check_bf16("dQ", host(dq), dQ)
    check_bf16("dK", host(dk), dK)
    check_bf16("dV", host(dv), dV)


def test_workload_long_context_causal(fa):
    """Full size on the GPU; the oracle checks sampled rows: 512 forward rows
    over all heads, and on two heads dQ for 64 query rows and dK, dV for 64
    key rows (these need every row's statistics, computed by the oracle from
    the definition)."""
    w = workloads.WORKLOADS["long_context_causal"]
    inp = workloads.make_inputs(w)
    say(f"  {w.name}")
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    B, H, N, d = q.shape
    rng = np.random.default_rng(2024)
    rows = np.sort(rng.choice(B * H * N, 512, replace=False))
    rows = np.concatenate([rows, [0, N - 1, N, B * H * N - 1]])
    qf, kf, vf, dof = (f64(inp[n]) for n in ("q", "k", "v", "dout"))
    Or, Lr = oracle.fwd_rows(qf, kf, vf, rows, causal=True, scale=w.scale)
    check_bf16("O[rows]", host(o).reshape(-1, d)[rows], Or)
    check_lse("LSE[rows]", host(lse).reshape(-1)[rows], Lr)
    for h in (0, H - 1):
        qr = np.concatenate([[0, 1, N - 1], rng.choice(N, 61, replace=False)])
        kr = np.concatenate([[0, 1, N - 1], rng.choice(N, 61, replace=False)])
        sq, sk, sv = oracle.bwd_sample(qf[0, h], kf[0, h], vf[0, h], dof[0, h], qr, kr,
                                       causal=True, scale=w.scale)
        check_bf16(f"dQ[h={h}]", host(dq)[0, h, qr], sq)
        check_bf16(f"dK[h={h}]", host(dk)[0, h, kr], sk)
        check_bf16(f"dV[h={h}]", host(dv)[0, h, kr], sv)


@pytest.mark.timeout(900)
def test_workload_long_context_causal_full(fa):
    """The same long-context causal forward and backward compared on every
    element: O, LSE, dQ, dK and dV of all 16 heads against the oracle's full
    fp64 forward and backward (about a minute of CPU time on 16 cores)."""
    w = workloads.WORKLOADS["long_context_causal"]
    inp = workloads.make_inputs(w)
    say(f"  {w.name} full tensors (oracle on {oracle.threads()} threads)")
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (host(t) for t in (o, lse, dq, dk, dv))
    qf, kf, vf, dof = (f64(inp[n]) for n in ("q", "k", "v", "dout"))
    O, L = oracle.fwd(qf, kf, vf, causal=True, scale=w.scale)
    check_bf16("O", o, O)
    check_lse("LSE", lse, L)
    del O, L
    dQ, dK, dV, _ = oracle.bwd(qf, kf, vf, dof, causal=True, scale=w.scale)
    check_bf16("dQ", dq, dQ)
    check_bf16("dK", dk, dK)
    check_bf16("dV", dv, dV)


@pytest.mark.parametrize("tile_n", [64, 128])
def test_workload_long_context_bwd_tiles(fa, tile_n):
    """The backward's query-tile choices at the long-context size (two
    heads): dQ for 64 query rows and dK, dV for 64 key rows of each head."""
    w = workloads.WORKLOADS["long_context_causal"]
    inp = workloads.make_inputs(w, H=2)
    say(f"  {w.name} H=2 backward tile={tile_n}")
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=True, tile_n=tile_n)
    torch.cuda.synchronize()
    N = w.N
    rng = np.random.default_rng(17)
    qf, kf, vf, dof = (f64(inp[n]) for n in ("q", "k", "v", "dout"))
    for h in (0, 1):
        qr = np.concatenate([[0, 1, N - 1], rng.choice(N, 61, replace=False)])
        kr = np.concatenate([[0, 1, N - 1], rng.choice(N, 61, replace=False)])
        sq, sk, sv = oracle.bwd_sample(qf[0, h], kf[0, h], vf[0, h], dof[0, h], qr, kr,
                                       causal=True, scale=w.scale)
        check_bf16(f"dQ[h={h}] tile={tile_n}", host(dq)[0, h, qr], sq)
        check_bf16(f"dK[h={h}] tile={tile_n}", host(dk)[0, h, kr], sk)
        check_bf16(f"dV[h={h}] tile={tile_n}", host(dv)[0, h, kr], sv)


@pytest.mark.parametrize("tile_n", [32, 64, 128, 256])
def test_workload_long_context_tiles(fa, tile_n):
    """The key-tile sweep: every tile length gives the same forward."""
    w = workloads.WORKLOADS["long_context_causal"]
    inp = workloads.make_inputs(w, H=2)
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    o, lse = fa.fwd(q, k, v, causal=True, tile_n=tile_n)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = rng.choice(2 * w.N, 256, replace=False)
    Or, Lr = oracle.fwd_rows(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), rows, causal=True,
                             scale=w.scale)
    check_bf16(f"O[rows] tile={tile_n}", host(o).reshape(-1, w.d)[rows], Or)
    check_lse("LSE[rows]", host(lse).reshape(-1)[rows], Lr)


@pytest.mark.timeout(600)
def test_workload_block_sparse_backward(fa):
    """The block-sparse workload with a backward pass (dO drawn after Q, K,
    V from the same seed): dQ, dK and dV compared on every element with the
    oracle's full backward under the same block mask."""
    w = workloads.WORKLOADS["block_sparse_fwdbwd"]
    inp = workloads.make_inputs(w)
    say(f"  {w.name}")
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    mask = inp["block_mask"]
    dm = dev(mask)
    o, lse = fa.fwd_blocksparse(q, k, v, dm)
    dq, dk, dv = fa.bwd_blocksparse(q, k, v, o, do, lse, dm)
    torch.cuda.synchronize()
    qf, kf, vf, dof = (f64(inp[n]) for n in ("q", "k", "v", "dout"))
    dQ, dK, dV, _ = oracle.bwd(qf, kf, vf, dof, scale=w.scale, block_mask=mask.numpy(),
                               mask_block=128)
    check_bf16("dQ", host(dq), dQ)
    check_bf16("dK", host(dk), dK)
    check_bf16("dV", host(dv), dV)


def test_workload_block_sparse(fa):
    w = workloads.WORKLOADS["block_sparse"]
    inp = workloads.make_inputs(w)
    say(f"  {w.name}")
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    mask = inp["block_mask"]
    assert int(mask.sum()) == round(0.25 * mask.numel())
    o, lse = fa.fwd_blocksparse(q, k, v, dev(mask))
    torch.cuda.synchronize()
    O, L = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale=w.scale,
                      block_mask=mask.numpy(), mask_block=128)
    check_bf16("O", host(o), O)
    check_lse("LSE", host(lse), L)
