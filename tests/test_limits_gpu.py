"""GPU checks at the documented size limits, where byte offsets approach
2^31 and the mask lists are longest, with references that stay cheap:

  * split-KV decode over a 2^24-row cache (d = 64, one head: 2 GiB of K and
    2 GiB of V, B*H*Nk*d = 2^30): every key equal, so softmax weights are
    uniform over the filled rows and O is the mean of V over them, LSE =
    scale q.k + ln(len) -- the closed form of identical keys, summed in fp64
    chunk by chunk on the host;
  * block-sparse forward and backward at N = 65536 (the largest the API
    takes) with a block-diagonal mask: every 128-row block is then an
    independent attention problem, which the oracle solves exactly for a
    few blocks;
  * the dense forward (every key tile) and backward (every query tile) with
    B*H*N*d just under 2^31 elements (H = 16, N = 1024, B = 1000 at d = 128
    and 500 at d = 256: 3.9 GiB per tensor, byte offsets past 2^31): every
    (b, h) is an independent problem, so the oracle checks whole heads,
    the last among them;
  * the block-sparse forward and backward at the same size (d = 128, a
    random 8 x 8 mask of 128-blocks with its diagonal on), whole heads
    against the oracle under the same mask;
  * the FP8 quantiser and forward at the same size (1.95 GiB of codes per
    tensor): the codes and descales of whole heads equal the oracle
    quantiser's bit for bit, and the forward of those heads stays within the
    derived E4M3 bounds.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as ofp8
import workloads
from test_fp8_gpu import check_bound, check_lse_bound
from test_parity_gpu import check_bf16, check_lse, f64, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import exact_io_aware_36_amd as fa

    return fa


def test_splitkv_two_gib_cache(fa):
    Nk, d = 1 << 24, 64
    length = Nk - 37
    say(f"  decode: Nk={Nk} d={d} (K, V {Nk * d * 2 / 2**30:.1f} GiB each), kv_len={length}")
    gen = torch.Generator(device="cuda").manual_seed(77)
    krow = torch.randn((d,), generator=gen, device="cuda").to(torch.bfloat16)
    k = krow.expand(Nk, d).contiguous().view(1, 1, Nk, d)
    v = torch.randn((1, 1, Nk, d), generator=gen, device="cuda").to(torch.bfloat16)
    q = torch.randn((1, 1, 1, d), generator=gen, device="cuda").to(torch.bfloat16)
    lens = torch.tensor([length], dtype=torch.int32, device="cuda")
    o, lse = fa.fwd_splitkv(q, k, v, kv_lens=lens)
    torch.cuda.synchronize()
    # reference: the mean of V's filled rows, fp64, in chunks
    acc = np.zeros(d)
    step = 1 << 22
    for a in range(0, length, step):
        b = min(length, a + step)
        acc += v[0, 0, a:b].double().sum(dim=0).cpu().numpy()
    O_ref = acc / length
    scale = 1.0 / math.sqrt(d)
    L_ref = scale * float(q.double().cpu().numpy().ravel() @ krow.double().cpu().numpy()) + math.log(length)
    check_bf16("O", host(o).reshape(d), O_ref)
    check_lse("LSE", host(lse).reshape(1), np.array([L_ref]))
    del k, v


def test_blocksparse_largest_n(fa):
    N, d = 65536, 64
    nb = N // 128
    say(f"  block-sparse N={N} d={d}: block-diagonal mask of {nb} blocks")
    inp = workloads.random_qkv(1, 1, N, d, seed=65536)
    mask = torch.eye(nb, dtype=torch.uint8)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "dout"))
    dm = mask.cuda()
    o, lse = fa.fwd_blocksparse(q, k, v, dm)
    dq, dk, dv = fa.bwd_blocksparse(q, k, v, o, do, lse, dm)
    torch.cuda.synchronize()
    for blk in (0, 1, nb // 2, nb - 1):
        sl = slice(blk * 128, (blk + 1) * 128)
        qs, ks, vs, ds = (f64(inp[n][:, :, sl]) for n in ("q", "k", "v", "dout"))
        O, L = oracle.fwd(qs, ks, vs)
        dQ, dK, dV, _ = oracle.bwd(qs, ks, vs, ds)
        check_bf16(f"O[blk {blk}]", host(o)[:, :, sl], O)
        check_lse(f"LSE[blk {blk}]", host(lse)[:, :, sl], L)
        check_bf16(f"dQ[blk {blk}]", host(dq)[:, :, sl], dQ)
        check_bf16(f"dK[blk {blk}]", host(dk)[:, :, sl], dK)
        check_bf16(f"dV[blk {blk}]", host(dv)[:, :, sl], dV)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_dense_at_element_limit(fa, causal, d):
    B, H, N = 1000 * 128 // d, 16, 1024
    fwd_tiles, bwd_tiles = ((32, 64, 128, 256), (64, 128)) if d == 128 else ((32, 64), (64,))
    assert B * H * N * d < 2**31 and (B * H - 1) * N * d * 2 > 2**31
    say(f"  dense B={B} H={H} N={N} d={d} causal={causal}: {B * H * N * d * 2 / 2**30:.2f} GiB per tensor")
    gen = torch.Generator(device="cuda").manual_seed(2031 + causal)

    def draw(scale):
        return (torch.randn((B, H, N, d), generator=gen, device="cuda") * scale).to(torch.bfloat16)

    q, k, v = draw(0.5), draw(0.5), draw(1.0)
    do = draw(1.0)
    heads = (0, B * H // 2 - 223, B * H - 1)

    def head(t, bh):
        return t.view(B * H, N, d)[bh].double().cpu().numpy()[None, None]

    refs = {}
    for bh in heads:
        qs, ks, vs, ds = head(q, bh), head(k, bh), head(v, bh), head(do, bh)
        O, L = oracle.fwd(qs, ks, vs, causal=causal)
        dQ, dK, dV, _ = oracle.bwd(qs, ks, vs, ds, causal=causal)
        refs[bh] = (O, L, dQ, dK, dV)
    o64 = lse64 = None
    for tile in fwd_tiles:
        say(f"    forward, key tile {tile}")
        o, lse = fa.fwd(q, k, v, causal=causal, tile_n=tile)
        torch.cuda.synchronize()
        for bh in heads:
            O, L = refs[bh][:2]
            check_bf16(f"O[{bh}] tile={tile}", host(o.view(B * H, N, d)[bh])[None, None], O)
            check_lse(f"LSE[{bh}] tile={tile}", host(lse.view(B * H, N)[bh])[None, None], L)
        if tile == 64:
            o64, lse64 = o, lse
        del o, lse
    for tile in bwd_tiles:
        say(f"    backward, query tile {tile}")
        dq, dk, dv = fa.bwd(q, k, v, o64, do, lse64, causal=causal, tile_n=tile)
        torch.cuda.synchronize()
        for bh in heads:
            dQ, dK, dV = refs[bh][2:]
            check_bf16(f"dQ[{bh}] tile={tile}", host(dq.view(B * H, N, d)[bh])[None, None], dQ)
            check_bf16(f"dK[{bh}] tile={tile}", host(dk.view(B * H, N, d)[bh])[None, None], dK)
            check_bf16(f"dV[{bh}] tile={tile}", host(dv.view(B * H, N, d)[bh])[None, None], dV)
        del dq, dk, dv
    del q, k, v, do, o64, lse64
    torch.cuda.empty_cache()


def test_fp8_at_element_limit(fa):
    B, H, N, d = 1000, 16, 1024, 128
    say(f"  fp8 B={B} H={H} N={N} d={d} causal: {B * H * N * d / 2**30:.2f} GiB of codes per tensor")
    gen = torch.Generator(device="cuda").manual_seed(2033)

    def draw(scale):
        return (torch.randn((B, H, N, d), generator=gen, device="cuda") * scale).to(torch.bfloat16)

    q, k, v = draw(0.5), draw(0.5), draw(1.0)
    signs = workloads.random_signs(d, 2033)
    q8, qs = fa.quantize_fp8(q, 128, signs=signs.cuda())
    k8, ks = fa.quantize_fp8(k, 128, signs=signs.cuda())
    v8t, vs = fa.quantize_fp8(v, 0, transpose=True)
    o, lse = fa.fwd_fp8(q8, k8, v8t, qs, ks, vs, causal=True)
    torch.cuda.synchronize()
    nblk = N // 128
    for bh in (0, 7777, B * H - 1):
        x = {n: t.view(B * H, N, d)[bh].float().cpu().numpy()[None, None] for n, t in (("q", q), ("k", k), ("v", v))}
        cq, dq_ = ofp8.quantize(x["q"], 128, signs.numpy())
        ck, dk_ = ofp8.quantize(x["k"], 128, signs.numpy())
        cv, dv_ = ofp8.quantize(x["v"], 0)
        assert np.array_equal(q8.view(B * H, N, d)[bh].cpu().numpy(), cq[0, 0]), f"q codes of head {bh}"
        assert np.array_equal(k8.view(B * H, N, d)[bh].cpu().numpy(), ck[0, 0]), f"k codes of head {bh}"
        assert np.array_equal(v8t.view(B * H, d, N)[bh].cpu().numpy().T, cv[0, 0]), f"v codes of head {bh}"
        assert np.array_equal(qs.view(B * H, nblk)[bh].cpu().numpy(), dq_.reshape(nblk))
        assert np.array_equal(ks.view(B * H, nblk)[bh].cpu().numpy(), dk_.reshape(nblk))
        assert np.array_equal(vs.view(B * H)[bh].cpu().numpy().reshape(1), dv_.reshape(1))
        O, L, (Qd, Kd, Vd) = ofp8.reference(cq, ck, cv, dq_, dk_, dv_, causal=True)
        check_bound(f"O[{bh}]", host(o.view(B * H, N, d)[bh])[None, None], O,
                    ofp8.p_quant_bound(Qd, Kd, Vd, L, causal=True))
        check_lse_bound(f"LSE[{bh}]", host(lse.view(B * H, N)[bh])[None, None], L,
                        ofp8.lse_bound(cq, dq_, ck, dk_, L, causal=True))
    del q, k, v, q8, k8, v8t, o, lse
    torch.cuda.empty_cache()


def test_blocksparse_at_element_limit(fa):
    B, H, N, d = 1000, 16, 1024, 128
    nb = N // 128
    mask_np = workloads.random_block_mask(nb, 0.4, 2035).numpy()
    say(f"  block-sparse B={B} H={H} N={N} d={d}: {int(mask_np.sum())} of {nb * nb} blocks on")
    gen = torch.Generator(device="cuda").manual_seed(2035)

    def draw(scale):
        return (torch.randn((B, H, N, d), generator=gen, device="cuda") * scale).to(torch.bfloat16)

    q, k, v, do = draw(0.5), draw(0.5), draw(1.0), draw(1.0)
    dm = torch.from_numpy(mask_np).cuda()
    o, lse = fa.fwd_blocksparse(q, k, v, dm)
    dq, dk, dv = fa.bwd_blocksparse(q, k, v, o, do, lse, dm)
    torch.cuda.synchronize()

    def head(t, bh):
        return t.view(B * H, N, d)[bh]

    for bh in (0, 5555, B * H - 1):
        qs, ks, vs, ds = (head(t, bh).double().cpu().numpy()[None, None] for t in (q, k, v, do))
        O, L = oracle.fwd(qs, ks, vs, block_mask=mask_np, mask_block=128)
        dQ, dK, dV, _ = oracle.bwd(qs, ks, vs, ds, block_mask=mask_np, mask_block=128)
        check_bf16(f"O[{bh}]", host(head(o, bh))[None, None], O)
        check_lse(f"LSE[{bh}]", host(lse.view(B * H, N)[bh])[None, None], L)
        check_bf16(f"dQ[{bh}]", host(head(dq, bh))[None, None], dQ)
        check_bf16(f"dK[{bh}]", host(head(dk, bh))[None, None], dK)
        check_bf16(f"dV[{bh}]", host(head(dv, bh))[None, None], dV)
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
