"""The benchmark's accounting against the worked IO example printed by
"01 · FlashAttention" (step 5 of 5 "The payoff", panel "show the accounting"),
stored in tests/golden/io_accounting_n8192_d128_m65536.txt with its citation,
and the flop convention against closed forms."""
from __future__ import annotations

import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "io_accounting_n8192_d128_m65536.txt")


def load_golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                vals[k] = float(v)
    return vals


def test_io_accounting_matches_the_page():
    g = load_golden()
    N, d, M = int(g["N"]), int(g["d"]), int(g["M"])
    std = bench.standard_io_elements(N, d)
    fl = bench.flash_io_elements(N, d, M)
    assert N * N == g["score_entries_per_head"]
    assert std == g["standard_elements"]
    assert fl == g["flash_elements"]
    assert round(std / fl, 1) == g["traffic_reduction"]
    # the page's bars: 2-byte elements at 2 TB/s, 2 N^2 d flops at 312 TFLOP/s
    wait_std = std * 2 / 2e12 * 1e6
    wait_fl = fl * 2 / 2e12 * 1e6
    compute = 2 * N * N * d / 312e12 * 1e6
    assert round(wait_std) == g["standard_wait_us"]
    assert round(wait_fl) == g["flash_wait_us"]
    assert round(compute) == g["compute_us"]
    assert round(wait_std + compute) == g["standard_total_us"]
    assert round(wait_fl + compute) == g["flash_total_us"]
    assert round((wait_std + compute) / (wait_fl + compute), 1) == g["speedup"]


def test_flop_convention():
    # forward: two products of 2 N^2 d flops per head
    assert bench.fwd_flops(1, 1, 256, 64) == 4 * 256 * 256 * 64
    assert bench.fwd_flops(8, 16, 1024, 64, causal=True) == 17179869184
    assert bench.fwd_flops(1, 16, 16384, 128, causal=True) == 1099511627776
    assert bench.fwd_flops(4, 16, 4096, 64, sparse_frac=0.25) == 68719476736
    assert bench.step_flops(16, 16, 512, 64, backward=True) == 2.5 * 17179869184
    # per-kernel products: dK/dV four, dQ three, forward two
    f = bench.fwd_flops(1, 2, 512, 64, causal=True)
    assert bench.kernel_flops("bwd_dkdv", 1, 2, 512, 64, causal=True) == 2 * f
    assert bench.kernel_flops("bwd_dq", 1, 2, 512, 64, causal=True) == 1.5 * f


def test_floor_bytes():
    B, H, N, d = 1, 16, 16384, 128
    assert bench.floor_bytes("fwd", B, H, N, d) == 269484032
    t = B * H * N * d * 2
    assert bench.floor_bytes("bwd_dkdv", B, H, N, d) == 6 * t + 8 * B * H * N


def test_gpus_above_one_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_kvouter_bytes_closed_form():
    """The key/value-outer byte model against its closed form when N is a
    multiple of 128 (every query block full): per head, T_c = N/64 blocks,
    each moving Q (2 B) and O, l, m out (4 d + 8 B per row), the blocks after
    the first also reading O, l, m back; K, V once; the last pass."""
    for N, d in ((1024, 64), (8192, 128)):
        tc = N // 64
        per_head = (tc * (2 * N * d + 4 * N * d + 8 * N) + (tc - 1) * (4 * N * d + 8 * N)
                    + 4 * N * d + (4 * N * d + 8 * N + 2 * N * d + 4 * N))
        assert bench.kvouter_bytes(2, 3, N, d, False) == 6 * per_head


def test_kvouter_bytes_grows_quadratically_and_causal_halves():
    r = bench.kvouter_bytes(1, 1, 16384, 128, False) / bench.kvouter_bytes(1, 1, 8192, 128, False)
    assert 3.9 < r < 4.0
    c = bench.kvouter_bytes(1, 1, 8192, 128, True) / bench.kvouter_bytes(1, 1, 8192, 128, False)
    assert 0.5 < c < 0.52
    # against the queries-outer floor: two orders of magnitude at N = 8192
    assert bench.kvouter_bytes(1, 16, 8192, 128, False) > 100 * bench.floor_bytes("fwd", 1, 16, 8192, 128)


def test_step_percentiles_nearest_rank():
    # nearest-rank on the sorted sample, whatever the input order
    assert bench.percentiles([5.0, 1.0, 3.0, 2.0, 4.0]) == {10: 1.0, 50: 3.0, 90: 5.0}
    xs = [float(i) for i in range(101)]
    assert bench.percentiles(xs[::-1]) == {10: 10.0, 50: 50.0, 90: 90.0}
    assert bench.percentiles([7.0]) == {10: 7.0, 50: 7.0, 90: 7.0}


def test_l2_read_model_closed_forms():
    B, H, N, d, blk = 2, 3, 1024, 64, 128
    nb = N // blk
    row = d * 2
    # non-causal: the streamed pair is read once per block
    assert bench.l2_read_model("fwd", B, H, N, d, False, blk) == B * H * (N * row + 2 * nb * N * row)
    assert bench.l2_read_model("bwd_dq", B, H, N, d, False, blk) == B * H * (N * (2 * row + 8) + 2 * nb * N * row)
    assert bench.l2_read_model("bwd_dkdv", B, H, N, d, False, blk) == B * H * (2 * N * row + nb * N * (2 * row + 8))
    # causal: query block i sees (i + 1) blk keys; key block j is seen by N - j blk rows
    seen = blk * nb * (nb + 1) // 2
    seen_t = N * nb - blk * nb * (nb - 1) // 2
    assert seen == seen_t      # the same triangle, counted from either side
    assert bench.l2_read_model("fwd", B, H, N, d, True, blk) == B * H * (N * row + 2 * seen * row)
    assert bench.l2_read_model("bwd_dkdv", B, H, N, d, True, blk) == B * H * (2 * N * row + seen_t * (2 * row + 8))
    # one block covering everything: each operand read once, as the O(Nd) floor counts them
    assert bench.l2_read_model("fwd", 1, 1, 256, 64, False, 256) == 3 * 256 * 64 * 2
