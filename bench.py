#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input: the
forward kernel and the three backward launches (D = rowsum(dO * O), the
keys-outer dK/dV kernel, the queries-outer dQ kernel), each through the C ABI
on torch's current stream.  Default workload: long-context causal attention,
B=1, H=16, N=16384, d=128, bf16 (inputs N(0,1) * 0.5, dO N(0,1)).

FLOP convention: forward = 4 N^2 d B H, halved when causal, times the
nonzero-block fraction when block-sparse; forward + backward = 2.5 x forward.
value = (flops of one step) / (wall time of one step), in TFLOP/s.

The JSON line also carries
  roofline: the dominant kernel (largest average launch time, measured with
            HIP events on the launch stream over the timed steps): its
            algorithmic flops per launch / its average duration, against the
            bf16 dense MFMA peak of 2.5 PFLOP/s; traffic is the HBM bytes per
            launch from the committed rocprofv3 counter summary when it was
            taken on the current kernel source, else null;
  cpu_baseline: the fp64 oracle timed on this host's cores on a bounded
            random sample of query rows of the same workload (forward rows
            plus the backward dQ of those rows), scaled to TFLOP/s with the
            same convention.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
HBM_PEAK_GBS = 8000.0               # MI355X HBM3E

# kernel name (as rocprofv3 reports it) -> source file, for the traffic
# summaries' staleness check
KERNEL_SOURCES = {
    "fwd": ("exact_io_aware_36_amd/csrc/fa_fwd.hip", "exact_io_aware_36_amd/csrc/fa_fwd_pp.hip"),
    "bwd_dot": "exact_io_aware_36_amd/csrc/fa_bwd.hip",
    "bwd_dkdv": "exact_io_aware_36_amd/csrc/fa_bwd_dkdv.hip",
    "bwd_dq": "exact_io_aware_36_amd/csrc/fa_bwd.hip",
    "bwd_sparse": ("exact_io_aware_36_amd/csrc/fa_bwd.hip", "exact_io_aware_36_amd/csrc/fa_bwd_dkdv.hip"),
    "decode": "exact_io_aware_36_amd/csrc/fa_decode.hip",
    "fwd_fp8": "exact_io_aware_36_amd/csrc/fa_fp8.hip",
}


# ---------------------------------------------------------------------------
# accounting (no attention arithmetic: counts only)

def fwd_flops(B, H, N, d, causal=False, sparse_frac=None) -> float:
    f = 4.0 * N * N * d * B * H
    if causal:
        f *= 0.5
    if sparse_frac is not None:
        f *= sparse_frac
    return f


def step_flops(B, H, N, d, causal=False, sparse_frac=None, backward=False) -> float:
    f = fwd_flops(B, H, N, d, causal, sparse_frac)
    return 2.5 * f if backward else f


def kernel_flops(stage, B, H, N, d, causal=False, sparse_frac=None) -> float:
    """Algorithmic matrix-product flops one launch performs: the forward does
    two products per (query, allowed key) pair (S and P V), the dK/dV kernel
    four (S, dP, dV, dK), the dQ kernel three (S, dP, dQ); 2 d flops each."""
    f = fwd_flops(B, H, N, d, causal, sparse_frac)
    return {"fwd": f, "bwd_dkdv": 2.0 * f, "bwd_dq": 1.5 * f, "bwd_dot": 0.0,
            "bwd_sparse": 3.5 * f}[stage]


def floor_bytes(stage, B, H, N, d, elem=2) -> float:
    """The O(N d) input/output floor of one launch."""
    t = B * H * N * d * elem
    rows = B * H * N * 4
    return {
        "fwd": 4 * t + rows,                 # Q, K, V in; O out; LSE out
        "bwd_dot": 2 * t + 3 * rows,         # O, dO, LSE in; D, LSE*log2e out
        "bwd_dkdv": 6 * t + 2 * rows,        # Q, K, V, dO, LSE*log2e, D in; dK, dV out
        "bwd_dq": 5 * t + 2 * rows,          # Q, K, V, dO, LSE*log2e, D in; dQ out
        "bwd_sparse": 8 * t + 4 * rows,      # the three launches of the sparse backward
        # E4M3 Q, K, V in (1 byte each); O bf16 and LSE out; the 128-row scales
        "fwd_fp8": 3 * (t // elem) + t + rows + 2 * 4 * B * H * ((N + 127) // 128) + 4 * B * H,
    }[stage]


def l2_read_model(stage, B, H, N, d, causal, block, elem=2) -> float:
    """Bytes one launch reads from L2 under the blocked schedule, before any
    L1 reuse: the operand that stays on chip is read once; the streamed pair
    is read once per block of `block` rows that needs it (causal: only the
    rows or keys on the block's side of the diagonal), plus the per-row fp32
    statistics that come with it.
      fwd       Q once; K, V per query block of `block` rows
      bwd_dkdv  K, V once; Q, dO, LSE log2(e), D per key block of `block` keys
      bwd_dq    Q, dO, LSE log2(e), D once; K, V per query block of `block` rows"""
    nb = (N + block - 1) // block
    if causal:
        # query block i sees keys [0, (i+1) block); key block j is seen by rows [j block, N)
        seen = sum(min(N, (i + 1) * block) for i in range(nb))
        seen_t = sum(N - j * block for j in range(nb))
    else:
        seen = seen_t = nb * N
    row = d * elem
    if stage == "fwd":
        return B * H * (N * row + 2 * seen * row)
    if stage == "bwd_dkdv":
        return B * H * (2 * N * row + seen_t * (2 * row + 8))
    if stage == "bwd_dq":
        return B * H * (N * (2 * row + 8) + 2 * seen * row)
    raise ValueError(stage)


def standard_io_elements(N, d) -> float:
    """Standard attention's HBM traffic in elements, 2N^2 + 4Nd, as the
    worked accounting of "01 · FlashAttention" (step 5 of 5, "show the
    accounting") counts it."""
    return 2.0 * N * N + 4.0 * N * d


def flash_io_elements(N, d, M) -> float:
    """The same page's tiled count, 4Nd + 2 N^2 d^2 / M, with M the number
    of elements that fit on chip."""
    return 4.0 * N * d + 2.0 * N * N * d * d / M


def kvouter_bytes(B, H, N, d, causal) -> float:
    """Algorithmic HBM bytes of one fa_fwd_kvouter call (the key/value-outer
    loop order): per 64-key block j, every 128-row query block that sees it
    reads its Q rows (bf16) and, from the second block on, its fp32 O
    accumulator and the two fp32 statistics, then writes them back; K_j and
    V_j count once; a last pass reads the accumulator and statistics and
    writes O (bf16) and LSE."""
    tc = (N + 63) // 64
    total = 0.0
    for qb in range((N + 127) // 128):
        rows = min(128, N - 128 * qb)
        n_j = min(tc, (128 * qb + 127) // 64 + 1) if causal else tc
        per = rows * d * 2 + rows * d * 4 + 8 * rows          # Q in, O and m, l out
        total += n_j * per + (n_j - 1) * (rows * d * 4 + 8 * rows)   # reads after block 0
    total += 2 * N * d * 2                                     # K, V once
    total += N * d * 4 + 8 * N + N * d * 2 + 4 * N             # the last pass
    return B * H * total


# ---------------------------------------------------------------------------

# what else decides a kernel's machine code: the two headers every kernel
# includes and the build script that holds the compiler flags
KERNEL_HEADERS = ("exact_io_aware_36_amd/csrc/fa_tile.h", "exact_io_aware_36_amd/csrc/fa_internal.h",
                  "exact_io_aware_36_amd/build.py")


def source_digest(path) -> str:
    """First 16 hex digits of the sha256 over the kernel source (one path, or
    a tuple of them for a stage spanning several files) followed by the two
    headers every kernel includes and the build script (compiler flags)."""
    h = hashlib.sha256()
    paths = (path,) if isinstance(path, str) else tuple(path)
    for p in paths + KERNEL_HEADERS:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(stage: str, workload: str):
    """HBM bytes per launch from profiles/traffic_<stage>_<workload>.txt, or
    None when absent or taken on another version of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_digest(KERNEL_SOURCES[stage]):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def percentiles(xs, qs=(10, 50, 90)):
    """Nearest-rank percentiles of a list of floats."""
    ys = sorted(xs)
    out = {}
    for q in qs:
        i = min(len(ys) - 1, max(0, int(round(q / 100 * (len(ys) - 1)))))
        out[q] = ys[i]
    return out


def cpu_baseline(inp, w, metric_flops, budget_s=15.0, seed=99):
    """Time the oracle on a random sample of query rows (forward rows, and for
    workloads with a backward also dQ of the same rows); credit the sample
    with its share of the step's metric flops."""
    import numpy as np

    import oracle

    B, H, N, d = inp["B"], inp["H"], inp["N"], inp["d"]
    total_rows = B * H * N
    f64 = {n: inp[n].double().numpy() for n in ("q", "k", "v") if inp.get(n) is not None}
    if w.backward:
        f64["dout"] = inp["dout"].double().numpy()
    lens = inp["kv_lens"].numpy() if inp.get("kv_lens") is not None else None
    mask = inp["block_mask"].numpy() if inp.get("block_mask") is not None else None
    rng = np.random.default_rng(seed)

    def run(rows):
        oracle.fwd_rows(f64["q"], f64["k"], f64["v"], rows, causal=w.causal, scale=w.scale,
                        kv_lens=lens, block_mask=mask, mask_block=w.mask_block)
        if w.backward:
            # dQ of the sampled rows, head by head
            bh = rows // N
            for g in np.unique(bh):
                b, h = divmod(int(g), H)
                sel = rows[bh == g] % N
                oracle.bwd_sample(f64["q"][b, h], f64["k"][b, h], f64["v"][b, h],
                                  f64["dout"][b, h], sel, np.zeros(0, np.int64), causal=w.causal,
                                  scale=w.scale, kv_len=None if lens is None else int(lens[b]),
                                  block_mask=mask, mask_block=w.mask_block)

    # batches of random rows (doubling) until the budget is spent
    done = 0
    dt = 0.0
    batch = 64
    while dt < budget_s and done < total_rows:
        rows = np.sort(rng.choice(total_rows, min(batch, total_rows - done), replace=False))
        t0 = time.perf_counter()
        run(rows)
        dt += time.perf_counter() - t0
        done += rows.size
        batch *= 2
    n = done
    flops = metric_flops * n / total_rows
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"{n} of {total_rows} query rows drawn uniformly at random (batches of 64, 128, "
                   f"... until {budget_s:.0f} s): oracle fp64 forward "
                   f"rows{' + backward dQ rows' if w.backward else ''}, {dt:.1f} s; credited "
                   f"{n}/{total_rows} of one step's {metric_flops:.4g} flops"),
        "seconds": dt,
    }


def decode_accounting(B, H, nq, d, lens, causal=False):
    """Flops and algorithmic bytes of one decode-shaped forward call: each
    query row against the keys it sees (2 products, 2 d flops each per pair);
    bytes = the visible K and V rows once + Q, O (bf16) + LSE (fp32)."""
    pairs = 0
    for L in lens:
        for t in range(nq):
            pairs += max(0, (L - nq + t + 1) if causal else L)
    flops = 4.0 * d * H * pairs
    kv_rows = H * sum(int(L) for L in lens)
    nbytes = 2 * kv_rows * d * 2 + 2 * B * H * nq * d * 2 + B * H * nq * 4
    return flops, nbytes


def cpu_baseline_decode(inp, w, budget_s=15.0):
    """Time the oracle's decode forward over the whole workload, repeated
    until the budget is spent."""
    import numpy as np

    import oracle

    q = inp["q"].double().numpy()
    k = inp["k"].double().numpy()
    v = inp["v"].double().numpy()
    lens = inp["kv_lens"].numpy() if inp["kv_lens"] is not None else None
    reps, dt = 0, 0.0
    while dt < budget_s:
        t0 = time.perf_counter()
        oracle.decode(q, k, v, causal=w.causal, scale=w.scale, kv_lens=lens)
        dt += time.perf_counter() - t0
        reps += 1
    flops, _ = decode_accounting(inp["B"], inp["H"], w.nq, inp["d"],
                                 lens if lens is not None else [inp["N"]] * inp["B"], w.causal)
    return {"value": flops * reps / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"the whole workload, {reps} oracle fp64 decode call(s) in {dt:.1f} s",
            "seconds": dt}


def bench_decode(args, w, inp, fa, torch):
    """One step = one fa_fwd_splitkv call (the split kernel and the merge)."""
    B, H, N, d, nq = inp["B"], inp["H"], inp["N"], inp["d"], w.nq
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    lens_h = inp["kv_lens"] if inp["kv_lens"] is not None else torch.full((B,), N, dtype=torch.int32)
    lens = lens_h.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, nq), dtype=torch.float32, device=dev)
    nbytes_ws = fa.fa_fwd_splitkv_workspace_bytes(B, H, nq, N, d, 0)
    ws = torch.empty(max(nbytes_ws, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def launch():
        fa.fa_fwd_splitkv(q, k, v, o, lse, ws, causal=w.causal, scale=w.scale, kv_lens=lens)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        launch()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    call_ms = sum(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)) / args.steps
    flops, nbytes = decode_accounting(B, H, nq, d, lens_h.tolist(), w.causal)
    gbs = nbytes / (call_ms * 1e-3) / 1e9
    traffic = read_traffic("decode", w.name)
    roofline = {"kernel": "decode", "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "avg_launch_ms": round(call_ms, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_decode(inp, w, budget_s=args.cpu_budget)
        cpu = {k2: (round(v2, 6) if isinstance(v2, float) else v2) for k2, v2 in cpu.items()}
    line = {
        "metric": "attention TFLOP/s fwd & fwd+bwd, % bf16 MFMA peak, N=256-16K, d=64/128",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "Nq": nq, "Nk": N, "d": d,
                   "causal": w.causal, "pass": "fwd (decode, split keys)",
                   "splits": fa.fa_splitkv_splits(B, H, N, 0), "flops_per_step": flops,
                   "bytes_per_step": nbytes,
                   "flop_convention": "4 d flops per (query row, visible key) pair"},
        "roofline": roofline, "cpu_baseline": cpu,
        "detail": {"call_ms": round(call_ms, 4), "hbm_gbs": round(gbs, 1)},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_fp8(args, w, inp, fa, torch):
    """One step = one fa_fwd_fp8 call on inputs already quantised in HBM
    (Q, K rotated with random signs; the quantiser is timed on the side)."""
    import workloads

    B, H, N, d = inp["B"], inp["H"], inp["N"], inp["d"]
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    signs = workloads.random_signs(d, w.seed).to(dev)
    stream = torch.cuda.current_stream(dev)

    def quantize():
        q8, qs = fa.quantize_fp8(q, 128, signs)
        k8, ks = fa.quantize_fp8(k, 128, signs)
        v8t, vs = fa.quantize_fp8(v, 0, None, transpose=True)
        return q8, qs, k8, ks, v8t, vs

    q8, qs, k8, ks, v8t, vs = quantize()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def launch():
        fa.fa_fwd_fp8(q8, k8, v8t, qs, ks, vs, o, lse, causal=w.causal, scale=w.scale)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        launch()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    call_ms = sum(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)) / args.steps
    flops = fwd_flops(B, H, N, d, w.causal)
    achieved = flops / (call_ms * 1e-3) / 1e12
    # the quantiser, for context (not part of the step)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        quantize()
    e1.record(stream)
    torch.cuda.synchronize()
    roofline = {"kernel": "fwd_fp8", "bound": "mfma", "achieved": round(achieved, 2),
                "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_FP8_PEAK_TFLOPS, 4),
                "traffic": read_traffic("fwd_fp8", w.name), "avg_launch_ms": round(call_ms, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, w, flops, budget_s=args.cpu_budget)
        cpu = {k2: (round(v2, 6) if isinstance(v2, float) else v2) for k2, v2 in cpu.items()}
    line = {
        "metric": "attention TFLOP/s fwd & fwd+bwd, % bf16 MFMA peak, N=256-16K, d=64/128",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "pass": "fwd (FP8 E4M3 operands, fp32 accumulation)", "flops_per_step": flops,
                   "pct_fp8_mfma_peak": round(100 * achieved / MFMA_FP8_PEAK_TFLOPS, 2),
                   "flop_convention": "fwd 4N^2dBH (x1/2 causal)"},
        "roofline": roofline, "cpu_baseline": cpu,
        "detail": {"call_ms": round(call_ms, 4), "quantize_qkv_ms": round(e0.elapsed_time(e1) / 5, 4)},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_sweep(args, fa, torch):
    """The metric's range: N = 256 ... 16384 with 16384 tokens per batch
    (B = 16384 / N), H = 16, d = 64, 128 and 256, causal and not; seeded
    N(0,1) inputs (x 0.5 for Q, K, V), dO N(0,1).  For each point: the
    forward alone and forward + backward (dense stages), HIP events over
    args.steps calls after args.warmup."""
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for d in (64, 128, 256):
        for N in (256, 512, 1024, 2048, 4096, 8192, 16384):
            B, H = max(1, 16384 // N), 16
            inp = workloads.random_qkv(B, H, N, d, seed=2000 + N + d, input_scale=0.5)
            q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
            o = torch.empty_like(q)
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
            ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
            for causal in (False, True):
                scale = 1.0 / math.sqrt(d)

                def fwd():
                    fa.fa_fwd(q, k, v, o, lse, causal=causal, scale=scale)

                def step():
                    fwd()
                    fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=causal, scale=scale)

                f = fwd_flops(B, H, N, d, causal)
                t_f = timed(fwd, args.steps)
                t_s = timed(step, args.steps)
                print(json.dumps({
                    "sweep": "attention fwd / fwd+bwd", "B": B, "H": H, "N": N, "d": d,
                    "causal": causal, "fwd_ms": round(t_f, 4),
                    "fwd_tflops": round(f / (t_f * 1e-3) / 1e12, 1),
                    "fwd_pct_peak": round(100 * f / (t_f * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 1),
                    "fwd_bwd_ms": round(t_s, 4),
                    "fwd_bwd_tflops": round(2.5 * f / (t_s * 1e-3) / 1e12, 1)}), flush=True)
            del q, k, v, do, o, lse, dq, dk, dv, ws
    return 0


def bench_io_ablation(args, fa, torch):
    """The loop-order ablation: for N = 2048, 4096, 8192 (d = 128, H = 16,
    B = 1, non-causal, seeded N(0,1) inputs x 0.5) the forward (queries
    outer, O and the statistics in registers) against fa_fwd_kvouter (keys
    outer, O and the statistics through HBM once per 64-key block), with
    each one's algorithmic HBM bytes and the pages' element counts for the
    same N (M = 65536 elements on chip)."""
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    d, H, B = 128, 16, 1
    for N in (2048, 4096, 8192):
        inp = workloads.random_qkv(B, H, N, d, seed=2500 + N, input_scale=0.5, with_dout=False)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_fwd_kvouter_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
        t_q = timed(lambda: fa.fa_fwd(q, k, v, o, lse, causal=False), args.steps)
        t_k = timed(lambda: fa.fa_fwd_kvouter(q, k, v, o, lse, ws, causal=False), max(2, args.steps // 4))
        f = fwd_flops(B, H, N, d, False)
        print(json.dumps({
            "io_ablation": "forward loop order", "B": B, "H": H, "N": N, "d": d, "causal": False,
            "queries_outer_ms": round(t_q, 4), "keys_outer_ms": round(t_k, 4),
            "queries_outer_tflops": round(f / (t_q * 1e-3) / 1e12, 1),
            "keys_outer_tflops": round(f / (t_k * 1e-3) / 1e12, 1),
            "queries_outer_floor_bytes": floor_bytes("fwd", B, H, N, d),
            "keys_outer_model_bytes": kvouter_bytes(B, H, N, d, False),
            "page_standard_elements_per_head": standard_io_elements(N, d),
            "page_tiled_elements_per_head_m65536": flash_io_elements(N, d, 65536)}), flush=True)
        del q, k, v, o, lse, ws
    return 0


def _timed(torch, stream, fn, warmup, reps):
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def metric_range(fa, torch, steps=5, warmup=2, ds=(64, 128)):
    """The metric's range, compactly: N = 256 ... 16384 with 16384 tokens per
    batch (B = 16384 / N), H = 16, d = 64 and 128, causal and not; for each
    point the forward alone and forward + backward (default kernels), HIP
    events over `steps` calls.  Inputs N(0,1) x 0.5 (dO N(0,1)) drawn on the
    GPU from a fixed seed (timing only; parity is tested elsewhere)."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev)
    out = []
    for d in ds:
        for N in (256, 512, 1024, 2048, 4096, 8192, 16384):
            B, H = max(1, 16384 // N), 16
            gen.manual_seed(3000 + N + d)
            shape = (B, H, N, d)
            q, k, v = ((torch.randn(shape, generator=gen, device=dev) * 0.5).to(torch.bfloat16)
                       for _ in range(3))
            do = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
            o = torch.empty_like(q)
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
            ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
            for causal in (False, True):
                def fwd():
                    fa.fa_fwd(q, k, v, o, lse, causal=causal)

                def step():
                    fwd()
                    fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=causal)

                f = fwd_flops(B, H, N, d, causal)
                t_f = _timed(torch, stream, fwd, warmup, steps)
                t_s = _timed(torch, stream, step, warmup, steps)
                out.append({"N": N, "d": d, "B": B, "causal": causal, "fwd_ms": round(t_f, 4),
                            "fwd_tflops": round(f / (t_f * 1e-3) / 1e12, 1),
                            "fwd_pct_peak": round(100 * f / (t_f * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 1),
                            "fwd_bwd_ms": round(t_s, 4),
                            "fwd_bwd_tflops": round(2.5 * f / (t_s * 1e-3) / 1e12, 1)})
            del q, k, v, do, o, lse, dq, dk, dv, ws
    return out


def next_rows(fa, torch, workloads, steps=5, warmup=2):
    """The extensions beyond the dense path, once each at their workloads'
    shapes (timing only; parity is tested elsewhere): the block-sparse forward +
    backward, the split-KV decode step, the d = 256 forward + backward and the
    FP8 forward.  Q, K, V (and dO) are drawn on the GPU from a fixed seed at the
    workload's input scale; key lengths and the block mask come from the
    workload's own CPU generator.  Compute-bound rows give metric-convention
    TFLOP/s against their MFMA peak, the decode step HBM GB/s against 8 TB/s."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev)
    res = {}

    def draw(w, shape, scale=None):
        sc = w.input_scale if scale is None else scale
        return (torch.randn(shape, generator=gen, device=dev) * sc).to(torch.bfloat16)

    # block-sparse forward + backward
    w = workloads.WORKLOADS["block_sparse_fwdbwd"]
    gen.manual_seed(w.seed)
    B, H, N, d = w.B, w.H, w.N, w.d
    q, k, v = (draw(w, (B, H, N, d)) for _ in range(3))
    do = draw(w, (B, H, N, d), 1.0)
    mask = workloads.block_mask(N // w.mask_block, w.sparse_frac,
                                torch.Generator().manual_seed(w.seed)).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)

    def sp_fwd():
        fa.fa_fwd_blocksparse(q, k, v, o, lse, mask, mask_block=w.mask_block, scale=w.scale)

    def sp_bwd():
        fa.fa_bwd_blocksparse(q, k, v, o, do, lse, dq, dk, dv, ws, mask,
                              mask_block=w.mask_block, scale=w.scale)

    sp_fwd()
    t_f = _timed(torch, stream, sp_fwd, warmup, steps)
    t_b = _timed(torch, stream, sp_bwd, warmup, steps)
    ff = fwd_flops(B, H, N, d, False, w.sparse_frac)
    res["block_sparse_fwdbwd"] = {
        "fwd_ms": round(t_f, 4), "bwd_ms": round(t_b, 4),
        "fwd_bwd_tflops": round(2.5 * ff / ((t_f + t_b) * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100 * 2.5 * ff / ((t_f + t_b) * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2)}
    del q, k, v, do, o, dq, dk, dv, ws

    # split-KV decode step
    w = workloads.WORKLOADS["decode_splitkv"]
    gen.manual_seed(w.seed)
    B, H, N, d, nq = w.B, w.H, w.N, w.d, w.nq
    q = draw(w, (B, H, nq, d))
    k, v = draw(w, (B, H, N, d)), draw(w, (B, H, N, d))
    lo, hi = w.kv_len_range
    lens_h = torch.randint(lo, hi + 1, (B,), generator=torch.Generator().manual_seed(w.seed),
                           dtype=torch.int32)
    lens = lens_h.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, nq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(fa.fa_fwd_splitkv_workspace_bytes(B, H, nq, N, d, 0), 256),
                     dtype=torch.uint8, device=dev)

    def dec():
        fa.fa_fwd_splitkv(q, k, v, o, lse, ws, causal=w.causal, scale=w.scale, kv_lens=lens)

    t = _timed(torch, stream, dec, warmup, steps)
    _, nbytes = decode_accounting(B, H, nq, d, lens_h.tolist(), w.causal)
    gbs = nbytes / (t * 1e-3) / 1e9
    res["decode_splitkv"] = {"call_ms": round(t, 4), "hbm_gbs": round(gbs, 1),
                             "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
    del q, k, v, o, ws

    # d = 256 forward + backward
    w = workloads.WORKLOADS["d256_fwdbwd"]
    gen.manual_seed(w.seed)
    B, H, N, d = w.B, w.H, w.N, w.d
    q, k, v = (draw(w, (B, H, N, d)) for _ in range(3))
    do = draw(w, (B, H, N, d), 1.0)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)

    def f256():
        fa.fa_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale)

    def b256():
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=w.causal, scale=w.scale)

    f256()
    t_f = _timed(torch, stream, f256, warmup, steps)
    t_b = _timed(torch, stream, b256, warmup, steps)
    ff = fwd_flops(B, H, N, d, w.causal)
    res["d256_fwdbwd"] = {
        "fwd_ms": round(t_f, 4), "fwd_tflops": round(ff / (t_f * 1e-3) / 1e12, 2),
        "bwd_ms": round(t_b, 4),
        "fwd_bwd_tflops": round(2.5 * ff / ((t_f + t_b) * 1e-3) / 1e12, 2)}
    del q, k, v, do, o, dq, dk, dv, ws

    # FP8 forward on quantised inputs (Q, K rotated with the workload's signs)
    w = workloads.WORKLOADS["long_context_fp8"]
    gen.manual_seed(w.seed)
    B, H, N, d = w.B, w.H, w.N, w.d
    q, k, v = (draw(w, (B, H, N, d)) for _ in range(3))
    signs = workloads.random_signs(d, w.seed).to(dev)
    q8, qs = fa.quantize_fp8(q, 128, signs)
    k8, ks = fa.quantize_fp8(k, 128, signs)
    v8t, vs = fa.quantize_fp8(v, 0, None, transpose=True)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    def f8():
        fa.fa_fwd_fp8(q8, k8, v8t, qs, ks, vs, o, lse, causal=w.causal, scale=w.scale)

    t = _timed(torch, stream, f8, warmup, steps)
    ff = fwd_flops(B, H, N, d, w.causal)
    res["long_context_fp8"] = {"fwd_ms": round(t, 4), "fwd_tflops": round(ff / (t * 1e-3) / 1e12, 2),
                               "pct_fp8_peak": round(100 * ff / (t * 1e-3) / 1e12 / MFMA_FP8_PEAK_TFLOPS, 2)}
    return res


def other_configs(fa, torch, workloads, steps=10, warmup=3):
    """The other measured workloads once each (default kernels, their seeded
    inputs): the single-head fp32 forward, the GPT-2-shaped causal forward,
    the BERT-shaped padded forward + backward and the block-sparse forward;
    metric-convention TFLOP/s and per-stage times."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name in ("single_head_fp32", "gpt2_medium_causal", "bert_large_padded", "block_sparse"):
        w = workloads.WORKLOADS[name]
        inp = workloads.make_inputs(w)
        B, H, N, d = inp["B"], inp["H"], inp["N"], inp["d"]
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        lens = inp["kv_lens"].to(dev) if inp["kv_lens"] is not None else None
        mask = inp["block_mask"].to(dev) if inp["block_mask"] is not None else None
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

        def fwd():
            if mask is not None:
                fa.fa_fwd_blocksparse(q, k, v, o, lse, mask, mask_block=w.mask_block, scale=w.scale)
            else:
                fa.fa_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale, kv_lens=lens)

        t_f = _timed(torch, stream, fwd, warmup, steps)
        ff = fwd_flops(B, H, N, d, w.causal, w.sparse_frac)
        r = {"fwd_ms": round(t_f, 4), "fwd_tflops": round(ff / (t_f * 1e-3) / 1e12, 2)}
        if w.backward:
            do = inp["dout"].to(dev)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
            ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)

            def step():
                fwd()
                fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=w.causal, scale=w.scale,
                          kv_lens=lens)

            t_s = _timed(torch, stream, step, warmup, steps)
            r.update({"fwd_bwd_ms": round(t_s, 4),
                      "fwd_bwd_tflops": round(2.5 * ff / (t_s * 1e-3) / 1e12, 2)})
        res[name] = r
    return res


# ---------------------------------------------------------------------------
# profiler summaries: rocprofv3 CSVs (under gpurun_out/) -> profiles/*.txt

DIGEST_PATTERNS = {"fwd": ["fwd_bf16_kernel", "fwd_pp_kernel", "fwd_bf16_t256_kernel"],
                   "bwd_dot": ["bwd_dot_kernel"], "bwd_dkdv": ["bwd_dkdv_kernel"],
                   "bwd_dq": ["bwd_dq_kernel"],
                   "bwd_sparse": ["bwd_dot_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"],
                   "fwd_fp8": ["fwd_fp8_kernel"], "decode": ["decode_kernel", "merge_kernel"]}
SQ_GROUP = ("GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
            "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS")


def _short_kernel(name):
    import re
    import subprocess

    if name.startswith("_Z"):
        name = subprocess.run(["c++filt", name], capture_output=True, text=True).stdout.strip() or name
    name = re.sub(r"^void ", "", name).replace("(anonymous namespace)::", "")
    return re.sub(r"\([^()]*\)$", "", name)


def digest(workload, stages, root=ROOT, steps=10, warmup=3):
    """Write profiles/kernel_stats_<workload>.txt from the kernel trace of
    `rocprofv3 --kernel-trace --stats ... -o <workload> -- python3 bench.py
    --workload <workload> --steps 10 --warmup 3 --quick` (stdout of that run
    in gpurun_out/<workload>_stats.log), and for each stage
    profiles/traffic_<stage>_<workload>.txt from three counter runs
    (<workload>_p1: FETCH_SIZE, _p2: WRITE_SIZE, _p3: the SQ group) of
    `bench.py --workload <workload> --steps 2 --warmup 1 --quick
    --copy-calibration 512`, the counters scaled by what they read for the
    512 MiB copy."""
    import csv
    from collections import defaultdict

    import workloads

    w = workloads.WORKLOADS[workload]
    go = os.path.join(root, "gpurun_out")
    wdesc = (f"B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} {'causal' if w.causal else 'non-causal'}"
             + (f", kv_len U{{{w.kv_len_range[0]}..{w.kv_len_range[1]}}}" if w.kv_len_range else "")
             + (", block mask" if w.sparse_frac else "") + (", fp8" if w.fp8 else ""))
    trace_csv = os.path.join(go, "prof", f"{workload}_kernel_trace.csv")
    if os.path.exists(trace_csv):
        per = defaultdict(list)
        for r in csv.DictReader(open(trace_csv)):
            if "fa::" in r["Kernel_Name"] or r["Kernel_Name"].startswith("_ZN2fa"):
                per[_short_kernel(r["Kernel_Name"])].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        tot = sum(sum(v) for v in per.values())
        line = None
        for ln in open(os.path.join(go, f"{workload}_stats.log")):
            if ln.startswith("{"):
                line = json.loads(ln)
        det = line["detail"] if line else {}
        ev = (", ".join(f"{k} {v}" for k, v in det["stage_ms"].items()) if "stage_ms" in det
              else f"whole call {det.get('call_ms')}")
        out = [f"# rocprofv3 kernel statistics: {workload} ({wdesc})",
               "# command (from the repository root, on one MI355X):",
               f"#   rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof -o {workload} "
               f"-- python3 bench.py --workload {workload} --steps {steps} --warmup {warmup} --quick",
               f"# summary: python3 bench.py --digest {workload} (CPU; reads gpurun_out/)",
               f"# {steps + warmup} calls per kernel = {warmup} warm-up + {steps} timed steps. Durations in microseconds.",
               f"# HIP-event averages over the timed steps printed by that same bench run (ms): {ev}",
               "# timed_avg_us: average over the last calls (the timed steps), from the kernel trace of the same run.",
               "",
               f"{'kernel':<60}{'calls':>6}{'avg_us':>11}{'min_us':>11}{'max_us':>11}{'pct':>7}{'timed_avg_us':>14}"]
        for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            tv = v[-steps:]
            out.append(f"{k:<60}{len(v):>6}{sum(v)/len(v):>11.1f}{min(v):>11.1f}{max(v):>11.1f}"
                       f"{100*sum(v)/tot:>7.2f}{sum(tv)/len(tv):>14.1f}")
        with open(os.path.join(root, "profiles", f"kernel_stats_{workload}.txt"), "w") as f:
            f.write("\n".join(out) + "\n")
        print("\n".join(out))

    def rows(p):
        return list(csv.DictReader(open(os.path.join(go, "pmc", f"{workload}_p{p}_counter_collection.csv"))))

    def per_launch(rs, pats, counter):
        d = defaultdict(float)
        names = {}
        for r in rs:
            if r["Counter_Name"] == counter and any(pt in r["Kernel_Name"] for pt in pats):
                d[r["Dispatch_Id"]] += float(r["Counter_Value"])
                names[r["Dispatch_Id"]] = _short_kernel(r["Kernel_Name"])
        by = defaultdict(list)
        for k, v in d.items():
            by[names[k]].append(v)
        return sum(sum(v) / len(v) for v in by.values()), sorted(by)

    def copy_kib(rs, counter):
        return max((float(r["Counter_Value"]) for r in rs
                    if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower()), default=0.0)

    if not stages:
        return
    p1, p2, p3 = rows(1), rows(2), rows(3)
    cf, cw = copy_kib(p1, "FETCH_SIZE"), copy_kib(p2, "WRITE_SIZE")
    ff, fw = 512 * 1024 / cf, 512 * 1024 / cw
    # optional fourth run: L2 read sectors (32 B), scaled by what the copy reads
    p4_path = os.path.join(go, "pmc", f"{workload}_p4_counter_collection.csv")
    p4 = rows(4) if os.path.exists(p4_path) else None
    L2C = "TCC_READ_SECTORS_sum"
    if p4 is not None:
        cs = max((float(r["Counter_Value"]) for r in p4
                  if r["Counter_Name"] == L2C and "copy" in r["Kernel_Name"].lower()), default=0.0)
        fs = 512 * (1 << 20) / (32 * cs) if cs else 0.0
    for stage in stages:
        pats = DIGEST_PATTERNS[stage]
        fetch, kn = per_launch(p1, pats, "FETCH_SIZE")
        write, _ = per_launch(p2, pats, "WRITE_SIZE")
        c3 = {c: per_launch(p3, pats, c)[0] for c in SQ_GROUP.split()}
        if stage == "decode":
            lens = workloads.make_inputs(w)["kv_lens"].numpy()
            floor = decode_accounting(w.B, w.H, w.nq, w.d, lens, w.causal)[1]
        else:
            floor = floor_bytes(stage, w.B, w.H, w.N, w.d)
        hbm = fetch * 1024 * ff + write * 1024 * fw
        what = "one launch" if len(kn) == 1 else f"one call (its {len(kn)} launches)"
        groups = [(1, "FETCH_SIZE"), (2, "WRITE_SIZE"), (3, SQ_GROUP)] + ([(4, L2C)] if p4 is not None else [])
        cmd = [f"#   rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc -o {workload}_p{i} -- "
               f"python3 bench.py --workload {workload} --steps 2 --warmup 1 --quick --copy-calibration 512"
               for i, c in groups]
        busy = c3["SQ_BUSY_CU_CYCLES"]
        out = [f"# HBM traffic of {what} of the {stage} stage ({' + '.join(kn)}), {workload}",
               f"# ({wdesc}), from rocprofv3 counters.",
               "# commands (from the repository root, on one MI355X; one counter group per run):", *cmd,
               f"# summary: python3 bench.py --digest {workload} {stage} (CPU; reads gpurun_out/)",
               "# Scaling: the same runs first copy 512 MiB with a plain device copy; its counters read",
               f"# FETCH_SIZE {cf:.0f} KiB and WRITE_SIZE {cw:.0f} KiB for 524288 KiB moved each way, so",
               f"# FETCH_SIZE is multiplied by {ff:.4f} and WRITE_SIZE by {fw:.4f}.",
               "# source_sha256 is the first 16 hex digits of the sha256 over the kernel source, the two shared",
               "# kernel headers and the build script (compiler flags) when measured; bench.py reports this",
               "# traffic only while they are unchanged.",
               f"source_sha256: {source_digest(KERNEL_SOURCES[stage])}",
               f"fetch_size_kib_per_launch: {fetch:.1f}",
               f"write_size_kib_per_launch: {write:.1f}",
               f"fetch_bytes_scaled: {fetch*1024*ff:.0f}",
               f"write_bytes_scaled: {write*1024*fw:.0f}",
               f"hbm_bytes_per_launch: {hbm:.0f}",
               f"floor_bytes_per_launch: {floor:.0f}   # O(Nd) inputs + outputs once",
               f"ratio_to_floor: {hbm/floor:.3f}",
               f"mfma_busy_fraction: {c3['SQ_VALU_MFMA_BUSY_CYCLES']/(4*busy) if busy else 0:.3f}"
               "   # SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES)",
               f"busy_cycles_per_cu: {busy/256:.3g}",
               f"gpu_clock_cycles_per_xcd: {c3['GRBM_GUI_ACTIVE']/8:.4g}   # GRBM_GUI_ACTIVE / 8 XCDs",
               f"insts_valu: {c3['SQ_INSTS_VALU']:.4g}",
               f"insts_mfma: {c3['SQ_INSTS_MFMA']:.4g}",
               f"insts_lds: {c3['SQ_INSTS_LDS']:.4g}",
               f"lds_bank_conflict_cycles: {c3['SQ_LDS_BANK_CONFLICT']:.0f}",
               f"wait_inst_lds: {c3['SQ_WAIT_INST_LDS']:.4g}"]
        if p4 is not None and fs:
            sec, _ = per_launch(p4, pats, L2C)
            l2 = sec * 32 * fs
            out += ["# L2 read bytes: TCC_READ_SECTORS_sum (32-byte sectors) x 32, scaled by the same",
                    f"# copy ({cs:.0f} sectors for 512 MiB read: factor {fs:.4f}).",
                    f"l2_read_bytes_per_launch: {l2:.0f}"]
            block = {"fwd": 256 if any("fwd_pp_kernel" in k for k in kn) else 128,
                     "bwd_dkdv": 128, "bwd_dq": 128}.get(stage)
            if block and not w.sparse_frac and not w.fp8:
                model = l2_read_model(stage, w.B, w.H, w.N, w.d, w.causal, block)
                out += [f"l2_read_model_bytes: {model:.0f}   # blocked schedule, {block}-row blocks "
                        "(bench.l2_read_model)",
                        f"l2_read_ratio_to_model: {l2/model:.3f}"]
        with open(os.path.join(root, "profiles", f"traffic_{stage}_{workload}.txt"), "w") as f:
            f.write("\n".join(out) + "\n")
        print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_context_causal")
    ap.add_argument("--tile", type=int, default=0, help="forward key tile (0 = default)")
    ap.add_argument("--tile-sweep", default="32,64,128,256",
                    help="forward key tiles to time on the side ('' to skip)")
    ap.add_argument("--bwd-tile-sweep", default="64,128",
                    help="backward (dK/dV query) tiles to time on the side ('' to skip)")
    ap.add_argument("--quick", action="store_true",
                    help="only the workload's own step: no tile sweeps, no metric range, no other "
                         "workloads, no CPU baseline (for profiler runs)")
    ap.add_argument("--digest", nargs="+", metavar=("WORKLOAD", "STAGE"),
                    help="instead of running: summarise rocprofv3 CSVs under gpurun_out/ into "
                         "profiles/ (CPU only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the single workload: one JSON line per (N, d, causal) with "
                         "N = 256..16384, d = 64/128/256, H = 16, B = 16384/N, fwd and fwd+bwd")
    ap.add_argument("--io-ablation", action="store_true",
                    help="instead of the single workload: the forward against the key/value-outer "
                         "loop order (fa_fwd_kvouter) at N = 2048, 4096, 8192, d = 128")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="first run one plain device copy of MB MiB (a known-size kernel "
                         "for scaling the profiler's FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args(argv)

    if args.digest:
        digest(args.digest[0], args.digest[1:])
        return 0
    if args.quick:
        args.tile_sweep = ""
        args.bwd_tile_sweep = ""
        args.no_cpu_baseline = True
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(heads and batch shard across GPUs with no communication; see the design notes)",
              file=sys.stderr)
        return 2

    import torch

    import exact_io_aware_36_amd as fa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.sweep:
        return bench_sweep(args, fa, torch)
    if args.io_ablation:
        return bench_io_ablation(args, fa, torch)
    w = workloads.WORKLOADS[args.workload]
    inp = workloads.make_inputs(w)
    if w.nq is not None:
        return bench_decode(args, w, inp, fa, torch)
    if w.fp8:
        return bench_fp8(args, w, inp, fa, torch)
    B, H, N, d = inp["B"], inp["H"], inp["N"], inp["d"]
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    dout = inp["dout"].to(dev) if w.backward else None
    lens = inp["kv_lens"].to(dev) if inp["kv_lens"] is not None else None
    mask = inp["block_mask"].to(dev) if inp["block_mask"] is not None else None
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if w.backward:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    if not w.backward:
        stages = ["fwd"]
    elif mask is None:
        stages = ["fwd", "bwd_dot", "bwd_dkdv", "bwd_dq"]
    else:
        stages = ["fwd", "bwd_sparse"]     # fa_bwd_blocksparse: its three launches together

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def launch(stage, tile=args.tile):
        if stage == "fwd":
            if mask is not None:
                fa.fa_fwd_blocksparse(q, k, v, o, lse, mask, mask_block=w.mask_block, scale=w.scale)
            else:
                fa.fa_fwd_ex(q, k, v, o, lse, causal=w.causal, scale=w.scale, kv_lens=lens,
                             tile_n=tile)
        elif stage == "bwd_dot":
            fa.fa_bwd_preprocess(o, dout, lse, ws)
        elif stage == "bwd_dkdv":
            fa.fa_bwd_dkdv(q, k, v, dout, lse, dk, dv, ws, causal=w.causal, scale=w.scale,
                           kv_lens=lens)
        elif stage == "bwd_dq":
            fa.fa_bwd_dq(q, k, v, dout, lse, dq, ws, causal=w.causal, scale=w.scale, kv_lens=lens)
        elif stage == "bwd_sparse":
            fa.fa_bwd_blocksparse(q, k, v, o, dout, lse, dq, dk, dv, ws, mask,
                                  mask_block=w.mask_block, scale=w.scale)

    for _ in range(args.warmup):
        for s in stages:
            launch(s)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        for j, s in enumerate(stages):
            launch(s)
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    stage_ms = {s: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)) / args.steps
                for j, s in enumerate(stages)}

    sf = w.sparse_frac
    flops = step_flops(B, H, N, d, w.causal, sf, w.backward)
    value = flops / (ms_per_step * 1e-3) / 1e12
    dom = max(stages, key=lambda s: stage_ms[s])
    dom_flops = kernel_flops(dom, B, H, N, d, w.causal, sf)
    achieved = dom_flops / (stage_ms[dom] * 1e-3) / 1e12
    traffic = read_traffic(dom, w.name)
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                "avg_launch_ms": round(stage_ms[dom], 4)}

    fflops = fwd_flops(B, H, N, d, w.causal, sf)
    # per-step spread from the same events (first stage's start to last stage's end)
    step_ev = [evs[i][0].elapsed_time(evs[i][-1]) for i in range(args.steps)]
    pc = percentiles(step_ev)
    detail = {
        "stage_ms": {s: round(t, 4) for s, t in stage_ms.items()},
        "step_ms_events": {"p10": round(pc[10], 4), "median": round(pc[50], 4), "p90": round(pc[90], 4)},
        "fwd_tflops": round(fflops / (stage_ms["fwd"] * 1e-3) / 1e12, 2),
        "kernel_tflops": {s: round(kernel_flops(s, B, H, N, d, w.causal, sf) / (stage_ms[s] * 1e-3) / 1e12, 2)
                          for s in stages if s != "bwd_dot"},
        "floor_bytes_per_step": sum(floor_bytes(s, B, H, N, d) for s in stages),
    }
    if w.backward:
        bwd_ms = sum(stage_ms[s] for s in stages if s != "fwd")
        detail["bwd_tflops_1.5x"] = round(1.5 * fflops / (bwd_ms * 1e-3) / 1e12, 2)
        detail["fwd_bwd_tflops_3.5x"] = round(3.5 * fflops / (ms_per_step * 1e-3) / 1e12, 2)

    sweep = [int(t) for t in args.tile_sweep.split(",") if t.strip()] if mask is None else []
    if d == 256 and sweep:   # the key tiles built at head dim 256
        sweep = [32, 64]
    if w.dtype != "bf16":
        sweep = []
    if sweep:
        res = {}
        for t in sweep:
            for _ in range(3):
                launch("fwd", tile=t)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(3, args.steps // 2)
            e0.record(stream)
            for _ in range(reps):
                launch("fwd", tile=t)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            res[str(t)] = {"fwd_ms": round(ms, 4), "fwd_tflops": round(fflops / (ms * 1e-3) / 1e12, 2)}
        detail["fwd_tile_sweep"] = res
    bsweep = [int(t) for t in args.bwd_tile_sweep.split(",") if t.strip()]
    if w.backward and mask is None and bsweep:
        res = {}
        for t in bsweep:
            if d == 256 and t != 64:
                continue

            def bwd_call(t=t):
                fa.fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, ws, causal=w.causal, scale=w.scale,
                             kv_lens=lens, tile_n=t)

            ms = _timed(torch, stream, bwd_call, 3, max(3, args.steps // 2))
            res[str(t)] = {"bwd_ms": round(ms, 4),
                           "bwd_tflops_2.5x": round(2.5 * fflops / (ms * 1e-3) / 1e12, 2),
                           "fwd_bwd_tflops": round(2.5 * fflops / ((ms + stage_ms["fwd"]) * 1e-3) / 1e12, 2)}
        detail["bwd_tile_sweep"] = res
    if not args.quick and args.workload == "long_context_causal":
        detail["sweep"] = metric_range(fa, torch)
        detail["configs"] = other_configs(fa, torch, workloads)
        detail["next_rows"] = next_rows(fa, torch, workloads)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, w, flops, budget_s=args.cpu_budget)
        cpu = {k2: (round(v2, 6) if isinstance(v2, float) else v2) for k2, v2 in cpu.items()}

    line = {
        "metric": "attention TFLOP/s fwd & fwd+bwd, % bf16 MFMA peak, N=256-16K, d=64/128",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "pass": "fwd+bwd" if w.backward else "fwd",
                   "flops_per_step": flops, "pct_mfma_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 2),
                   "flop_convention": "fwd 4N^2dBH (x1/2 causal, x s sparse); fwd+bwd 2.5x fwd"},
        "roofline": roofline, "cpu_baseline": cpu, "detail": detail,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
