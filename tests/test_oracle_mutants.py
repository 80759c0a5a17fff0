"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle (its C source or the
Python E4M3 reference) inside a scratch directory, rebuilds that copy and runs
the oracle's pin tests (tests/test_oracle.py, test_oracle_decode.py,
test_oracle_fp8.py, copied beside it) against it in a child process: at least
one pin must fail.  The unmodified copy, run the same way, must pass.  Every
mistake is applied to all the places the oracle repeats the same arithmetic
(the full backward and the sampled one), so the mutant is self-consistent and
only the pins -- not a disagreement between two oracle functions -- can catch
it.  CPU only."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ("test_oracle.py", "test_oracle_decode.py", "test_oracle_fp8.py")

C, PY = "oracle/fa_oracle.c", "oracle/fp8.py"
# (name, file, [(text, replacement), ...]); every occurrence is replaced
MUTANTS = [
    ("causal_includes_diagonal_wrongly", C, [("if (causal && j > i)", "if (causal && j >= i)")]),
    ("score_transposed", C, [("s[j] = scale * dot(qi, kh + (size_t)j * d, d);\n            if (!any",
                              "s[j] = scale * dot(qi - ((long)i - j) * d, kh + (size_t)i * d, d);\n"
                              "            if (!any")]),
    ("max_shift_dropped", C, [("l += exp(s[j] - m);\n    for (int j = 0; j < N; ++j)\n"
                               "        p[j] = ok[j] ? exp(s[j] - m) / l : 0.0;\n    return m + log(l);",
                               "l += exp(s[j]);\n    for (int j = 0; j < N; ++j)\n"
                               "        p[j] = ok[j] ? exp(s[j]) / l : 0.0;\n    return log(l);")]),
    ("row_sum_offset", C, [("double l = 0.0;\n    for (int j = 0; j < N; ++j)\n        if (ok[j])",
                            "double l = 1e-3;\n    for (int j = 0; j < N; ++j)\n        if (ok[j])")]),
    ("mask_read_transposed", C, [("mask[(size_t)(i / mask_block) * nb + (size_t)(j / mask_block)]",
                                  "mask[(size_t)(j / mask_block) * nb + (size_t)(i / mask_block)]")]),
    ("padding_keeps_one_key_too_many", C, [("if (j >= kv_len)", "if (j > kv_len)")]),
    ("backward_D_term_dropped", C, [("const double ds = p[j] * (dp[j] - D);",
                                     "const double ds = p[j] * dp[j];")]),
    ("dK_scale_dropped", C, [("dkj[t] += scale * ds * qi[t];", "dkj[t] += ds * qi[t];"),
                             ("dk_loc[(size_t)r * d + t] += scale * ds * qi[t];",
                              "dk_loc[(size_t)r * d + t] += ds * qi[t];")]),
    ("dV_probability_dropped", C, [("dvj[t] += p[j] * doi[t];", "dvj[t] += doi[t];"),
                                   ("dv_loc[(size_t)r * d + t] += p[j] * doi[t];",
                                    "dv_loc[(size_t)r * d + t] += doi[t];")]),
    ("dQ_uses_queries", C, [("dqi[t] += scale * ds * kj[t];", "dqi[t] += scale * ds * qi[t];"),
                            ("dqi[t] += scale * ds * k[(size_t)j * d + t];",
                             "dqi[t] += scale * ds * qi[t];")]),
    ("decode_causal_off_by_one", C, [("int visible = causal ? len - Nq + t + 1 : len;",
                                      "int visible = causal ? len - Nq + t : len;")]),
    ("decode_queries_top_aligned", C, [("int visible = causal ? len - Nq + t + 1 : len;",
                                        "int visible = causal ? t + 1 : len;")]),
    ("merge_weights_unnormalised", C, [("const double w1 = exp(L - Lnew), w2 = exp(Ls - Lnew);",
                                        "const double w1 = exp(L - mx), w2 = exp(Ls - mx);")]),
    ("e4m3_subnormal_round_half_up", PY, [("np.rint(a / 2.0 ** -9)", "np.floor(a / 2.0 ** -9 + 0.5)")]),
    ("e4m3_normal_round_half_up", PY, [("mant = np.rint((np.where(sub, 1.0, a)",
                                        "mant = np.floor(0.5 + (np.where(sub, 1.0, a)")]),
    ("e4m3_bias_8", PY, [("np.exp2(e - 7.0)", "np.exp2(e - 8.0)")]),
    ("e4m3_subnormal_threshold", PY, [("sub = a < 2.0 ** -6", "sub = a < 2.0 ** -7")]),
    ("e4m3_max_240", PY, [("E4M3_MAX = 448.0", "E4M3_MAX = 240.0")]),
    ("e4m3_negative_zero_dropped", PY, [("sign = np.signbit(x).astype(np.int64) << 7",
                                         "sign = (x < 0).astype(np.int64) << 7")]),
    ("rotation_unscaled", PY, [("return np.float32(1.0 / np.sqrt(np.float64(d)))",
                                "return np.float32(1.0)")]),
    ("rotation_butterfly_sign", PY, [("v[..., 1, :] = a - b", "v[..., 1, :] = b - a")]),
    ("probability_bound_halved", PY, [("w = np.maximum(2.0 ** -4 * P,", "w = np.maximum(2.0 ** -5 * P,")]),
    ("score_truncation_window_too_narrow", PY, [("WINDOW_BITS = 13", "WINDOW_BITS = 18")]),
    ("lse_bound_weights_dropped", PY, [("first = 1.05 * (P * delta).sum(axis=1)",
                                        "first = 1.05 * (P * delta).max(axis=1)")]),
]


def make_copy(dst, mutation=None):
    """Scratch copy of the oracle, the pins and what they import; with a
    mutation (file, [(text, replacement), ...]) applied."""
    os.makedirs(os.path.join(dst, "tests"))
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "*.so.tmp", "__pycache__"))
    shutil.copy(os.path.join(ROOT, "workloads.py"), dst)
    for f in ("conftest.py",) + PINS:
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests"))
    if mutation is not None:
        path, edits = mutation
        p = os.path.join(dst, path)
        src = open(p).read()
        for text, repl in edits:
            assert src.count(text) >= 1, f"mutation site not found in {path}: {text!r}"
            src = src.replace(text, repl)
        with open(p, "w") as f:
            f.write(src)
    # build the copy's C oracle now, so a compile error cannot pass for a caught mutant
    r = subprocess.run([sys.executable, "-c", "from oracle.build import build_oracle; build_oracle()"],
                       cwd=dst, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def run_pins(dst):
    env = dict(os.environ, OMP_NUM_THREADS="4", PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "-m", "not gpu", *[os.path.join("tests", f) for f in PINS]],
                          cwd=dst, env=env, capture_output=True, text=True, timeout=600)


def _check_mutant(base, name, path, edits):
    dst = os.path.join(base, name)
    make_copy(dst, (path, edits))
    r = run_pins(dst)
    failed = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
    return name, r.returncode, failed[:1], r.stdout[-1500:]


def test_unmodified_copy_passes(tmp_path):
    make_copy(str(tmp_path / "clean"))
    r = run_pins(str(tmp_path / "clean"))
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]


def test_every_mutant_fails_a_pin(tmp_path):
    """The mutants run in parallel child processes (a few at a time)."""
    from concurrent.futures import ThreadPoolExecutor

    workers = max(1, min(8, (os.cpu_count() or 2) // 2))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda m: _check_mutant(str(tmp_path), *m), MUTANTS))
    missed = []
    for name, rc, failed, tail in results:
        print(f"{name}: rc={rc} caught by {failed}")
        if rc != 1:
            missed.append((name, rc, tail))
    assert not missed, "mutants no pin caught: " + "; ".join(f"{n} (rc {rc})\n{t}" for n, rc, t in missed)
