"""FP8 (OCP E4M3FN) quantisation and the FP8 attention reference, for the
block-quantised FP8 forward.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: used by the tests, the
smoke check and the benchmark's CPU-baseline leg, never by the product path,
and sharing no code with the GPU library.

What the pages fix and what they leave open
-------------------------------------------
"FlashAttention: Mathematical Foundations, IO-Aware Tiling, Online Softmax,
and Recomputation Dynamics" (section "FlashAttention-3: Hopper ...", item on
low-precision FP8 support) describes block-quantised FP8 matrix products with
dynamic scaling; the "Attention" chapter of learn-kernels.com (paragraph on
Hopper) adds block quantisation with incoherent processing.  Neither gives
the format, the block shape, the scale rule or the rotation.  The readings
taken here (each also stated in the design notes):

  * format: OCP 8-bit floating point E4M3 ("FN": 4 exponent bits, bias 7,
    3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448,
    smallest normal 2^-6, smallest subnormal 2^-9); round to nearest, ties
    to even; a value beyond the largest finite one is NaN (no saturation);
  * dynamic per-block scale: the block's largest magnitude maps to 448:
    inv = 448 / amax, code = E4M3(x * inv), descale = amax / 448, all in
    fp32 (the decision that produces a code is taken in fp32 on both sides);
    an all-zero block gets inv = descale = 1;
  * blocks: Q and K per 128 consecutive rows of one (b, h); V per (b, h), so
    that its scale factors out of the P V sum;
  * incoherent processing: Q and K (never V) are multiplied by the same
    orthogonal R = diag(signs) H_d / sqrt(d), H_d the Sylvester Hadamard
    matrix and signs a random +-1 vector passed in.  Q R (K R)^T = Q K^T, so
    the scores are unchanged in exact arithmetic while outliers are spread
    over all d coordinates before quantisation.  The product is taken with
    the fast Walsh-Hadamard butterflies in fp32 (stages of width 1, 2, 4, ...,
    each pair (a, b) -> (a + b, a - b)), then multiplied by the fp32 constant
    1/sqrt(d);
  * the attention itself is the plain definition evaluated on the
    dequantised values (``reference``); the kernel differs from it by
    quantising the probabilities to E4M3 for the P V product, whose effect
    on O ``p_quant_bound`` bounds element by element, and by the way the
    hardware sums E4M3 products (each 64-product block truncates its
    products below the largest one's binade), whose effect on the scores and
    on LSE ``score_error_bound`` and ``lse_bound`` bound.  The pages say
    nothing of that summation; the bound rests on its measured behaviour,
    and the CPU tests pin it to a direct simulation of that behaviour.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK_ROWS = 128


# ---------------------------------------------------------------- format

def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each E4M3FN code (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """E4M3FN code of each float32 value, round to nearest even; magnitudes
    that round beyond 448 become NaN (0x7F with the sign bit)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)   # exact
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.abs(x)
    out = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9 (the code's low bits are the count;
    # a count of 8 is exactly the smallest normal, code 0x08)
    out = np.where(sub, np.rint(a / 2.0 ** -9).astype(np.int64), out)
    # normal range: 3 mantissa bits below the leading one
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(sub, 1.0, a))).astype(np.int64)
        mant = np.rint((np.where(sub, 1.0, a) / np.exp2(e.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8
    e = np.where(carry, e + 1, e)
    mant = np.where(carry, 0, mant)
    normal = ((e + 7) << 3) | mant
    normal = np.where((e + 7 > 15) | (((e + 7) == 15) & (mant == 7)), 0x7F, normal)
    out = np.where(sub, out, normal)
    out = np.where(np.isnan(x), 0x7F, out)
    return (out | sign).astype(np.uint8)


# ---------------------------------------------------------------- rotation

def rotation_scale(d: int) -> np.float32:
    """The fp32 constant 1/sqrt(d) (double result rounded once to fp32)."""
    return np.float32(1.0 / np.sqrt(np.float64(d)))


def rotate_fp32(x, signs) -> np.ndarray:
    """x R with R = diag(signs) H_d / sqrt(d), computed in fp32: signs, then
    the Walsh-Hadamard butterflies of widths 1, 2, 4, ..., d/2, then the
    1/sqrt(d) multiply."""
    y = np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    d = y.shape[-1]
    assert d & (d - 1) == 0
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = v[..., 0, :].copy(), v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        y = v.reshape(y.shape)
        h *= 2
    return (y * rotation_scale(d)).astype(np.float32)


# ---------------------------------------------------------------- quantisation

def quantize(x, block_rows: int = BLOCK_ROWS, signs=None):
    """Quantise x [B, H, N, d] (any float dtype, taken as float32) in blocks of
    block_rows rows of one (b, h) (block_rows = 0: one block per (b, h)).
    Returns (codes uint8 [B, H, N, d], descale float32 [B, H, nblk])."""
    x = np.asarray(x, dtype=np.float32)
    if signs is not None:
        x = rotate_fp32(x, signs)
    B, H, N, d = x.shape
    br = N if block_rows == 0 else block_rows
    nblk = -(-N // br)
    codes = np.empty(x.shape, dtype=np.uint8)
    descale = np.empty((B, H, nblk), dtype=np.float32)
    for i in range(nblk):
        blk = x[:, :, i * br:(i + 1) * br, :]
        amax = np.abs(blk).max(axis=(2, 3)).astype(np.float32)
        safe = np.where(amax > 0, amax, np.float32(1.0))
        inv = np.where(amax > 0, np.float32(E4M3_MAX) / safe, np.float32(1.0)).astype(np.float32)
        ds = np.where(amax > 0, safe / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        y = (blk * inv[:, :, None, None]).astype(np.float32)
        codes[:, :, i * br:(i + 1) * br, :] = e4m3_encode(y)
        descale[:, :, i] = ds
    return codes, descale


def dequantize(codes, descale, block_rows: int = BLOCK_ROWS) -> np.ndarray:
    """float64 values of quantised [B, H, N, d] codes."""
    c = e4m3_decode(codes)
    N = c.shape[2]
    br = N if block_rows == 0 else block_rows
    rows = np.arange(N) // br
    return c * np.asarray(descale, np.float64)[:, :, rows][..., None]


# ---------------------------------------------------------------- attention

def reference(q8, k8, v8, q_descale, k_descale, v_descale, causal=False, scale=None, kv_lens=None):
    """Exact attention (the fp64 oracle) of the dequantised inputs.  q8, k8,
    v8 are codes [B, H, N, d] (V in its natural layout), q/k descales
    [B, H, N/128], v descale [B, H] (or [B, H, 1]).  Returns (O, LSE, (Q, K, V))
    with the dequantised operands."""
    import oracle

    Q = dequantize(q8, q_descale)
    K = dequantize(k8, k_descale)
    V = dequantize(v8, np.asarray(v_descale, np.float32).reshape(v8.shape[0], v8.shape[1], 1), 0)
    O, L = oracle.fwd(Q, K, V, causal=causal, scale=scale, kv_lens=kv_lens)
    return O, L, (Q, K, V)


def p_quant_bound_rows(q_rows, i_rows, K, V, lse_rows, causal=False, scale=None, kv_len=None,
                       n_slack=None) -> np.ndarray:
    """Element-wise bound on |O_kernel - O_reference| for some query rows of
    one head (q_rows [n, d] at positions i_rows, K and V [N, d], lse_rows
    their reference LSE), caused by rounding the probabilities to E4M3 before
    the P V product.

    The kernel forms p~_ij = 2^(s_ij log2 e - m) with a reference m no larger
    than the row's true maximum, so p~_ij >= P_ij l*_i with
    l*_i = sum_j exp(s_ij - max_j s_ij) >= 1.  Rounding p~ to E4M3 changes it
    by at most 2^-4 p~ when p~ >= 2^-6 (3 mantissa bits) and by at most 2^-10
    below (subnormal spacing 2^-9); after the division by the row sum (taken
    on the unrounded p~) the change of O_i is at most
        sum_j |v_j| max(2^-4 P_ij, [P_ij l*_i < 2^-6] 2^-10 / l*_i).
    A relative slack of (1e-4 + n 2^-24) on sum_j P_ij |v_j| covers the fp32
    exponentials and sums (n = number of keys)."""
    N, d = K.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    kvl = N if kv_len is None else int(kv_len)
    j = np.arange(N)
    i = np.asarray(i_rows)
    s = scale * (np.asarray(q_rows, np.float64) @ K.T)
    allowed = (j[None, :] < kvl) & ((j[None, :] <= i[:, None]) | (not causal))
    s = np.where(allowed, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    fin = np.isfinite(mx)
    mx = np.where(fin, mx, 0.0)
    lstar = np.exp(s - mx).sum(axis=1, keepdims=True)
    lse = np.asarray(lse_rows, np.float64)
    P = np.where(fin & allowed, np.exp(s - np.where(np.isfinite(lse), lse, 0.0)[:, None]), 0.0)
    small = (P * lstar) < 2.0 ** -6
    w = np.maximum(2.0 ** -4 * P, np.where(small & allowed, 2.0 ** -10 / np.maximum(lstar, 1.0), 0.0))
    n = N if n_slack is None else n_slack
    return w @ np.abs(V) + (1e-4 + n * 2.0 ** -24) * (P @ np.abs(V))


def p_quant_bound(Q, K, V, lse, causal=False, scale=None, kv_lens=None, n_slack=None) -> np.ndarray:
    """p_quant_bound_rows for every row of [B, H, N, d] operands."""
    B, H, N, d = Q.shape
    bound = np.empty((B, H, N, d))
    rows = np.arange(N)
    for b in range(B):
        kvl = None if kv_lens is None else int(kv_lens[b])
        for h in range(H):
            bound[b, h] = p_quant_bound_rows(Q[b, h], rows, K[b, h], V[b, h], lse[b, h], causal,
                                             scale, kvl, n_slack)
    return bound


# ---------------------------------------------------------------- scores and LSE

# The E4M3 matrix product sums K_BLOCK = 64 products per instruction.  Measured
# on gfx950 (v_mfma_f32_32x32x64_f8f6f4, one large and one small product, and
# 64 random products): every product is exact, is aligned to the binade E of
# the block's largest product and truncated toward zero to a multiple of
# 2^(E - 14) (products 15 or more binades below vanish); the block's sum is
# then added to the fp32 accumulator (one fp32 rounding).  The bound below
# takes the window one bit narrower (2^(E - WINDOW_BITS), WINDOW_BITS = 13),
# twice the measured truncation.
K_BLOCK = 64
WINDOW_BITS = 13


def score_error_bound(q8_rows, k8, window_bits: int = WINDOW_BITS) -> np.ndarray:
    """Bound on |s_kernel - s_exact| for raw E4M3 scores sum_k q_ik k_jk (codes,
    before the descales), per row of q8_rows [n, d] and key of k8 [N, d]:
    per 64-product block, sum_k (|p_k| mod 2^(E - window_bits)) -- the
    largest truncation each product can suffer -- plus one fp32 rounding
    (2^-23 relative) of the running sum per block."""
    a = e4m3_decode(q8_rows).astype(np.float64)
    b = e4m3_decode(k8).astype(np.float64)
    n, d = a.shape
    nblk = -(-d // K_BLOCK)
    out = np.zeros((n, b.shape[0]))
    absum = np.zeros((n, b.shape[0]))
    for r0 in range(0, n, 32):
        ar = a[r0:r0 + 32]
        for c in range(0, d, K_BLOCK):
            p = np.abs(ar[:, None, c:c + K_BLOCK] * b[None, :, c:c + K_BLOCK])   # exact in fp64
            mx = p.max(axis=-1)
            with np.errstate(divide="ignore"):
                e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
            lsb = np.exp2(e - window_bits)[..., None]
            out[r0:r0 + 32] += (p - np.floor(p / lsb) * lsb).sum(axis=-1)
            absum[r0:r0 + 32] += p.sum(axis=-1)
    return out + nblk * 2.0 ** -23 * absum


def lse_bound_rows(q8_rows, i_rows, q_descale_rows, k8, k_descale, lse_rows, causal=False,
                   scale=None, kv_len=None, window_bits: int = WINDOW_BITS) -> np.ndarray:
    """Bound on |LSE_kernel - LSE_reference| of the FP8 forward for some query
    rows of one head: codes q8_rows [n, d] at positions i_rows with their row
    descales [n], codes k8 [N, d] with per-key descales k_descale [N], and
    the reference LSE of those rows.

    The kernel's score of (i, j) in log2 units is t = s_raw c with
    c = scale log2(e) dq_i dk_j formed in fp32 (three roundings) and s_raw the
    E4M3 product sum (error bounded by score_error_bound).  LSE is smooth with
    gradient P_ij in the scores, so to first order a score error Delta_j
    moves it by sum_j P_ij Delta_j (x 1.05 for the second order: the errors
    are below 0.05 nats).  Then the row sum l = sum_j 2^(t_j - m) in fp32
    (exp2 within 2^-21 relative, at most N + 64 roundings of 2^-24 over the
    sum and the lazy rescales), and LSE = ln2 (m + log2 l) in fp32 (a few
    roundings of 2^-24 |LSE|, 1e-5 for log2's own error)."""
    N, d = k8.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    kvl = N if kv_len is None else int(kv_len)
    i = np.asarray(i_rows)
    j = np.arange(N)
    a = e4m3_decode(q8_rows).astype(np.float64)
    b = e4m3_decode(k8).astype(np.float64)
    craw = scale * np.asarray(q_descale_rows, np.float64)[:, None] * np.asarray(k_descale, np.float64)[None, :]
    s = craw * (a @ b.T)                                   # natural units
    allowed = (j[None, :] < kvl) & ((j[None, :] <= i[:, None]) | (not causal))
    lse = np.asarray(lse_rows, np.float64)
    fin = np.isfinite(lse)
    P = np.where(allowed & fin[:, None], np.exp(np.where(allowed, s, 0.0) - np.where(fin, lse, 0.0)[:, None]), 0.0)
    delta = craw * score_error_bound(q8_rows, k8, window_bits) + 4 * 2.0 ** -24 * np.abs(s)
    first = 1.05 * (P * delta).sum(axis=1)
    slack = 1e-5 + 2.0 ** -21 + (N + 64) * 2.0 ** -24 + 4 * 2.0 ** -24 * np.abs(np.where(fin, lse, 0.0))
    return np.where(fin, first + slack, 0.0)


def lse_bound(q8, qs, k8, ks, lse, causal=False, scale=None, kv_lens=None) -> np.ndarray:
    """lse_bound_rows for every row of [B, H, N, d] codes with 128-row
    descales qs, ks [B, H, ceil(N/128)] (the quantiser's layout)."""
    B, H, N, d = q8.shape
    rows = np.arange(N)
    out = np.empty((B, H, N))
    for b in range(B):
        kvl = None if kv_lens is None else int(kv_lens[b])
        for h in range(H):
            out[b, h] = lse_bound_rows(q8[b, h], rows, np.asarray(qs)[b, h][rows // BLOCK_ROWS], k8[b, h],
                                       np.asarray(ks)[b, h][rows // BLOCK_ROWS], lse[b, h], causal,
                                       scale, kvl)
    return out

