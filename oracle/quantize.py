"""Plain CPU reference of the VBQ per-group quantizer and of the fixed recipe.

TEST INFRASTRUCTURE ONLY: imported by the tests and by the quantizer
benchmark's CPU-baseline leg, never by the product path. Plain numpy, no
code shared with the HIP library.

VBQ paper (arXiv 2607.02893):
  - §3.1 Eq. (1): a group of 64 weights quantized to b >= 2 bits has scale
    s = max|w| / (2^(b-1) - 1), and each weight becomes
    s * clip(round(w / s), -(2^(b-1) - 1), 2^(b-1) - 1); at 1 bit a weight
    keeps its sign and the group's scale is the mean magnitude.
  - §3.4 "From discovery to a fixed recipe": first-block MLP projections at
    4 bits, every other attention and MLP projection at 2 bits, and the LM
    head tiered per row by token frequency: the top 0.5% of the vocabulary
    (by descending frequency) at 8 bits, the next 1.5% at 4, the next 10% at
    2, the bottom 88% at 1 (mean 1.18 bits).

Readings (the pages leave these open):
  Q1 precision: magnitudes, the largest magnitude, the b >= 2 scale s and
     the ratios w / s are fp32 (IEEE, correctly rounded division); the
     1-bit mean magnitude is summed in fp64 (exact here) and divided by 64.
  Q2 the stored scale is the fp16 rounding (to nearest, ties to even) of
     that value: of the fp32 quotient at b >= 2, of the fp64 mean at 1 bit
     (one rounding, no fp32 step in between); the codes are computed with
     the stored scale, so s * q is exactly what decode multiplies.
  Q3 round half away from zero; sign(0) = +1, also for -0.0.
  Q4 a stored scale of 0 (an all-zero group, or a largest magnitude too
     small for fp16) gives codes 0 at b >= 2 (+1 at 1 bit); a scale beyond
     the largest finite fp16 is stored as 65504.
  Q5 head tiers: rows ranked by descending frequency, ties by lower row
     index; with N rows, ranks below round(0.005 N) get 8 bits, below
     round(0.02 N) 4 bits, below round(0.12 N) 2 bits, the rest 1 bit
     (round = half up).
"""
from __future__ import annotations

import numpy as np

FP16_MAX = np.float16(65504.0)


def _stored_scale(s: np.ndarray) -> np.ndarray:
    """fp32 or fp64 scales -> fp16 in one rounding (nearest even), saturated at the largest finite value (Q2, Q4)."""
    with np.errstate(over="ignore"):
        s16 = s.astype(np.float16)
    return np.where(np.isinf(s16), FP16_MAX, s16)


def _round_half_away(r: np.ndarray) -> np.ndarray:
    """Q3 on fp32 ratios: |r| + 0.5 taken in fp64, where it is exact for every fp32 |r| < 2^28
    (in fp32 the sum would round 0.5 - 2^-25 up to 1); larger ratios are clipped anyway."""
    a = np.abs(r).astype(np.float64)
    return np.sign(r) * np.floor(a + 0.5)


def quantize(w: np.ndarray, bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Eq. (1) over every group of w (fp32 [n][k]) at widths bits (uint8 [n][k/64]).

    Returns (codes int8 [n][k], scales uint16 [n][k/64] as binary16 bit patterns).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % 64 == 0
    g = w.reshape(n * (k // 64), 64)
    b = np.asarray(bits, dtype=np.uint8).reshape(-1)
    assert b.size == g.shape[0] and np.all(np.isin(b, (1, 2, 4, 8)))
    codes = np.zeros(g.shape, np.int8)
    scales = np.zeros(g.shape[0], np.float16)
    mag = np.abs(g)
    one = b == 1
    if one.any():
        mean = mag[one].astype(np.float64).sum(axis=1) / 64.0                         # Q1
        scales[one] = _stored_scale(mean)
        codes[one] = np.where(g[one] < 0, -1, 1)                                      # Q3
    for width in (2, 4, 8):
        sel = b == width
        if not sel.any():
            continue
        qmax = np.float32(2 ** (width - 1) - 1)
        s16 = _stored_scale(mag[sel].max(axis=1) / qmax)                              # Q1, Q2
        s32 = s16.astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = g[sel] / s32[:, None]
        q = np.clip(_round_half_away(r), -qmax, qmax)
        q = np.where(s32[:, None] == 0, 0, q)                                         # Q4
        codes[sel] = q.astype(np.int8)
        scales[sel] = s16
    return codes.reshape(n, k), scales.view(np.uint16).reshape(n, k // 64)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """w_hat = s * q per group (fp64)."""
    n, k = codes.shape
    s = np.asarray(scales, dtype=np.uint16).view(np.float16).astype(np.float64).reshape(n, k // 64, 1)
    return (codes.astype(np.float64).reshape(n, k // 64, 64) * s).reshape(n, k)


def projection_bits(first_block_mlp: bool) -> int:
    """§3.4: first-block MLP (gate, up, down) at 4 bits, every other projection at 2."""
    return 4 if first_block_mlp else 2


def head_bits(freq: np.ndarray) -> np.ndarray:
    """§3.4 frequency-tiered head: one width per row (uint8 [rows]), Q5."""
    freq = np.asarray(freq)
    rows = freq.size
    order = np.lexsort((np.arange(rows), -freq.astype(np.float64)))   # descending frequency, then row index
    cut = [(per_mille * rows + 500) // 1000 for per_mille in (5, 20, 120)]
    out = np.empty(rows, np.uint8)
    rank = np.empty(rows, np.int64)
    rank[order] = np.arange(rows)
    out[:] = 1
    out[rank < cut[2]] = 2
    out[rank < cut[1]] = 4
    out[rank < cut[0]] = 8
    return out


# ---------------------------------------------------------------- soft quantizer (training side)
# VBQ §3.2 "Differentiable bit selection": each group has logits over the widths (1, 2, 4, 8); a
# Gumbel-Softmax sample pi = softmax((logits + e) / tau) mixes the group's reconstructions at the four
# widths, w_soft = sum_k pi_k * w_hat^(B_k), and the expected bit cost is the mean over groups of
# sum_k pi_k * B_k. Readings (the pages leave these open):
#   S1 the Gumbel noise e is an input (drawn by the caller), one value per group and width;
#   S2 w_hat^(b) is Eq. (1) at training time: the scale stays fp32 (no binary16 rounding), computed as in
#      Q1 (fp32 max and division; the 1-bit mean summed in fp64 and rounded once to fp32), codes as in
#      Q3/Q4 with that scale; the code decisions are taken in fp32, as the device takes them;
#   S3 the softmax, the mixture and the bit cost are fp64 here;
#   S4 the mean in the bit cost runs over groups (every group has 64 weights, so it is also the mean
#      over weights).
WIDTHS = (1, 2, 4, 8)


def training_reconstruction(w: np.ndarray, b: int) -> np.ndarray:
    """w_hat^(b) per group of w (fp32 [n][k]) with fp32 scales (S2); returns float64 [n][k]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    g = w.reshape(-1, 64)
    mag = np.abs(g)
    if b == 1:
        s = (mag.astype(np.float64).sum(axis=1) / 64.0).astype(np.float32)
        q = np.where(g < 0, -1.0, 1.0)
    else:
        qmax = np.float32(2 ** (b - 1) - 1)
        s = mag.max(axis=1) / qmax
        with np.errstate(divide="ignore", invalid="ignore"):
            r = g / s[:, None]
        q = np.clip(_round_half_away(r), -qmax, qmax)
        q = np.where(s[:, None] == 0, 0.0, q)
    return (q.astype(np.float64) * s.astype(np.float64)[:, None]).reshape(n, k)


def soft_quantize(w: np.ndarray, logits: np.ndarray, gumbel: np.ndarray, tau: float):
    """Returns (w_soft float64 [n][k], pi float64 [groups][4], mean expected bits)."""
    n, k = w.shape
    z = (np.asarray(logits, np.float64).reshape(-1, 4) + np.asarray(gumbel, np.float64).reshape(-1, 4)) / tau
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    pi = e / e.sum(axis=1, keepdims=True)
    recon = [training_reconstruction(w, b).reshape(-1, 64) for b in WIDTHS]
    w_soft = sum(pi[:, i:i + 1] * recon[i] for i in range(4)).reshape(n, k)
    bits = float((pi * np.array(WIDTHS, np.float64)).sum(axis=1).mean()) if pi.size else 0.0
    return w_soft, pi, bits
