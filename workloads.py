"""Seeded synthetic inputs for the VBQ packed GEMV / small-batch GEMM.

This module is the ONLY code shared by the oracle side and the HIP side. It
draws inputs - per-group bit widths, integer codes on each width's grid, fp16
scales and fp16 activations - and holds none of the method's arithmetic: no
packing, no decoding, no dot products.

Workload shapes follow the layer sets the VBQ paper measures decode on
("Variable Bit-width Quantization: Learning Per-Group Precision for
'Bigger-but-Smaller' Language Models", arXiv 2607.02893, §6 and Figure 5:
131M, 1.0B and 9B models; §5.1 for the learned width mix and the head's
near-1-bit allocation). Trained weights are not available, so every matrix is
a synthetic stand-in with the paper's group size (§3.1: G = 64) and a width
mix drawn i.i.d. per group:

* standard mix {1: 0.69, 2: 0.16, 4: 0.10, 8: 0.05} (1.81 mean bits);
* first-block MLP of the 131M set {1: 0.35, 2: 0.30, 4: 0.25, 8: 0.10};
* LM head {1: 0.97, 2: 0.02, 4: 0.01}.

Scales are |N(0, 0.02)| rounded to fp16 (round-to-nearest-even), codes are
uniform over the width's grid (b = 1: {-1, +1}; b >= 2: the symmetric
integers |q| <= 2^(b-1) - 1 of §3.1 Eq. (1)), activations are N(0, 1) rounded
to fp16. Every draw is keyed by a numpy SeedSequence tuple so both sides can
regenerate identical inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GROUP = 64

STD_MIX = {1: 0.69, 2: 0.16, 4: 0.10, 8: 0.05}
FIRST_MLP_MIX = {1: 0.35, 2: 0.30, 4: 0.25, 8: 0.10}
HEAD_MIX = {1: 0.97, 2: 0.02, 4: 0.01}

# input roles: which matrices of a decoder layer read the same activation
ROLE_ATTN_IN, ROLE_O_IN, ROLE_MLP_IN, ROLE_DOWN_IN, ROLE_HEAD_IN = range(5)


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    n: int
    k: int
    mix: dict
    seed: tuple
    layer: int = 0
    role: int = ROLE_ATTN_IN


@dataclass(frozen=True)
class ConfigSpec:
    cid: int
    name: str
    matrices: list = field(default_factory=list)
    batches: tuple = (1,)

    @property
    def weights(self) -> int:
        return sum(m.n * m.k for m in self.matrices)


def _decoder_layers(cid, n_layers, d, mlp, gated, first_mix=None):
    mats = []
    idx = 0
    for layer in range(n_layers):
        mlp_mix = first_mix if (first_mix is not None and layer == 0) else STD_MIX
        names = [("q", d, d, STD_MIX, ROLE_ATTN_IN), ("k", d, d, STD_MIX, ROLE_ATTN_IN),
                 ("v", d, d, STD_MIX, ROLE_ATTN_IN), ("o", d, d, STD_MIX, ROLE_O_IN)]
        if gated:
            names.append(("gate", mlp, d, mlp_mix, ROLE_MLP_IN))
        names += [("up", mlp, d, mlp_mix, ROLE_MLP_IN), ("down", d, mlp, mlp_mix, ROLE_DOWN_IN)]
        for nm, n, k, mix, role in names:
            mats.append(MatrixSpec(f"L{layer}.{nm}", n, k, mix, (cid, idx), layer, role))
            idx += 1
    return mats


def config(cid: int) -> ConfigSpec:
    """Workload c (1-based): 1 single linear, 2 131M set, 3 1.0B set, 4 9B layer, 5 LM head."""
    if cid == 1:
        return ConfigSpec(1, "single_768x768", [MatrixSpec("w", 768, 768, STD_MIX, (1, 0))], (1,))
    if cid == 2:
        return ConfigSpec(2, "decoder_131m_12L", _decoder_layers(2, 12, 768, 3072, False, FIRST_MLP_MIX), (1,))
    if cid == 3:
        return ConfigSpec(3, "decoder_1b_22L", _decoder_layers(3, 22, 2048, 5632, True), (1, 8))
    if cid == 4:
        return ConfigSpec(4, "layer_9b", _decoder_layers(4, 1, 4096, 14336, True), (1,))
    if cid == 5:
        return ConfigSpec(5, "lm_head_32000x4096",
                          [MatrixSpec("head", 32000, 4096, HEAD_MIX, (5, 0), 0, ROLE_HEAD_IN)], (1, 16, 64))
    raise ValueError(f"unknown workload {cid}")


ALL_CONFIGS = (1, 2, 3, 4, 5)


def draw_group_widths(rng: np.random.Generator, n: int, groups: int, mix: dict) -> np.ndarray:
    ws = np.array(sorted(mix), dtype=np.uint8)
    p = np.array([mix[w] for w in sorted(mix)], dtype=np.float64)
    p = p / p.sum()
    return ws[rng.choice(len(ws), size=(n, groups), p=p)]


def draw_codes(rng: np.random.Generator, bits: np.ndarray) -> np.ndarray:
    """Integer codes uniform over each group's grid; returns int8 [n, groups*64]."""
    n, groups = bits.shape
    u = rng.random((n, groups, GROUP), dtype=np.float32)
    b = bits.astype(np.int32)[:, :, None]
    lim = (1 << np.maximum(b - 1, 0)) - 1                 # 2^(b-1) - 1 (0 for b = 1)
    span = 2 * lim + 1
    q = np.floor(u * span).astype(np.int32)
    q = np.minimum(q, span - 1) - lim
    one = np.where(u < 0.5, -1, 1).astype(np.int32)
    q = np.where(b == 1, one, q)
    return q.reshape(n, groups * GROUP).astype(np.int8)


def draw_scales(rng: np.random.Generator, n: int, groups: int, sigma: float = 0.02) -> np.ndarray:
    s = np.abs(rng.normal(0.0, sigma, size=(n, groups))).astype(np.float16)
    return s.view(np.uint16)


def draw_matrix(spec: MatrixSpec):
    """(bits uint8 [n,G], codes int8 [n,K], scales uint16 [n,G]) for one matrix."""
    if spec.k % GROUP:
        raise ValueError("K must be a multiple of 64")
    rng = np.random.default_rng(np.random.SeedSequence(spec.seed))
    g = spec.k // GROUP
    bits = draw_group_widths(rng, spec.n, g, spec.mix)
    scales = draw_scales(rng, spec.n, g)
    codes = draw_codes(rng, bits)
    return bits, codes, scales


def draw_random_matrix(seed, n: int, k: int, mix=None):
    """Same recipe for an arbitrary shape (tests)."""
    return draw_matrix(MatrixSpec("t", n, k, mix or STD_MIX, tuple(np.atleast_1d(seed).tolist())))


def draw_weights(seed, n: int, k: int, sigma: float = 0.02, outlier_frac: float = 0.002) -> np.ndarray:
    """fp32 weights [n, k] for the quantizer: N(0, sigma), with a small fraction of
    entries scaled up 10-50x (the heavy tail trained projections show, which
    is what sets a group's absmax)."""
    rng = np.random.default_rng(np.random.SeedSequence(tuple(np.atleast_1d(seed).tolist()) + (104729,)))
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)
    hit = rng.random((n, k), dtype=np.float32) < outlier_frac
    w[hit] *= rng.uniform(10.0, 50.0, size=int(hit.sum())).astype(np.float32)
    return w


def draw_x(seed, k: int, m: int = 1) -> np.ndarray:
    """fp16 N(0,1) activations as uint16 bit patterns, shape [m, k]."""
    rng = np.random.default_rng(np.random.SeedSequence(tuple(np.atleast_1d(seed).tolist()) + (7919,)))
    return rng.standard_normal((m, k)).astype(np.float16).view(np.uint16)


def draw_x_offset(seed, k: int, m: int = 1, mean: float = 1.0, sigma: float = 0.1) -> np.ndarray:
    """fp16 activations mean + sigma * N(0,1) (a common mode, as post-activation or un-centred
    inputs have) as uint16 bit patterns, shape [m, k]."""
    rng = np.random.default_rng(np.random.SeedSequence(tuple(np.atleast_1d(seed).tolist()) + (6007,)))
    return (mean + sigma * rng.standard_normal((m, k))).astype(np.float16).view(np.uint16)


def draw_signed_scales(seed, n: int, groups: int, sigma: float = 0.02) -> np.ndarray:
    """fp16 scales N(0, sigma) with either sign (the format allows negative scales)."""
    rng = np.random.default_rng(np.random.SeedSequence(tuple(np.atleast_1d(seed).tolist()) + (4421,)))
    return rng.normal(0.0, sigma, size=(n, groups)).astype(np.float16).view(np.uint16)


def x_seed(spec: MatrixSpec) -> tuple:
    """Matrices of one layer that read the same input share this key."""
    return (spec.seed[0], 10_000 + spec.layer, spec.role)
