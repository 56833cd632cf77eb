"""Shared test helpers: tolerance checks and oracle/library side-by-side setup."""
import numpy as np

import oracle
import workloads as W

REL_L2 = 1e-3        # relative L2 error bound per output vector
MAX_ABS_K = 2e-3     # max abs error bound = MAX_ABS_K * ||x_m||_2 * max|scale|


def xf64(x_bits):
    return np.asarray(x_bits, np.uint16).view(np.float16).astype(np.float64)


def tolerance_report(y_gpu, y_ref, x_bits, scales_bits):
    """Per output vector: (rel_l2, max_abs, abs_bound). y arrays are [m, n] (n may be a row subset)."""
    y_gpu = np.atleast_2d(np.asarray(y_gpu, np.float64))
    y_ref = np.atleast_2d(np.asarray(y_ref, np.float64))
    xs = np.atleast_2d(xf64(x_bits))
    smax = float(np.abs(np.asarray(scales_bits, np.uint16).view(np.float16).astype(np.float64)).max()) \
        if np.size(scales_bits) else 0.0
    out = []
    for i in range(y_ref.shape[0]):
        d = y_gpu[i] - y_ref[i]
        nref = np.linalg.norm(y_ref[i])
        rel = float(np.linalg.norm(d) / nref) if nref > 0 else 0.0
        out.append((rel, float(np.abs(d).max()) if d.size else 0.0,
                    MAX_ABS_K * float(np.linalg.norm(xs[i])) * smax))
    return out


def assert_within_tolerance(y_gpu, y_ref, x_bits, scales_bits, what=""):
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    for i, (rel, mx, bound) in enumerate(tolerance_report(y_gpu, y_ref, x_bits, scales_bits)):
        assert rel <= REL_L2, f"{what}[{i}]: rel L2 {rel:.3e} > {REL_L2}"
        assert mx <= bound, f"{what}[{i}]: max abs {mx:.3e} > {bound:.3e}"


def make_case(seed, n, k, mix=None):
    bits, codes, scales = W.draw_random_matrix(seed, n, k, mix or W.STD_MIX)
    return bits, codes, scales, oracle.pack(n, k, bits, codes, scales)
