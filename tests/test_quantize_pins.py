"""Pins for the CPU reference of the per-group quantizer and the fixed recipe.

VBQ paper (arXiv 2607.02893) §3.1 Eq. (1) (absmax scale over 2^(b-1) - 1,
round and clip; 1-bit sign with the mean magnitude as scale) and §3.4 (the
recipe: 4-bit first-block MLP, 2-bit projections, frequency-tiered head at a
mean of 1.18 bits). Each test checks the reference against something it does
not share code with: a brute-force search over the code grid, the nearest
binary16 value found by scanning all 65536 patterns, hand-built groups with
known answers, and the head mean the pages print.
"""
import numpy as np
import pytest

from oracle import quantize as Q

ALL_HALVES = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
FINITE_HALVES = ALL_HALVES[np.isfinite(ALL_HALVES)].astype(np.float64)


def nearest_half(v: float) -> float:
    """Nearest finite binary16 value to v by scanning every pattern (ties to the even mantissa)."""
    d = np.abs(FINITE_HALVES - v)
    cand = FINITE_HALVES[d == d.min()]
    if cand.size == 1:
        return float(cand[0])
    pats = cand.astype(np.float16).view(np.uint16)
    return float(cand[(pats & 1) == 0][0])


def one_group(values, b):
    w = np.zeros((1, 64), np.float32)
    w[0, :len(values)] = values
    codes, scales = Q.quantize(w, np.array([[b]], np.uint8))
    return codes[0], float(scales.view(np.float16)[0, 0])


@pytest.mark.parametrize("b", [2, 4, 8])
def test_codes_are_the_nearest_grid_point_of_the_stored_scale(b):
    # brute force: every code minimises |w - s q| over the whole grid for the stored scale
    rng = np.random.default_rng(b)
    w = (rng.standard_normal((40, 64 * 8)) * 0.02).astype(np.float32)
    bits = np.full((40, 8), b, np.uint8)
    codes, scales = Q.quantize(w, bits)
    qmax = 2 ** (b - 1) - 1
    grid = np.arange(-qmax, qmax + 1, dtype=np.float64)
    s = scales.view(np.float16).astype(np.float64)
    for r in range(40):
        for j in range(8):
            wg = w[r, 64 * j:64 * j + 64].astype(np.float64)
            err = np.abs(wg[:, None] - s[r, j] * grid[None, :])
            best = grid[err.argmin(axis=1)]
            tie = np.sort(err, axis=1)[:, 1] - err.min(axis=1) < 1e-12
            assert np.array_equal(codes[r, 64 * j:64 * j + 64][~tie], best[~tie])
            # the largest magnitude lands on the end of the grid
            i = np.abs(wg).argmax()
            assert abs(int(codes[r, 64 * j + i])) == qmax


@pytest.mark.parametrize("b", [2, 4, 8])
def test_scale_is_the_nearest_half_of_max_over_grid_end(b):
    rng = np.random.default_rng(10 + b)
    for _ in range(20):
        vals = (rng.standard_normal(64) * rng.choice([1e-3, 0.02, 3.0])).astype(np.float32)
        _, s = one_group(vals, b)
        s32 = np.float32(np.abs(vals).max()) / np.float32(2 ** (b - 1) - 1)
        assert s == nearest_half(float(s32))


def test_one_bit_is_sign_and_mean_magnitude():
    vals = np.array([0.5, -0.25, 0.0, -0.0, 1.0, -2.0] + [0.25] * 58, np.float32)
    codes, s = one_group(vals, 1)
    assert list(codes[:6]) == [1, -1, 1, 1, 1, -1]   # sign(0) = +1, also for -0.0
    assert np.all(codes[6:] == 1)
    assert s == nearest_half(float(np.abs(vals.astype(np.float64)).sum() / 64))
    # equal magnitudes: the mean is that magnitude exactly
    codes, s = one_group(np.array([0.75, -0.75] * 32, np.float32), 1)
    assert s == 0.75 and list(codes[:4]) == [1, -1, 1, -1]


def test_one_bit_scale_is_rounded_once_from_the_mean():
    # M is the midpoint of two adjacent halves; 63 weights at M and one an fp32 ulp below
    # give a mean of M - 2^-36: nearest half is the lower one, whereas rounding the mean
    # to fp32 first lands on M and then ties to the even (upper) half
    lo, hi = np.array([0x237F, 0x2380], np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2
    vals = np.array([mid] * 63 + [mid - 2.0 ** -30], np.float32)
    assert float(vals[0]) == mid and float(vals[63]) == mid - 2.0 ** -30
    _, s = one_group(vals, 1)
    assert s == lo == nearest_half(float(np.abs(vals.astype(np.float64)).sum() / 64))


def test_ties_round_away_from_zero():
    # b = 4: largest magnitude 7 gives scale 1, so every ratio is the weight itself
    codes, s = one_group([7, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 3.5, -3.5, 0.49], 4)
    assert s == 1.0
    assert list(codes[:10]) == [7, 3, -3, 1, -1, 2, -2, 4, -4, 0]


def test_rounding_just_below_a_half():
    # scale 1 (b = 8, largest magnitude 127): each code is round-half-away of the weight itself
    below_half = np.nextafter(np.float32(0.5), np.float32(0))          # 0.5 - 2^-25
    below_1_5 = np.nextafter(np.float32(1.5), np.float32(0))
    above_half = np.nextafter(np.float32(0.5), np.float32(1))
    vals = [127, below_half, -below_half, 0.5, -0.5, below_1_5, -below_1_5, above_half, 126.5, -126.5]
    codes, s = one_group(np.array(vals, np.float32), 8)
    assert s == 1.0
    assert list(codes[:10]) == [127, 0, 0, 1, -1, 1, -1, 1, 127, -127]


def test_codes_use_the_stored_half_scale():
    # max/127 = 1 + 3 * 2^-13 rounds to the half 1.0; 100.52 / 1.0 rounds to 101,
    # whereas 100.52 over the unrounded scale would round to 100
    amax = np.float32(127) * np.float32(1 + 3 * 2 ** -13)
    codes, s = one_group([amax, 100.52], 8)
    assert s == 1.0
    assert codes[0] == 127 and codes[1] == 101


def test_zero_group_and_tiny_and_huge_scales():
    for b in (2, 4, 8):
        codes, s = one_group([], b)
        assert s == 0.0 and np.all(codes == 0)
        codes, s = one_group([1e-10, -1e-10], b)   # the scale underflows fp16
        assert s == 0.0 and np.all(codes == 0)
        codes, s = one_group([1e9, -3e8, 2.0], b)   # the scale saturates at the largest finite half
        qmax = 2 ** (b - 1) - 1
        assert s == 65504.0
        assert codes[0] == qmax and codes[2] == 0
        assert codes[1] == -min(qmax, int(np.floor(3e8 / 65504 + 0.5)))
    codes, s = one_group([], 1)
    assert s == 0.0 and np.all(codes == 1)


def test_mixed_widths_pick_each_groups_rule():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((3, 256)) * 0.05).astype(np.float32)
    bits = np.array([[1, 2, 4, 8], [8, 4, 2, 1], [2, 2, 1, 8]], np.uint8)
    codes, scales = Q.quantize(w, bits)
    for r in range(3):
        for j in range(4):
            c, s = one_group(w[r, 64 * j:64 * j + 64], int(bits[r, j]))
            assert np.array_equal(codes[r, 64 * j:64 * j + 64], c)
            assert float(scales.view(np.float16)[r, j]) == s


def test_head_recipe_mean_is_the_pages_1_18_bits():
    rows = 32000
    freq = np.random.default_rng(3).permutation(rows) + 1   # distinct frequencies
    bits = Q.head_bits(freq)
    counts = {b: int((bits == b).sum()) for b in (8, 4, 2, 1)}
    assert counts == {8: 160, 4: 480, 2: 3200, 1: 28160}
    assert bits.astype(np.float64).mean() == pytest.approx(1.18, abs=1e-12)
    # the most frequent rows get the most bits, monotonically
    order = np.argsort(-freq, kind="stable")
    assert np.all(np.diff(bits[order].astype(int)) <= 0)
    assert bits[freq.argmax()] == 8 and bits[freq.argmin()] == 1


def test_head_recipe_ties_go_to_the_lower_row():
    bits = Q.head_bits(np.zeros(1000))   # all tied: rank = row index
    assert list(bits[:5]) == [8] * 5 and bits[5] == 4 and bits[19] == 4 and bits[20] == 2
    assert bits[119] == 2 and bits[120] == 1


def test_head_recipe_rounds_tier_edges_half_up():
    # 300 rows: 0.5% is 1.5 rows -> 2, 2% is 6, 12% is 36; 100 rows: 0.5 -> 1, 2, 12
    for rows, counts in ((300, {8: 2, 4: 4, 2: 30, 1: 264}), (100, {8: 1, 4: 1, 2: 10, 1: 88})):
        bits = Q.head_bits(np.arange(rows)[::-1])
        assert {b: int((bits == b).sum()) for b in (8, 4, 2, 1)} == counts


def test_projection_recipe():
    assert Q.projection_bits(True) == 4 and Q.projection_bits(False) == 2


def test_dequantize_error_bound():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((8, 512)) * 0.02).astype(np.float32)
    bits = rng.choice(np.array([2, 4, 8], np.uint8), size=(8, 8))
    codes, scales = Q.quantize(w, bits)
    wh = Q.dequantize(codes, scales)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 64, axis=1)
    # inside the grid the error is at most half a step; the clipped end is the largest magnitude
    qmax = np.repeat((2 ** (bits.astype(int) - 1) - 1), 64, axis=1)
    inside = np.abs(codes) < qmax
    assert np.all(np.abs(w - wh)[inside] <= s[inside] / 2 * (1 + 1e-6))


# ---------------------------------------------------------------- soft quantizer (§3.2)

def test_training_reconstruction_is_the_nearest_grid_point_with_fp32_scale():
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((6, 256)) * 0.03).astype(np.float32)
    for b in (2, 4, 8):
        wh = Q.training_reconstruction(w, b)
        qmax = 2 ** (b - 1) - 1
        for r in range(6):
            for j in range(4):
                g = w[r, 64 * j:64 * j + 64]
                s = float(np.float32(np.abs(g).max()) / np.float32(qmax))
                grid = s * np.arange(-qmax, qmax + 1)
                err = np.abs(g.astype(np.float64)[:, None] - grid[None, :])
                best = grid[err.argmin(axis=1)]
                tie = np.sort(err, axis=1)[:, 1] - err.min(axis=1) < 1e-12
                assert np.allclose(wh[r, 64 * j:64 * j + 64][~tie], best[~tie], rtol=0, atol=1e-12)
    one = Q.training_reconstruction(w, 1)
    assert np.allclose(np.abs(one[:, :64]), np.abs(w[:, :64]).astype(np.float64).mean(axis=1, keepdims=True),
                       rtol=1e-7)
    assert np.array_equal(np.sign(one), np.where(w < 0, -1.0, 1.0))


def test_soft_quantizer_limits_and_bit_cost():
    rng = np.random.default_rng(22)
    n, k = 5, 192
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    groups = n * k // 64
    zero = np.zeros((groups, 4))
    # a dominant logit: the mixture is that width's reconstruction and the cost is that width
    for i, b in enumerate(Q.WIDTHS):
        logits = np.full((groups, 4), -60.0)
        logits[:, i] = 60.0
        ws, pi, bits = Q.soft_quantize(w, logits, zero, 1.0)
        assert np.allclose(ws, Q.training_reconstruction(w, b), rtol=0, atol=1e-12)
        assert bits == pytest.approx(b, abs=1e-12)
    # equal logits: each width weighs 1/4, the cost is the mean width 3.75
    ws, pi, bits = Q.soft_quantize(w, zero, zero, 5.0)
    assert np.allclose(pi, 0.25) and bits == pytest.approx(3.75, abs=1e-12)
    assert np.allclose(ws, sum(Q.training_reconstruction(w, b) for b in Q.WIDTHS) / 4, rtol=0, atol=1e-15)
    # softmax of (l + e) / tau: shifting all four by a constant changes nothing; a lower tau sharpens
    l = rng.standard_normal((groups, 4))
    e = -np.log(-np.log(rng.random((groups, 4))))
    a = Q.soft_quantize(w, l, e, 0.7)
    b2 = Q.soft_quantize(w, l + 3.0, e - 1.0, 0.7)
    assert np.allclose(a[1], b2[1], rtol=1e-13) and np.allclose(a[0], b2[0], rtol=1e-12)
    z = (l + e) / 0.7
    assert np.allclose(a[1], np.exp(z) / np.exp(z).sum(axis=1, keepdims=True), rtol=1e-12)
    sharp = Q.soft_quantize(w, l, e, 0.05)[1]
    assert np.all(sharp.max(axis=1) >= a[1].max(axis=1) - 1e-12)
    # the mixture is a convex combination: it lies between the smallest and largest reconstruction
    rec = np.stack([Q.training_reconstruction(w, b) for b in Q.WIDTHS])
    assert np.all(a[0] >= rec.min(axis=0) - 1e-15) and np.all(a[0] <= rec.max(axis=0) + 1e-15)
