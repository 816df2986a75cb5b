"""CPU model of the f32 latent kernel's f16-part products (no GPU).

The f32-cache latent kernel feeds f16 matrix products: every f32 operand x
(cache entries, q * scale * log2(e), the softmax weights P) becomes two f16
parts, hi = round(x) and lo = round((x - hi) * 2^11), and each product of two
split operands is taken as three products of parts, a_hi b_hi + 2^-11 (a_hi
b_lo + a_lo b_hi), with f32 accumulation (a_lo b_lo, below 2^-22 of the
whole, is left out). For the output product the weights' hi part enters as
hi * 2^11, so all three products share one accumulator scaled by 2^11; that
needs hi * 2^11 finite in f16, which holds for weights up to 2^4 (the
kernel's lazy-maximum threshold). These tests model that arithmetic in numpy
(float64 sums of exactly widened parts) and pin:

* hi + lo * 2^-11 equals x within 2^-22 |x| + 2^-36 over f16's whole range,
  and magnitudes from 65,520 up give an infinite hi and the opposite
  infinity as lo, so every product such a value enters is NaN;
* latent scores (576 columns) from three products stay within 1e-6 of the
  exact score relative to sum |q| |c|, while hi products alone miss by far
  more;
* weighted value sums from the single scaled accumulator stay within 2^-20
  of sum P |V|, for caches of unit and of 1e-4 magnitude, and hi * 2^11 is
  exact for every weight up to 16 but overflows at 32.
"""

import numpy as np

LOG2E = 1.4426950408889634


def _parts(x32):
    """The kernel's split of f32 values: hi = f16(x), lo = f16(x 2^11 - hi 2^11)
    (both products exact in f32, the difference exact by construction)."""
    x32 = np.asarray(x32, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        hi = x32.astype(np.float16)
        res = x32 * np.float32(2048.0) - hi.astype(np.float32) * np.float32(2048.0)
        return hi, res.astype(np.float16)


def _recombine(hi, lo):
    return hi.astype(np.float64) + lo.astype(np.float64) / 2048.0


def test_two_f16_parts_carry_22_bits_over_f16_range():
    g = np.random.default_rng(5)
    mag = np.exp2(g.uniform(-40.0, 15.9, 200_000))
    x = (mag * g.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    hi, lo = _parts(x)
    err = np.abs(_recombine(hi, lo) - x.astype(np.float64))
    bound = 2.0**-22 * np.abs(x.astype(np.float64)) + 2.0**-36
    assert np.all(err <= bound), float((err / bound).max())
    # without the 2^11 the residuals of small values are f16 subnormals and
    # lose bits
    unscaled = (x - hi.astype(np.float32)).astype(np.float16)
    err_u = np.abs(hi.astype(np.float64) + unscaled.astype(np.float64) - x.astype(np.float64))
    assert np.mean(err_u > bound) > 0.2


def test_f16_range_boundary_of_the_split():
    hi, lo = _parts(np.array([65504.0, 65519.0, 65520.0, -70000.0], dtype=np.float32))
    assert np.isfinite(hi[:2].astype(np.float64)).all()
    assert np.isinf(hi[2:].astype(np.float64)).all()
    # past the range, lo is the opposite infinity: a product of parts,
    # a_hi b_hi + 2^-11 (a_hi b_lo + a_lo b_hi), then sums inf and -inf
    assert np.all(np.sign(lo[2:].astype(np.float64)) == -np.sign(hi[2:].astype(np.float64)))
    g = np.random.default_rng(3)
    b = g.standard_normal(64).astype(np.float32)
    bh, bl = _parts(b)
    with np.errstate(invalid="ignore", over="ignore"):
        for k in (2, 3):
            a_hi, a_lo = np.float64(hi[k]), np.float64(lo[k])
            mixed = a_hi * bl.astype(np.float64) + a_lo * bh.astype(np.float64)  # one accumulator
            prod = a_hi * bh.astype(np.float64) + mixed / 2048.0
            assert np.all(np.isnan(prod))


def _latent(rows=512, heads=96, dk=576, seed=17, c_scale=1.0):
    g = np.random.default_rng(seed)
    q = g.standard_normal((heads, dk), dtype=np.float32)
    c = (g.standard_normal((rows, dk), dtype=np.float32) * np.float32(c_scale)).astype(np.float32)
    qs = (q * np.float32(np.float32(1.0 / np.sqrt(dk)) * np.float32(LOG2E))).astype(np.float32)
    return qs, c


def test_latent_scores_from_three_products_keep_f32_accuracy():
    qs, c = _latent()
    qh, ql = _parts(qs)
    ch, cl = _parts(c)
    f = lambda a: a.astype(np.float64)
    three = f(ch) @ f(qh).T + (f(ch) @ f(ql).T + f(cl) @ f(qh).T) / 2048.0
    exact = f(c) @ f(qs).T
    scale = np.abs(f(c)) @ np.abs(f(qs)).T
    rel = np.abs(three - exact) / scale
    assert rel.max() <= 1e-6, rel.max()
    hi_only = f(ch) @ f(qh).T
    assert (np.abs(hi_only - exact) / scale).max() >= 100 * rel.max()


def test_weighted_values_from_one_scaled_accumulator():
    g = np.random.default_rng(23)
    rows, cols = 1024, 512
    # weights up to 2^4 (lazy maximum), many far below 1, some zero
    p = np.exp2(g.uniform(-30.0, 4.0, rows)).astype(np.float32)
    p[::97] = 0.0
    for v_scale in (1.0, 1e-4):
        v = (g.standard_normal((rows, cols), dtype=np.float32) * np.float32(v_scale)).astype(np.float32)
        ph, pl = _parts(p)
        phs = (ph.astype(np.float32) * np.float32(2048.0)).astype(np.float16)
        assert np.array_equal(phs.astype(np.float64), ph.astype(np.float64) * 2048.0)  # exact, finite
        vh, vl = _parts(v)
        f = lambda a: a.astype(np.float64)
        acc = f(phs) @ f(vh) + f(ph) @ f(vl) + f(pl) @ f(vh)
        got = acc / 2048.0
        exact = f(p) @ f(v)
        scale = f(p) @ np.abs(f(v))
        assert np.all(np.abs(got - exact) <= 2.0**-20 * scale), float((np.abs(got - exact) / scale).max())
    # a weight of 2^5 would overflow: hi * 2^11 = 65,536 is past f16's range
    with np.errstate(over="ignore"):
        assert np.isinf(np.float16(np.float32(32.0) * np.float32(2048.0)).astype(np.float64))
