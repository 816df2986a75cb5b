"""CPU model of the query-tile kernel's 16-bit part split of q (no GPU).

The MFMA inputs are 16-bit, so the kernel splits x = q * scale * log2(e) into
parts: f16 hi = round(x), lo = round((x - hi) * 2^11) (added back times
2^-11), or three bf16 parts. These tests model that arithmetic in numpy
(float64 sums of exactly widened parts) and pin three facts about it:

* the split as the kernel does it keeps each score within 1e-6 of the exact
  score, well inside f32 accuracy;
* without the 2^11 scaling, the f16 residual is a subnormal (x is about 0.1,
  so x - hi is below f16's smallest normal, 2^-14) and loses bits;
* when hi is rounded twice (x to f32, then f16) for the MFMA operand but once
  (the exact product straight to f16, as a fused mixed-precision multiply
  does) for the residual, the two disagree about once in 2^14 elements and
  the parts then miss x by a whole f16 step: single scores err by 1e-5 to
  3e-4. That is the fault the kernel's split guards against.
"""

import numpy as np

LN2 = float(np.log(2.0))
LOG2E = np.float32(1.4426950408889634)


def _inputs(rows=4096, D=256, seed=11):
    g = np.random.default_rng(seed)
    q = g.standard_normal((rows, D), dtype=np.float32)
    k = g.standard_normal((rows, D), dtype=np.float32).astype(np.float16)
    qscale = np.float32(np.float32(1.0 / np.sqrt(D)) * LOG2E)
    exact = q.astype(np.float64) * np.float64(qscale)  # the exact product (48 bits)
    x32 = exact.astype(np.float32)  # the product rounded to f32, as the kernel computes it
    return k.astype(np.float64), exact, x32


def _score_err(parts_sum, k, x32):
    # Scores in natural-log units, against the exact sum over the f32 values.
    got = (parts_sum * k).sum(-1) * LN2
    ref = (x32.astype(np.float64) * k).sum(-1) * LN2
    return np.abs(got - ref)


def test_f16_split_with_scaled_residual_keeps_scores_within_1e6():
    k, _, x32 = _inputs()
    hi = x32.astype(np.float16)
    lo = ((x32 - hi.astype(np.float32)) * np.float32(2048.0)).astype(np.float16)
    parts = hi.astype(np.float64) + lo.astype(np.float64) / 2048.0
    # 11 + 11 bits: the parts carry x to within 2^-22 of |x| (plus f16's floor)
    assert np.all(np.abs(parts - x32) <= 2.0 ** -22 * np.abs(x32) + 2.0 ** -35)
    err = _score_err(parts, k, x32)
    assert err.max() <= 1e-6 and np.median(err) <= 5e-8, (err.max(), np.median(err))


def test_unscaled_f16_residual_is_subnormal_and_coarser():
    k, _, x32 = _inputs()
    hi = x32.astype(np.float16)
    res = x32 - hi.astype(np.float32)
    assert np.mean(np.abs(res) < 2.0 ** -14) > 0.99  # almost every residual is an f16 subnormal
    lo = res.astype(np.float16)
    coarse = _score_err(hi.astype(np.float64) + lo.astype(np.float64), k, x32)
    scaled_lo = (res * np.float32(2048.0)).astype(np.float16)
    fine = _score_err(hi.astype(np.float64) + scaled_lo.astype(np.float64) / 2048.0, k, x32)
    assert np.median(coarse) >= 3 * np.median(fine), (np.median(coarse), np.median(fine))


def test_mixed_rounding_of_hi_gives_rare_whole_step_errors():
    k, exact, x32 = _inputs()
    hi_operand = x32.astype(np.float16)  # rounded twice: to f32, then to f16
    hi_residual = exact.astype(np.float16)  # rounded once (fused multiply straight to f16)
    mismatch = hi_operand != hi_residual
    rate = mismatch.mean()
    assert 2.0 ** -16 < rate < 2.0 ** -12, rate  # about once in 2^14 elements
    lo = (exact - hi_residual.astype(np.float64)).astype(np.float32).astype(np.float16)
    err = _score_err(hi_operand.astype(np.float64) + lo.astype(np.float64), k, x32)
    rows = mismatch.any(-1)
    # every score off by 1e-5 or more holds a mismatched element, and the
    # scores that hold one are typically off by tens of times the others
    assert np.all(rows[err >= 1e-5]) and err.max() >= 1e-4, err.max()
    assert np.median(err[rows]) >= 30 * np.median(err[~rows]), (np.median(err[rows]), np.median(err[~rows]))


def test_bf16_three_parts_carry_24_bits_and_are_never_subnormal():
    import torch

    k, _, x32 = _inputs(rows=1024)
    x = torch.from_numpy(x32)
    parts = []
    r = x.clone()
    for _ in range(3):
        p = r.to(torch.bfloat16).to(torch.float32)
        parts.append(p)
        r = r - p
    total = (parts[0].double() + parts[1].double() + parts[2].double()).numpy()
    assert np.all(np.abs(total - x32) <= 2.0 ** -24 * np.abs(x32))
    nz = parts[1].abs() > 0
    assert torch.all(parts[1].abs()[nz] >= 2.0 ** -126)  # bf16 has f32's exponent range
    assert _score_err(total, k, x32).max() <= 1e-6
