"""The batched prefill's fp16 split of an fp32 activation a (the decode
kernel keeps fp32): hi = fp16(a), lo = fp16((a - hi) * 2^11), products of
lo scaled back by 2^-11.  Written out here with numpy's IEEE binary16
rounding, independently of the kernel, to pin the range the ABI documents:
hi + 2^-11 lo equals a to 2^-22 relative for 2^-14 <= |a| <= 65504 (hi is
the nearest fp16, lo the nearest fp16 to the exact remainder times 2^11,
each within half an fp16 ulp, 2^-11 relative); above that hi is infinite,
which the kernel reports as KIE_ERR_RANGE."""
import numpy as np


def split(a: np.ndarray):
    a = a.astype(np.float32)
    hi = a.astype(np.float16)
    lo = ((a - hi.astype(np.float32)) * np.float32(2048.0)).astype(np.float16)
    return hi, lo


def rebuild(hi, lo):
    return hi.astype(np.float64) + lo.astype(np.float64) / 2048.0


def test_split_error_within_2_pow_minus_22_over_the_documented_range():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-14.0, np.log2(65504.0), 400_000))
    a = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    a = np.concatenate([a, np.float32([2.0 ** -14, -(2.0 ** -14), 65504.0, -65504.0, 1.0, 0.1])])
    hi, lo = split(a)
    assert np.isfinite(hi).all() and np.isfinite(lo).all()
    err = np.abs(rebuild(hi, lo) - a.astype(np.float64)) / np.abs(a.astype(np.float64))
    assert err.max() <= 2.0 ** -22, err.max()
    # the bound is attained in order of magnitude: the split is not exact
    assert err.max() > 2.0 ** -26


def test_split_of_fp16_values_is_exact_and_plain_fp16_is_not_enough():
    rng = np.random.default_rng(8)
    h = rng.standard_normal(10_000).astype(np.float16)
    hi, lo = split(h.astype(np.float32))
    assert np.array_equal(hi, h) and not lo.any()
    # rounding the activation to fp16 alone leaves up to 2^-11 relative
    a = rng.standard_normal(100_000).astype(np.float32)
    one = np.abs(a.astype(np.float16).astype(np.float64) - a) / np.abs(a)
    assert one.max() > 2.0 ** -13


def test_split_overflows_above_the_fp16_range():
    with np.errstate(over="ignore"):
        hi, _ = split(np.float32([65520.0, -70000.0, 1e6]))
    assert np.isinf(hi).all()
    hi, lo = split(np.float32([65519.0]))
    assert np.isfinite(hi).all() and abs(rebuild(hi, lo)[0] - 65519.0) <= 65519.0 * 2.0 ** -22
