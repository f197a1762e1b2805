"""Pins for the oracle's fp64 -> fp16 / bf16 / fp32 round-to-nearest-even.

fp16 and fp32 are checked against numpy's conversions from float64 (a
library routine that rounds directly from fp64); bf16, which numpy lacks, is
checked against a brute-force nearest-value search over every finite bf16
bit pattern (ties to the even pattern), which is the definition itself.
"""
import numpy as np
import pytest

from oracle import oracle as O


def _all_f16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return bits.view(np.float16).astype(np.float64)


def _all_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        return (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)


def test_f16_exhaustive_round_trip():
    v = _all_f16()
    r = O.round_to(v, "float16")
    fin = np.isfinite(v)
    np.testing.assert_array_equal(r[fin], v[fin])
    assert np.all(np.isnan(r[np.isnan(v)]))
    np.testing.assert_array_equal(r[np.isinf(v)], v[np.isinf(v)])
    # signed zero is kept
    assert np.signbit(O.round_scalar(-0.0, "float16"))


def test_f16_midpoints_and_random_match_numpy():
    v = np.unique(_all_f16()[np.isfinite(_all_f16())])
    mids = (v[:-1] + v[1:]) / 2            # exact in fp64
    rng = np.random.default_rng(0)
    rnd = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 5, 200000),
        rng.uniform(65000, 66000, 20000), -rng.uniform(65000, 66000, 20000),
        mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
    ])
    with np.errstate(over="ignore"):
        ref = rnd.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(O.round_to(rnd, "float16"), ref)


def _bf16_nearest(vals):
    # brute force: nearest finite bf16 value, ties to the even bit pattern;
    # beyond the largest finite value, round-to-nearest overflows to inf at
    # max + half an ulp (ties there also go to the even pattern, i.e. inf).
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        allv = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    fin = np.isfinite(allv)
    pos = fin & (allv >= 0) & ~((allv == 0) & (bits >= 0x8000))
    table = allv[pos]
    tbits = bits[pos]
    order = np.argsort(table)
    table, tbits = table[order], tbits[order]
    out = np.empty_like(vals)
    a = np.abs(vals)
    idx = np.clip(np.searchsorted(table, a), 1, len(table) - 1)
    lo, hi = table[idx - 1], table[idx]
    dlo, dhi = a - lo, hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (tbits[idx] % 2 == 0))
    res = np.where(pick_hi, hi, lo)
    maxv = table[-1]
    ulp = maxv - table[-2]
    res = np.where(a >= maxv + ulp / 2, np.inf, res)
    out[:] = np.copysign(res, vals)
    return out


def test_bf16_exhaustive_round_trip():
    v = _all_bf16()
    r = O.round_to(v, "bfloat16")
    fin = np.isfinite(v)
    np.testing.assert_array_equal(r[fin], v[fin])
    assert np.all(np.isnan(r[np.isnan(v)]))


def test_bf16_matches_brute_force_nearest():
    v = _all_bf16()
    v = np.unique(v[np.isfinite(v) & (v >= 0)])
    mids = (v[:-1] + v[1:]) / 2
    rng = np.random.default_rng(1)
    rnd = np.concatenate([
        rng.standard_normal(300000) * 10.0 ** rng.integers(-40, 38, 300000),
        mids, -mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
        np.array([3.3895313892515355e38, 3.39e38, 3.4e38, 1e-45, 9.18e-41]),
    ])
    np.testing.assert_array_equal(O.round_to(rnd, "bfloat16"), _bf16_nearest(rnd))


def test_f32_matches_numpy():
    rng = np.random.default_rng(2)
    v = rng.standard_normal(200000) * 10.0 ** rng.integers(-45, 38, 200000)
    f = rng.standard_normal(1000).astype(np.float32).astype(np.float64)
    step = np.spacing(np.abs(f).astype(np.float32)).astype(np.float64)
    v = np.concatenate([v, f + step / 2, f - step / 2])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(O.round_to(v, "float32"), ref)


@pytest.mark.parametrize("dtype,val,exp", [
    ("float16", 1.0 + 2 ** -11, 1.0),              # tie -> even
    ("float16", 1.0 + 3 * 2 ** -11, 1.0 + 2 ** -9),  # tie -> even (up)
    ("float16", 65519.999, 65504.0),
    ("float16", 65520.0, np.inf),
    ("float16", 2.0 ** -25, 0.0),                  # half the smallest subnormal, tie -> 0
    ("float16", 3 * 2.0 ** -26, 2.0 ** -24),
    ("bfloat16", 1.0 + 2 ** -8, 1.0),
    ("bfloat16", 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -6),
])
def test_rounding_special_values(dtype, val, exp):
    assert O.round_scalar(val, dtype) == exp
