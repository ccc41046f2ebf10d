"""The error bound stated for LIK_F32_BF16X3, checked on the CPU.

include/lik.h states that splitting float32 values into a bfloat16 high part
hi = bf16(x) and a bfloat16 low part lo = bf16(x - hi) (both rounded to
nearest even) and taking hi_q*hi_d + hi_q*lo_d + lo_q*hi_d leaves a product
within 3 * 2^-16 * |q d| of the exact one (the GPU parity tests use that
bound, with slack, per similarity).  This test rounds to bfloat16 with its own
integer arithmetic (independent of the library) and checks, in float64:
  - the parts: |x - hi - lo| <= 2^-16 |x| and hi, lo are bfloat16 values;
  - every product of two split values against the bound, over random values
    across many binades and over the worst cases (values just under a
    rounding boundary);
  - values with at most 8 significant bits are their own high part (lo = 0),
    so integer inputs split exactly.
"""

import numpy as np


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (r.astype(np.uint32) << 16).view(np.float32)


def split(x: np.ndarray):
    x = np.asarray(x, dtype=np.float32)
    hi = bf16_rne(x)
    lo = bf16_rne((x - hi).astype(np.float32))   # x - hi is exact in float32
    return hi, lo


def _is_bf16(v: np.ndarray) -> bool:
    return bool(np.all((np.ascontiguousarray(v, dtype=np.float32).view(np.uint32) & 0xFFFF) == 0))


def test_rounding_helper_matches_known_values():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even gives 1;
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: gives 1 + 2^-6
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5], np.float32)
    want = np.array([1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -2.5], np.float32)
    assert np.array_equal(bf16_rne(x), want)


def test_parts_and_products_stay_within_the_bound():
    rng = np.random.default_rng(7)
    n = 200_000
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
    y = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
    # values just under and over rounding boundaries of both parts
    edge = (1 + np.arange(1, 2001) * 2.0 ** -8 + 2.0 ** -17).astype(np.float32)
    x = np.concatenate([x, edge, -edge])
    y = np.concatenate([y, edge[::-1], edge])
    hx, lx = split(x)
    hy, ly = split(y)
    assert _is_bf16(hx) and _is_bf16(lx) and _is_bf16(hy) and _is_bf16(ly)
    X, Y = x.astype(np.float64), y.astype(np.float64)
    assert np.all(np.abs(X - hx - lx) <= 2.0 ** -16 * np.abs(X))
    approx = (hx.astype(np.float64) * hy + hx.astype(np.float64) * ly
              + lx.astype(np.float64) * hy)
    err = np.abs(X * Y - approx)
    bound = 3 * 2.0 ** -16 * np.abs(X * Y)
    assert np.all(err <= bound), float(np.max(err / np.abs(X * Y)))
    # the bound is not loose by orders of magnitude: the worst case comes
    # within a factor of a few of it
    assert float(np.max(err / bound)) > 0.05


def test_short_values_split_exactly():
    rng = np.random.default_rng(8)
    ints = rng.integers(-255, 256, 10_000).astype(np.float32)
    hi, lo = split(ints)
    assert np.array_equal(hi, ints) and not np.any(lo)
    # a dot product of such values is exact in the split form
    q, d = ints[:128].astype(np.float64), ints[128:256].astype(np.float64)
    hq, lq = split(ints[:128])
    hd, ld = split(ints[128:256])
    approx = float(np.sum(hq.astype(np.float64) * hd + hq.astype(np.float64) * ld
                          + lq.astype(np.float64) * hd))
    assert approx == float(np.sum(q * d))
