"""Pins of the FP8 GEMM oracle (oracle/fp8_gemm.py) against things other than itself.

* brute force: integer-valued operands that e4m3fn holds exactly, multiplied with Python integers;
  random codes summed with exact rational arithmetic (fractions.Fraction) -- the float64 product
  must equal both exactly;
* hand-computed codes: the row maximum maps to +-448 (code 0x7E / 0xFE), ties round to the even
  mantissa (17 -> 16, code 0x58), 134.4 -> 128 (code 0x70), zero and negative-zero rows, values that
  overflow 448 in float32 saturate;
* relations: scaling a row of X (or all of W) by a power of two scales the codes' scale, not the
  codes, and the product by the same factor;
* a bound against the unquantised product (each e4m3fn rounding moves a value by at most 2^-4 of
  it, or 2^-10 of the scale in the subnormal range);
* planted mistakes (a divided scale, an untransposed W, a per-tensor X scale) that the pins catch.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle.fp8_gemm as g
from oracle.numerics import e4m3fn_decode

F32 = np.float32


def _int_operands(m, n, k, seed):
    """Integer operands in [-16, 16] (exact in e4m3fn) with the maximum magnitude 448 placed in
    every row of X and once in W, so that every inverse scale is exactly 1."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-16, 17, (m, k)).astype(F32)
    w = rng.integers(-16, 17, (n, k)).astype(F32)
    x[np.arange(m), rng.integers(0, k, m)] = 448.0 * rng.choice([-1, 1], m)
    w[rng.integers(0, n), rng.integers(0, k)] = -448.0
    return x, w


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (3, 5, 7), (8, 4, 64), (17, 9, 130)])
def test_integer_product_brute_force(m, n, k):
    x, w = _int_operands(m, n, k, 10 * m + n)
    xc, xs = g.quantize_rows(x)
    wc, ws = g.quantize_tensor(w)
    assert np.all(xs == 1.0) and ws == 1.0
    assert np.array_equal(e4m3fn_decode(xc), x) and np.array_equal(e4m3fn_decode(wc), w)
    y = g.gemm(xc, xs, wc, ws)
    xi = x.astype(np.int64).tolist()
    wi = w.astype(np.int64).tolist()
    for i in range(m):
        for j in range(n):
            assert y[i, j] == sum(a * b for a, b in zip(xi[i], wi[j]))


def test_exact_sum_of_random_codes():
    rng = np.random.default_rng(5)
    codes_x = rng.integers(0, 256, (4, 300)).astype(np.uint8)
    codes_w = rng.integers(0, 256, (3, 300)).astype(np.uint8)
    # drop the NaN codes S.1111.111
    codes_x[(codes_x & 0x7F) == 0x7F] = 0x7E
    codes_w[(codes_w & 0x7F) == 0x7F] = 0x7E
    y = g.gemm(codes_x, np.ones(4, F32), codes_w, F32(1))
    xv, wv = e4m3fn_decode(codes_x), e4m3fn_decode(codes_w)
    for i in range(4):
        for j in range(3):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xv[i], wv[j]))
            assert Fraction(float(y[i, j])) == exact


def test_hand_computed_codes():
    x = np.array([[448.0 * 0.3, 448.0, 17.0, -448.0],     # amax 448: inv = scale = 1
                  [0.0, 0.0, 0.0, 0.0],                     # zero row
                  [-0.0, -0.0, -0.0, -0.0],                  # negative zeros
                  [3.0, 3.0, 3.0, 3.0]], dtype=F32)          # constant row
    c, s = g.quantize_rows(x)
    assert list(c[0]) == [0x70, 0x7E, 0x58, 0xFE]
    assert s[0] == 1.0 and s[1] == 1.0 and s[2] == 1.0
    assert list(c[1]) == [0, 0, 0, 0] and list(c[2]) == [0x80] * 4
    assert list(c[3]) == [0x7E] * 4 and s[3] == F32(F32(3.0) / F32(448.0))


def test_saturation():
    # amax * (448 / amax) rounds above 448 in float32 for some amax; the code must still be 0x7E
    amaxes = np.array([1.0 + i / 997.0 for i in range(2000)], F32)
    over = [a for a in amaxes if F32(a * F32(F32(448.0) / a)) > F32(448.0)]
    assert over, "no float32 amax that overflows 448 in this range"
    x = np.array([[a, -a] for a in over[:50]], F32)
    c, _ = g.quantize_rows(x)
    assert np.all(c[:, 0] == 0x7E) and np.all(c[:, 1] == 0xFE)


def test_tensor_scale_is_global():
    w = np.array([[1.0, 2.0], [100.0, -3.0]], F32)
    c, s = g.quantize_tensor(w)
    assert s == F32(F32(100.0) / F32(448.0))
    inv = F32(F32(448.0) / F32(100.0))
    # 1 * 4.48 = 4.48 -> 4.5 (spacing 0.5 in [4, 8)); 2 * 4.48 = 8.96 -> 9 (spacing 1 in [8, 16))
    assert F32(F32(1.0) * inv) == F32(4.48) and list(c[0]) == [0x49, 0x51]
    assert c[1, 0] == 0x7E


@pytest.mark.parametrize("j", [-5, -1, 3, 6])
def test_power_of_two_scaling(j):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 96)).astype(F32)
    w = rng.standard_normal((5, 96)).astype(F32)
    xc, xs = g.quantize_rows(x)
    wc, ws = g.quantize_tensor(w)
    y = g.gemm(xc, xs, wc, ws)
    x2 = x.copy()
    x2[2] *= F32(2.0 ** j)
    xc2, xs2 = g.quantize_rows(x2)
    assert np.array_equal(xc2, xc) and xs2[2] == F32(xs[2] * F32(2.0 ** j))
    y2 = g.gemm(xc2, xs2, wc, ws)
    assert np.array_equal(y2[2], y[2] * 2.0 ** j) and np.array_equal(np.delete(y2, 2, 0), np.delete(y, 2, 0))
    wc3, ws3 = g.quantize_tensor(w * F32(2.0 ** j))
    assert np.array_equal(wc3, wc) and ws3 == F32(ws * F32(2.0 ** j))
    assert np.allclose(g.gemm(xc, xs, wc3, ws3), y * 2.0 ** j, rtol=1e-15, atol=0)


def test_close_to_unquantised_product():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((20, 256)).astype(F32)
    w = rng.standard_normal((12, 256)).astype(F32)
    y = g.linear(x, w)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    xc, xs = g.quantize_rows(x)
    wc, ws = g.quantize_tensor(w)
    # |x - x~ s| <= 2^-4 |x| + 2^-10 s  (normal and subnormal ranges), likewise for w
    ex = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * xs[:, None]
    ew = 2.0 ** -4 * np.abs(w) + 2.0 ** -10 * ws
    bound = ex @ np.abs(w).T + np.abs(x) @ ew.T + ex @ ew.T
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-9))
    assert np.abs(e4m3fn_decode(xc) * xs[:, None] - x).max() <= ex.max()


def test_rows_and_accumulation_bound():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((9, 128)).astype(F32)
    w = rng.standard_normal((4, 128)).astype(F32)
    xc, xs = g.quantize_rows(x)
    wc, ws = g.quantize_tensor(w)
    rows = [8, 0, 3]
    assert np.array_equal(g.gemm_rows(xc, xs, wc, ws, rows), g.gemm(xc, xs, wc, ws)[rows])
    b = g.accumulation_bound(xc, xs, wc, ws, rows)
    y = g.gemm_rows(xc, xs, wc, ws, rows)
    assert b.shape == y.shape and np.all(b >= 128 * 2.0 ** -24 * np.abs(y) * (1 - 1e-12))


def _mutant_divided_scale(xc, xs, wc, ws):
    return (e4m3fn_decode(xc) @ e4m3fn_decode(wc).T) / np.asarray(xs, np.float64)[:, None] * ws


def _mutant_untransposed(xc, xs, wc, ws):
    return (e4m3fn_decode(xc) @ e4m3fn_decode(wc)) * np.asarray(xs, np.float64)[:, None] * ws


def test_planted_mistakes_are_caught(monkeypatch):
    # a divided activation scale fails the power-of-two relation
    rng = np.random.default_rng(17)
    x = rng.standard_normal((4, 64)).astype(F32)
    w = rng.standard_normal((64, 64)).astype(F32)
    x2 = x.copy()
    x2[1] *= F32(8.0)
    xc, xs = g.quantize_rows(x)
    xc2, xs2 = g.quantize_rows(x2)
    wc, ws = g.quantize_tensor(w)
    y, y2 = _mutant_divided_scale(xc, xs, wc, ws), _mutant_divided_scale(xc2, xs2, wc, ws)
    assert not np.array_equal(y2[1], y[1] * 8.0)
    # an untransposed (square) W fails the brute-force integer product
    xi, wi = _int_operands(3, 8, 8, 3)
    xci, xsi = g.quantize_rows(xi)
    wci, wsi = g.quantize_tensor(wi)
    ref = xi.astype(np.int64) @ wi.astype(np.int64).T
    assert not np.array_equal(_mutant_untransposed(xci, xsi, wci, wsi), ref)
    # a per-tensor activation scale gives different codes for rows below the tensor maximum
    monkeypatch.setattr(g, "quantize_rows", lambda a: g.quantize_tensor(a))
    xcm, _ = g.quantize_rows(x2)
    assert not np.array_equal(xcm, xc2)
