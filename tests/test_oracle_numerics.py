"""Pins of the oracle's bit-level rounding: bfloat16 and e4m3fn against torch's casts (a library
routine implementing the same formats), exhaustively over all 2^16 bfloat16 bit patterns plus the
midpoints between neighbours; e4m3fn decoding over all 256 codes; int8 codes on hand-checked cases.
"""

import numpy as np
import torch

import oracle
from oracle.numerics import E4M3_MAX


def _all_bf16_as_f32():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    return x[np.isfinite(x)]


def _torch_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def test_bf16_round_exhaustive_and_midpoints():
    x = _all_bf16_as_f32()
    np.testing.assert_array_equal(oracle.bf16_round(x), x)            # already bf16: unchanged
    u = x.view(np.uint32)
    cases = []
    for delta in (0x7FFF, 0x8000, 0x8001, 0x0001, 0xFFFF, 0x4000):   # below, at, above midpoint
        y = (u.astype(np.uint64) + delta).astype(np.uint32).view(np.float32)
        cases.append(y[np.isfinite(y)])
    rng = np.random.default_rng(0)
    r = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
    cases.append(r[np.isfinite(r)])
    y = np.concatenate(cases)
    np.testing.assert_array_equal(oracle.bf16_round(y), _torch_bf16(y))


def test_bf16_ties_to_even_examples():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to the even significand, 1.0
    assert oracle.bf16_round(np.float32(1 + 2 ** -8)) == np.float32(1.0)
    assert oracle.bf16_round(np.float32(1 + 3 * 2 ** -8)) == np.float32(1 + 2 ** -6)
    mid = np.float32(2.0 ** 127 * (2 - 2 ** -8))      # halfway between the largest bf16 and 2^128
    assert np.isinf(oracle.bf16_round(mid))
    assert oracle.bf16_round(np.nextafter(mid, np.float32(0))) == np.float32(2.0 ** 127 * (2 - 2 ** -7))


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).float().numpy()


def test_e4m3fn_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    fin = ours[~nan]
    assert fin.max() == 448.0 and np.min(np.abs(fin[fin != 0])) == 2.0 ** -9
    finite = codes[~nan]
    np.testing.assert_array_equal(oracle.e4m3fn_encode(oracle.e4m3fn_decode(finite)), finite)


def test_e4m3fn_round_against_torch():
    x = _all_bf16_as_f32()
    inside = x[np.abs(x) <= E4M3_MAX]
    np.testing.assert_array_equal(oracle.e4m3fn_round(inside), _torch_e4m3(inside))
    vals = np.unique(oracle.e4m3fn_decode(np.arange(256, dtype=np.uint8)))
    vals = vals[np.isfinite(vals)]
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)        # exact ties
    near = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(-np.inf))]).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3fn_round(near), _torch_e4m3(near))
    outside = x[np.abs(x) > E4M3_MAX]                               # saturating reading
    np.testing.assert_array_equal(oracle.e4m3fn_round(outside), np.sign(outside) * E4M3_MAX)


def test_e4m3fn_examples():
    assert oracle.e4m3fn_round(2.0 ** -10) == 0.0                 # half the smallest subnormal
    assert oracle.e4m3fn_round(3 * 2.0 ** -10) == 2.0 ** -8       # tie between 1 and 2 quanta -> 2
    assert oracle.e4m3fn_round(500.0) == 448.0
    assert oracle.e4m3fn_encode(np.array([448.0]))[0] == 0x7E
    assert oracle.e4m3fn_encode(np.array([-0.0]))[0] == 0x80


def test_int8_codes():
    inv = np.float32(1.0)
    x = np.array([2.5, 3.5, -2.5, -3.5, 0.49, 126.5, 127.4, 200.0, -300.0], np.float32)
    np.testing.assert_array_equal(oracle.int8_codes(x, inv),
                                  np.array([2, 4, -2, -4, 0, 126, 127, 127, -127], np.int8))
    # the product is taken in float32 before rounding
    x = np.array([1.0], np.float32)
    inv = np.float32(127.0) / np.float32(3.0)
    assert oracle.int8_codes(x, inv)[0] == np.rint(np.float32(x[0] * inv))
