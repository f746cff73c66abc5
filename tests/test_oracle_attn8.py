"""Pins of the 8-bit scheme emulator (oracle.attn8) against things other than itself.

* Quantisation against its defining bounds: every int8 code is within half a step of x * inv, the
  block maximum maps to +-127, every e4m3 value is within the format's relative half-step of
  V * inv, the channel maximum maps to +-448; exactly representable inputs round-trip exactly.
* Smoothing balances the per-channel maxima of Q' and K' and leaves QK^T unchanged (fp64 check).
* Special cases that reduce to the exact attention: one key returns its V row; a V that is the same
  in every key returns it exactly (the normaliser sums the same FP8 weights that multiply V); with
  exactly representable operands -- also with a distinct power-of-two scale in every Q and K block --
  the only error left is the FP8 rounding of P, within a bound derived from e4m3's half step; planted
  mistakes (a dropped P or V scale, block scales shifted by a block or a token, the normaliser taken
  from P before its FP8 rounding) break these pins.
* The 8-bit path's accuracy bounds (rel-L2 <= 6e-2, cosine >= 0.995 against exact attention) on
  a small seeded workload with 1% outlier channels at 8 sigma, and that the literal scheme without
  smoothing is worse there.
"""

import numpy as np
import pytest

import oracle
from oracle import attn8


def _bf16(x):
    return oracle.bf16_round(np.asarray(x, np.float32))


def _gauss(shape, seed, sigma=1.0):
    return _bf16(np.random.default_rng(seed).standard_normal(shape) * sigma)


def _metrics(got, ref):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    cos = got @ ref / (np.linalg.norm(got) * np.linalg.norm(ref))
    return rel, cos


def test_int8_block_quantisation_bounds():
    x = _gauss((200, 128), 1, 3.0)
    codes, scales = attn8._block_int8(x, 64)
    assert codes.shape == x.shape and scales.shape == (4,)
    for blk in range(4):
        xb = x[blk * 64:(blk + 1) * 64].astype(np.float64)
        cb = codes[blk * 64:(blk + 1) * 64].astype(np.float64)
        amax = np.abs(xb).max()
        assert np.isclose(scales[blk], amax / 127, rtol=2 ** -23)
        assert np.max(np.abs(cb)) == 127
        assert np.max(np.abs(cb - xb * (127 / amax))) <= 0.5 + 1e-4
    z, zs = attn8._block_int8(np.zeros((70, 128), np.float32), 64)
    assert not z.any() and np.all(zs == 1)


def test_int8_exact_roundtrip():
    x = np.random.default_rng(2).integers(-127, 128, size=(64, 128)).astype(np.float32)
    x[3, 7] = 127.0
    codes, scales = attn8._block_int8(x, 64)
    np.testing.assert_array_equal(codes, x.astype(np.int8))
    assert scales[0] == 1.0


def test_e4m3_channel_quantisation_bounds():
    v = _gauss((300, 128), 3, 2.0)
    codes, scale = attn8._channel_e4m3(v)
    vals = oracle.e4m3fn_decode(codes)
    amax = np.abs(v).max(axis=0).astype(np.float64)
    np.testing.assert_allclose(scale, amax / 448, rtol=2 ** -23)
    assert np.all(np.abs(vals).max(axis=0) == 448)
    t = v.astype(np.float64) * (448 / amax)
    normal = np.abs(t) >= 2 ** -6
    assert np.all(np.abs(vals - t)[normal] <= np.abs(t)[normal] * 2 ** -4 * (1 + 1e-6))
    assert np.all(np.abs(vals - t)[~normal] <= 2 ** -10 * (1 + 1e-6))


def test_smoothing_balances_and_preserves_products():
    rng = np.random.default_rng(4)
    q = _bf16(rng.standard_normal((100, 128)) * rng.uniform(0.1, 10, 128))
    k = _bf16(rng.standard_normal((90, 128)) * rng.uniform(0.1, 10, 128))
    z = attn8.quantize_head(q, k, k, smooth=True)
    a = z["alpha"].astype(np.float64)
    qs, ks = q * a, k / a
    np.testing.assert_allclose(np.abs(qs).max(0), np.abs(ks).max(0), rtol=1e-6)
    np.testing.assert_allclose(qs @ ks.T, q.astype(np.float64) @ k.astype(np.float64).T,
                               rtol=1e-6, atol=1e-9)


def test_single_key_returns_value_row():
    q = _gauss((1, 10, 2, 128), 5)
    k = _gauss((1, 1, 2, 128), 6)
    # V values are e4m3 values and each channel's maximum is 448, so V quantises exactly
    v = oracle.e4m3fn_round(np.random.default_rng(7).standard_normal((1, 1, 2, 128)) * 100)
    v[..., :] = np.where(np.abs(v) > 0, np.sign(v) * 448.0, 448.0)
    rows = np.array([[0, h, i] for h in range(2) for i in range(10)])
    got = oracle.attn8_emulate(q, k, v.astype(np.float32), rows)
    np.testing.assert_array_equal(got, v[0, 0][rows[:, 1]].astype(np.float32))


def test_exact_operands_leave_only_fp8_rounding_of_p():
    rng = np.random.default_rng(8)
    s, d = 256, 128
    # int8-exact Q, K: integers with a 127 in every 64-row block; no smoothing
    q = rng.integers(-127, 128, (1, 64, 1, d)).astype(np.float32) / 64
    k = rng.integers(-127, 128, (1, s, 1, d)).astype(np.float32) / 64
    q[0, 0, 0, 0] = 127 / 64
    k[0, ::64, 0, 0] = 127 / 64
    vv = oracle.e4m3fn_round(rng.standard_normal((1, s, 1, d)) * 50)
    vv[0, 0, 0, :] = 448.0
    v = vv.astype(np.float32)
    rows = np.array([[0, 0, i] for i in range(64)])
    got = oracle.attn8_emulate(q, k, v, rows, smooth=False).astype(np.float64)
    ref = oracle.attention_rows(q, k, v, rows)
    bound = _exact_operand_bound(q, k, v, rows, ref, got)
    assert np.all(np.abs(got - ref) <= bound)
    # and the bound is not trivially loose: the mean error is far below it
    assert np.mean(np.abs(got - ref)) < 0.25 * np.mean(bound)


def _outlier_case(seed, H=4, s=8192, d=128, n_rows=48):
    rng = np.random.default_rng(seed)
    def draw():
        x = rng.standard_normal((1, s, H, d))
        cols = rng.choice(H * d, size=max(1, round(0.01 * H * d)), replace=False)
        x.reshape(1, s, H * d)[:, :, cols] *= 8
        return _bf16(x)
    q, k, v = draw(), draw(), draw()
    rows = np.array([[0, h, i] for h in range(H) for i in rng.choice(s, n_rows, replace=False)])
    return q, k, v, rows


def test_accuracy_bounds_with_outliers_and_literal_scheme_is_worse():
    q, k, v, rows = _outlier_case(9)
    ref = oracle.attention_rows(q, k, v, rows)
    rel_s, cos_s = _metrics(oracle.attn8_emulate(q, k, v, rows, smooth=True), ref)
    rel_l, cos_l = _metrics(oracle.attn8_emulate(q, k, v, rows, smooth=False), ref)
    assert rel_s <= 6e-2 and cos_s >= 0.995
    assert rel_l > rel_s


def test_kv_block_size_changes_only_rounding():
    q, k, v, rows = _outlier_case(10, H=2, s=2048, n_rows=32)
    a = oracle.attn8_emulate(q, k, v, rows, kv_block=64)
    b = oracle.attn8_emulate(q, k, v, rows, kv_block=128)
    rel, _ = _metrics(a, b)
    assert rel < 2e-2


@pytest.mark.parametrize("where", ["p_scale", "v_scale"])
def test_planted_mistakes_are_caught(monkeypatch, where):
    """A dropped factor in the emulator breaks the exact-operand pin above."""
    rng = np.random.default_rng(11)
    q = _gauss((1, 64, 1, 128), 12)
    k = _gauss((1, 128, 1, 128), 13)
    v = _gauss((1, 128, 1, 128), 14)
    rows = np.array([[0, 0, i] for i in range(64)])
    ref = oracle.attention_rows(q, k, v, rows)
    if where == "p_scale":
        monkeypatch.setattr(attn8, "e4m3fn_round", lambda x: oracle.e4m3fn_round(np.asarray(x) / 256.0))
    else:
        orig = attn8._channel_e4m3
        monkeypatch.setattr(attn8, "_channel_e4m3", lambda vh: (orig(vh)[0], np.ones(vh.shape[1], np.float32)))
    bad = oracle.attn8_emulate(q, k, v, rows)
    rel, _ = _metrics(bad, ref)
    assert rel > 0.2
    del rng


def _pow2_blocks(rng, s, d, exps, sigma=20.0):
    """int8-exact operand with a distinct power-of-two scale per 64-token block: block i holds
    integer codes (one of them 127, so the block maximum is 127 * 2^exps[i]) times 2^exps[i].  The
    block quantisation then gives inv = 2^-exps[i], the codes themselves and scale 2^exps[i]."""
    x = np.clip(np.rint(rng.standard_normal((s, d)) * sigma), -127, 127)
    for i in range(-(-s // 64)):
        x[64 * i, i % d] = 127
        x[64 * i:64 * (i + 1)] *= 2.0 ** exps[i]
    return x.astype(np.float32)


def _exact_operand_case(seed):
    """Q (150 tokens: blocks of 64, 64, 22) and K (300 tokens: 4 x 64 + 44) with distinct block
    scales, V in e4m3 with every channel's maximum 448 (so its codes are exact with scale 1)."""
    rng = np.random.default_rng(seed)
    q = _pow2_blocks(rng, 150, 128, [-3, -6, -4])[None, :, None, :]
    k = _pow2_blocks(rng, 300, 128, [-5, -2, -6, -3, -4])[None, :, None, :]
    vv = oracle.e4m3fn_round(rng.standard_normal((1, 300, 1, 128)) * 60)
    vv[0, 7, 0, :] = 448.0
    return q, k, vv.astype(np.float32)


def _exact_operand_bound(q, k, v, rows, ref, got):
    """Per-element bound on |emulated - exact| when only P~ = e4m3(256 p) is rounded.  With
    P~_j = 256 p_j + delta_j, |delta_j| <= max(2^-4 * 256 p_j, 2^-10) (half a step of e4m3fn in its
    normal and subnormal range), L = sum_j p_j and O the exact output row, the emulator's
    sum_j P~_j V_j / sum_j P~_j differs from O by sum_j delta_j (V_j - O) / sum_j P~_j, so
    |O~ - O| <= sum_j |delta_j| |V_j - O| / (256 L - sum_j |delta_j|); then half a bf16 ulp."""
    out = np.empty(ref.shape)
    vv = v[0, :, 0, :].astype(np.float64)
    for r, (_, _, i) in enumerate(rows):
        s = (q[0, i, 0, :].astype(np.float64) @ k[0, :, 0, :].astype(np.float64).T) / np.sqrt(128.0)
        p = np.exp(s - s.max())
        dlt = np.maximum(2.0 ** -4 * 256.0 * p, 2.0 ** -10)
        out[r] = (dlt @ np.abs(vv - ref[r][None, :])) / (256.0 * p.sum() - dlt.sum())
    return out + 2.0 ** -8 * (np.abs(ref) + out)


def test_exact_operands_with_distinct_block_scales():
    q, k, v = _exact_operand_case(15)
    rows = np.array([[0, 0, i] for i in range(150)])
    z = attn8.attn8_quantize(q, k, v, smooth=False)[(0, 0)]
    # the quantisation reproduces the codes and the power-of-two scales exactly
    np.testing.assert_array_equal(z["q_scale"], 2.0 ** np.array([-3, -6, -4], np.float64))
    np.testing.assert_array_equal(z["k_scale"], 2.0 ** np.array([-5, -2, -6, -3, -4], np.float64))
    np.testing.assert_array_equal(z["q_codes"].astype(np.float64) * np.repeat(z["q_scale"], 64)[:150, None],
                                  q[0, :, 0, :])
    got = oracle.attn8_emulate(q, k, v, rows, smooth=False).astype(np.float64)
    ref = oracle.attention_rows(q, k, v, rows)
    bound = _exact_operand_bound(q, k, v, rows, ref, got)
    assert np.all(np.abs(got - ref) <= bound)
    assert np.mean(np.abs(got - ref)) < 0.25 * np.mean(bound)


class _RollScales:
    """attn8._block_int8 whose returned scales are shifted by one block on the n-th call of every
    quantize_head (0: Q, 1: K): a block scale applied to the neighbouring block."""

    def __init__(self, which):
        self.which, self.calls, self.orig = which, 0, attn8._block_int8

    def __call__(self, x, block):
        codes, scales = self.orig(x, block)
        hit = self.calls % 2 == self.which
        self.calls += 1
        return codes, (np.roll(scales, 1) if hit else scales)


class _NumpyWithRepeat:
    """numpy whose repeat is off by one token (the per-key scale expansion misaligned)."""

    def __getattr__(self, name):
        if name == "repeat":
            return lambda a, r: np.roll(np.repeat(a, r), 1)
        return getattr(np, name)


@pytest.mark.parametrize("where", ["q_block_scale", "k_block_scale", "k_scale_token_shift"])
def test_misaligned_block_scales_are_caught(monkeypatch, where):
    q, k, v = _exact_operand_case(15)
    rows = np.array([[0, 0, i] for i in range(150)])
    ref = oracle.attention_rows(q, k, v, rows)
    if where == "q_block_scale":
        monkeypatch.setattr(attn8, "_block_int8", _RollScales(0))
    elif where == "k_block_scale":
        monkeypatch.setattr(attn8, "_block_int8", _RollScales(1))
    else:
        monkeypatch.setattr(attn8, "np", _NumpyWithRepeat())
    bad = oracle.attn8_emulate(q, k, v, rows, smooth=False).astype(np.float64)
    assert np.any(np.abs(bad - ref) > _exact_operand_bound(q, k, v, rows, ref, bad))


def _uniform_v_case():
    q = _gauss((1, 70, 2, 128), 31, 2.0)
    k = _gauss((1, 300, 2, 128), 32, 2.0)
    row = _bf16(np.random.default_rng(33).standard_normal(128) * 3)
    v = np.broadcast_to(row, (1, 300, 2, 128)).astype(np.float32).copy()
    rows = np.array([[0, h, i] for h in range(2) for i in range(70)])
    return q, k, v, row, rows


def test_uniform_values_return_that_row_exactly():
    # every key's V row equal: sum_j P~_j v / sum_j P~_j = v whatever the weights
    q, k, v, row, rows = _uniform_v_case()
    got = oracle.attn8_emulate(q, k, v, rows)
    np.testing.assert_array_equal(got, np.broadcast_to(row, got.shape))


def test_normaliser_before_rounding_is_caught(monkeypatch):
    # the other reading (l from p before its FP8 rounding) breaks the uniform-V pin
    q, k, v, row, rows = _uniform_v_case()
    def old_normaliser(qz, qi, kv_block, block):
        qc = qz["q_codes"][qi].astype(np.float64)
        sq = qz["q_scale"][qi // block].astype(np.float64)
        kc = qz["k_codes"].astype(np.float64)
        sk = np.repeat(qz["k_scale"].astype(np.float64), block)[:kc.shape[0]]
        vt = oracle.e4m3fn_decode(qz["v_codes"])
        s = (qc @ kc.T) * sq[:, None] * sk[None, :] / np.sqrt(128.0)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        pt = oracle.e4m3fn_round(p * 256.0)
        out = (pt @ vt) * qz["v_scale"].astype(np.float64)[None, :] / (256.0 * p.sum(axis=1)[:, None])
        return oracle.bf16_round(out.astype(np.float32))

    monkeypatch.setattr(attn8, "_attend_head", old_normaliser)
    bad = oracle.attn8_emulate(q, k, v, rows)
    assert not np.array_equal(bad, np.broadcast_to(row, bad.shape))
