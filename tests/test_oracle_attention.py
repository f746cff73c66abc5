"""Pins of the exact fp64 attention oracle against things other than itself.

* brute force: a scalar Python triple loop with exactly-rounded sums (math.fsum) on tiny inputs;
* a library routine: torch's scaled_dot_product_attention in float64 on the CPU (same definition,
  default scale 1/sqrt(d));
* closed forms: one key, zero query, two keys in one dimension (logistic weights), identical V rows;
* invariants: rows of P sum to one, joint permutation of (K, V) rows, K + 1 u^T, affine V;
* planted mistakes: the pins above must catch a wrong scale or a wrong exponential base.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.exact as oatt


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def brute_force(q, k, v):
    """Scalar loops; every sum is math.fsum (correctly rounded)."""
    b, s_q, H, d = q.shape
    s_kv = k.shape[1]
    out = np.zeros((b, s_q, H, d))
    for bb in range(b):
        for hh in range(H):
            for i in range(s_q):
                s = [math.fsum(float(q[bb, i, hh, c]) * float(k[bb, j, hh, c]) for c in range(d))
                     / math.sqrt(d) for j in range(s_kv)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                l = math.fsum(e)
                for c in range(d):
                    out[bb, i, hh, c] = math.fsum(e[j] * float(v[bb, j, hh, c])
                                                  for j in range(s_kv)) / l
    return out


@pytest.mark.parametrize("b,H,s_q,s_kv,d", [
    (1, 1, 1, 1, 1), (1, 2, 3, 5, 2), (2, 1, 4, 7, 3), (1, 2, 5, 16, 128), (2, 2, 16, 9, 128)])
def test_brute_force(b, H, s_q, s_kv, d):
    q = _rand((b, s_q, H, d), 1, 2.0)
    k = _rand((b, s_kv, H, d), 2, 2.0)
    v = _rand((b, s_kv, H, d), 3)
    got = oracle.attention(q, k, v)
    ref = brute_force(q, k, v)
    assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("b,H,s_q,s_kv,d", [(1, 3, 257, 129, 128), (2, 2, 65, 300, 128), (1, 1, 8, 1, 16)])
def test_against_sdpa_fp64(b, H, s_q, s_kv, d):
    q = _rand((b, s_q, H, d), 11)
    k = _rand((b, s_kv, H, d), 12)
    v = _rand((b, s_kv, H, d), 13)
    got = oracle.attention(q, k, v)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v)).permute(0, 2, 1, 3).numpy()
    rel = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    assert rel <= 1e-12


def test_rows_match_full():
    q, k, v = _rand((2, 40, 3, 128), 21), _rand((2, 70, 3, 128), 22), _rand((2, 70, 3, 128), 23)
    full = oracle.attention(q, k, v)
    rows = np.array([[0, 0, 0], [1, 2, 39], [0, 1, 17], [1, 0, 5], [0, 1, 3]])
    got = oracle.attention_rows(q, k, v, rows)
    for r, (bb, hh, i) in enumerate(rows):
        np.testing.assert_allclose(got[r], full[bb, i, hh], rtol=0, atol=1e-14)
    assert oracle.attention_rows(q, k, v, np.zeros((0, 3), np.int64)).shape == (0, 128)


def test_single_key_returns_its_value_row():
    q, k, v = _rand((1, 9, 2, 128), 31, 5.0), _rand((1, 1, 2, 128), 32), _rand((1, 1, 2, 128), 33)
    out = oracle.attention(q, k, v)
    np.testing.assert_array_equal(out, np.broadcast_to(v, out.shape))


def test_zero_query_gives_mean_of_values():
    q = np.zeros((1, 3, 1, 128))
    k, v = _rand((1, 50, 1, 128), 41, 3.0), _rand((1, 50, 1, 128), 42)
    out = oracle.attention(q, k, v)
    np.testing.assert_allclose(out[0, :, 0], np.broadcast_to(v[0, :, 0].mean(0), (3, 128)), rtol=0, atol=1e-14)


def test_two_keys_one_dim_logistic():
    rng = np.random.default_rng(5)
    for _ in range(20):
        qv, k0, k1, v0, v1 = rng.standard_normal(5) * 3
        q = np.array(qv).reshape(1, 1, 1, 1)
        k = np.array([k0, k1]).reshape(1, 2, 1, 1)
        v = np.array([v0, v1]).reshape(1, 2, 1, 1)
        delta = qv * (k0 - k1)            # d = 1, scale 1/sqrt(1)
        w0 = 1.0 / (1.0 + math.exp(-delta))
        expect = w0 * v0 + (1 - w0) * v1
        got = oracle.attention(q, k, v)[0, 0, 0, 0]
        assert abs(got - expect) <= 1e-14 * max(1.0, abs(v0), abs(v1))


def test_identical_value_rows():
    q, k = _rand((1, 20, 2, 128), 51), _rand((1, 33, 2, 128), 52)
    row = _rand((128,), 53)
    v = np.broadcast_to(row, (1, 33, 2, 128)).copy()
    out = oracle.attention(q, k, v)
    np.testing.assert_allclose(out, np.broadcast_to(row, out.shape), rtol=0, atol=1e-14)


def test_probability_rows_sum_to_one():
    q, k = _rand((1, 17, 2, 128), 61, 4.0), _rand((1, 300, 2, 128), 62, 4.0)
    p = oracle.attention_probs(q, k, 0, 1, np.arange(17))
    assert p.shape == (17, 300)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_key_value_permutation_invariance():
    q, k, v = _rand((2, 30, 2, 128), 71), _rand((2, 90, 2, 128), 72), _rand((2, 90, 2, 128), 73)
    perm = np.random.default_rng(74).permutation(90)
    a = oracle.attention(q, k, v)
    b = oracle.attention(q, k[:, perm], v[:, perm])
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_key_shift_invariance():
    q, k, v = _rand((1, 25, 1, 128), 81), _rand((1, 60, 1, 128), 82), _rand((1, 60, 1, 128), 83)
    u = _rand((128,), 84)
    a = oracle.attention(q, k, v)
    b = oracle.attention(q, k + u, v)          # adds q.u / sqrt(d) to every score of a row
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_affine_values():
    q, k, v = _rand((1, 25, 2, 128), 91), _rand((1, 60, 2, 128), 92), _rand((1, 60, 2, 128), 93)
    a, c = -2.5, _rand((128,), 94)
    np.testing.assert_allclose(oracle.attention(q, k, a * v + c), a * oracle.attention(q, k, v) + c,
                               rtol=0, atol=1e-12)


class _NumpyWithMistake:
    """numpy with one function replaced, to plant a mistake in the oracle."""

    def __init__(self, **over):
        self._over = over

    def __getattr__(self, name):
        return self._over.get(name, getattr(np, name))


@pytest.mark.parametrize("mistake", [
    dict(sqrt=lambda x: x),                      # scale 1/d instead of 1/sqrt(d)
    dict(exp=lambda x: np.exp2(x)),              # wrong exponential base
])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    q, k, v = _rand((1, 4, 1, 8), 101, 2.0), _rand((1, 6, 1, 8), 102, 2.0), _rand((1, 6, 1, 8), 103)
    ref = brute_force(q, k, v)
    monkeypatch.setattr(oatt, "np", _NumpyWithMistake(**mistake))
    bad = oatt.attention(q, k, v)
    assert np.max(np.abs(bad - ref)) > 1e-6


def test_probabilities_brute_force():
    q, k = _rand((1, 4, 2, 6), 111, 2.0), _rand((1, 9, 2, 6), 112, 2.0)
    p = oracle.attention_probs(q, k, 0, 1, np.arange(4))
    for i in range(4):
        s = [math.fsum(float(q[0, i, 1, c]) * float(k[0, j, 1, c]) for c in range(6)) / math.sqrt(6)
             for j in range(9)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        l = math.fsum(e)
        for j in range(9):
            assert abs(p[i, j] - e[j] / l) <= 1e-14


def test_probabilities_times_values_give_the_output():
    # P V is the attention output, which the brute-force and SDPA pins fix independently
    q, k, v = _rand((2, 33, 3, 128), 121, 2.0), _rand((2, 70, 3, 128), 122, 2.0), _rand((2, 70, 3, 128), 123)
    out = oracle.attention(q, k, v)
    for bb, hh in ((0, 0), (1, 2)):
        p = oracle.attention_probs(q, k, bb, hh, np.arange(33))
        np.testing.assert_allclose(p @ v[bb, :, hh, :], out[bb, :, hh, :], rtol=0, atol=1e-13)


@pytest.mark.parametrize("mistake", [
    dict(sqrt=lambda x: 1.0),                    # 1/sqrt(d) dropped
    dict(sqrt=lambda x: x),                      # scale 1/d instead of 1/sqrt(d)
    dict(exp=lambda x: np.exp2(x)),              # wrong exponential base
])
def test_probabilities_planted_mistakes_are_caught(monkeypatch, mistake):
    q, k, v = _rand((1, 5, 1, 16), 131, 2.0), _rand((1, 7, 1, 16), 132, 2.0), _rand((1, 7, 1, 16), 133)
    out = oracle.attention(q, k, v)          # taken before the mistake is planted
    monkeypatch.setattr(oatt, "np", _NumpyWithMistake(**mistake))
    bad = oatt.attention_probs(q, k, 0, 0, np.arange(5))
    assert np.max(np.abs(bad @ v[0, :, 0, :] - out[0, :, 0, :])) > 1e-6
