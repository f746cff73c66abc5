"""Pins of the float64 attention backward oracle against things other than itself.

* automatic differentiation: torch autograd in float64 on the CPU through the forward definition
  softmax(q k^T / sqrt(d)) v -- it differentiates the forward, not the oracle's written-out chain rule;
* finite differences: central differences of sum(O * dO) on tiny inputs, element by element;
* brute force: the row log-sum-exp with exactly rounded sums (math.fsum);
* identities that hold at any size: sum_j dK_j = 0 (every row of dS sums to zero), sum_j dV_j =
  sum_i dO_i (every row of P sums to one); one key, or identical value rows, give dQ = dK = 0;
* planted mistakes: a flipped sign of the row term, a dropped 1/sqrt(d), a transposed dS, and a row
  term without P must each fail the autograd pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.backward as obw


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _inputs(b, H, s_q, s_kv, d, seed, scale=1.0):
    return (_rand((b, s_q, H, d), seed, scale), _rand((b, s_kv, H, d), seed + 1, scale),
            _rand((b, s_kv, H, d), seed + 2), _rand((b, s_q, H, d), seed + 3))


def _autograd(q, k, v, do):
    """Gradients of sum(O * dO) by torch autograd, float64, forward written from the definition."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    d = q.shape[-1]
    # [b, s, H, d] -> [b, H, s, d]
    qh, kh, vh = (t.permute(0, 2, 1, 3) for t in (tq, tk, tv))
    s = qh @ kh.transpose(-1, -2) / math.sqrt(d)
    o = torch.softmax(s, dim=-1) @ vh
    o.permute(0, 2, 1, 3).backward(torch.tensor(do, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("b,H,s_q,s_kv,d,scale", [
    (1, 1, 1, 1, 1, 1.0), (1, 2, 3, 5, 4, 1.0), (2, 1, 7, 4, 3, 2.0), (1, 2, 16, 9, 128, 1.0),
    (2, 2, 33, 70, 128, 1.0), (1, 1, 20, 20, 128, 3.0)])
def test_against_autograd(b, H, s_q, s_kv, d, scale):
    q, k, v, do = _inputs(b, H, s_q, s_kv, d, 10 * s_q + s_kv, scale)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do)
    aq, ak, av = _autograd(q, k, v, do)
    for got, ref in ((dq, aq), (dk, ak), (dv, av)):
        assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_finite_differences():
    q, k, v, do = _inputs(1, 1, 3, 4, 2, 7, 1.5)

    def loss(qq, kk, vv):
        return float((oracle.attention(qq, kk, vv) * do).sum())

    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do)
    h = 1e-6
    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in np.ndindex(x.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[idx]) < 1e-7


def test_lse_brute_force():
    q, k, _, _ = _inputs(2, 2, 5, 9, 6, 41, 2.0)
    _, _, _, lse = oracle.attention_backward(q, k, k, q)
    for bb in range(2):
        for hh in range(2):
            for i in range(5):
                s = [math.fsum(q[bb, i, hh, c] * k[bb, j, hh, c] for c in range(6)) / math.sqrt(6)
                     for j in range(9)]
                m = max(s)
                ref = m + math.log(math.fsum(math.exp(x - m) for x in s))
                assert abs(lse[bb, hh, i] - ref) < 1e-13


def test_row_functions_match_full():
    q, k, v, do = _inputs(2, 3, 40, 30, 128, 61)
    dq, _, _, lse = oracle.attention_backward(q, k, v, do)
    rows = np.array([[0, 0, 0], [1, 2, 39], [0, 1, 17], [1, 0, 5], [1, 2, 0]])
    got = oracle.dq_rows(q, k, v, do, rows)
    for r, (bb, hh, i) in enumerate(rows):
        assert np.allclose(got[r], dq[bb, i, hh], rtol=1e-12, atol=1e-14)
    assert np.allclose(oracle.lse_rows(q, k, rows), [lse[bb, hh, i] for bb, hh, i in rows], rtol=1e-14)
    assert oracle.dq_rows(q, k, v, do, np.zeros((0, 3), np.int64)).shape == (0, 128)


def test_identities():
    q, k, v, do = _inputs(2, 2, 25, 37, 128, 71)
    _, dk, dv, _ = oracle.attention_backward(q, k, v, do)
    # rows of dS sum to zero, so the keys' gradients cancel; rows of P sum to one
    assert np.abs(dk.sum(axis=1)).max() < 1e-12
    assert np.allclose(dv.sum(axis=1), do.sum(axis=1), rtol=1e-12, atol=1e-12)


def test_single_key():
    q, k, v, do = _inputs(1, 2, 6, 1, 128, 81)
    dq, dk, dv, lse = oracle.attention_backward(q, k, v, do)
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() < 1e-15
    assert np.allclose(dv[:, 0], do.sum(axis=1), rtol=1e-14)
    s = np.einsum("bihc,bjhc->bhij", q, k)[..., 0] / math.sqrt(128)
    assert np.allclose(lse, s, rtol=1e-14)


def test_identical_value_rows():
    q, k, v, do = _inputs(1, 1, 9, 12, 16, 91)
    v[:] = v[:, :1]
    dq, dk, _, _ = oracle.attention_backward(q, k, v, do)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14


class _Mutant:
    """obw._head with one planted mistake."""

    def __init__(self, kind):
        self.kind = kind

    def __call__(self, q, k, v, do, bb, hh):
        d = q.shape[-1]
        qq, kk, vv, gg = (np.asarray(x[bb, :, hh, :], np.float64) for x in (q, k, v, do))
        inv = 1.0 / np.sqrt(d)
        s = (qq @ kk.T) * inv
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dv = p.T @ gg
        dp = gg @ vv.T
        dd = (p * dp).sum(axis=1, keepdims=True) if self.kind != "row_term_without_p" else dp.sum(axis=1, keepdims=True)
        ds = p * (dp + dd) if self.kind == "sign" else p * (dp - dd)
        dq = (ds @ kk) * (1.0 if self.kind == "scale" else inv)
        dk = ((ds if self.kind == "transpose" else ds.T) @ qq) * inv
        return dq, dk, dv, np.zeros(q.shape[1])


@pytest.mark.parametrize("kind", ["sign", "scale", "transpose", "row_term_without_p"])
def test_planted_mistakes_are_caught(monkeypatch, kind):
    q, k, v, do = _inputs(1, 1, 8, 8, 16, 101, 1.5)
    aq, ak, _ = _autograd(q, k, v, do)
    monkeypatch.setattr(obw, "_head", _Mutant(kind))
    dq, dk, _, _ = obw.attention_backward(q, k, v, do)
    assert max(np.abs(dq - aq).max(), np.abs(dk - ak).max()) > 1e-6


@pytest.mark.parametrize("b,H,s_q,s_kv,d", [(2, 3, 40, 30, 128), (1, 2, 129, 70, 128), (1, 1, 1, 5, 16),
                                            (1, 1, 7, 1, 8)])
def test_key_row_functions_match_full_and_autograd(b, H, s_q, s_kv, d):
    q, k, v, do = _inputs(b, H, s_q, s_kv, d, 500 + s_q)
    _, dk, dv, _ = oracle.attention_backward(q, k, v, do)
    _, ak, av = _autograd(q, k, v, do)
    rng = np.random.default_rng(501)
    n = 12
    rows = np.stack([rng.integers(0, b, n), rng.integers(0, H, n), rng.integers(0, s_kv, n)], 1)
    rows[0] = [0, 0, 0]
    rows[1] = [b - 1, H - 1, s_kv - 1]
    gk, gv = oracle.dkdv_rows(q, k, v, do, rows)
    for r, (bb, hh, j) in enumerate(rows):
        assert np.allclose(gk[r], dk[bb, j, hh], rtol=1e-11, atol=1e-13)
        assert np.allclose(gv[r], dv[bb, j, hh], rtol=1e-11, atol=1e-13)
        assert np.allclose(gk[r], ak[bb, j, hh], rtol=1e-10, atol=1e-12)
        assert np.allclose(gv[r], av[bb, j, hh], rtol=1e-10, atol=1e-12)
    ek, ev = oracle.dkdv_rows(q, k, v, do, np.zeros((0, 3), np.int64))
    assert ek.shape == (0, d) and ev.shape == (0, d)


def test_key_row_statistics_chunks():
    # the query-row statistics are taken in chunks of rows; a chunk boundary inside the head
    # (and a partial last chunk) must not change them
    q, k, v, do = _inputs(1, 1, 1100, 50, 32, 511)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x[0, :, 0, :], np.float64))
    lse, dd = obw._query_row_stats(t(q), t(k), t(v), t(do), 1.0 / math.sqrt(32), chunk=512)
    _, _, _, rlse = oracle.attention_backward(q, k, v, do)
    assert np.allclose(lse.numpy(), rlse[0, 0], rtol=1e-13)
    p = oracle.attention_probs(q, k, 0, 0, np.arange(1100))
    dp = do[0, :, 0, :] @ v[0, :, 0, :].T
    assert np.allclose(dd.numpy(), (p * dp).sum(axis=1), rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("kind", ["lse_shift", "no_row_term", "no_scale"])
def test_key_row_planted_mistakes_are_caught(monkeypatch, kind):
    q, k, v, do = _inputs(1, 2, 20, 24, 16, 521, 1.5)
    _, ak, av = _autograd(q, k, v, do)
    rows = np.array([[0, h, j] for h in range(2) for j in range(24)])
    orig = obw._query_row_stats
    if kind == "lse_shift":        # P built from a wrong normaliser
        monkeypatch.setattr(obw, "_query_row_stats", lambda *a, **kw: (orig(*a, **kw)[0] + 0.5, orig(*a, **kw)[1]))
    elif kind == "no_row_term":    # dS without the softmax Jacobian's row term
        monkeypatch.setattr(obw, "_query_row_stats", lambda *a, **kw: (orig(*a, **kw)[0], 0 * orig(*a, **kw)[1]))
    else:                          # 1/sqrt(d) dropped everywhere
        monkeypatch.setattr(obw, "np", _NumpyWithSqrt(lambda x: np.ones_like(np.asarray(x, np.float64))))
    gk, gv = obw.dkdv_rows(q, k, v, do, rows)
    ref_k = ak[0][rows[:, 2], rows[:, 1]]
    ref_v = av[0][rows[:, 2], rows[:, 1]]
    assert max(np.abs(gk - ref_k).max(), np.abs(gv - ref_v).max()) > 1e-6


class _NumpyWithSqrt:
    """numpy with sqrt replaced, to plant a mistake in the oracle."""

    def __init__(self, sqrt):
        self._sqrt = sqrt

    def __getattr__(self, name):
        return self._sqrt if name == "sqrt" else getattr(np, name)
