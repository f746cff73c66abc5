"""Exact multi-head attention in float64 -- test infrastructure (see the package docstring).

Definition followed (standard scaled dot-product attention; the Wan pages name the operation --
non-causal, full spatio-temporal, "Wan 2.1: VBench 86.22% ..." explainer, sections "先看现象" and
"干预与形式化" -- but print no formula):

    s_j = (q . k_j) / sqrt(d)          for every key j (no mask, no causality)
    m   = max_j s_j
    e_j = exp(s_j - m)
    l   = sum_j e_j
    o   = (sum_j e_j v_j) / l

Two passes over the keys (first the global maximum, then exponentials and sums), in float64, on
an exact upcast of whatever values the caller passes (for bf16 inputs: the bf16 values themselves).
Layouts: q is [b, s_q, H, d]; k and v are [b, s_kv, H, d]; the output has q's shape.
"""

import numpy as np


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _head_rows(q, k, v, bb, hh, qi):
    """Exact attention for query rows ``qi`` of one (batch, head) pair -> [len(qi), d] float64."""
    d = q.shape[-1]
    kk = _as_f64(k[bb, :, hh, :])                  # [s_kv, d]
    vv = _as_f64(v[bb, :, hh, :])                  # [s_kv, d]
    qq = _as_f64(q[bb, qi, hh, :])                 # [n, d]
    s = (qq @ kk.T) / np.sqrt(np.float64(d))       # scores, [n, s_kv]
    m = s.max(axis=1, keepdims=True)               # pass 1: global row maximum
    e = np.exp(s - m)                              # pass 2: exponentials ...
    l = e.sum(axis=1, keepdims=True)               # ... their sum ...
    return (e @ vv) / l                            # ... and the normalised weighted sum of V


def attention(q, k, v):
    """Full attention output [b, s_q, H, d] in float64."""
    b, s_q, H, d = q.shape
    assert k.shape[0] == b and k.shape[2] == H and k.shape[3] == d and v.shape == k.shape
    out = np.empty((b, s_q, H, d), dtype=np.float64)
    all_i = np.arange(s_q)
    for bb in range(b):
        for hh in range(H):
            out[bb, :, hh, :] = _head_rows(q, k, v, bb, hh, all_i)
    return out


def attention_rows(q, k, v, rows):
    """Attention for selected query rows.

    rows: integer array [n, 3] of (batch, head, query index) triples.
    Returns [n, d] float64, row r being O[rows[r,0], rows[r,2], rows[r,1], :].
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    d = q.shape[-1]
    out = np.empty((rows.shape[0], d), dtype=np.float64)
    if rows.shape[0] == 0:
        return out
    pairs = np.unique(rows[:, :2], axis=0)
    for bb, hh in pairs:
        sel = np.nonzero((rows[:, 0] == bb) & (rows[:, 1] == hh))[0]
        out[sel] = _head_rows(q, k, v, int(bb), int(hh), rows[sel, 2])
    return out


def attention_probs(q, k, bb, hh, qi):
    """The softmax weights P[i, j] for query rows ``qi`` of one (batch, head) -> [n, s_kv] float64.

    Exposed so that tests can check that every row of P sums to one.
    """
    d = q.shape[-1]
    s = (_as_f64(q[bb, qi, hh, :]) @ _as_f64(k[bb, :, hh, :]).T) / np.sqrt(np.float64(d))
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)
