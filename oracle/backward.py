"""Exact attention backward in float64 -- test infrastructure (see the package docstring).

What it computes: the gradients of the non-causal multi-head attention O = softmax(Q K^T/sqrt(d)) V
with respect to Q, K and V, given the upstream gradient dO, per (batch, head).  The pages fix the
operation and its cost -- the backward of non-causal attention is the beta = 8 term of the DiT cost
model, twice the forward's 4, and attention is 95% of training time at 1M tokens ("Wan 2.1: VBench
86.22% ..." explainer of the Wan technical report, section "先看现象") -- but print no gradient
formula.  The oracle writes out the chain rule through the row softmax:

    S    = Q K^T / sqrt(d)
    P    = softmax over each row of S
    dV   = P^T dO
    dP   = dO V^T
    D_i  = sum_j P_ij dP_ij                 (the softmax Jacobian's row term)
    dS   = P * (dP - D)                     (elementwise, D broadcast along the row)
    dQ   = dS K / sqrt(d)
    dK   = dS^T Q / sqrt(d)

and the row log-sum-exp lse_i = log sum_j exp(S_ij) (natural log), the statistic a forward pass
hands to the backward so that P_ij = exp(S_ij - lse_i).  Everything is float64 on an exact upcast of
the inputs; layouts are [b, s, H, d] for the tensors and [b, H, s_q] for lse.
"""

import numpy as np
import torch


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _head(q, k, v, do, bb, hh):
    """All gradients of one (batch, head): returns dq [s_q, d], dk [s_kv, d], dv [s_kv, d], lse [s_q]."""
    d = q.shape[-1]
    qq = _f64(q[bb, :, hh, :])
    kk = _f64(k[bb, :, hh, :])
    vv = _f64(v[bb, :, hh, :])
    gg = _f64(do[bb, :, hh, :])
    inv = 1.0 / np.sqrt(np.float64(d))
    s = (qq @ kk.T) * inv                             # [s_q, s_kv]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l                                         # softmax rows
    lse = (m + np.log(l))[:, 0]
    dv = p.T @ gg                                     # dV = P^T dO
    dp = gg @ vv.T                                    # dP = dO V^T
    dd = (p * dp).sum(axis=1, keepdims=True)          # D_i = sum_j P_ij dP_ij
    ds = p * (dp - dd)                                # dS = P * (dP - D)
    dq = (ds @ kk) * inv
    dk = (ds.T @ qq) * inv
    return dq, dk, dv, lse


def attention_backward(q, k, v, do):
    """Full gradients (dq, dk, dv) in float64 with the shapes of q, k, v, plus lse [b, H, s_q]."""
    b, s_q, H, d = q.shape
    s_kv = k.shape[1]
    assert k.shape == (b, s_kv, H, d) and v.shape == k.shape and do.shape == q.shape
    dq = np.empty((b, s_q, H, d))
    dk = np.empty((b, s_kv, H, d))
    dv = np.empty((b, s_kv, H, d))
    lse = np.empty((b, H, s_q))
    for bb in range(b):
        for hh in range(H):
            gq, gk, gv, ls = _head(q, k, v, do, bb, hh)
            dq[bb, :, hh, :] = gq
            dk[bb, :, hh, :] = gk
            dv[bb, :, hh, :] = gv
            lse[bb, hh, :] = ls
    return dq, dk, dv, lse


def _row_terms(q, k, v, do, bb, hh, qi):
    """P rows, dP rows and the scaled score rows of query rows qi of one (batch, head)."""
    d = q.shape[-1]
    kk = _f64(k[bb, :, hh, :])
    inv = 1.0 / np.sqrt(np.float64(d))
    s = (_f64(q[bb, qi, hh, :]) @ kk.T) * inv
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    dp = _f64(do[bb, qi, hh, :]) @ _f64(v[bb, :, hh, :]).T
    return p, dp, (m + np.log(l))[:, 0], kk, inv


def lse_rows(q, k, rows):
    """Row log-sum-exp of the scaled scores for (batch, head, query) triples -> [n] float64."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    d = q.shape[-1]
    out = np.empty(rows.shape[0])
    for r, (bb, hh, i) in enumerate(rows):
        s = (_f64(q[bb, i, hh, :]) @ _f64(k[bb, :, hh, :]).T) / np.sqrt(np.float64(d))
        m = s.max()
        out[r] = m + np.log(np.exp(s - m).sum())
    return out


def dq_rows(q, k, v, do, rows):
    """dQ for (batch, head, query) triples -> [n, d] float64.  Each row needs only its own softmax
    row, so this runs at any sequence length in O(s_kv * d) per row."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], q.shape[-1]))
    if rows.shape[0] == 0:
        return out
    pairs = np.unique(rows[:, :2], axis=0)
    for bb, hh in pairs:
        sel = np.nonzero((rows[:, 0] == bb) & (rows[:, 1] == hh))[0]
        p, dp, _, kk, inv = _row_terms(q, k, v, do, int(bb), int(hh), rows[sel, 2])
        dd = (p * dp).sum(axis=1, keepdims=True)
        out[sel] = ((p * (dp - dd)) @ kk) * inv
    return out


def _query_row_stats(qq, kk, vv, gg, inv, chunk=1024):
    """lse_i and D_i = sum_j P_ij dP_ij of every query row of one head (float64 torch CPU tensors
    qq, gg [s_q, d] and kk, vv [s_kv, d]), in chunks of query rows so that no full [s_q, s_kv]
    matrix is held.  torch's CPU ops here only spread the elementwise work over the host's cores."""
    s_q = qq.shape[0]
    lse = torch.empty(s_q, dtype=torch.float64)
    dd = torch.empty(s_q, dtype=torch.float64)
    for i0 in range(0, s_q, chunk):
        i1 = min(i0 + chunk, s_q)
        s = (qq[i0:i1] @ kk.T) * inv
        m = s.max(dim=1, keepdim=True).values
        e = torch.exp(s - m)
        l = e.sum(dim=1, keepdim=True)
        dp = gg[i0:i1] @ vv.T
        lse[i0:i1] = (m + torch.log(l))[:, 0]
        dd[i0:i1] = ((e / l) * dp).sum(dim=1)
    return lse, dd


def dkdv_rows(q, k, v, do, rows):
    """dK and dV for (batch, head, key index) triples -> (dk [n, d], dv [n, d]) float64.

    Key row j of a head gathers over every query row i:  P_ij = exp(S_ij - lse_i),
    dV_j = sum_i P_ij dO_i,  dS_ij = P_ij (dP_ij - D_i),  dK_j = sum_i dS_ij Q_i / sqrt(d),
    with lse_i and D_i taken from the whole query row first (one pass over the head's keys per
    head that the triples touch), so a few key rows cost about one forward of their heads."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    d = q.shape[-1]
    out_k = np.empty((rows.shape[0], d))
    out_v = np.empty((rows.shape[0], d))
    if rows.shape[0] == 0:
        return out_k, out_v
    inv = 1.0 / np.sqrt(np.float64(d))
    t64 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    for bb, hh in np.unique(rows[:, :2], axis=0):
        bb, hh = int(bb), int(hh)
        sel = np.nonzero((rows[:, 0] == bb) & (rows[:, 1] == hh))[0]
        qq, kk, vv, gg = (t64(x[bb, :, hh, :]) for x in (q, k, v, do))
        lse, dd = _query_row_stats(qq, kk, vv, gg, inv)
        j = torch.from_numpy(rows[sel, 2])
        p = torch.exp((qq @ kk[j].T) * inv - lse[:, None])     # [s_q, n]: column j of P
        dp = gg @ vv[j].T                                      # column j of dP
        ds = p * (dp - dd[:, None])                            # column j of dS
        out_v[sel] = (p.T @ gg).numpy()
        out_k[sel] = ((ds.T @ qq) * inv).numpy()
    return out_k, out_v
