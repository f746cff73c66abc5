"""Parity of the bf16 attention backward (through the C ABI) with the fp64 oracle, on the GPU.

The forward that feeds it (wan_attn_fwd_lse) is checked first: its row log-sum-exp against the
oracle's, its output against wan_attn_fwd's (bit for bit).  Gradients: small and ragged shapes
compare every element of dQ, dK and dV with the oracle's exact gradients; the Wan-1.3B 480p and
Wan-14B 720p shapes compare sampled dQ rows, and 64 sampled key rows of dK and dV per checked head
(every head at 480p, two at 720p; each key row's gradient gathers every query row of its head), with
the oracle, and check dK and dV over the whole tensors through identities that hold at any size
(sum_j dK_j = 0, sum_j dV_j = sum_i dO_i).
Bounds, per tensor over all checked elements: rel-L2 <= BWD_REL_L2 and max-abs <= BWD_MAX_REL times
the largest magnitude of the exact gradient.
"""

import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_wan_amd as wan
import wan_inputs
from _util import BWD_MAX_REL, BWD_REL_L2, ensure_built, metrics, to_np

pytestmark = pytest.mark.gpu

LSE_MAX_ABS = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _inputs(b, H, s_q, s_kv, seed, sigma=1.0):
    q, k, v = wan_inputs.random_qkv(b, H, s_q, s_kv, seed, sigma=sigma, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(seed + 7)
    d_o = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, d_o


def _check_grad(name, got, ref):
    """rel-L2 and scaled max-abs; an exact gradient that is zero (one key: softmax is constant)
    is checked against the floor 1e-2 of the scale (inputs are N(0, 1))."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = max(float(np.max(np.abs(ref))), 1e-2)
    mx = float(np.max(np.abs(got - ref)))
    if np.linalg.norm(ref) > 1e-12:
        rel, _, _ = metrics(got, ref)
    else:
        rel = 0.0
    print(f"  {name}: rel-L2 {rel:.2e}  max-abs {mx:.2e} (scale {scale:.2e})", flush=True)
    assert rel <= BWD_REL_L2 and mx <= BWD_MAX_REL * scale, (name, rel, mx, scale)


def _full_case(b, H, s_q, s_kv, seed, sigma=1.0):
    print(f"backward b={b} H={H} s_q={s_q} s_kv={s_kv} sigma={sigma}", flush=True)
    q, k, v, d_o = _inputs(b, H, s_q, s_kv, seed, sigma)
    o, lse = wan.attention_with_lse(q, k, v)
    dq, dk, dv = wan.attention_backward(q, k, v, o, lse, d_o)
    torch.cuda.synchronize()
    rq, rk, rv, rlse = oracle.attention_backward(to_np(q), to_np(k), to_np(v), to_np(d_o))
    assert np.max(np.abs(to_np(lse) - rlse)) <= LSE_MAX_ABS
    _check_grad("dq", to_np(dq), rq)
    _check_grad("dk", to_np(dk), rk)
    _check_grad("dv", to_np(dv), rv)


@pytest.mark.parametrize("b,H,s_q,s_kv", [(1, 2, 600, 4000), (2, 3, 513, 700), (1, 40, 300, 512)])
def test_forward_lse(b, H, s_q, s_kv):
    # (1, 2, 600, 4000) runs the split key-range path, the others the one-pass kernel
    q, k, v, _ = _inputs(b, H, s_q, s_kv, 5)
    o, lse = wan.attention_with_lse(q, k, v)
    o_plain = wan.attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)
    rows = np.array([[bb, hh, i] for bb in range(b) for hh in range(H) for i in range(s_q)])
    ref = oracle.lse_rows(to_np(q), to_np(k), rows)
    got = to_np(lse).reshape(-1)
    assert np.max(np.abs(got - ref)) <= LSE_MAX_ABS


@pytest.mark.parametrize("s_q,s_kv", [(1, 1), (1, 200), (64, 64), (65, 63), (127, 129), (129, 127), (300, 1),
                                      (200, 300), (256, 256), (257, 320), (511, 257)])
def test_backward_ragged(s_q, s_kv):
    _full_case(1, 2, s_q, s_kv, seed=3000 + 7 * s_q + s_kv)


@pytest.mark.parametrize("b,H,s_q,s_kv", [(2, 3, 300, 500), (1, 4, 1000, 1000), (1, 2, 2000, 150)])
def test_backward_batches_heads(b, H, s_q, s_kv):
    _full_case(b, H, s_q, s_kv, seed=b * 1000 + H * 100 + s_q)


@pytest.mark.parametrize("sigma", [2.0, 3.0])
def test_backward_peaky(sigma):
    """Q, K, V with N(0, sigma^2) entries: the scores have standard deviation sigma^2, so one key
    holds 43% (sigma 2) or 75% (sigma 3) of a row's softmax on average.  The dK/dV kernel passes
    P * 2^15 between its waves as a half: here the largest P bring that near its top (32,768) while
    most P fall far below the half's normal range.  (The error grows with the peak: D = dO . O is
    taken from the bf16 O, and dP - D cancels at the dominant key; a model of that arithmetic in
    numpy gives rel-L2 4e-3 and 6e-3 for dQ.)"""
    _full_case(1, 2, 700, 900, seed=int(100 * sigma), sigma=sigma)


@pytest.fixture(scope="module")
def wan13b_grads():
    """Wan2.1-1.3B at 480p, 81 frames: 12 heads x 32,760 tokens, one batch entry."""
    b, H, s = 1, 12, 32760
    print(f"backward b={b} H={H} s={s}", flush=True)
    q, k, v, d_o = _inputs(b, H, s, s, 77)
    o, lse = wan.attention_with_lse(q, k, v)
    dq, dk, dv = wan.attention_backward(q, k, v, o, lse, d_o)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, d_o=d_o, dq=dq, dk=dk, dv=dv)


@pytest.fixture(scope="module")
def wan14b_grads():
    """The backward the bench times: Wan-14B-shaped 720p, 81 frames, b=2, with the bench's own inputs
    (make_qkv of the workload, dO from a generator seeded with the workload seed + 11)."""
    w = wan_inputs.WORKLOADS["wan14b_720p81f_self"]
    print(f"backward b={w.batch} H={w.heads} s={w.s_q}", flush=True)
    q, k, v = wan_inputs.make_qkv(w, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(w.seed + 11)
    d_o = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    o, lse = wan.attention_with_lse(q, k, v)
    dq, dk, dv = wan.attention_backward(q, k, v, o, lse, d_o)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, d_o=d_o, dq=dq, dk=dk, dv=dv, w=w)


def test_backward_wan_sized(wan13b_grads):
    g = wan13b_grads
    q, k, v, d_o, dq, dk, dv = (g[n] for n in ("q", "k", "v", "d_o", "dq", "dk", "dv"))
    b, s, H, _ = q.shape
    rng = np.random.default_rng(78)
    rows = np.stack([np.zeros(48, np.int64), rng.integers(0, H, 48), rng.integers(0, s, 48)], 1)
    rows[0] = [0, 0, 0]
    rows[1] = [0, H - 1, s - 1]
    qn, kn, vn, gn = to_np(q), to_np(k), to_np(v), to_np(d_o)
    ref = oracle.dq_rows(qn, kn, vn, gn, rows)
    got = to_np(dq[0, rows[:, 2], rows[:, 1], :])
    _check_grad("dq rows", got, ref)
    # identities: sum over keys of dK is zero; sum over keys of dV is the sum over queries of dO
    dk64 = dk.double().sum(dim=1)
    scale = dk.double().abs().sum(dim=1)
    assert float((dk64.abs() / scale).max()) < 2e-2
    sum_dv = dv.double().sum(dim=1)
    sum_do = d_o.double().sum(dim=1)
    rel = float((sum_dv - sum_do).norm() / sum_do.norm())
    print(f"  sum dK / sum |dK| max {float((dk64.abs() / scale).max()):.2e}, sum dV vs sum dO rel {rel:.2e}")
    assert rel < 1e-2


def _key_rows(s, n, seed):
    """n distinct key rows of a head, the first and the last among them."""
    j = np.random.default_rng(seed).choice(np.arange(1, s - 1), n - 2, replace=False)
    return np.sort(np.concatenate([[0, s - 1], j]))


def _check_key_rows(g, pairs, n_rows, seed):
    """dK and dV of sampled key rows of the (batch, head) pairs against the oracle's chain rule per key
    row (every query row of the head enters each key row's gradient), on host copies of those heads."""
    q, k, v, d_o, dk, dv = (g[n] for n in ("q", "k", "v", "d_o", "dk", "dv"))
    s = k.shape[1]
    got_k, got_v, ref_k, ref_v = [], [], [], []
    for bb, hh in pairs:
        head = [t[bb, :, hh, :].double().cpu().numpy()[None, :, None, :] for t in (q, k, v, d_o)]
        j = _key_rows(s, n_rows, seed + 97 * bb + hh)
        rows = np.stack([np.zeros_like(j), np.zeros_like(j), j], 1)
        rk, rv = oracle.dkdv_rows(*head, rows)
        ref_k.append(rk)
        ref_v.append(rv)
        got_k.append(dk[bb, torch.as_tensor(j, device=dk.device), hh, :].double().cpu().numpy())
        got_v.append(dv[bb, torch.as_tensor(j, device=dv.device), hh, :].double().cpu().numpy())
        print(f"  head (b={bb}, h={hh}): {len(j)} key rows", flush=True)
    _check_grad("dk rows", np.concatenate(got_k), np.concatenate(ref_k))
    _check_grad("dv rows", np.concatenate(got_v), np.concatenate(ref_v))


@pytest.mark.parametrize("heads", [(0, 1, 2, 3), (4, 5, 6, 7), (8, 9, 10, 11)])
def test_backward_wan_sized_key_rows(wan13b_grads, heads):
    # 64 key rows (the first and last included) of every head, element by element
    _check_key_rows(wan13b_grads, [(0, h) for h in heads], 64, 79)


def test_backward_wan14b_720p_bench_inputs(wan14b_grads):
    g = wan14b_grads
    q, k, v, d_o, dq, dk, dv = (g[n] for n in ("q", "k", "v", "d_o", "dq", "dk", "dv"))
    w = g["w"]
    b, H, s = w.batch, w.heads, w.s_q
    # sampled dQ rows on 4 heads of both batch entries (the first and last rows among them), against
    # the oracle on host copies of those heads only
    heads = [0, 13, 27, H - 1]
    rng = np.random.default_rng(w.seed + 12)
    rows = np.stack([rng.integers(0, b, 32), rng.integers(0, len(heads), 32), rng.integers(0, s, 32)], 1)
    rows[0] = [0, 0, 0]
    rows[1] = [b - 1, len(heads) - 1, s - 1]
    hsel = torch.tensor(heads, device="cuda")
    sub = [t.index_select(2, hsel).double().cpu().numpy() for t in (q, k, v, d_o)]
    ref = oracle.dq_rows(*sub, rows)
    got = dq.index_select(2, hsel).double().cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]]
    _check_grad("dq rows", got, ref)
    # identities over the whole tensors: sum over keys of dK is zero; sum over keys of dV is the sum
    # over queries of dO (per batch entry, head and channel)
    dk_sum = dk.double().sum(dim=1)
    dk_scale = dk.double().abs().sum(dim=1)
    ratio = float((dk_sum.abs() / dk_scale).max())
    rel = float((dv.double().sum(dim=1) - d_o.double().sum(dim=1)).norm() / d_o.double().sum(dim=1).norm())
    print(f"  sum dK / sum |dK| max {ratio:.2e}, sum dV vs sum dO rel {rel:.2e}", flush=True)
    assert ratio < 2e-2 and rel < 1e-2


@pytest.mark.parametrize("pair", [(0, 0), (1, 39)])
def test_backward_wan14b_720p_key_rows(wan14b_grads, pair):
    # 64 key rows (the first and last included) of the first head of batch entry 0 and the last head
    # of batch entry 1, element by element
    _check_key_rows(wan14b_grads, [pair], 64, 80)
