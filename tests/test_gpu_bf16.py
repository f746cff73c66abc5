"""Parity of the bf16 HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Bounds (both on all checked elements, global): rel-L2 <= 1e-2 and max-abs <= 3e-2.
Small shapes compare every output row; the Wan workloads compare all rows (single 480p frame) or
4096 seeded rows plus every row of the last, partial query tile of two heads.
"""

import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_wan_amd as wan
import wan_inputs
from _util import (BF16_MAX_ABS, BF16_REL_L2, ensure_built, gather_rows, metrics, tail_rows, to_np)

pytestmark = pytest.mark.gpu

TAILS = [1, 2, 63, 64, 65, 127, 129, 255, 256, 257, 300]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _run_full(b, H, s_q, s_kv, seed, sigma=1.0):
    q, k, v = wan_inputs.random_qkv(b, H, s_q, s_kv, seed, sigma=sigma, device="cuda")
    out = wan.attention(q, k, v)
    torch.cuda.synchronize()
    ref = oracle.attention(to_np(q), to_np(k), to_np(v))
    return to_np(out), ref


@pytest.mark.parametrize("s_q", TAILS)
def test_tails_all_rows(s_q):
    print(f"tails s_q={s_q}", flush=True)
    for j, s_kv in enumerate(TAILS):
        got, ref = _run_full(1, 2, s_q, s_kv, seed=1000 + 17 * s_q + j)
        rel, mx, _ = metrics(got, ref)
        assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS, (s_q, s_kv, rel, mx)


@pytest.mark.parametrize("b,H,s_q,s_kv", [(2, 3, 513, 700), (1, 1, 1000, 64), (2, 2, 90, 4097)])
def test_batches_and_heads(b, H, s_q, s_kv):
    got, ref = _run_full(b, H, s_q, s_kv, seed=b * 100 + H * 10 + s_q)
    rel, mx, _ = metrics(got, ref)
    assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS, (rel, mx)


def _growing_keys(s_q, s_kv, seed, growth, damped=None, q_scale=1.0, heads=2):
    """Q, K, V ~ N(0, 1) with every key from the second 64-key block on multiplied by growth
    (and the query rows `damped` by q_scale): scores after the first tile outgrow the reference
    maximum the kernel takes from it."""
    q, k, v = wan_inputs.random_qkv(1, heads, s_q, s_kv, seed, device="cuda")
    k = k.clone()
    k[:, 64:] = (k[:, 64:].float() * growth).to(torch.bfloat16)
    if damped is not None:
        q = q.clone()
        q[:, damped] = (q[:, damped].float() * q_scale).to(torch.bfloat16)
    return q, k, v


@pytest.mark.parametrize("growth,damped,s_kv,heads,s_q", [(6.0, None, 1000, 2, 300), (40.0, None, 1000, 2, 300),
                                                           (40.0, "first100", 1000, 2, 300),
                                                           (40.0, "every32", 1000, 2, 300),
                                                           (40.0, "every32", 20000, 2, 300),
                                                           (40.0, "every32", 1000, 64, 600)])
def test_scores_outgrowing_the_first_tile(growth, damped, s_kv, heads, s_q):
    # growth 6: later scores exceed the first tile's maximum by up to ~2^30 in P, which the fixed
    # reference absorbs; growth 40: P would overflow (row sums past 2^64), so the query tiles take
    # the exact path (row max sweep, then softmax against it).  damped rows do not overflow:
    # "first100" = rows 0-99; "every32" = rows 0, 32, 64, ..., lane 0 of every wave, so that only
    # other lanes' rows call for the exact path.  s_kv 1000 runs with the keys split into ranges
    # (2 heads x 2 query tiles are too few to fill the GPU), s_kv 20000 as well with longer ranges;
    # 64 heads x 3 query tiles run unsplit.
    print(f"growing keys x{growth}, damped {damped}, s_kv {s_kv}, heads {heads}, s_q {s_q}", flush=True)
    rows = {None: None, "first100": np.arange(100), "every32": np.arange(0, s_q, 32)}[damped]
    q, k, v = _growing_keys(s_q, s_kv, seed=91, growth=growth, damped=rows, q_scale=0.02, heads=heads)
    out = wan.attention(q, k, v)
    torch.cuda.synchronize()
    got = to_np(out)
    assert np.isfinite(got).all()
    rel, mx, _ = metrics(got, oracle.attention(to_np(q), to_np(k), to_np(v)))
    assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS, (rel, mx)


def test_large_logits_keep_accuracy():
    # Q, K ~ N(0, 9) make score spreads of tens, far above the first tile's maximum
    q, k, _ = wan_inputs.random_qkv(1, 2, 300, 2000, seed=77, sigma=3.0, device="cuda")
    _, _, v = wan_inputs.random_qkv(1, 2, 300, 2000, seed=78, device="cuda")
    out = wan.attention(q, k, v)
    torch.cuda.synchronize()
    rel, mx, _ = metrics(to_np(out), oracle.attention(to_np(q), to_np(k), to_np(v)))
    assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS, (rel, mx)


def test_uniform_values_return_that_row():
    q, k, _ = wan_inputs.random_qkv(1, 3, 200, 333, seed=5, device="cuda")
    row = torch.randn(3, 128, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    v = row.to("cuda").view(1, 1, 3, 128).expand(1, 333, 3, 128).contiguous()
    out = wan.attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), v[:, :1].expand(1, 200, 3, 128).cpu())


def test_single_key_returns_its_value():
    q, k, v = wan_inputs.random_qkv(2, 2, 77, 1, seed=8, device="cuda")
    out = wan.attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), v.expand(2, 77, 2, 128).cpu())


def test_key_value_permutation_invariance():
    q, k, v = wan_inputs.random_qkv(1, 2, 256, 640, seed=9, device="cuda")
    perm = torch.randperm(640, generator=torch.Generator().manual_seed(10)).cuda()
    a = wan.attention(q, k, v)
    b = wan.attention(q, k[:, perm].contiguous(), v[:, perm].contiguous())
    torch.cuda.synchronize()
    rel, mx, _ = metrics(to_np(a), to_np(b))
    assert rel <= 5e-3 and mx <= 2e-2


def test_deterministic():
    q, k, v = wan_inputs.random_qkv(1, 4, 1000, 1500, seed=11, device="cuda")
    a = wan.attention(q, k, v)
    b = wan.attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_runs_on_a_side_stream():
    q, k, v = wan_inputs.random_qkv(1, 2, 129, 65, seed=12, device="cuda")
    ref = wan.attention(q, k, v)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = wan.attention(q, k, v)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def _workload_parity(name, n_rows=4096):
    w = wan_inputs.WORKLOADS[name]
    print(f"workload {name}: generating", flush=True)
    q, k, v = wan_inputs.make_qkv(w, device="cuda")
    out = wan.attention(q, k, v)
    torch.cuda.synchronize()
    print(f"workload {name}: kernel done, oracle on sampled rows", flush=True)
    rows = wan_inputs.sample_rows(w, n_rows).numpy()
    rows = np.concatenate([rows, tail_rows(w.batch, w.heads, w.s_q)])
    qn, kn, vn = to_np(q.cpu()), to_np(k.cpu()), to_np(v.cpu())
    del q, k, v
    ref = oracle.attention_rows(qn, kn, vn, rows)
    got = gather_rows(out, rows)
    rel, mx, cos = metrics(got, ref)
    print(f"workload {name}: rel-L2 {rel:.3e} max-abs {mx:.3e} cos {cos:.6f}", flush=True)
    assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS


def test_frame480_all_rows():
    w = wan_inputs.WORKLOADS["frame480_self"]
    q, k, v = wan_inputs.make_qkv(w, device="cuda")
    out = wan.attention(q, k, v)
    torch.cuda.synchronize()
    ref = oracle.attention(to_np(q), to_np(k), to_np(v))
    rel, mx, cos = metrics(to_np(out), ref)
    print(f"workload frame480_self (every row): rel-L2 {rel:.3e} max-abs {mx:.3e} cos {cos:.6f}", flush=True)
    assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS


def test_wan13b_480p_sampled():
    _workload_parity("wan1.3b_480p81f_self")


def test_wan14b_text_cross_sampled():
    _workload_parity("wan14b_text_cross")


def test_wan14b_720p_sampled():
    _workload_parity("wan14b_720p81f_self")
