"""Parity of the block-sparse (VSA-style) attention path (through the C ABI) with the oracle, on the GPU.

* Coarse stage.  The GPU decides the selection from float32 block means and scores, the oracle from
  float64 ones, so the GPU's list is checked to be a valid top-keep set of the oracle's scores within
  the float32 rounding of those scores (oracle.block_sparse.is_valid_selection), bound per score
  (u = 2^-24, n <= 64 tokens per block, d = 128):
      |mean error| <= 65 u mean|x|                   (4 in-order sums of 16 tokens, their sum, the division)
      |score error| <= u (20 sum_c |mq_c mk_c| + 66 sum_c (mean|q|_c |mk_c| + |mq_c| mean|k|_c)) / sqrt(d)
  (16 in-order products per lane and a 3-level butterfly; the mean errors carried through), twice
  over for the two scores compared.  Where the scores are exact in float32 (constant blocks of small
  integers) the GPU must return the oracle's list itself, ties to the lower index included.
* Fine stage: the output against oracle.block_sparse.sparse_attention_rows on the GPU's own list (or a
  given one), with the bf16 path's bounds (rel-L2 <= 1e-2, max-abs <= 3e-2).
* Shapes: ragged sequence lengths (partial last blocks on either side, an odd number of query blocks,
  which leaves half of the last workgroup idle), keep from 1 to every block, and the two Wan workloads
  on sampled heads and rows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.block_sparse as bs
import video_diffusion_transformer_wan_amd as wan
import wan_inputs
from _util import BF16_MAX_ABS, BF16_REL_L2, ensure_built, metrics, to_np

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _score_tol(q, k):
    """Per (b, H, query block): twice the largest float32 rounding bound of that block's scores."""
    mq, mk = bs.block_means(q), bs.block_means(k)
    aq, ak = bs.block_means(np.abs(q)), bs.block_means(np.abs(k))
    d = q.shape[-1]
    prod = np.einsum("bhic,bhjc->bhij", np.abs(mq), np.abs(mk))
    carry = np.einsum("bhic,bhjc->bhij", aq, np.abs(mk)) + np.einsum("bhic,bhjc->bhij", np.abs(mq), ak)
    bound = U * (20 * prod + 66 * carry) / math.sqrt(d) + U * np.abs(bs.block_scores(q, k))
    return 2 * bound.max(axis=-1)


def _check_selection(sel, q, k, keep):
    sel = np.asarray(sel, np.int64)
    n_kb = bs.n_blocks(k.shape[1])
    assert sel.shape == (q.shape[0], q.shape[2], bs.n_blocks(q.shape[1]), keep)
    assert sel.min() >= 0 and sel.max() < n_kb
    assert np.all(np.diff(sel, axis=-1) > 0) if keep > 1 else True        # ascending, distinct
    scores = bs.block_scores(q, k)
    tol = _score_tol(q, k)
    ok = bs.is_valid_selection(sel, scores, tol)
    assert np.all(ok), f"{int((~ok).sum())} of {ok.size} query blocks with an invalid selection"
    same = np.mean(np.all(sel == bs.select_blocks(q, k, keep), axis=-1))
    print(f"  selection valid; equal to the oracle's in {same:.4f} of the query blocks", flush=True)


def _check_output(got, ref):
    rel, mx, _ = metrics(got, ref)
    print(f"  rel-L2 {rel:.3e}  max-abs {mx:.3e}", flush=True)
    assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS, (rel, mx)


def _all_rows(b, H, s):
    return np.array([[bb, hh, i] for bb in range(b) for hh in range(H) for i in range(s)], np.int64)


def _gather(o, rows):
    o = to_np(o)
    return o[rows[:, 0], rows[:, 2], rows[:, 1]]


CASES = [
    # b, H, s_q, s_kv, keep
    (1, 2, 64, 64, 1),
    (1, 2, 65, 130, 2),
    (1, 1, 100, 700, 3),          # 2 query blocks, 11 key blocks (last of 60 keys)
    (2, 3, 513, 1000, 4),         # 9 query blocks: half of the last workgroup idle
    (1, 2, 300, 129, 3),          # every key block, the last with one key
    (1, 2, 1000, 4097, 9),        # a one-key last block among 65
    (1, 1, 200, 4160, 65),        # keep = n_kb: dense
    (2, 2, 257, 2048, 1),
]


@pytest.mark.parametrize("b,H,s_q,s_kv,keep", CASES)
def test_select_and_attend(b, H, s_q, s_kv, keep):
    print(f"vsa b={b} H={H} s_q={s_q} s_kv={s_kv} keep={keep}", flush=True)
    seed = 40000 + 7 * s_q + s_kv + keep
    q, k, v = wan_inputs.random_qkv(b, H, s_q, s_kv, seed, device="cuda")
    sel = wan.vsa_select(q, k, keep)
    o = wan.vsa_attention(q, k, v, sel)
    torch.cuda.synchronize()
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    sel_np = sel.cpu().numpy().astype(np.int64)
    _check_selection(sel_np, qn, kn, keep)
    rows = _all_rows(b, H, s_q)
    _check_output(_gather(o, rows), bs.sparse_attention_rows(qn, kn, vn, sel_np, rows))
    # both stages in one call: the same kernels, so the same bits
    o2 = wan.vsa_forward(q, k, v, keep)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


def test_keep_all_is_dense():
    q, k, v = wan_inputs.random_qkv(1, 2, 333, 600, 41000, device="cuda")
    n_kb = bs.n_blocks(600)
    o = wan.vsa_forward(q, k, v, n_kb)
    torch.cuda.synchronize()
    _check_output(to_np(o), oracle.attention(to_np(q), to_np(k), to_np(v)))


def test_exact_scores_and_ties():
    # query blocks of constant rows e0; key block j constant c_j e0: scores c_j / sqrt(128), exact in
    # float32, so the GPU must pick the oracle's blocks, equal scores going to the lower index
    d = 128
    c = np.array([0.5, 3.0, -1.0, 2.0, 3.0, 0.0, 1.0, 2.0, 5.0, -2.0], np.float32)
    q = np.zeros((1, 130, 1, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 64 * len(c), 1, d), np.float32)
    for j, cj in enumerate(c):
        k[0, 64 * j:64 * (j + 1), 0, 0] = cj
    qt = torch.tensor(q, dtype=torch.bfloat16, device="cuda")
    kt = torch.tensor(k, dtype=torch.bfloat16, device="cuda")
    for keep, want in ((1, [8]), (3, [1, 4, 8]), (4, [1, 3, 4, 8]), (10, list(range(10)))):
        sel = wan.vsa_select(qt, kt, keep).cpu().numpy()
        assert np.array_equal(sel[0, 0], np.array([want] * 3)), (keep, sel)
        assert np.array_equal(sel[0, 0, 0], bs.select_blocks(q, k, keep)[0, 0, 0])
    # every score equal: the lowest indices
    sel = wan.vsa_select(qt, torch.zeros_like(kt), 4).cpu().numpy()
    assert np.array_equal(sel[0, 0], np.array([[0, 1, 2, 3]] * 3))


def test_given_lists_and_skipped_entries():
    b, H, s_q, s_kv = 1, 2, 300, 1000          # 5 query blocks, 16 key blocks (last of 40 keys)
    q, k, v = wan_inputs.random_qkv(b, H, s_q, s_kv, 41001, device="cuda")
    rng = np.random.default_rng(5)
    n_qb, n_kb = bs.n_blocks(s_q), bs.n_blocks(s_kv)
    valid = np.stack([np.stack([np.sort(rng.choice(n_kb, 4, replace=False)) for _ in range(n_qb)])
                      for _ in range(b * H)]).reshape(b, H, n_qb, 4)
    valid[0, 0, 0] = [0, 5, 9, n_kb - 1]       # the first and the partial last block
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    rows = _all_rows(b, H, s_q)
    ref = bs.sparse_attention_rows(qn, kn, vn, valid, rows)
    o = wan.vsa_attention(q, k, v, torch.tensor(valid, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    _check_output(_gather(o, rows), ref)
    # the same lists with out-of-range entries mixed in: skipped
    bad = np.array([-1, n_kb, 1 << 30], np.int64)
    mixed = np.concatenate([valid[..., :2], np.broadcast_to(bad, valid.shape[:3] + (3,)), valid[..., 2:]], axis=-1)
    o2 = wan.vsa_attention(q, k, v, torch.tensor(mixed, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    _check_output(_gather(o2, rows), ref)
    # a repeated block counts twice (its keys enter the softmax twice)
    dup = valid.copy()
    dup[..., 1] = dup[..., 0]
    o3 = wan.vsa_attention(q, k, v, torch.tensor(dup, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    _check_output(_gather(o3, rows), bs.sparse_attention_rows(qn, kn, vn, dup, rows))


def test_side_stream_and_determinism():
    q, k, v = wan_inputs.random_qkv(1, 3, 700, 900, 41002, device="cuda")
    ref = wan.vsa_forward(q, k, v)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = torch.empty_like(q)
        wan.vsa_forward(q, k, v, out=out, stream=s)
    s.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("name", sorted(wan_inputs.VSA_WORKLOADS))
def test_wan_workload_sampled(name):
    w = wan_inputs.VSA_WORKLOADS[name]
    print(f"{name}: b={w.batch} H={w.heads} s={w.s} keep={w.keep}", flush=True)
    q, k, v = wan_inputs.make_vsa(w, device="cuda")
    sel = wan.vsa_select(q, k, w.keep)
    o = wan.vsa_attention(q, k, v, sel)
    torch.cuda.synchronize()
    heads = [0, w.heads - 1]
    hsel = torch.tensor(heads, device="cuda")
    qn = to_np(q.index_select(2, hsel))
    kn = to_np(k.index_select(2, hsel))
    vn = to_np(v.index_select(2, hsel))
    sel_np = sel.index_select(1, hsel).cpu().numpy().astype(np.int64)
    _check_selection(sel_np, qn, kn, w.keep)
    rng = np.random.default_rng(w.seed + 2)
    rows = []
    for j in range(len(heads)):
        r = rng.choice(w.s, 512, replace=False)
        r = np.concatenate([r, np.arange(64 * ((w.s - 1) // 64), w.s)])   # the last query block
        rows += [[0, j, i] for i in np.unique(r)]
    rows = np.array(rows, np.int64)
    ref = bs.sparse_attention_rows(qn, kn, vn, sel_np, rows)
    got = to_np(o.index_select(2, hsel))[rows[:, 0], rows[:, 2], rows[:, 1]]
    _check_output(got, ref)


def test_largest_key_block_count():
    # 4,096 key blocks (262,144 keys), the selection's largest: the scores of its 8 query blocks fill
    # 128 KB of LDS (the launch raises the dynamic LDS limit)
    b, H, s_q, s_kv, keep = 1, 1, 100, 4096 * 64, 512
    print(f"vsa b={b} H={H} s_q={s_q} s_kv={s_kv} keep={keep}", flush=True)
    q, k, v = wan_inputs.random_qkv(b, H, s_q, s_kv, 41003 + keep, device="cuda")
    sel = wan.vsa_select(q, k, keep)
    o = wan.vsa_attention(q, k, v, sel)
    torch.cuda.synchronize()
    # float64 copies made by torch (exact for bf16; numpy's own cast of large torch-backed arrays is slow)
    qn, kn, vn = (t.double().cpu().numpy() for t in (q, k, v))
    sel_np = sel.cpu().numpy().astype(np.int64)
    _check_selection(sel_np, qn, kn, keep)
    rows = _all_rows(b, H, s_q)[::7]
    _check_output(_gather(o, rows), bs.sparse_attention_rows(qn, kn, vn, sel_np, rows))


def test_many_query_blocks_every_row():
    # 8 heads x 65 query blocks = 520 workgroups: more than one round of the XCD numbering (8 x 64), with
    # rounds that straddle heads; every output row is checked
    b, H, s_q, s_kv, keep = 1, 8, 4160, 640, 2
    print(f"vsa b={b} H={H} s_q={s_q} s_kv={s_kv} keep={keep}", flush=True)
    q, k, v = wan_inputs.random_qkv(b, H, s_q, s_kv, 41004, device="cuda")
    sel = wan.vsa_select(q, k, keep)
    o = wan.vsa_attention(q, k, v, sel)
    torch.cuda.synchronize()
    qn, kn, vn = (t.double().cpu().numpy() for t in (q, k, v))
    sel_np = sel.cpu().numpy().astype(np.int64)
    _check_selection(sel_np, qn, kn, keep)
    rows = _all_rows(b, H, s_q)
    _check_output(_gather(o, rows), bs.sparse_attention_rows(qn, kn, vn, sel_np, rows))
