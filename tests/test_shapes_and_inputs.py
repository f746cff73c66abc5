"""Host arithmetic (token lengths, cost model) against the hand-worked fixtures under
tests/golden/, and the determinism of the seeded input generators."""

import os

import numpy as np
import pytest
import torch

from video_diffusion_transformer_wan_amd import shapes
import wan_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [list(map(int, l.split())) for l in f if l.strip() and not l.startswith("#")]


def test_token_counts_match_fixture():
    for T, H, W, lt, lh, lw, s in _rows("token_counts.txt"):
        assert shapes.latent_shape(T, H, W) == (lt, lh, lw, 16)
        assert shapes.video_tokens(T, H, W) == s
    with pytest.raises(ValueError):
        shapes.video_tokens(3, 480, 832)


def test_cost_model_matches_fixture():
    for b, H, sq, skv, flops in _rows("cost_model.txt"):
        assert shapes.attention_flops(b, H, sq, skv) == flops


def test_workloads_use_the_page_shapes():
    w = wan_inputs.WORKLOADS
    assert w["frame480_self"].s_q == shapes.video_tokens(0, 480, 832)
    assert w["wan1.3b_480p81f_self"].s_q == shapes.video_tokens(80, 480, 832)
    assert w["wan14b_720p81f_self"].s_q == shapes.video_tokens(80, 720, 1280)
    assert w["wan14b_text_cross"].s_kv == shapes.TEXT_TOKENS
    flops = {r[:4] and tuple(r[:4]): r[4] for r in _rows("cost_model.txt")}
    for x in w.values():
        assert x.flops == flops[(x.batch, x.heads, x.s_q, x.s_kv)]


def test_inputs_are_deterministic_and_bf16():
    a = wan_inputs.make_qkv("frame480_self")
    b = wan_inputs.make_qkv("frame480_self")
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and torch.equal(x, y)
    q, k, v = a
    assert q.shape == (1, 1560, 2, 128) and k.shape == v.shape == (1, 1560, 2, 128)
    assert not torch.equal(q, k)
    assert abs(q.float().std().item() - 1.0) < 0.01


def test_batched_draw_equals_one_shot():
    q, k, v = wan_inputs.random_qkv(3, 2, 50, 40, seed=7)
    g = torch.Generator().manual_seed(7)
    one = torch.randn((3, 50, 2, 128), generator=g).to(torch.bfloat16)
    assert torch.equal(q, one)


def test_outlier_columns_and_rows():
    w = wan_inputs.WORKLOADS["wan14b_720p81f_self_int8fp8"]
    cols = [wan_inputs.outlier_columns(w, t) for t in range(3)]
    assert all(c.numel() == 51 and c.unique().numel() == 51 for c in cols)
    assert not torch.equal(cols[0], cols[1])
    rows = wan_inputs.sample_rows(w)
    assert rows.shape == (4096, 3)
    flat = (rows[:, 0] * w.heads + rows[:, 1]) * w.s_q + rows[:, 2]
    assert flat.unique().numel() == 4096
    assert rows[:, 1].max() < w.heads and rows[:, 2].max() < w.s_q
    small = wan_inputs.sample_rows("frame480_self")
    assert small.shape == (3120, 3)


def test_outliers_scale_the_chosen_columns():
    w = wan_inputs.Workload("t", 1, 4, 300, 300, 128, 1.0, 1.0, "int8_fp8", 0.01, 99, "")
    q, k, v = wan_inputs.make_qkv(w)
    cols = wan_inputs.outlier_columns(w, 0)
    qf = q.float().reshape(300, 4 * 128)
    std = qf.std(dim=0)
    mask = torch.zeros(512, dtype=torch.bool)
    mask[cols] = True
    assert std[mask].min() > 4 and std[~mask].max() < 2


def test_vsa_workloads_and_default_keep():
    # the block-sparse workloads: the 16x28x52 token grid and the 720p 81-frame sequence, 87.5% of the
    # 64-token key blocks dropped; the binding's default keep is the oracle's
    import oracle.block_sparse as bs
    import video_diffusion_transformer_wan_amd as wan
    assert wan_inputs.VSA_WORKLOADS["wan1.3b_vsa_16x28x52"].s == 16 * 28 * 52
    assert wan_inputs.VSA_WORKLOADS["wan14b_720p81f_vsa"].s == shapes.video_tokens(80, 720, 1280)
    for w in wan_inputs.VSA_WORKLOADS.values():
        assert w.keep == bs.default_keep(w.s)
    for s in (1, 63, 64, 65, 512, 513, 4096, 23296, 32760, 75600, 262144):
        assert wan.vsa_default_keep(s) == bs.default_keep(s), s
