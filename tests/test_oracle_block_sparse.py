"""Pins of the block-sparse (VSA-style) attention oracle against things other than itself.

* brute force: block means and block scores with math.fsum loops, including a partial last block;
* reduction to the dense definition: keeping every key block gives oracle.attention (itself pinned
  to brute force and torch SDPA), and keeping one block gives the dense attention over that block's
  keys alone;
* the selection: a constructed score matrix whose top-k is known, the tie rule (constant blocks ->
  the lowest indices), equivariance under a permutation of whole key blocks (indices follow, O does
  not change), and the validity check used against the GPU;
* planted mistakes (bottom-k instead of top-k, all keys instead of the selected ones) that fail.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.block_sparse as bs


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_default_keep():
    assert bs.default_keep(64) == 1 and bs.default_keep(65) == 1
    assert bs.default_keep(8 * 64) == 1 and bs.default_keep(9 * 64) == 2
    assert bs.default_keep(75600) == 148          # 1,182 key blocks at 720p
    assert bs.default_keep(32760) == 64           # 512 key blocks at 480p


def test_block_means_and_scores_brute_force():
    b, s, H, d = 2, 150, 3, 5                      # blocks of 64, 64, 22 tokens
    q = _rand((b, s, H, d), 1)
    k = _rand((b, 130, H, d), 2)                   # blocks of 64, 64, 2 tokens
    mq = bs.block_means(q)
    for bb in range(b):
        for hh in range(H):
            for j, (lo, hi) in enumerate([(0, 64), (64, 128), (128, 150)]):
                for c in range(d):
                    assert abs(mq[bb, hh, j, c] - math.fsum(q[bb, lo:hi, hh, c]) / (hi - lo)) < 1e-14
    sc = bs.block_scores(q, k)
    mk = bs.block_means(k)
    for bb in range(b):
        for hh in range(H):
            for i in range(3):
                for j in range(3):
                    ref = math.fsum(mq[bb, hh, i, c] * mk[bb, hh, j, c] for c in range(d)) / math.sqrt(d)
                    assert abs(sc[bb, hh, i, j] - ref) < 1e-13


def test_keep_all_is_dense_attention():
    q, k, v = _rand((1, 200, 2, 128), 3), _rand((1, 300, 2, 128), 4), _rand((1, 300, 2, 128), 5)
    sel = bs.select_blocks(q, k, keep=bs.n_blocks(300))
    assert np.array_equal(sel[0, 0, 0], np.arange(5))
    o = bs.sparse_attention(q, k, v, sel)
    assert np.allclose(o, oracle.attention(q, k, v), rtol=1e-12, atol=1e-13)


def test_keep_one_is_attention_over_that_block():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 64, 1, 128))
    k = rng.standard_normal((1, 256, 1, 128))
    v = rng.standard_normal((1, 256, 1, 128))
    # key block 2 points along the queries' mean: its block score is by far the largest
    k[0, 128:192, 0, :] += 3.0 * q[0, :, 0, :].mean(axis=0) / np.linalg.norm(q[0, :, 0, :].mean(axis=0)) * 4
    sel = bs.select_blocks(q, k, keep=1)
    assert sel.shape == (1, 1, 1, 1) and sel[0, 0, 0, 0] == 2
    o = bs.sparse_attention(q, k, v, sel)
    ref = oracle.attention(q, k[:, 128:192], v[:, 128:192])
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_known_top_k_and_ties():
    # query-block mean e0; key blocks constant vectors c_j * e0 with scores proportional to c_j
    d = 128
    q = np.zeros((1, 64, 1, d))
    q[..., 0] = 1.0
    c = np.array([0.5, 3.0, -1.0, 2.0, 3.0, 0.0, 1.0, 2.0, 5.0, -2.0])
    k = np.zeros((1, 64 * len(c), 1, d))
    for j, cj in enumerate(c):
        k[0, 64 * j:64 * (j + 1), 0, 0] = cj
    assert np.array_equal(bs.select_blocks(q, k, keep=3)[0, 0, 0], [1, 4, 8])   # 5, 3, 3
    assert np.array_equal(bs.select_blocks(q, k, keep=4)[0, 0, 0], [1, 3, 4, 8])  # tie 2.0: index 3 before 7
    k[:] = 0.0                                                                    # all scores equal
    assert np.array_equal(bs.select_blocks(q, k, keep=4)[0, 0, 0], [0, 1, 2, 3])


def test_block_permutation():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 128, 2, 128))
    k = rng.standard_normal((1, 512, 2, 128))
    v = rng.standard_normal((1, 512, 2, 128))
    perm = rng.permutation(8)
    kp = k.reshape(1, 8, 64, 2, 128)[:, perm].reshape(k.shape)
    vp = v.reshape(1, 8, 64, 2, 128)[:, perm].reshape(v.shape)
    sel = bs.select_blocks(q, k, keep=3)
    selp = bs.select_blocks(q, kp, keep=3)
    inv = np.argsort(perm)                         # block j of k sits at position inv[j] of kp
    assert np.array_equal(np.sort(inv[sel], axis=-1), selp)
    assert np.allclose(bs.sparse_attention(q, k, v, sel), bs.sparse_attention(q, kp, vp, selp), rtol=1e-12, atol=1e-13)


def test_validity_check():
    scores = np.array([[0.0, 1.0, 2.0, 3.0, 4.0]])
    assert bs.is_valid_selection(np.array([[3, 4]]), scores, 0.0)[0]
    assert not bs.is_valid_selection(np.array([[2, 4]]), scores, 0.5)[0]
    assert bs.is_valid_selection(np.array([[2, 4]]), scores, 1.0)[0]         # within tolerance
    assert not bs.is_valid_selection(np.array([[4, 4]]), scores, 10.0)[0]    # repeated index
    q, k = _rand((2, 300, 3, 128), 9), _rand((2, 700, 3, 128), 10)
    assert np.all(bs.is_valid_selection(bs.select_blocks(q, k), bs.block_scores(q, k), 0.0))


def test_planted_mistakes_are_caught():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 64, 1, 128))
    k = rng.standard_normal((1, 256, 1, 128))
    v = rng.standard_normal((1, 256, 1, 128))
    k[0, 128:192, 0, :] += 12.0 * q[0, :, 0, :].mean(axis=0) / np.linalg.norm(q[0, :, 0, :].mean(axis=0))
    # bottom-k instead of top-k
    c = bs.block_scores(q, k)
    bottom = np.sort(np.argsort(c, axis=-1, kind="stable")[..., :1], axis=-1)
    assert not np.all(bs.is_valid_selection(bottom, c, 0.0))
    # attending to all keys instead of the selected block
    sel = bs.select_blocks(q, k, keep=1)
    dense = oracle.attention(q, k, v)
    ref = oracle.attention(q, k[:, 128:192], v[:, 128:192])
    assert np.allclose(bs.sparse_attention(q, k, v, sel), ref, rtol=1e-12, atol=1e-13)
    assert not np.allclose(dense, ref, rtol=1e-3, atol=1e-3)
