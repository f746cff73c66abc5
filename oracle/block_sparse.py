"""Block-sparse attention in the style of Video Sparse Attention (VSA) -- test infrastructure (see
the package docstring).

What the pages fix (the FastWan / VSA article, sections "传统稀疏注意力，为何会在蒸馏中失效？" and
"一张卡，秒生视频"): VSA is a dynamic sparse attention with a coarse stage that finds the key
tokens that matter and a fine stage that runs block-sparse attention over them; at 87.5% sparsity it
cuts attention FLOPs 8x; its mask is made of 64 x 64 blocks (the block size FlexAttention was given
for the comparison).  What they leave open, and the reading taken here (each one also lives in the
GPU path, which is written separately):

  1. Blocks are 64 consecutive tokens of the flattened sequence, starting at token 0; the last
     block of a sequence may be partial.
  2. Coarse stage, per (batch, head): the mean of Q over each query block and of K over each key
     block (over the block's real tokens), block scores C[i, j] = mean_q[i] . mean_k[j] / sqrt(d),
     and for every query block the `keep` key blocks with the largest scores; keep = ceil(n_kb / 8)
     (87.5% sparsity) unless given.  Ties go to the lower key-block index.
  3. Fine stage: every query row attends to the keys of its query block's selected key blocks only:
     O[i] = sum_{j in selected} softmax_j(q_i . k_j / sqrt(d)) v_j, the softmax taken over those
     keys alone.  Nothing is added for the unselected blocks.

Everything is float64 on an exact upcast of the bf16 inputs.  Which blocks the GPU selects is
decided by float32 scores there; the tests check that the GPU's choice is a valid top-k of the
float64 scores within the rounding of the float32 ones, and run the fine stage of this oracle on
the GPU's own choice.
"""

import math

import numpy as np

BLOCK = 64


def n_blocks(s, block=BLOCK):
    return (s + block - 1) // block


def default_keep(s_kv, block=BLOCK):
    """ceil(n_kb / 8): 87.5% of the key blocks dropped."""
    return max(1, -(-n_blocks(s_kv, block) // 8))


def block_means(x, block=BLOCK):
    """Reading 2: x [b, s, H, d] -> the mean of each block's real tokens, [b, H, n_blocks, d] float64."""
    x = np.asarray(x, np.float64)
    b, s, H, d = x.shape
    nb = n_blocks(s, block)
    out = np.empty((b, H, nb, d))
    for j in range(nb):
        seg = x[:, j * block:min((j + 1) * block, s)]          # [b, t, H, d]
        out[:, :, j, :] = seg.mean(axis=1)
    return out


def block_scores(q, k, block=BLOCK):
    """C [b, H, n_qb, n_kb] = mean_q . mean_k^T / sqrt(d) (float64)."""
    mq = block_means(q, block)
    mk = block_means(k, block)
    d = mq.shape[-1]
    return np.einsum("bhid,bhjd->bhij", mq, mk) / math.sqrt(d)


def select_blocks(q, k, keep=None, block=BLOCK):
    """The selected key blocks of every query block, [b, H, n_qb, keep] int64, in ascending block order
    (the top `keep` scores; ties to the lower index)."""
    c = block_scores(q, k, block)
    keep = default_keep(k.shape[1], block) if keep is None else keep
    # stable sort on -score: equal scores keep ascending index order
    order = np.argsort(-c, axis=-1, kind="stable")[..., :keep]
    return np.sort(order, axis=-1)


def is_valid_selection(sel, scores, tol):
    """True where the selection `sel` [..., keep] is a top-keep set of `scores` [..., n_kb] up to `tol`
    (every selected score >= every unselected score - tol), per query block -> bool [...]."""
    n_kb = scores.shape[-1]
    mask = np.zeros(scores.shape, bool)
    np.put_along_axis(mask, np.asarray(sel, np.int64), True, axis=-1)
    sel_min = np.where(mask, scores, np.inf).min(axis=-1)
    unsel_max = np.where(mask, -np.inf, scores).max(axis=-1) if sel.shape[-1] < n_kb else np.full(sel_min.shape, -np.inf)
    distinct = np.all(np.sort(sel, axis=-1)[..., 1:] != np.sort(sel, axis=-1)[..., :-1], axis=-1) if sel.shape[-1] > 1 \
        else np.ones(sel_min.shape, bool)
    return (sel_min >= unsel_max - tol) & distinct


def sparse_attention_rows(q, k, v, sel, rows, block=BLOCK):
    """Reading 3 for (batch, head, query row) triples -> [n, d] float64, given the selection `sel`
    [b, H, n_qb, keep] (block indices)."""
    rows = np.asarray(rows, np.int64).reshape(-1, 3)
    s_kv = k.shape[1]
    d = q.shape[-1]
    out = np.empty((rows.shape[0], d))
    for r, (bb, hh, i) in enumerate(rows):
        blocks = np.asarray(sel[bb, hh, i // block], np.int64)
        keys = np.concatenate([np.arange(j * block, min((j + 1) * block, s_kv)) for j in blocks])
        qq = np.asarray(q[bb, i, hh, :], np.float64)
        kk = np.asarray(k[bb, keys, hh, :], np.float64)
        vv = np.asarray(v[bb, keys, hh, :], np.float64)
        s = kk @ qq / math.sqrt(d)
        p = np.exp(s - s.max())
        out[r] = (p @ vv) / p.sum()
    return out


def sparse_attention(q, k, v, sel, block=BLOCK):
    """Reading 3 for every row: O [b, s_q, H, d] float64."""
    b, s_q, H, d = q.shape
    rows = np.array([[bb, hh, i] for bb in range(b) for hh in range(H) for i in range(s_q)], np.int64)
    o = sparse_attention_rows(q, k, v, sel, rows, block)
    out = np.empty((b, s_q, H, d))
    out[rows[:, 0], rows[:, 2], rows[:, 1]] = o
    return out
