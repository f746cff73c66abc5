"""Seeded synthetic inputs for the Wan attention workloads (shared by tests, bench and smoke).

This module holds only shapes, seeds and random draws -- none of the attention arithmetic.  Both
the HIP path and the CPU oracle receive what it produces; neither is imported here.

Token lengths come from the Wan VAE and patchify shapes ("Wan 2.1: VBench 86.22% ..." explainer,
section "先看现象": a (1+T) x H x W x 3 video becomes a [1+T/4, H/8, W/8, 16] latent, then a
(1,2,2) patchify): 480x832 gives 30 x 52 = 1,560 tokens per latent frame, 720x1280 gives
45 x 80 = 3,600, and 81 frames give 21 latent frames.  The text context is the 512-token umT5
embedding (same page, section "干预与形式化").  The pages print no activation statistics, so the
values are Gaussian stand-ins for Wan's real Q/K/V activations.

Recipe (the same on every machine with this torch version):
  * Q, K, V are drawn in that order from one ``torch.Generator`` seeded with the workload's seed,
    on the device that will hold them, as float32 N(0, 1) of shape [b, s, H, d], scaled by the
    workload's sigma and rounded to bfloat16 (round to nearest even).  Each tensor is drawn one
    batch entry at a time, which equals a one-shot draw of the whole tensor.
  * Outlier channels (the 8-bit workload): from a CPU generator seeded with seed + 1, for Q, K
    and V in turn, round(0.01 * H * d) distinct (head, channel) columns are picked without
    replacement and multiplied by 8 before the bfloat16 rounding.
  * Sampled query rows: from a CPU generator seeded with seed + 2, distinct (batch, head, row)
    triples uniformly without replacement.
"""

from dataclasses import dataclass

import torch

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    s_q: int
    s_kv: int
    head_dim: int
    sigma_q: float
    sigma_kv: float
    path: str          # "bf16" or "int8_fp8"
    outlier_frac: float
    seed: int
    description: str

    @property
    def flops(self):
        """Attention forward FLOPs: the two products, 2 * s_q * s_kv * d each, per (batch, head)."""
        return 4 * self.batch * self.heads * self.s_q * self.s_kv * self.head_dim


WORKLOADS = {
    w.name: w for w in [
        Workload("frame480_self", 1, 2, 1560, 1560, HEAD_DIM, 1.0, 1.0, "bf16", 0.0, 20250000,
                 "one 480x832 latent frame (1x30x52 tokens), self-attention, 2 heads"),
        Workload("wan1.3b_480p81f_self", 1, 12, 32760, 32760, HEAD_DIM, 1.0, 1.0, "bf16", 0.0,
                 20250001, "Wan-1.3B-shaped self-attention, 480x832x81 frames (21x30x52 tokens)"),
        Workload("wan14b_text_cross", 2, 40, 32760, 512, HEAD_DIM, 1.0, 0.5, "bf16", 0.0,
                 20250002, "Wan-14B-shaped text cross-attention, 32760 video x 512 umT5 tokens, "
                 "b=2 (cond/uncond)"),
        Workload("wan14b_720p81f_self", 2, 40, 75600, 75600, HEAD_DIM, 1.0, 1.0, "bf16", 0.0,
                 20250003, "Wan-14B-shaped self-attention, 720x1280x81 frames (21x45x80 tokens), "
                 "b=2 (cond/uncond)"),
        Workload("wan14b_720p81f_self_int8fp8", 1, 40, 75600, 75600, HEAD_DIM, 1.0, 1.0,
                 "int8_fp8", 0.01, 20250004,
                 "8-bit path at the 720p 14B shape, N(0,1) plus 1% outlier channels at 8 sigma"),
    ]
}


def _draw(gen, shape, sigma, device, col_scale=None):
    b = shape[0]
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    for bb in range(b):
        x = torch.randn(shape[1:], generator=gen, dtype=torch.float32, device=device)
        if sigma != 1.0:
            x.mul_(sigma)
        if col_scale is not None:
            x.mul_(col_scale)
        out[bb].copy_(x)          # float32 -> bfloat16, round to nearest even
        del x
    return out


def outlier_columns(w, which):
    """(head, channel) columns scaled by 8 for tensor ``which`` in (0: Q, 1: K, 2: V)."""
    n = int(round(w.outlier_frac * w.heads * w.head_dim))
    if n == 0:
        return torch.empty(0, dtype=torch.long)
    g = torch.Generator().manual_seed(w.seed + 1)
    cols = None
    for _ in range(which + 1):
        cols = torch.randperm(w.heads * w.head_dim, generator=g)[:n]
    return cols


def _col_scale(w, which, device):
    cols = outlier_columns(w, which)
    if cols.numel() == 0:
        return None
    s = torch.ones(w.heads * w.head_dim, dtype=torch.float32)
    s[cols] = 8.0
    return s.view(w.heads, w.head_dim).to(device)


def make_qkv(w, device="cpu"):
    """Q [b, s_q, H, d], K and V [b, s_kv, H, d], bfloat16 on ``device``."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    gen = torch.Generator(device=device).manual_seed(w.seed)
    q = _draw(gen, (w.batch, w.s_q, w.heads, w.head_dim), w.sigma_q, device, _col_scale(w, 0, device))
    k = _draw(gen, (w.batch, w.s_kv, w.heads, w.head_dim), w.sigma_kv, device, _col_scale(w, 1, device))
    v = _draw(gen, (w.batch, w.s_kv, w.heads, w.head_dim), w.sigma_kv, device, _col_scale(w, 2, device))
    return q, k, v


def random_qkv(batch, heads, s_q, s_kv, seed, head_dim=HEAD_DIM, sigma=1.0, device="cpu"):
    """Ad-hoc seeded shapes (parity sweeps over tails): N(0, sigma^2) rounded to bfloat16."""
    w = Workload("adhoc", batch, heads, s_q, s_kv, head_dim, sigma, sigma, "bf16", 0.0, seed, "")
    return make_qkv(w, device)


def sample_rows(w, n=4096):
    """``n`` distinct (batch, head, query row) triples, int64 [n, 3] (all rows if fewer exist)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    total = w.batch * w.heads * w.s_q
    g = torch.Generator().manual_seed(w.seed + 2)
    flat = torch.randperm(total, generator=g)[:min(n, total)]
    bh, i = flat // w.s_q, flat % w.s_q
    return torch.stack([bh // w.heads, bh % w.heads, i], dim=1)


# ---------------------------------------------------------------------------------------------
# FP8 GEMM of the DiT linear layers (y = x w^T).  The pages give the model width only through the
# attention shape: 40 heads x 128 channels = 5,120 for the 14B model (12 x 128 = 1,536 for 1.3B);
# they print no FFN width, so the workloads are the width-preserving projections (the Q, K, V and
# output projections of a block), m = the 75,600 video tokens of one 720p, 81-frame sample.
# Recipe: activations x [m, k] are N(0, 1) with 1% of the input-feature columns (picked without
# replacement from a CPU generator seeded with seed + 1) multiplied by 8 -- outlier channels, the
# reason activations get a scale per token; weights w [n, k] are N(0, 1/k).  Each is drawn from
# its own torch.Generator on the target device (x with seed, w with seed + 2), rounded to bf16.


@dataclass(frozen=True)
class LinearWorkload:
    name: str
    m: int
    n: int
    k: int
    outlier_frac: float
    seed: int
    description: str

    @property
    def flops(self):
        return 2 * self.m * self.n * self.k


LINEAR_WORKLOADS = {
    w.name: w for w in [
        LinearWorkload("wan14b_720p_proj_fp8", 75600, 5120, 5120, 0.01, 20250010,
                       "Wan-14B width-preserving projection (5120 -> 5120) over the 75,600 tokens "
                       "of a 720x1280x81 sample, FP8 e4m3 with per-token / per-tensor scales"),
        LinearWorkload("wan1.3b_480p_proj_fp8", 32760, 1536, 1536, 0.01, 20250011,
                       "Wan-1.3B width-preserving projection (1536 -> 1536) over the 32,760 tokens "
                       "of a 480x832x81 sample"),
    ]
}


def random_activations(m, k, seed, outlier_frac=0.01, device="cpu"):
    """x [m, k] bfloat16: N(0, 1), round(outlier_frac * k) columns scaled by 8."""
    gen = torch.Generator(device=device).manual_seed(seed)
    x = torch.randn((m, k), generator=gen, dtype=torch.float32, device=device)
    n_out = int(round(outlier_frac * k))
    if n_out:
        cols = torch.randperm(k, generator=torch.Generator().manual_seed(seed + 1))[:n_out]
        x[:, cols.to(device)] *= 8.0
    return x.to(torch.bfloat16)


def random_weights(n, k, seed, device="cpu"):
    """w [n, k] bfloat16: N(0, 1/k)."""
    gen = torch.Generator(device=device).manual_seed(seed + 2)
    w = torch.randn((n, k), generator=gen, dtype=torch.float32, device=device)
    return w.mul_(k ** -0.5).to(torch.bfloat16)


def make_linear(w, device="cpu"):
    """(x [m, k], w [n, k]) bfloat16 for a linear workload (name or LinearWorkload)."""
    if isinstance(w, str):
        w = LINEAR_WORKLOADS[w]
    return random_activations(w.m, w.k, w.seed, w.outlier_frac, device), random_weights(w.n, w.k, w.seed, device)


# ---------------------------------------------------------------------------------------------
# Block-sparse (VSA-style) attention.  The FastWan / VSA article fine-tunes Wan-1.3B with VSA on a
# 16 x 28 x 52 video latent (taken here as the token grid: 16 latent frames of 28 x 52 tokens,
# 23,296 tokens; the 1.3B model has 12 heads of 128) and quotes the fine kernel's speed against
# dense attention on long sequences, so the second workload is the 720p, 81-frame 14B shape
# (75,600 tokens, 40 heads).  Both keep ceil(n_kb / 8) of the 64-token key blocks (87.5% sparsity).
# Q, K, V follow make_qkv's recipe (N(0, 1) in bf16, one generator seeded with the seed).


@dataclass(frozen=True)
class VsaWorkload:
    name: str
    batch: int
    heads: int
    s: int
    keep: int
    seed: int
    description: str

    @property
    def dense_flops(self):
        return 4 * self.batch * self.heads * self.s * self.s * HEAD_DIM


VSA_WORKLOADS = {
    w.name: w for w in [
        VsaWorkload("wan1.3b_vsa_16x28x52", 1, 12, 16 * 28 * 52, 46, 20250020,
                    "Wan-1.3B-shaped self-attention over a 16x28x52 latent token grid, keep 46 of 364 "
                    "key blocks"),
        VsaWorkload("wan14b_720p81f_vsa", 1, 40, 75600, 148, 20250021,
                    "Wan-14B-shaped self-attention, 720x1280x81 frames (21x45x80 tokens), keep 148 of "
                    "1,182 key blocks"),
    ]
}


def make_vsa(w, device="cpu"):
    """Q, K, V [b, s, H, 128] bfloat16 for a block-sparse workload (name or VsaWorkload)."""
    if isinstance(w, str):
        w = VSA_WORKLOADS[w]
    return random_qkv(w.batch, w.heads, w.s, w.s, w.seed, device=device)
