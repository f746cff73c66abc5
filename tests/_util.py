"""Shared test helpers: loading the built library, moving tensors to the oracle, error metrics."""

import os

import numpy as np

import video_diffusion_transformer_wan_amd as wan


def ensure_built():
    """Build the HIP library only if nothing is built yet (the build is a separate step)."""
    if not os.path.exists(wan.LIB_PATH):
        from video_diffusion_transformer_wan_amd import build
        build.build()
    return wan.lib()


def to_np(t):
    """bf16 / fp32 torch tensor (any device) -> float32 numpy (exact for bf16)."""
    return t.detach().float().cpu().numpy()


def metrics(got, ref):
    """Global rel-L2, max-abs and cosine over all checked elements, in float64."""
    g = np.asarray(got, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    d = g - r
    rel = float(np.linalg.norm(d) / np.linalg.norm(r))
    maxabs = float(np.max(np.abs(d))) if d.size else 0.0
    cos = float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r)))
    return rel, maxabs, cos


# Bounds of the bf16 path against the exact oracle, and of the 8-bit path (the latter also
# requires cosine similarity >= 0.995).
BF16_REL_L2 = 1e-2
BF16_MAX_ABS = 3e-2
INT8_REL_L2 = 6e-2
INT8_COS = 0.995
# Bounds of the bf16 backward's dQ, dK, dV against the exact gradients (per tensor): rel-L2, and
# max-abs as a fraction of the largest exact magnitude.  The final rounding to bf16 alone gives a
# relative RMS error of about 2^-7/sqrt(12) = 2.3e-3 and a worst case of 2^-8 = 0.4% at the largest
# element; P and dS rounded to bf16 before their products add errors of the same size that average
# out over the sums.  The bounds leave a factor of about 4 and 5 above that.
BWD_REL_L2 = 1e-2
BWD_MAX_REL = 2e-2


def gather_rows(out, rows):
    """out [b, s_q, H, d] torch -> numpy [n, d] at (b, h, i) triples."""
    import torch
    r = torch.as_tensor(rows, dtype=torch.long, device=out.device)
    return to_np(out[r[:, 0], r[:, 2], r[:, 1], :])


def tail_rows(b, H, s_q, tile=256):
    """Every row of the last (partial) query tile for (b=0, h=0) and (b=last, h=last)."""
    start = (s_q - 1) // tile * tile
    i = np.arange(start, s_q)
    a = np.stack([np.zeros_like(i), np.zeros_like(i), i], 1)
    z = np.stack([np.full_like(i, b - 1), np.full_like(i, H - 1), i], 1)
    return np.concatenate([a, z])
