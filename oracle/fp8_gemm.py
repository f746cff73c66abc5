"""FP8 GEMM of the DiT linear layers -- test infrastructure (see the package docstring).

What the pages fix: at inference the matrix multiplications of the model's linear layers (the
alpha term of the DiT cost model) run in FP8, the weights quantised per tensor and the
activations per token, which almost doubles the speed of those modules ("Wan模型是什么它能做什么"
explainer, section 4.2; "Wan 2.1: VBench 86.22% ..." explainer, section "干预与形式化": FP8 GEMM,
1.13x end to end).  What they leave open, and the reading taken here (each one also lives in the
GPU path, which is written separately):

  1. Format: OCP e4m3fn, the format of the 8-bit attention's FP8 operands.
  2. Activations X [M, K] (tokens x input features), per token (row) m: amax = max_k |X[m, k]|,
     inv = 448 / amax, code = e4m3fn(clamp(X * inv, +-448)), scale = amax / 448; a zero row takes
     inv = scale = 1, so its codes are zeros (0x80 for a negative zero).
  3. Weights W [N, K] (output features x input features, the layout of y = x W^T): one scale for
     the whole tensor, by the same rule with amax over all of W.
  4. Y[m, n] = (sum_k X~[m, k] * W~[n, k]) * scale_x[m] * scale_w, then rounded to bf16.  No bias:
     the pages do not mention one, and a bias add is not part of the product.

Quantisation decisions are taken in float32, as the GPU path takes them, so that codes and scales
compare bit for bit.  The product is exact here: a product of two e4m3fn values is a multiple of
2^-18 below 2^17.6 in magnitude, so for K < 2^21 every partial sum of K such products is an
integer multiple of 2^-18 below 2^53 * 2^-18 -- exactly representable in float64, whatever the
summation order of the library matmul.  The scaling runs in float64.
"""

import numpy as np

from .numerics import e4m3fn_decode, e4m3fn_encode, e4m3fn_round

F32 = np.float32
E4M3_MAX = F32(448.0)


def _codes(x, amax):
    """e4m3fn codes of x (float32) against amax (float32 scalar or column), and the scale."""
    x = np.asarray(x, F32)
    amax = np.asarray(amax, F32)
    ok = amax > 0
    inv = np.where(ok, (E4M3_MAX / np.where(ok, amax, F32(1))).astype(F32), F32(1)).astype(F32)
    scale = np.where(ok, (amax / E4M3_MAX).astype(F32), F32(1)).astype(F32)
    prod = (x * inv).astype(F32)
    return e4m3fn_encode(e4m3fn_round(prod)), scale


def quantize_rows(x):
    """Reading 2: per-token (row) quantisation of X [M, K] -> (codes uint8 [M, K], scales float32 [M])."""
    x = np.asarray(x, F32)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], F32)
    codes, scale = _codes(x, amax[:, None].astype(F32))
    return codes, scale[:, 0]


def quantize_tensor(w):
    """Reading 3: per-tensor quantisation of W [N, K] -> (codes uint8 [N, K], scale float32)."""
    w = np.asarray(w, F32)
    amax = F32(np.abs(w).max()) if w.size else F32(0)
    codes, scale = _codes(w, amax)
    return codes, F32(scale)


def gemm(x_codes, x_scales, w_codes, w_scale):
    """Reading 4 without the final rounding: Y [M, N] float64 = (X~ W~^T) * scale_x[m] * scale_w,
    the product exact (see the module docstring)."""
    xv = e4m3fn_decode(x_codes)
    wv = e4m3fn_decode(w_codes)
    assert xv.shape[1] == wv.shape[1] and xv.shape[1] < 2 ** 21
    acc = xv @ wv.T
    return acc * np.asarray(x_scales, np.float64)[:, None] * np.float64(w_scale)


def gemm_rows(x_codes, x_scales, w_codes, w_scale, rows):
    """The rows `rows` of gemm(...) -> [len(rows), N] float64."""
    rows = np.asarray(rows, np.int64)
    return gemm(np.asarray(x_codes)[rows], np.asarray(x_scales)[rows], w_codes, w_scale)


def accumulation_bound(x_codes, x_scales, w_codes, w_scale, rows=None):
    """Per-element bound [len(rows), N] on the error of a float32 accumulation of the same
    products in any order: K * 2^-24 * sum_k |X~[m,k] W~[n,k]| * scale_x[m] * scale_w (the
    standard worst-case bound for a recursive sum of K terms)."""
    xc = np.asarray(x_codes) if rows is None else np.asarray(x_codes)[np.asarray(rows, np.int64)]
    xs = np.asarray(x_scales, np.float64) if rows is None else np.asarray(x_scales, np.float64)[np.asarray(rows, np.int64)]
    xa = np.abs(e4m3fn_decode(xc))
    wa = np.abs(e4m3fn_decode(w_codes))
    k = xa.shape[1]
    return k * 2.0 ** -24 * (xa @ wa.T) * xs[:, None] * np.float64(w_scale)


def linear(x, w):
    """Both quantisations, then the product: Y [M, N] float64 for bf16 inputs x [M, K], w [N, K]."""
    xc, xs = quantize_rows(x)
    wc, ws = quantize_tensor(w)
    return gemm(xc, xs, wc, ws)
