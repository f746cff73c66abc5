"""The 8-bit attention scheme, step by step -- test infrastructure (see the package docstring).

What the pages fix: the Wan 8-bit FlashAttention multiplies Q and K in int8, runs the second,
output-producing product in FP8, and accumulates in FP32 across KV blocks ("Wan 2.1: VBench
86.22% ..." explainer, section "干预与形式化", DiT backbone paragraph; "Wan模型是什么它能做什么"
explainer, section 4.2).  What they leave open, and the reading taken here (each one also lives in
the 8-bit GPU path, which is written separately):

  1. Channel smoothing.  Per (batch, head, channel c): a_q = max_t |Q[t,c]|, a_k = max_t |K[t,c]|,
     alpha_c = sqrt(a_k / a_q) (1 when either is 0), Q' = Q * alpha, K' = K * (1 / alpha).
     Q'K'^T equals QK^T in real arithmetic; it only balances the int8 range of the two operands.
  2. Q' and K': one symmetric int8 scale per (batch, head, 64-token block starting at token 0)
     over all 128 channels; a partial last block uses its real tokens.  amax = max |x| over the
     block, inv = 127 / amax, code = clamp(round_half_even(x * inv), -127, 127), scale = amax / 127
     (amax = 0 gives code 0 and scale 1).
  3. V: one scale per (batch, head, channel) over all keys.  inv = 448 / amax, code =
     e4m3fn(clamp(V * inv, +-448)), scale = amax / 448.
  4. Per KV block: S = (int32 sum_c q_code * k_code) * scale_q * scale_k / sqrt(128).
  5. m' = max(m, row max of S); alpha = exp(m - m'); p = exp(S - m').
  6. P~ = e4m3fn(p * 2^8): the power-of-two factor keeps p in the normal range of e4m3fn and is
     removed again at the end.
  7. O = alpha * O + P~ . V~ ; l = alpha * l + sum P~ (the row sum adds the same FP8 weights that
     multiply V, so the output is a weighted mean whose weights sum to one; the pages fix only that
     the accumulation across KV blocks is FP32, not whether the normaliser uses P before or after
     its FP8 rounding).
  8. Out = bf16(O * scale_v[c] / l)   (l carries the factor 2^8 of P~).

Quantisation decisions (steps 1-3) are taken in float32, as the GPU path takes them, so that the
int8 and e4m3 codes can be compared bit for bit.  Steps 4-8 run in float64: this emulator is a
diagnostic reference; the 8-bit path's accuracy bounds are still taken against the exact attention.
"""

import numpy as np

from .numerics import bf16_round, e4m3fn_round, e4m3fn_encode, e4m3fn_decode, int8_codes

F32 = np.float32


def _smoothing(qh, kh):
    """Per-channel smoothing factors alpha (float32 [d]) for one head's q [s_q,d], k [s_kv,d]."""
    aq = np.abs(qh).max(axis=0).astype(F32)
    ak = np.abs(kh).max(axis=0).astype(F32)
    alpha = np.ones_like(aq)
    ok = (aq > 0) & (ak > 0)
    alpha[ok] = np.sqrt((ak[ok] / aq[ok]).astype(F32)).astype(F32)
    return alpha


def _block_int8(x, block):
    """Step 2 for one head: x [s, d] float32 -> (codes int8 [s, d], scales float32 [nblocks])."""
    s = x.shape[0]
    nb = (s + block - 1) // block
    codes = np.zeros(x.shape, dtype=np.int8)
    scales = np.ones(nb, dtype=F32)
    for blk in range(nb):
        xb = x[blk * block:(blk + 1) * block]
        amax = F32(np.abs(xb).max()) if xb.size else F32(0)
        if amax > 0:
            inv = F32(F32(127.0) / amax)
            codes[blk * block:(blk + 1) * block] = int8_codes(xb, inv)
            scales[blk] = F32(amax / F32(127.0))
    return codes, scales


def _channel_e4m3(vh):
    """Step 3 for one head: v [s_kv, d] float32 -> (e4m3 codes uint8 [s_kv, d], scales [d])."""
    amax = np.abs(vh).max(axis=0).astype(F32)
    inv = np.ones_like(amax)
    scale = np.ones_like(amax)
    ok = amax > 0
    inv[ok] = (F32(448.0) / amax[ok]).astype(F32)
    scale[ok] = (amax[ok] / F32(448.0)).astype(F32)
    prod = (vh.astype(F32) * inv[None, :]).astype(F32)
    return e4m3fn_encode(e4m3fn_round(prod)), scale


def quantize_head(qh, kh, vh, block=64, smooth=True):
    """Steps 1-3 for one (batch, head); inputs float32 [s, d] holding the bf16 input values."""
    qh = np.asarray(qh, F32)
    kh = np.asarray(kh, F32)
    vh = np.asarray(vh, F32)
    d = qh.shape[1]
    alpha = _smoothing(qh, kh) if smooth else np.ones(d, F32)
    beta = (F32(1.0) / alpha).astype(F32)
    qs = (qh * alpha[None, :]).astype(F32)
    ks = (kh * beta[None, :]).astype(F32)
    q_codes, q_scale = _block_int8(qs, block)
    k_codes, k_scale = _block_int8(ks, block)
    v_codes, v_scale = _channel_e4m3(vh)
    return dict(q_codes=q_codes, q_scale=q_scale, k_codes=k_codes, k_scale=k_scale,
                v_codes=v_codes, v_scale=v_scale, alpha=alpha)


def attn8_quantize(q, k, v, block=64, smooth=True, heads=None):
    """Steps 1-3 over [b, s, H, d] arrays.  Returns a dict of per-(b, h) results keyed by (b, h);
    ``heads`` restricts the work to the given (b, h) pairs."""
    b, _, H, _ = q.shape
    pairs = heads if heads is not None else [(bb, hh) for bb in range(b) for hh in range(H)]
    return {(int(bb), int(hh)): quantize_head(q[bb, :, hh, :], k[bb, :, hh, :], v[bb, :, hh, :],
                                              block, smooth)
            for bb, hh in pairs}


def _attend_head(qz, qi, kv_block, block):
    """Steps 4-8 for query rows ``qi`` of one head, given its quantised operands."""
    qc = qz["q_codes"][qi].astype(np.float64)                 # [n, d] integer-valued
    sq = qz["q_scale"][qi // block].astype(np.float64)        # [n]
    kc = qz["k_codes"].astype(np.float64)                      # [s_kv, d]
    s_kv, d = kc.shape
    sk = np.repeat(qz["k_scale"].astype(np.float64), block)[:s_kv]   # [s_kv]
    vt = e4m3fn_decode(qz["v_codes"])                          # [s_kv, d] e4m3 values
    n = qc.shape[0]
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    o = np.zeros((n, d))
    inv_sqrt_d = 1.0 / np.sqrt(np.float64(d))
    for j0 in range(0, s_kv, kv_block):
        j1 = min(j0 + kv_block, s_kv)
        acc = qc @ kc[j0:j1].T          # integers below 128*127^2 < 2^53: exact in float64
        S = acc * sq[:, None] * sk[None, j0:j1] * inv_sqrt_d
        m_new = np.maximum(m, S.max(axis=1))
        a = np.exp(m - m_new)
        p = np.exp(S - m_new[:, None])
        pt = e4m3fn_round(p * 256.0)
        l = a * l + pt.sum(axis=1)
        o = a[:, None] * o + pt @ vt[j0:j1]
        m = m_new
    out = (o * qz["v_scale"].astype(np.float64)[None, :]) / l[:, None]
    return bf16_round(out.astype(F32))


def attn8_emulate(q, k, v, rows, kv_block=64, block=64, smooth=True, quantized=None):
    """8-bit attention output for selected rows (integer [n, 3] of (batch, head, query index)).
    Returns float32 [n, d] holding bf16 values.  ``quantized`` may pass a result of
    ``attn8_quantize`` covering the needed heads."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    d = q.shape[-1]
    out = np.empty((rows.shape[0], d), dtype=F32)
    if rows.shape[0] == 0:
        return out
    pairs = [tuple(p) for p in np.unique(rows[:, :2], axis=0)]
    qz_all = quantized if quantized is not None else attn8_quantize(q, k, v, block, smooth, pairs)
    for bb, hh in pairs:
        sel = np.nonzero((rows[:, 0] == bb) & (rows[:, 1] == hh))[0]
        out[sel] = _attend_head(qz_all[(int(bb), int(hh))], rows[sel, 2], kv_block, block)
    return out
