"""Sequence lengths and cost counts of the Wan DiT attention (host arithmetic, no GPU work).

* Token length: a (1+T) x H x W x 3 video is compressed by the Wan-VAE to a
  [1+T/4, H/8, W/8, 16] latent and patchified with a (1,2,2) kernel, so a DiT block sees
  s = (1 + T/4) * (H/16) * (W/16) video tokens; the text context is 512 umT5 tokens
  ("Wan 2.1: VBench 86.22% ..." explainer of the Wan technical report, section "先看现象" for the
  shapes, section "干预与形式化" for the umT5 context).
* Cost: the attention term of C = L(alpha*b*s*h^2 + beta*b*s^2*h) with beta = 4 for the
  non-causal forward pass (same page, section "先看现象"): per layer 4*b*s_q*s_kv*h FLOPs with
  h = heads * head_dim -- the two products QK^T and PV at 2*s_q*s_kv*head_dim each.
"""

TEXT_TOKENS = 512
PATCH = (1, 2, 2)
VAE_STRIDE = (4, 8, 8)


def latent_shape(frames_minus_one, height, width, channels=16):
    """Latent [1 + T/4, H/8, W/8, C] of a (1+T) x H x W video."""
    t, h, w = VAE_STRIDE
    if frames_minus_one % t or height % h or width % w:
        raise ValueError("T must be a multiple of 4 and H, W multiples of 8")
    return (1 + frames_minus_one // t, height // h, width // w, channels)


def video_tokens(frames_minus_one, height, width):
    """Sequence length after the (1,2,2) patchify of the latent."""
    lt, lh, lw, _ = latent_shape(frames_minus_one, height, width)
    pt, ph, pw = PATCH
    if lt % pt or lh % ph or lw % pw:
        raise ValueError("latent not divisible by the patch")
    return (lt // pt) * (lh // ph) * (lw // pw)


def attention_flops(batch, heads, s_q, s_kv, head_dim=128):
    """Forward FLOPs counted as beta * b * s_q * s_kv * h with beta = 4, h = heads * head_dim."""
    return 4 * batch * heads * s_q * s_kv * head_dim


def attention_bytes(batch, heads, s_q, s_kv, head_dim=128, in_bytes=2, out_bytes=2):
    """Algorithmic HBM bytes: Q, K, V read once and O written once."""
    return batch * heads * head_dim * (s_q * (in_bytes + out_bytes) + 2 * s_kv * in_bytes)


def attention8_kernel_bytes(batch, heads, s_q, s_kv, head_dim=128):
    """Algorithmic HBM bytes of the quantised-operand attention kernel: int8 Q and K, e4m3 V
    (one byte each), bf16 O, plus the fp32 scales."""
    nbq = -(-s_q // 64)
    nbk = -(-s_kv // 64)
    return (batch * heads * head_dim * (s_q * (1 + 2) + 2 * s_kv * 1)
            + 4 * batch * heads * (nbq + nbk + head_dim))


def exp_count(batch, heads, s_q, s_kv):
    """Exponentials of the softmax: one per (query, key) pair."""
    return batch * heads * s_q * s_kv
