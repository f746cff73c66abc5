"""Plain, slow CPU oracle for the Wan DiT attention forward -- TEST INFRASTRUCTURE ONLY.

What it computes is the non-causal, full spatio-temporal multi-head attention that every Wan DiT
block runs over its video tokens, and the cross-attention to the 512 umT5 text tokens:

    O[b, i, h, :] = sum_j softmax_j( Q[b,i,h,:] . K[b,j,h,:] / sqrt(d) ) * V[b, j, h, :]

Sources (page title, then section):
  * "Wan 2.1: VBench 86.22% ..." (paper-podcast explainer of the Wan technical report),
    section "先看现象" -- the attention is non-causal, and its forward cost is the beta = 4 term of
    C = L(alpha*b*s*h^2 + beta*b*s^2*h); section "干预与形式化", DiT backbone paragraph -- full
    spatio-temporal self-attention (not windowed), cross-attention injecting umT5, and the 8-bit
    FlashAttention scheme (mixed int8 / FP8, FP32 accumulation across KV blocks).
  * "Wan模型是什么它能做什么" (kwkr.cn explainer), section 4.2 -- int8 for Q and K, FP8 for the
    output-producing product, FP32 register accumulation.
  The pages do not print the softmax formula itself; the oracle uses the standard scaled
  dot-product definition above with d = 128 and scale 1/sqrt(d), and no mask.

Modules:
  exact     -- exact attention in float64, two passes (global row max, then exp / sum / weighted V).
  numerics  -- bit-level rounding to bfloat16, OCP FP8 E4M3 ("e4m3fn") and int8 codes.
  attn8     -- the 8-bit scheme, step by step, as a diagnostic reference for the 8-bit GPU path.
  backward  -- the exact gradients dQ, dK, dV (chain rule through the row softmax) and the row
               log-sum-exp, in float64: the attention backward (beta = 8 term of the cost model,
               same explainer, section "先看现象").
  fp8_gemm  -- the FP8 GEMM of the DiT linear layers (per-token activation and per-tensor weight
               e4m3fn quantisation, exact product): "Wan模型是什么它能做什么" explainer,
               section 4.2.
  block_sparse -- block-sparse attention in the style of Video Sparse Attention: 64-token block
               means, block scores, top-k key blocks per query block, exact attention over the
               selected keys (the FastWan / VSA article, sections on VSA and its kernel).

Who may use it: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``.  The product path (the HIP library and its Python binding) never imports, links or
calls anything here, and nothing here imports the product package.
"""

from .exact import attention, attention_rows, attention_probs  # noqa: F401
from .numerics import (  # noqa: F401
    round_to_binary,
    bf16_round,
    e4m3fn_round,
    e4m3fn_encode,
    e4m3fn_decode,
    int8_codes,
)
from .attn8 import attn8_emulate, attn8_quantize  # noqa: F401
from .backward import attention_backward, lse_rows, dq_rows, dkdv_rows  # noqa: F401
