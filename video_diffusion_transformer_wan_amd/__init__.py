"""Python binding of the Wan attention library (libwan_attn.so, hand-written HIP for gfx950).

Argument marshalling only: every step of the attention runs in the library's kernels.  The
functions below carry the C ABI's names (include/wan_attn.h) and take either raw device
addresses (ints) or torch tensors for the pointer arguments; torch serves for device memory and
streams.  ``attention`` is a convenience wrapper that allocates the output.

The library must have been built (``video_diffusion_transformer_wan_amd.build.build()``); there is
no fallback -- loading fails loudly when it is missing.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwan_attn.so")

WAN_ATTN_BF16 = 0
WAN_ATTN_INT8_FP8 = 1
DTYPES = {"bf16": WAN_ATTN_BF16, "int8_fp8": WAN_ATTN_INT8_FP8}

WAN_ATTN_OK = 0
WAN_ATTN_EINVAL = -1
WAN_ATTN_EALIGN = -2
WAN_ATTN_ENOMEM = -3
WAN_ATTN_ELAUNCH = -4
WAN_ATTN_EUNSUPPORTED = -5

QUANT_BLOCK = 64
HEAD_DIM = 128


class WanAttnError(RuntimeError):
    def __init__(self, code, fn):
        self.code = code
        super().__init__(f"{fn} failed with {code}: {wan_attn_strerror(code)}")


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64

_SIGNATURES = {
    "wan_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, ctypes.c_int, _P]),
    "wan_attn8_quantize": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                          _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "wan_attn8_quantize_scratch_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "wan_attn8_fwd_quantized": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P,
                                               _I64, _I64, _I64, _I64, _I64, _P]),
    "wan_attn_fwd_lse": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P]),
    "wan_attn_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P]),
    "wan_attn_bwd_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P]),
    "wan_fp8_quantize_rows": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "wan_fp8_quantize_tensor": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "wan_fp8_gemm": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "wan_vsa_select_scratch_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64]),
    "wan_vsa_select": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P]),
    "wan_vsa_attn": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P]),
    "wan_vsa_fwd": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P]),
    "wan_attn_release_scratch": (ctypes.c_int, []),
    "wan_attn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "wan_attn_version": (ctypes.c_int, []),
}


def lib():
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "video_diffusion_transformer_wan_amd.build.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc, fn):
    if rc != WAN_ATTN_OK:
        raise WanAttnError(rc, fn)


def wan_attn_strerror(code):
    return lib().wan_attn_strerror(code).decode()


def wan_attn_version():
    return lib().wan_attn_version()


def wan_attn_release_scratch():
    """Return the library's cached scratch memory to the driver (no call may be in flight)."""
    _check(lib().wan_attn_release_scratch(), "wan_attn_release_scratch")


def wan_attn_fwd(q, k, v, o, batch, heads, s_q, s_kv, head_dim, dtype, stream=None):
    dtype = DTYPES.get(dtype, dtype)
    rc = lib().wan_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), batch, heads, s_q, s_kv, head_dim,
                            dtype, _stream(stream))
    _check(rc, "wan_attn_fwd")


def wan_attn_fwd_lse(q, k, v, o, lse, batch, heads, s_q, s_kv, head_dim, stream=None):
    rc = lib().wan_attn_fwd_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), batch, heads, s_q, s_kv,
                                head_dim, _stream(stream))
    _check(rc, "wan_attn_fwd_lse")


def wan_attn_bwd(q, k, v, o, d_o, lse, dq, dk, dv, batch, heads, s_q, s_kv, head_dim, stream=None):
    rc = lib().wan_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk),
                            _ptr(dv), batch, heads, s_q, s_kv, head_dim, _stream(stream))
    _check(rc, "wan_attn_bwd")


def wan_attn_bwd_noalloc(q, k, v, o, d_o, lse, dq, dk, dv, batch, heads, s_q, s_kv, head_dim, stream=None):
    rc = lib().wan_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk),
                                    _ptr(dv), batch, heads, s_q, s_kv, head_dim, _stream(stream))
    _check(rc, "wan_attn_bwd_noalloc")


def wan_attn8_quantize_scratch_bytes(batch, heads):
    return lib().wan_attn8_quantize_scratch_bytes(batch, heads)


def wan_attn8_quantize(q, k, v, batch, heads, s_q, s_kv, head_dim, q_codes, q_scale, k_codes,
                       k_scale, v_codes, v_scale, smooth, scratch, stream=None):
    rc = lib().wan_attn8_quantize(_ptr(q), _ptr(k), _ptr(v), batch, heads, s_q, s_kv, head_dim,
                                  _ptr(q_codes), _ptr(q_scale), _ptr(k_codes), _ptr(k_scale),
                                  _ptr(v_codes), _ptr(v_scale), _ptr(smooth), _ptr(scratch),
                                  _stream(stream))
    _check(rc, "wan_attn8_quantize")


def wan_attn8_fwd_quantized(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, o, batch, heads,
                            s_q, s_kv, head_dim, stream=None):
    rc = lib().wan_attn8_fwd_quantized(_ptr(q_codes), _ptr(q_scale), _ptr(k_codes), _ptr(k_scale),
                                       _ptr(v_codes), _ptr(v_scale), _ptr(o), batch, heads, s_q,
                                       s_kv, head_dim, _stream(stream))
    _check(rc, "wan_attn8_fwd_quantized")


def _require(name, t, dtype, shape, device):
    """Every tensor handed to the library: a contiguous tensor of ``dtype`` and exactly ``shape`` on
    the CUDA device ``device`` (a wrong dtype or size, a strided view, host memory or another GPU
    raise ValueError before any library call)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    return t


def _check_tensors(q, k, v):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda
                or not t.is_contiguous() or t.dim() != 4):
            raise ValueError(f"{name} must be a contiguous 4-d bfloat16 CUDA tensor [b, s, H, d]")
    b, s_q, H, d = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[2] != H or k.shape[3] != d:
        raise ValueError("k and v must be [b, s_kv, H, d] matching q [b, s_q, H, d]")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on the same device")
    return b, H, s_q, k.shape[1], d


def attention(q, k, v, dtype="bf16", out=None, stream=None):
    """softmax(q k^T / sqrt(d)) v per (batch, head) for q [b, s_q, H, 128], k, v [b, s_kv, H, 128]
    bfloat16 CUDA tensors; returns a new (or fills ``out``) [b, s_q, H, 128] bfloat16 tensor."""
    import torch
    b, H, s_q, s_kv, d = _check_tensors(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _require("out", out, torch.bfloat16, q.shape, q.device)
    wan_attn_fwd(q, k, v, out, b, H, s_q, s_kv, d, dtype, stream)
    return out


def attention8_quantize(q, k, v, stream=None):
    """Stage 1 of the 8-bit path on torch tensors; returns a dict of the codes and scales
    (layouts as in include/wan_attn.h)."""
    import torch
    b, H, s_q, s_kv, d = _check_tensors(q, k, v)
    nbq = -(-s_q // QUANT_BLOCK)
    nbk = -(-s_kv // QUANT_BLOCK)
    dev = q.device
    out = dict(
        q_codes=torch.empty((b, s_q, H, d), dtype=torch.int8, device=dev),
        k_codes=torch.empty((b, s_kv, H, d), dtype=torch.int8, device=dev),
        q_scale=torch.empty((b, H, nbq), dtype=torch.float32, device=dev),
        k_scale=torch.empty((b, H, nbk), dtype=torch.float32, device=dev),
        v_codes=torch.empty((b, H, d, nbk * QUANT_BLOCK), dtype=torch.uint8, device=dev),
        v_scale=torch.empty((b, H, d), dtype=torch.float32, device=dev),
        smooth=torch.empty((b, H, d), dtype=torch.float32, device=dev),
    )
    scratch = torch.empty(wan_attn8_quantize_scratch_bytes(b, H) // 4, dtype=torch.float32, device=dev)
    wan_attn8_quantize(q, k, v, b, H, s_q, s_kv, d, out["q_codes"], out["q_scale"], out["k_codes"],
                       out["k_scale"], out["v_codes"], out["v_scale"], out["smooth"], scratch, stream)
    out["_scratch"] = scratch
    return out


def _quantized_shapes(b, H, s_q, s_kv):
    nbq = -(-s_q // QUANT_BLOCK)
    nbk = -(-s_kv // QUANT_BLOCK)
    import torch
    return dict(q_codes=((b, s_q, H, HEAD_DIM), torch.int8), k_codes=((b, s_kv, H, HEAD_DIM), torch.int8),
                q_scale=((b, H, nbq), torch.float32), k_scale=((b, H, nbk), torch.float32),
                v_codes=((b, H, HEAD_DIM, nbk * QUANT_BLOCK), torch.uint8), v_scale=((b, H, HEAD_DIM), torch.float32))


def attention8_from_quantized(z, b, H, s_q, s_kv, out=None, stream=None):
    """Stage 2 of the 8-bit path from the dict of ``attention8_quantize``."""
    import torch
    dev = z["q_codes"].device if isinstance(z.get("q_codes"), torch.Tensor) else None
    for name, (shape, dtype) in _quantized_shapes(b, H, s_q, s_kv).items():
        _require(name, z.get(name), dtype, shape, dev)
    if out is None:
        out = torch.empty((b, s_q, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    _require("out", out, torch.bfloat16, (b, s_q, H, HEAD_DIM), dev)
    wan_attn8_fwd_quantized(z["q_codes"], z["q_scale"], z["k_codes"], z["k_scale"], z["v_codes"],
                            z["v_scale"], out, b, H, s_q, s_kv, HEAD_DIM, stream)
    return out


def attention_with_lse(q, k, v, stream=None):
    """bf16 forward that also returns the row log-sum-exp: (o [b, s_q, H, 128] bf16,
    lse [b, H, s_q] float32)."""
    import torch
    b, H, s_q, s_kv, d = _check_tensors(q, k, v)
    out = torch.empty_like(q)
    lse = torch.empty((b, H, s_q), dtype=torch.float32, device=q.device)
    wan_attn_fwd_lse(q, k, v, out, lse, b, H, s_q, s_kv, d, stream)
    return out, lse


def attention_backward(q, k, v, o, lse, d_o, stream=None):
    """Gradients (dq, dk, dv) of the bf16 attention for upstream gradient d_o, from the forward's
    output o and row log-sum-exp lse (attention_with_lse); new bfloat16 tensors."""
    import torch
    b, H, s_q, s_kv, d = _check_tensors(q, k, v)
    _require("o", o, torch.bfloat16, q.shape, q.device)
    _require("d_o", d_o, torch.bfloat16, q.shape, q.device)
    _require("lse", lse, torch.float32, (b, H, s_q), q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wan_attn_bwd(q, k, v, o, d_o, lse, dq, dk, dv, b, H, s_q, s_kv, d, stream)
    return dq, dk, dv


def wan_fp8_quantize_rows(x, rows, cols, codes, scales, stream=None):
    rc = lib().wan_fp8_quantize_rows(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream))
    _check(rc, "wan_fp8_quantize_rows")


def wan_fp8_quantize_tensor(w, rows, cols, codes, scale, stream=None):
    rc = lib().wan_fp8_quantize_tensor(_ptr(w), rows, cols, _ptr(codes), _ptr(scale), _stream(stream))
    _check(rc, "wan_fp8_quantize_tensor")


def wan_fp8_gemm(x_codes, x_scales, w_codes, w_scale, y, m, n, k, stream=None):
    rc = lib().wan_fp8_gemm(_ptr(x_codes), _ptr(x_scales), _ptr(w_codes), _ptr(w_scale), _ptr(y), m, n, k,
                            _stream(stream))
    _check(rc, "wan_fp8_gemm")


def _check_matrix(name, t):
    import torch
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
        raise ValueError(f"{name} must be a contiguous 2-d bfloat16 CUDA tensor")
    return t.shape


def fp8_quantize_rows(x, stream=None):
    """Per-token e4m3fn quantisation of x [m, k] bf16: (codes [m, k] uint8, scales [m] float32)."""
    import torch
    m, k = _check_matrix("x", x)
    codes = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    scales = torch.empty((m,), dtype=torch.float32, device=x.device)
    wan_fp8_quantize_rows(x, m, k, codes, scales, stream)
    return codes, scales


def fp8_quantize_tensor(w, stream=None):
    """Per-tensor e4m3fn quantisation of w [n, k] bf16: (codes [n, k] uint8, scale [1] float32)."""
    import torch
    n, k = _check_matrix("w", w)
    codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    scale = torch.empty((1,), dtype=torch.float32, device=w.device)
    wan_fp8_quantize_tensor(w, n, k, codes, scale, stream)
    return codes, scale


def fp8_gemm(x_codes, x_scales, w_codes, w_scale, out=None, stream=None):
    """y [m, n] bf16 = (x_codes [m, k] . w_codes [n, k]^T) * x_scales[m] * w_scale, from the codes and
    scales of fp8_quantize_rows / fp8_quantize_tensor."""
    import torch
    if not isinstance(x_codes, torch.Tensor) or x_codes.dim() != 2:
        raise ValueError("x_codes must be a 2-d uint8 CUDA tensor [m, k]")
    if not isinstance(w_codes, torch.Tensor) or w_codes.dim() != 2:
        raise ValueError("w_codes must be a 2-d uint8 CUDA tensor [n, k]")
    m, k = x_codes.shape
    n = w_codes.shape[0]
    dev = x_codes.device
    _require("x_codes", x_codes, torch.uint8, (m, k), dev)
    _require("w_codes", w_codes, torch.uint8, (n, k), dev)
    _require("x_scales", x_scales, torch.float32, (m,), dev)
    _require("w_scale", w_scale, torch.float32, (1,), dev)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    _require("out", out, torch.bfloat16, (m, n), dev)
    wan_fp8_gemm(x_codes, x_scales, w_codes, w_scale, out, m, n, k, stream)
    return out


def fp8_linear(x, w_codes, w_scale, out=None, stream=None):
    """y = x w^T in FP8 for x [m, k] bf16 and a weight quantised once with fp8_quantize_tensor."""
    xc, xs = fp8_quantize_rows(x, stream)
    return fp8_gemm(xc, xs, w_codes, w_scale, out, stream)


VSA_BLOCK = 64


def vsa_default_keep(s_kv):
    """ceil(n_kb / 8) key blocks of 64 tokens: 87.5% sparsity."""
    return max(1, -(-(-(-s_kv // VSA_BLOCK)) // 8))


def wan_vsa_select_scratch_bytes(batch, heads, s_q, s_kv):
    return lib().wan_vsa_select_scratch_bytes(batch, heads, s_q, s_kv)


def wan_vsa_select(q, k, batch, heads, s_q, s_kv, head_dim, keep, block_idx, scratch, stream=None):
    rc = lib().wan_vsa_select(_ptr(q), _ptr(k), batch, heads, s_q, s_kv, head_dim, keep, _ptr(block_idx),
                              _ptr(scratch), _stream(stream))
    _check(rc, "wan_vsa_select")


def wan_vsa_attn(q, k, v, block_idx, o, batch, heads, s_q, s_kv, head_dim, keep, stream=None):
    rc = lib().wan_vsa_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(o), batch, heads, s_q, s_kv, head_dim,
                            keep, _stream(stream))
    _check(rc, "wan_vsa_attn")


def wan_vsa_fwd(q, k, v, o, batch, heads, s_q, s_kv, head_dim, keep, stream=None):
    rc = lib().wan_vsa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), batch, heads, s_q, s_kv, head_dim, keep,
                           _stream(stream))
    _check(rc, "wan_vsa_fwd")


def vsa_select(q, k, keep=None, stream=None):
    """Coarse stage of block-sparse attention: the `keep` key blocks (64 tokens) of largest block score
    for every query block, block_idx [b, H, ceil(s_q/64), keep] int32 in ascending order."""
    import torch
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a contiguous 4-d bfloat16 CUDA tensor [b, s, H, d]")
    b, s_q, H, d = q.shape
    _require("q", q, torch.bfloat16, q.shape, q.device)
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        raise ValueError("k must be a contiguous bfloat16 tensor [b, s_kv, H, d] matching q")
    s_kv = k.shape[1]
    _require("k", k, torch.bfloat16, (b, s_kv, H, d), q.device)
    keep = vsa_default_keep(s_kv) if keep is None else keep
    idx = torch.empty((b, H, -(-s_q // VSA_BLOCK), keep), dtype=torch.int32, device=q.device)
    scratch = torch.empty(max(wan_vsa_select_scratch_bytes(b, H, s_q, s_kv), 16) // 4, dtype=torch.float32,
                          device=q.device)
    wan_vsa_select(q, k, b, H, s_q, s_kv, d, keep, idx, scratch, stream)
    return idx


def vsa_attention(q, k, v, block_idx, out=None, stream=None):
    """Fine stage: attention of every query block over the keys of its listed key blocks
    (block_idx [b, H, ceil(s_q/64), keep] int32); returns o [b, s_q, H, 128] bfloat16."""
    import torch
    b, H, s_q, s_kv, d = _check_tensors(q, k, v)
    if not isinstance(block_idx, torch.Tensor) or block_idx.dim() != 4:
        raise ValueError("block_idx must be a contiguous int32 tensor [b, H, ceil(s_q/64), keep]")
    keep = block_idx.shape[3]
    _require("block_idx", block_idx, torch.int32, (b, H, -(-s_q // VSA_BLOCK), keep), q.device)
    if out is None:
        out = torch.empty_like(q)
    _require("out", out, torch.bfloat16, q.shape, q.device)
    wan_vsa_attn(q, k, v, block_idx, out, b, H, s_q, s_kv, d, keep, stream)
    return out


def vsa_forward(q, k, v, keep=None, out=None, stream=None):
    """Both stages in one call (the block list in library scratch); keep None: ceil(n_kb / 8)."""
    import torch
    b, H, s_q, s_kv, d = _check_tensors(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _require("out", out, torch.bfloat16, q.shape, q.device)
    wan_vsa_fwd(q, k, v, out, b, H, s_q, s_kv, d, 0 if keep is None else keep, stream)
    return out
