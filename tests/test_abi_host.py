"""The C ABI library on the host, without a GPU: it loads, exports every function that
include/wan_attn.h declares, and rejects bad arguments before any GPU work (the checks return
before the first HIP call, so these run on a machine without a GPU)."""

import ctypes
import os
import re

import pytest

import video_diffusion_transformer_wan_amd as wan
from _util import ensure_built

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "wan_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wan_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ensure_built()
    names = declared_functions()
    assert "wan_attn_fwd" in names and "wan_fp8_gemm" in names and len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror():
    ensure_built()
    assert wan.wan_attn_version() == 1
    for code in (0, -1, -2, -3, -4, -5):
        assert len(wan.wan_attn_strerror(code)) > 5
    assert wan.wan_attn_strerror(123) == "unknown status code"


def _fwd(q=16, k=32, v=48, o=4096, b=1, H=1, sq=1, skv=1, d=128, dtype=0):
    lib = ensure_built()
    return lib.wan_attn_fwd(q, k, v, o, b, H, sq, skv, d, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), wan.WAN_ATTN_EINVAL),
    (dict(o=None), wan.WAN_ATTN_EINVAL),
    (dict(b=0), wan.WAN_ATTN_EINVAL),
    (dict(H=-1), wan.WAN_ATTN_EINVAL),
    (dict(sq=0), wan.WAN_ATTN_EINVAL),
    (dict(skv=0), wan.WAN_ATTN_EINVAL),
    (dict(d=64), wan.WAN_ATTN_EUNSUPPORTED),
    (dict(d=0), wan.WAN_ATTN_EINVAL),
    (dict(dtype=2), wan.WAN_ATTN_EINVAL),
    (dict(dtype=-1), wan.WAN_ATTN_EINVAL),
    (dict(q=17), wan.WAN_ATTN_EALIGN),
    (dict(v=40), wan.WAN_ATTN_EALIGN),
    (dict(o=16), wan.WAN_ATTN_EINVAL),            # output overlaps q
    (dict(sq=1 << 31), wan.WAN_ATTN_EINVAL),      # token count beyond the kernels' counters
])
def test_argument_checks(kw, code):
    assert _fwd(**kw) == code


def test_quantize_argument_checks():
    lib = ensure_built()
    ptrs = [16 * (i + 1) for i in range(11)]
    args = ptrs[:3] + [1, 1, 64, 64, 128] + ptrs[3:] + [None]
    bad = list(args)
    bad[7] = 96
    assert lib.wan_attn8_quantize(*bad) == wan.WAN_ATTN_EUNSUPPORTED
    bad = list(args)
    bad[8] = None
    assert lib.wan_attn8_quantize(*bad) == wan.WAN_ATTN_EINVAL
    bad = list(args)
    bad[9] = 20
    assert lib.wan_attn8_quantize(*bad) == wan.WAN_ATTN_EALIGN
    assert lib.wan_attn8_quantize_scratch_bytes(2, 3) == 2 * 3 * 3 * 128 * 4
    assert lib.wan_attn8_quantize_scratch_bytes(0, 3) == 0
    fargs = [16 * (i + 1) for i in range(7)] + [1, 1, 64, 64, 128, None]
    bad = list(fargs)
    bad[6] = None
    assert lib.wan_attn8_fwd_quantized(*bad) == wan.WAN_ATTN_EINVAL
    bad = list(fargs)
    bad[10] = 0
    assert lib.wan_attn8_fwd_quantized(*bad) == wan.WAN_ATTN_EINVAL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(wan, "_lib", None)
    monkeypatch.setattr(wan, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        wan.lib()


def _bwd(**kw):
    """wan_attn_bwd with distinct, far-apart fake device addresses (never dereferenced: every case
    below fails a check before the first HIP call)."""
    lib = ensure_built()
    names = ["q", "k", "v", "o", "d_o", "lse", "dq", "dk", "dv"]
    args = {n: 4096 * (i + 1) for i, n in enumerate(names)}
    args.update(b=1, H=1, sq=1, skv=1, d=128)
    args.update(kw)
    return lib.wan_attn_bwd(*[args[n] for n in names], args["b"], args["H"], args["sq"], args["skv"],
                            args["d"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), wan.WAN_ATTN_EINVAL),
    (dict(lse=None), wan.WAN_ATTN_EINVAL),
    (dict(dv=None), wan.WAN_ATTN_EINVAL),
    (dict(d_o=4096 * 5 + 8), wan.WAN_ATTN_EALIGN),
    (dict(lse=4096 * 6 + 4), wan.WAN_ATTN_EALIGN),
    (dict(d=64), wan.WAN_ATTN_EUNSUPPORTED),
    (dict(skv=0), wan.WAN_ATTN_EINVAL),
    (dict(H=65537), wan.WAN_ATTN_EINVAL),         # a tile's 64 rows beyond a 32-bit byte offset
    (dict(dq=4096 * 1), wan.WAN_ATTN_EINVAL),     # dq overlaps q
    (dict(dk=4096 * 6), wan.WAN_ATTN_EINVAL),     # dk overlaps lse
    (dict(dv=4096 * 8), wan.WAN_ATTN_EINVAL),     # dv overlaps dk
])
def test_backward_argument_checks(kw, code):
    assert _bwd(**kw) == code


@pytest.mark.parametrize("args,code", [
    ((16, 32, 48, 4096, None), wan.WAN_ATTN_EINVAL),
    ((16, 32, 48, 4096, 8196), wan.WAN_ATTN_EALIGN),
    ((16, 32, 48, 4096, 4096), wan.WAN_ATTN_EINVAL),   # lse overlaps o
])
def test_forward_lse_argument_checks(args, code):
    lib = ensure_built()
    assert lib.wan_attn_fwd_lse(*args, 1, 1, 1, 1, 128, None) == code
    assert lib.wan_attn_fwd_lse(16, 32, 48, 4096, 8192, 1, 1, 1, 1, 96, None) == wan.WAN_ATTN_EUNSUPPORTED


def _fp8(fn, **kw):
    """The FP8 entry points with far-apart fake device addresses (never dereferenced: every case
    fails a check before the first HIP call)."""
    lib = ensure_built()
    if fn == "gemm":
        names = ["xc", "xs", "wc", "ws", "y"]
        args = {n: 1 << (20 + i) for i, n in enumerate(names)}
        args.update(m=1, n=4, k=64)
        args.update(kw)
        return lib.wan_fp8_gemm(*[args[n] for n in names], args["m"], args["n"], args["k"], None)
    args = dict(x=1 << 20, rows=1, cols=64, codes=1 << 21, scales=1 << 22)
    args.update(kw)
    f = lib.wan_fp8_quantize_rows if fn == "rows" else lib.wan_fp8_quantize_tensor
    return f(args["x"], args["rows"], args["cols"], args["codes"], args["scales"], None)


@pytest.mark.parametrize("fn", ["rows", "tensor"])
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), wan.WAN_ATTN_EINVAL),
    (dict(scales=None), wan.WAN_ATTN_EINVAL),
    (dict(rows=0), wan.WAN_ATTN_EINVAL),
    (dict(cols=0), wan.WAN_ATTN_EINVAL),
    (dict(cols=96), wan.WAN_ATTN_EUNSUPPORTED),        # not a multiple of 64
    (dict(cols=(1 << 20) + 64), wan.WAN_ATTN_EUNSUPPORTED),
    (dict(x=(1 << 20) + 8), wan.WAN_ATTN_EALIGN),
    (dict(scales=(1 << 22) + 2), wan.WAN_ATTN_EALIGN),
    (dict(codes=(1 << 20) + 64), wan.WAN_ATTN_EINVAL),  # codes overlap x
])
def test_fp8_quantize_argument_checks(fn, kw, code):
    assert _fp8(fn, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(y=None), wan.WAN_ATTN_EINVAL),
    (dict(ws=None), wan.WAN_ATTN_EINVAL),
    (dict(m=0), wan.WAN_ATTN_EINVAL),
    (dict(n=0), wan.WAN_ATTN_EINVAL),
    (dict(n=6), wan.WAN_ATTN_EUNSUPPORTED),            # n not a multiple of 4
    (dict(k=100), wan.WAN_ATTN_EUNSUPPORTED),
    (dict(xc=(1 << 20) + 4), wan.WAN_ATTN_EALIGN),
    (dict(xs=(1 << 21) + 1), wan.WAN_ATTN_EALIGN),
    (dict(y=1 << 20), wan.WAN_ATTN_EINVAL),            # y overlaps the activation codes
    (dict(m=1 << 40, n=1 << 30), wan.WAN_ATTN_EINVAL),  # work items beyond 32 bits
])
def test_fp8_gemm_argument_checks(kw, code):
    assert _fp8("gemm", **kw) == code


def _vsa(fn, **kw):
    """The block-sparse entry points with far-apart fake device addresses (every case fails a check
    before the first HIP call)."""
    lib = ensure_built()
    a = dict(q=1 << 24, k=1 << 25, v=1 << 26, idx=1 << 27, o=1 << 28, scratch=1 << 29,
             b=1, H=1, sq=64, skv=512, d=128, keep=1)
    a.update(kw)
    if fn == "select":
        return lib.wan_vsa_select(a["q"], a["k"], a["b"], a["H"], a["sq"], a["skv"], a["d"], a["keep"], a["idx"],
                                  a["scratch"], None)
    if fn == "attn":
        return lib.wan_vsa_attn(a["q"], a["k"], a["v"], a["idx"], a["o"], a["b"], a["H"], a["sq"], a["skv"], a["d"],
                                a["keep"], None)
    return lib.wan_vsa_fwd(a["q"], a["k"], a["v"], a["o"], a["b"], a["H"], a["sq"], a["skv"], a["d"], a["keep"], None)


@pytest.mark.parametrize("fn", ["select", "attn", "fwd"])
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), wan.WAN_ATTN_EINVAL),
    (dict(k=None), wan.WAN_ATTN_EINVAL),
    (dict(b=0), wan.WAN_ATTN_EINVAL),
    (dict(skv=0), wan.WAN_ATTN_EINVAL),
    (dict(d=64), wan.WAN_ATTN_EUNSUPPORTED),
    (dict(keep=9), wan.WAN_ATTN_EINVAL),                      # more than the 8 key blocks
    (dict(skv=4096 * 64 + 1), wan.WAN_ATTN_EUNSUPPORTED),     # beyond the selection's LDS capacity
    (dict(q=(1 << 24) + 8), wan.WAN_ATTN_EALIGN),
    (dict(b=1 << 20, H=4096), wan.WAN_ATTN_EINVAL),           # coarse-stage grid beyond 31 bits
])
def test_vsa_argument_checks(fn, kw, code):
    assert _vsa(fn, **kw) == code


@pytest.mark.parametrize("fn,kw,code", [
    ("select", dict(keep=0), wan.WAN_ATTN_EINVAL),
    ("attn", dict(keep=0), wan.WAN_ATTN_EINVAL),
    ("select", dict(idx=None), wan.WAN_ATTN_EINVAL),
    ("select", dict(scratch=None), wan.WAN_ATTN_EINVAL),
    ("select", dict(idx=(1 << 27) + 4), wan.WAN_ATTN_EALIGN),
    ("select", dict(idx=1 << 24), wan.WAN_ATTN_EINVAL),       # block list overlaps q
    ("select", dict(scratch=(1 << 25) + 16), wan.WAN_ATTN_EINVAL),   # scratch overlaps k
    ("attn", dict(idx=None), wan.WAN_ATTN_EINVAL),
    ("attn", dict(v=None), wan.WAN_ATTN_EINVAL),
    ("attn", dict(o=1 << 26), wan.WAN_ATTN_EINVAL),            # o overlaps v
    ("attn", dict(o=(1 << 27) - 64), wan.WAN_ATTN_EINVAL),     # o overlaps the block list
    ("fwd", dict(o=None), wan.WAN_ATTN_EINVAL),
])
def test_vsa_more_argument_checks(fn, kw, code):
    assert _vsa(fn, **kw) == code


def test_vsa_scratch_bytes():
    ensure_built()
    assert wan.wan_vsa_select_scratch_bytes(2, 3, 150, 700) == 2 * 3 * (3 + 11) * 512
    assert wan.wan_vsa_select_scratch_bytes(0, 3, 150, 700) == 0


def test_vsa_wrappers_reject_bad_tensors():
    # the torch wrappers check device, dtype, layout and shapes before calling the library
    import torch
    q = torch.zeros((1, 64, 1, 128), dtype=torch.bfloat16)            # host tensors: not CUDA
    idx = torch.zeros((1, 1, 1, 1), dtype=torch.int32)
    with pytest.raises(ValueError):
        wan.vsa_select(q, q, 1)
    with pytest.raises(ValueError):
        wan.vsa_attention(q, q, q, idx)
    with pytest.raises(ValueError):
        wan.vsa_forward(q, q, q)
    with pytest.raises(ValueError):
        wan.vsa_select(q.float(), q, 1)                                  # wrong dtype


def test_tensor_argument_helper_rejects_before_any_call():
    # the check every torch wrapper applies to each tensor it hands to the library (out, lse,
    # block_idx, FP8 codes and scales, the quantised operands): dtype, exact shape, contiguity,
    # then CUDA device
    import torch
    cuda0 = torch.device("cuda", 0)
    t = torch.zeros((2, 3, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="must be on cuda:0"):
        wan._require("block_idx", t, torch.int32, (2, 3, 4), cuda0)          # host memory
    with pytest.raises(ValueError, match="must be on cuda:0"):
        wan._require("lse", t.float(), torch.float32, (2, 3, 4), cuda0)       # host lse
    with pytest.raises(ValueError, match="shape"):
        wan._require("out", t, torch.int32, (2, 3, 5), cuda0)                 # undersized out
    with pytest.raises(ValueError, match="uint8"):
        wan._require("x_codes", t, torch.uint8, (2, 3, 4), cuda0)             # wrong dtype
    with pytest.raises(ValueError, match="contiguous"):
        wan._require("w_codes", t.transpose(0, 1), torch.int32, (3, 2, 4), cuda0)
    with pytest.raises(ValueError, match="torch tensor"):
        wan._require("x_scales", None, torch.float32, (1,), cuda0)


def test_torch_wrappers_reject_host_tensors(monkeypatch):
    # with host tensors every wrapper raises ValueError and never reaches the library
    import torch

    def no_library():
        raise AssertionError("the library was called")

    monkeypatch.setattr(wan, "lib", no_library)
    q = torch.zeros((1, 64, 1, 128), dtype=torch.bfloat16)
    lse = torch.zeros((1, 1, 64), dtype=torch.float32)
    codes = torch.zeros((64, 64), dtype=torch.uint8)
    scales = torch.ones((64,), dtype=torch.float32)
    calls = [
        lambda: wan.attention(q, q, q),
        lambda: wan.attention_with_lse(q, q, q),
        lambda: wan.attention_backward(q, q, q, q, lse, q),
        lambda: wan.attention8_quantize(q, q, q),
        lambda: wan.attention8_from_quantized({}, 1, 1, 64, 64),
        lambda: wan.fp8_gemm(codes, scales, codes, scales[:1]),
        lambda: wan.fp8_quantize_rows(q[0, :, 0, :]),
        lambda: wan.fp8_quantize_tensor(q[0, :, 0, :]),
        lambda: wan.vsa_attention(q, q, q, torch.zeros((1, 1, 1, 1), dtype=torch.int32)),
    ]
    for call in calls:
        with pytest.raises(ValueError):
            call()


def test_attn8_key_length_limit():
    # the 8-bit kernel's V-code descriptor spans 128 * ceil(s_kv/64)*64 bytes of one head: at 2^31 the
    # call is refused before anything is enqueued (fake, far-apart addresses, never dereferenced)
    lib = ensure_built()
    q, k, v, o = 1 << 40, 1 << 41, 1 << 42, 1 << 43
    assert lib.wan_attn_fwd(q, k, v, o, 1, 1, 1, 16777152 + 1, 128, 1, None) == wan.WAN_ATTN_EUNSUPPORTED
    assert lib.wan_attn_fwd(q, k, v, o, 1, 1, 1, 1 << 24, 128, 1, None) == wan.WAN_ATTN_EUNSUPPORTED
    assert lib.wan_attn8_fwd_quantized(q, q + (1 << 36), k, k + (1 << 36), v, v + (1 << 36), o, 1, 1, 1,
                                       1 << 24, 128, None) == wan.WAN_ATTN_EUNSUPPORTED


def _quantize_args(**kw):
    """wan_attn8_quantize with distinct, far-apart fake addresses; every case fails a check first."""
    names = ["q", "k", "v", "q_codes", "q_scale", "k_codes", "k_scale", "v_codes", "v_scale", "smooth", "scratch"]
    a = {n: (i + 1) << 32 for i, n in enumerate(names)}
    a.update(kw)
    return [a["q"], a["k"], a["v"], 1, 2, 300, 257, 128] + [a[n] for n in names[3:]] + [None]


@pytest.mark.parametrize("kw", [
    dict(q_codes=1 << 32),                    # q codes over q
    dict(k_scale=(2 << 32) + 4096),           # k scales inside k
    dict(v_codes=6 << 32),                    # v codes over the q scales
    dict(smooth=(9 << 32) + 256),             # smooth inside the v scales
    dict(scratch=(4 << 32) + 64),             # scratch inside the q codes
])
def test_quantize_output_overlap(kw):
    lib = ensure_built()
    assert lib.wan_attn8_quantize(*_quantize_args(**kw)) == wan.WAN_ATTN_EINVAL


@pytest.mark.parametrize("o", [1 << 32, (2 << 32) + 16, (5 << 32) + 4096, (6 << 32) + 16])
def test_quantized_forward_output_overlap(o):
    lib = ensure_built()
    ptrs = [(i + 1) << 32 for i in range(6)]
    assert lib.wan_attn8_fwd_quantized(*ptrs, o, 1, 2, 300, 257, 128, None) == wan.WAN_ATTN_EINVAL


def test_release_scratch_without_pools():
    # nothing allocated yet in this process: nothing to release
    ensure_built()
    assert wan.lib().wan_attn_release_scratch() == wan.WAN_ATTN_OK


def test_noalloc_backward_size_limit():
    # the static scratch holds 8 bytes per padded query row, 64 MiB: 8,388,608 rows; one tile more is
    # refused before any GPU work (fake, far-apart addresses, never dereferenced)
    lib = ensure_built()
    names = ["q", "k", "v", "o", "d_o", "lse", "dq", "dk", "dv"]
    ptrs = [(i + 1) << 40 for i in range(len(names))]
    assert lib.wan_attn_bwd_noalloc(*ptrs, 1, 1, 8388608 + 64, 1, 128, None) == wan.WAN_ATTN_EUNSUPPORTED
    assert lib.wan_attn_bwd_noalloc(*ptrs, 2, 64, 65537, 1, 128, None) == wan.WAN_ATTN_EUNSUPPORTED
    # the other checks are the allocating backward's
    bad = list(ptrs)
    bad[6] = ptrs[0]                      # dq over q
    assert lib.wan_attn_bwd_noalloc(*bad, 1, 1, 64, 64, 128, None) == wan.WAN_ATTN_EINVAL
    bad = list(ptrs)
    bad[5] = None
    assert lib.wan_attn_bwd_noalloc(*bad, 1, 1, 64, 64, 128, None) == wan.WAN_ATTN_EINVAL
    assert lib.wan_attn_bwd_noalloc(*ptrs, 1, 1, 64, 64, 64, None) == wan.WAN_ATTN_EUNSUPPORTED


def test_mfma_ceiling_library_rejects_bad_arguments():
    # the measurement library beside the attention library: it loads without a GPU and refuses
    # arguments it cannot launch with (null buffers, no workgroups, no iterations, unknown kind)
    # before touching the device
    from video_diffusion_transformer_wan_amd import build as wan_build
    ensure_built()
    if not os.path.exists(wan_build.CEILING_LIB):
        wan_build.build()
    lib = ctypes.CDLL(wan_build.CEILING_LIB)
    f = lib.wan_mfma_ceiling_run
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    fake = 4096   # never dereferenced: every call below is refused first
    assert f(0, None, fake, 256, 10, None) == 1
    assert f(0, fake, None, 256, 10, None) == 1
    assert f(0, fake, fake, 0, 10, None) == 1
    assert f(0, fake, fake, 256, 0, None) == 1
    assert f(6, fake, fake, 256, 10, None) == 1
    assert f(-1, fake, fake, 256, 10, None) == 1
