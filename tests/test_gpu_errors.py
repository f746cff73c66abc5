"""Error paths of the C ABI on the GPU: a failed scratch allocation is reported as WAN_ATTN_ENOMEM by
every entry point that allocates (the library's test hook WAN_ATTN_TEST_FAIL_ALLOC, read once per
process, makes each allocation fail: that part runs in a child process), nothing is written, and the
same calls succeed, with the same results, where allocation works.  The torch wrappers reject host,
wrong-dtype and wrong-size tensor arguments next to CUDA inputs before any library call."""

import os
import subprocess
import sys

import pytest
import torch

import video_diffusion_transformer_wan_amd as wan
import wan_inputs
from _util import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _calls(q, k, v, o, lse, d_o, grads, b, H, s_q, s_kv):
    lib = wan.lib()
    st = torch.cuda.current_stream().cuda_stream
    dq, dk, dv = grads
    return {
        # b * H * ceil(s_q / 256) = 4 query tiles: the bf16 forward splits the keys into ranges in scratch
        "bf16 split": lambda: lib.wan_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o["bf16"].data_ptr(), b, H,
                                               s_q, s_kv, 128, wan.WAN_ATTN_BF16, st),
        "int8_fp8": lambda: lib.wan_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o["int8"].data_ptr(), b, H,
                                             s_q, s_kv, 128, wan.WAN_ATTN_INT8_FP8, st),
        "backward": lambda: lib.wan_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o["ref"].data_ptr(),
                                             d_o.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                             dv.data_ptr(), b, H, s_q, s_kv, 128, st),
        "vsa": lambda: lib.wan_vsa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o["vsa"].data_ptr(), b, H, s_q,
                                       s_kv, 128, 0, st),
    }


def _case(with_forward=True):
    # b * H * ceil(s_q / 256) = 4 query tiles: the bf16 forward takes its split path, in scratch, so
    # with allocation failing the forward's output and lse stand in as zeros
    b, H, s_q, s_kv = 1, 2, 300, 257
    q, k, v = wan_inputs.random_qkv(b, H, s_q, s_kv, 50000, device="cuda")
    if with_forward:
        ref_o, lse = wan.attention_with_lse(q, k, v)
    else:
        ref_o, lse = torch.zeros_like(q), torch.zeros((b, H, s_q), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(50001)
    d_o = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    o = {"bf16": torch.zeros_like(q), "int8": torch.zeros_like(q), "vsa": torch.zeros_like(q), "ref": ref_o}
    grads = (torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v))
    torch.cuda.synchronize()
    return (q, k, v, o, lse, d_o, grads), (b, H, s_q, s_kv)


def child_main():
    """Run in a fresh process with WAN_ATTN_TEST_FAIL_ALLOC=1: every allocating call fails, nothing written."""
    ensure_built()
    tensors, dims = _case(with_forward=False)
    q, k, v, o, lse, d_o, grads = tensors
    for name, call in _calls(*tensors, *dims).items():
        print(f"  {name}", flush=True)
        assert call() == wan.WAN_ATTN_ENOMEM, name
    torch.cuda.synchronize()
    assert all(int(torch.count_nonzero(o[n])) == 0 for n in ("bf16", "int8", "vsa"))
    assert all(int(torch.count_nonzero(t)) == 0 for t in grads)
    print("CHILD_OK", flush=True)


def test_failed_scratch_allocation_is_reported():
    env = dict(os.environ, WAN_ATTN_TEST_FAIL_ALLOC="1")
    here = os.path.dirname(os.path.abspath(__file__))
    code = f"import sys; sys.path[:0] = [{here!r}, {os.path.dirname(here)!r}]; import test_gpu_errors as t; t.child_main()"
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    print(res.stdout[-2000:], res.stderr[-2000:], flush=True)
    assert res.returncode == 0 and "CHILD_OK" in res.stdout

    # here the hook is off: the same calls succeed with the wrappers' results
    tensors, dims = _case()
    q, k, v, o, lse, d_o, grads = tensors
    for name, call in _calls(*tensors, *dims).items():
        assert call() == wan.WAN_ATTN_OK, name
    torch.cuda.synchronize()
    ref_o = o["ref"]
    assert torch.equal(o["bf16"], ref_o)
    assert torch.equal(o["int8"], wan.attention(q, k, v, dtype="int8_fp8"))
    assert torch.equal(o["vsa"], wan.vsa_forward(q, k, v))
    dq, dk, dv = wan.attention_backward(q, k, v, ref_o, lse, d_o)
    assert torch.equal(grads[0], dq) and torch.equal(grads[1], dk) and torch.equal(grads[2], dv)
    torch.cuda.synchronize()
    assert wan.lib().wan_attn_release_scratch() == wan.WAN_ATTN_OK
    # after the release the pool allocates again
    assert torch.equal(wan.attention(q, k, v, dtype="int8_fp8"), o["int8"])


def test_wrappers_reject_bad_tensor_arguments(monkeypatch):
    q, k, v = wan_inputs.random_qkv(1, 2, 130, 70, 50002, device="cuda")
    o, lse = wan.attention_with_lse(q, k, v)
    idx = wan.vsa_select(q, k, 1)
    codes, scales = wan.fp8_quantize_rows(q[0, :, 0, :].contiguous())
    wcodes, wscale = wan.fp8_quantize_tensor(q[0, :64, 0, :].contiguous())
    torch.cuda.synchronize()

    def no_library():
        raise AssertionError("the library was called")

    monkeypatch.setattr(wan, "lib", no_library)
    bad = {
        "host block_idx": lambda: wan.vsa_attention(q, k, v, idx.cpu()),
        "int64 block_idx": lambda: wan.vsa_attention(q, k, v, idx.long()),
        "host lse": lambda: wan.attention_backward(q, k, v, o, lse.cpu(), o),
        "short lse": lambda: wan.attention_backward(q, k, v, o, lse[:, :, :-1].contiguous(), o),
        "undersized out": lambda: wan.attention(q, k, v, out=torch.empty_like(q)[:, :-1]),
        "strided out": lambda: wan.attention(q, k, v, out=torch.empty((1, 2, 130, 128), dtype=torch.bfloat16,
                                                                       device="cuda").transpose(1, 2)),
        "fp32 out": lambda: wan.vsa_forward(q, k, v, out=torch.empty(q.shape, device="cuda")),
        "host fp8 codes": lambda: wan.fp8_gemm(codes.cpu(), scales, wcodes, wscale),
        "host fp8 scales": lambda: wan.fp8_gemm(codes, scales.cpu(), wcodes, wscale),
        "short weight codes": lambda: wan.fp8_gemm(codes, scales, wcodes[:, :64].contiguous(), wscale),
        "incomplete quantised operands": lambda: wan.attention8_from_quantized(
            {"q_codes": codes}, 1, 2, 130, 70),
        "host k": lambda: wan.attention(q, k.cpu(), v),
    }
    for name, call in bad.items():
        with pytest.raises(ValueError):
            call()
        print(f"  rejected: {name}", flush=True)
