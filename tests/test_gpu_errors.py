"""Error paths of the C ABI on the GPU: a failed scratch allocation is reported as WAN_ATTN_ENOMEM by
every entry point that allocates (the library's test hook WAN_ATTN_TEST_FAIL_ALLOC makes each allocation
fail), nothing is left enqueued, and the same calls succeed, with the same results, once allocation
works again."""

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


def test_failed_scratch_allocation_is_reported(monkeypatch):
    b, H, s_q, s_kv = 1, 2, 300, 257
    q, k, v = wan_inputs.random_qkv(b, H, s_q, s_kv, 50000, device="cuda")
    ref_o, lse = wan.attention_with_lse(q, k, v)
    d_o = torch.randn(q.shape, device="cuda").to(torch.bfloat16)
    o = {"bf16": torch.zeros_like(q), "int8": torch.zeros_like(q), "vsa": torch.zeros_like(q), "ref": ref_o}
    grads = (torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v))
    torch.cuda.synchronize()
    calls = _calls(q, k, v, o, lse, d_o, grads, b, H, s_q, s_kv)

    monkeypatch.setenv("WAN_ATTN_TEST_FAIL_ALLOC", "1")
    for name, call in calls.items():
        assert call() == wan.WAN_ATTN_ENOMEM, name
    torch.cuda.synchronize()
    # nothing was written
    assert all(int(torch.count_nonzero(o[n])) == 0 for n in ("bf16", "int8", "vsa"))
    assert all(int(torch.count_nonzero(g)) == 0 for g in grads)

    monkeypatch.delenv("WAN_ATTN_TEST_FAIL_ALLOC")
    for name, call in calls.items():
        assert call() == wan.WAN_ATTN_OK, name
    torch.cuda.synchronize()
    assert torch.equal(o["bf16"], ref_o)
    assert torch.equal(o["int8"], wan.attention(q, k, v, dtype="int8_fp8"))
    assert torch.equal(o["vsa"], wan.vsa_forward(q, k, v))
    dq, dk, dv = wan.attention_backward(q, k, v, ref_o, lse, d_o)
    assert torch.equal(grads[0], dq) and torch.equal(grads[1], dk) and torch.equal(grads[2], dv)
