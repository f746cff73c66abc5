"""The 8-bit HIP path (through the C ABI) against the oracle, on the GPU.

* Stage 1 (quantisation) is integer / byte work: every int8 code, e4m3 code, scale and smoothing
  factor must equal the oracle's bit for bit (both take their decisions in fp32 with correctly
  rounded division and square root and round-half-even).
* Stage 2 against the step-by-step 8-bit emulator of the oracle: they differ only in fp32
  summation order and the hardware exp2, so they must agree to rel-L2 <= 5e-3 (a diagnostic bound
  of this repository).
* The accuracy bounds against the exact fp64 attention: rel-L2 <= 6e-2 and cosine >= 0.995.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import attn8 as oattn8
import video_diffusion_transformer_wan_amd as wan
import wan_inputs
from _util import INT8_COS, INT8_REL_L2, ensure_built, gather_rows, metrics, tail_rows, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _check_codes_head(z, qn, kn, vn, b, h, s_q, s_kv):
    ref = oattn8.quantize_head(qn[b, :, h], kn[b, :, h], vn[b, :, h])
    np.testing.assert_array_equal(z["smooth"][b, h].cpu().numpy(), ref["alpha"])
    np.testing.assert_array_equal(z["q_codes"][b, :, h].cpu().numpy(), ref["q_codes"])
    np.testing.assert_array_equal(z["k_codes"][b, :, h].cpu().numpy(), ref["k_codes"])
    np.testing.assert_array_equal(z["q_scale"][b, h].cpu().numpy(), ref["q_scale"])
    np.testing.assert_array_equal(z["k_scale"][b, h].cpu().numpy(), ref["k_scale"])
    np.testing.assert_array_equal(z["v_scale"][b, h].cpu().numpy(), ref["v_scale"])
    vt = z["v_codes"][b, h].cpu().numpy()               # [d, s_pad]
    np.testing.assert_array_equal(vt[:, :s_kv].T, ref["v_codes"])
    assert not vt[:, s_kv:].any()


@pytest.mark.parametrize("b,H,s_q,s_kv", [(1, 1, 1, 1), (1, 2, 63, 65), (2, 3, 200, 129),
                                          (1, 2, 1000, 1560), (2, 1, 64, 4097)])
def test_quantisation_codes_bit_exact(b, H, s_q, s_kv):
    q, k, v = wan_inputs.random_qkv(b, H, s_q, s_kv, seed=s_q + 7 * s_kv, device="cuda")
    z = wan.attention8_quantize(q, k, v)
    torch.cuda.synchronize()
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    for bb in range(b):
        for hh in range(H):
            _check_codes_head(z, qn, kn, vn, bb, hh, s_q, s_kv)


def test_quantisation_edge_values():
    # an all-zero channel, an all-zero 64-token block, large and tiny magnitudes
    q, k, v = wan_inputs.random_qkv(1, 2, 130, 140, seed=3, device="cuda")
    q[:, :, 0, 5] = 0
    k[:, :, 1, 7] = 0
    q[:, 64:128, 1, :] = 0
    v[:, :, 0, 3] = 0
    v[:, :, 1, 9] *= 1e-30
    k[:, :, 0, 11] *= 1e20
    z = wan.attention8_quantize(q.contiguous(), k.contiguous(), v.contiguous())
    torch.cuda.synchronize()
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    for hh in range(2):
        _check_codes_head(z, qn, kn, vn, 0, hh, 130, 140)


def _emulate(q, k, v, rows):
    return oracle.attn8_emulate(to_np(q), to_np(k), to_np(v), rows)


@pytest.mark.parametrize("b,H,s_q,s_kv", [(1, 2, 1, 1), (1, 2, 65, 63), (2, 2, 300, 257),
                                          (1, 1, 256, 2000), (1, 3, 129, 640)])
def test_fwd_matches_emulator_and_exact(b, H, s_q, s_kv):
    q, k, v = wan_inputs.random_qkv(b, H, s_q, s_kv, seed=11 * s_q + s_kv, device="cuda")
    out = wan.attention(q, k, v, dtype="int8_fp8")
    torch.cuda.synchronize()
    rows = np.array([[bb, hh, i] for bb in range(b) for hh in range(H) for i in range(s_q)])
    got = gather_rows(out, rows)
    emu = _emulate(q, k, v, rows)
    rel_e, _, _ = metrics(got, emu)
    assert rel_e <= 5e-3, rel_e
    ref = oracle.attention_rows(to_np(q), to_np(k), to_np(v), rows)
    rel, _, cos = metrics(got, ref)
    assert rel <= INT8_REL_L2 and cos >= INT8_COS, (rel, cos)


def test_two_stages_equal_the_single_call():
    q, k, v = wan_inputs.random_qkv(2, 2, 333, 444, seed=21, device="cuda")
    a = wan.attention(q, k, v, dtype="int8_fp8")
    z = wan.attention8_quantize(q, k, v)
    b = wan.attention8_from_quantized(z, 2, 2, 333, 444)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_deterministic():
    q, k, v = wan_inputs.random_qkv(1, 4, 700, 900, seed=22, device="cuda")
    a = wan.attention(q, k, v, dtype="int8_fp8")
    b = wan.attention(q, k, v, dtype="int8_fp8")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_wan14b_720p_int8fp8_sampled():
    w = wan_inputs.WORKLOADS["wan14b_720p81f_self_int8fp8"]
    print("8-bit workload: generating", flush=True)
    q, k, v = wan_inputs.make_qkv(w, device="cuda")
    out = wan.attention(q, k, v, dtype="int8_fp8")
    z = wan.attention8_quantize(q, k, v)
    torch.cuda.synchronize()
    print("8-bit workload: kernels done", flush=True)
    rows = np.concatenate([wan_inputs.sample_rows(w, 4096).numpy(), tail_rows(w.batch, w.heads, w.s_q)])
    qn, kn, vn = to_np(q.cpu()), to_np(k.cpu()), to_np(v.cpu())
    got = gather_rows(out, rows)
    ref = oracle.attention_rows(qn, kn, vn, rows)
    rel, mx, cos = metrics(got, ref)
    print(f"8-bit workload vs exact: rel-L2 {rel:.4e} max-abs {mx:.3e} cos {cos:.6f}", flush=True)
    assert rel <= INT8_REL_L2 and cos >= INT8_COS
    # codes of two heads, bit for bit, and the emulator on a subset of rows
    for hh in (0, w.heads - 1):
        _check_codes_head(z, qn, kn, vn, 0, hh, w.s_q, w.s_kv)
    sub = rows[np.isin(rows[:, 1], [0, 1])][:96]
    emu = oracle.attn8_emulate(qn, kn, vn, sub)
    rel_e, _, _ = metrics(gather_rows(out, sub), emu)
    print(f"8-bit workload vs emulator: rel-L2 {rel_e:.3e}", flush=True)
    assert rel_e <= 5e-3
