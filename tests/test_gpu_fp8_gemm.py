"""Parity of the FP8 GEMM path (through the C ABI) with the oracle, on the GPU.

* Quantisation: the GPU's e4m3fn codes and scales must equal the oracle's bit for bit (both take
  every decision in float32: amax, 448 / amax, the product, the saturating round to nearest even).
* Product: every checked element of Y against the oracle's exact Y (float64 from the same codes
  and scales).  The bound follows how the matrix core sums fp8 products, as measured on gfx950
  with single v_mfma_f32_32x32x64_f8f6f4 instructions on chosen operands: each group of 8
  consecutive products (k = 8g .. 8g+7) is summed aligned to its largest product, and bits below
  2^-13 of that product's power of two are dropped (with a largest product 2^8, seven products
  2^-6 in its group vanished and 2^-5 survived; products in other groups were exact).  Bound per
  element, with a factor 2 of margin on the window:
      E_mfma = sum_g sum_{k in g} min(|p_k|, 2^(floor(log2 max_g |p|) - 12))
      E_fp32 = 9 * (k / 64) * 2^-24 * sum_k |p_k|      (the group sums and the accumulator, per step)
      E      = (E_mfma + E_fp32) * scale_x * scale_w + 3 * 2^-24 |ref|   (the two scale roundings)
      |y - ref| <= 2^-8 (|ref| + E) + E                 (bf16 round to nearest: half an ulp)
* Shapes: ragged against the 256 x 256 output tile and the 64-byte K step (k = 64, 128, 192 run
  the pipeline with fewer stages than its depth), and the Wan projections on sampled rows.
"""

import numpy as np
import pytest
import torch

import oracle.fp8_gemm as og
import video_diffusion_transformer_wan_amd as wan
import wan_inputs
from _util import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _np(t):
    return t.detach().cpu().numpy()


def _f32(t):
    return t.detach().float().cpu().numpy()


def _bound(xc, xs, wc, ws, ref):
    """E of the module docstring for codes xc [r, k], wc [n, k] (row by row, to bound memory)."""
    from oracle.numerics import e4m3fn_decode
    xa = np.abs(e4m3fn_decode(xc))
    wa = np.abs(e4m3fn_decode(wc))
    k = wa.shape[1]
    out = np.empty(ref.shape)
    for i in range(xa.shape[0]):
        p = wa * xa[i][None, :]                                   # |products| [n, k]
        g = p.reshape(p.shape[0], k // 8, 8)
        mx = g.max(axis=2, keepdims=True)
        win = np.where(mx > 0, np.exp2(np.floor(np.log2(np.where(mx > 0, mx, 1.0))) - 12), 0.0)
        e_mfma = np.minimum(g, win).sum(axis=(1, 2))
        e_fp32 = 9 * (k // 64) * 2.0 ** -24 * p.sum(axis=1)
        out[i] = (e_mfma + e_fp32) * np.float64(xs[i]) * np.float64(ws)
    return out + 3 * 2.0 ** -24 * np.abs(ref)


def _check_product(y, xc, xs, wc, ws):
    ref = og.gemm(xc, xs, wc, ws)
    e = _bound(xc, xs, wc, ws, ref)
    bound = 2.0 ** -8 * (np.abs(ref) + e) + e
    err = np.abs(np.asarray(y, np.float64) - ref)
    worst = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    print(f"  max |y - ref| {err.max():.3e}, worst err/bound {worst:.3f}, "
          f"median bound/|ref| {float(np.median(bound / np.maximum(np.abs(ref), 1e-30))):.2e}", flush=True)
    assert np.all(err <= bound)


def _quantize_both(x, w):
    xc, xs = wan.fp8_quantize_rows(x)
    wc, ws = wan.fp8_quantize_tensor(w)
    torch.cuda.synchronize()
    return xc, xs, wc, ws


# row lengths on each register-resident path (up to 2, 4, 8 and 16 chunks of 8 values per lane) and
# past it (8,256 values: the two-pass kernel)
@pytest.mark.parametrize("m,k", [(1, 64), (3, 128), (37, 640), (5, 1536), (4, 4096), (300, 5120), (3, 8192),
                                 (3, 8256)])
def test_quantize_rows_bit_exact(m, k):
    x = wan_inputs.random_activations(m, k, seed=100 + m, device="cuda")
    x[0, :] = 0.0                                    # a zero row: scale 1, codes 0
    if m > 1:
        x[1, :] = -0.0                               # negative zeros: codes 0x80
    if m > 2:
        x[2, :7] = torch.tensor([3e4, -3e4, 1e-30, 7.0, -7.0, 448.0, 0.5])   # large and tiny values
    xc, xs = wan.fp8_quantize_rows(x)
    rc, rs = og.quantize_rows(_f32(x))
    assert np.array_equal(_np(xc), rc)
    assert np.array_equal(_np(xs).view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("n,k", [(1, 64), (5, 192), (300, 1024), (5120, 5120)])
def test_quantize_tensor_bit_exact(n, k):
    w = wan_inputs.random_weights(n, k, seed=200 + n, device="cuda")
    wc, ws = wan.fp8_quantize_tensor(w)
    rc, rs = og.quantize_tensor(_f32(w))
    assert np.array_equal(_np(wc), rc)
    assert _np(ws).view(np.uint32)[0] == np.float32(rs).view(np.uint32)


def test_quantize_tensor_zero():
    w = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    wc, ws = wan.fp8_quantize_tensor(w)
    assert float(ws[0]) == 1.0 and int(wc.sum()) == 0


@pytest.mark.parametrize("m,n,k", [(1, 4, 64), (5, 8, 64), (100, 260, 128), (257, 300, 192), (513, 516, 1024),
                                   (256, 256, 256), (1000, 1536, 1536)])
def test_gemm_against_exact(m, n, k):
    print(f"fp8 gemm m={m} n={n} k={k}", flush=True)
    x = wan_inputs.random_activations(m, k, seed=300 + m + k, device="cuda")
    w = wan_inputs.random_weights(n, k, seed=300 + n, device="cuda")
    xc, xs, wc, ws = _quantize_both(x, w)
    y = wan.fp8_gemm(xc, xs, wc, ws)
    torch.cuda.synchronize()
    rows = np.arange(m)
    if m * n * k > 2 ** 26:   # the bound costs n * k per row: check 40 rows, the first and last among them
        rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(m).choice(m, 38, replace=False)]))
    xcn, xsn = _np(xc)[rows], _np(xs)[rows]
    _check_product(_f32(y)[rows], xcn, xsn, _np(wc), _np(ws)[0])


def test_gemm_integer_operands_exact():
    # integer operands with the maximum 448 in every row of x and once in w: all scales are 1, and
    # each output (an integer of magnitude < 2^24 here) is exact in fp32 and rounds to bf16 once
    rng = np.random.default_rng(9)
    m, n, k = 70, 36, 128
    x = rng.integers(-4, 5, (m, k)).astype(np.float32)
    w = rng.integers(-4, 5, (n, k)).astype(np.float32)
    x[:, 0] = 448.0
    w[0, 1] = 448.0
    xt = torch.tensor(x, dtype=torch.bfloat16, device="cuda")
    wt = torch.tensor(w, dtype=torch.bfloat16, device="cuda")
    xc, xs, wc, ws = _quantize_both(xt, wt)
    assert torch.all(xs == 1.0) and float(ws[0]) == 1.0
    y = wan.fp8_gemm(xc, xs, wc, ws)
    ref = (x.astype(np.int64) @ w.astype(np.int64).T).astype(np.float64)
    want = torch.tensor(ref, dtype=torch.float32).to(torch.bfloat16).float().numpy()   # RNE to bf16
    assert np.array_equal(_f32(y), want)


def test_linear_and_determinism():
    x = wan_inputs.random_activations(333, 512, seed=7, device="cuda")
    w = wan_inputs.random_weights(260, 512, seed=7, device="cuda")
    wc, ws = wan.fp8_quantize_tensor(w)
    y1 = wan.fp8_linear(x, wc, ws)
    xc, xs = wan.fp8_quantize_rows(x)
    y2 = wan.fp8_gemm(xc, xs, wc, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_gemm_side_stream():
    x = wan_inputs.random_activations(300, 256, seed=8, device="cuda")
    w = wan_inputs.random_weights(64, 256, seed=8, device="cuda")
    xc, xs, wc, ws = _quantize_both(x, w)
    ref = wan.fp8_gemm(xc, xs, wc, ws)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = torch.empty_like(ref)
        wan.fp8_gemm(xc, xs, wc, ws, out=out, stream=s)
    s.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("name", sorted(wan_inputs.LINEAR_WORKLOADS))
def test_wan_projection_sampled(name):
    wl = wan_inputs.LINEAR_WORKLOADS[name]
    print(f"{name}: m={wl.m} n={wl.n} k={wl.k}", flush=True)
    x, w = wan_inputs.make_linear(wl, device="cuda")
    xc, xs, wc, ws = _quantize_both(x, w)
    y = wan.fp8_gemm(xc, xs, wc, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(wl.seed + 3)
    rows = np.sort(rng.choice(wl.m, 48, replace=False))
    rows[0], rows[-1] = 0, wl.m - 1
    # codes and scales of the sampled rows against the oracle's per-row quantisation
    xr = _f32(x[torch.as_tensor(rows, device="cuda")])
    rc, rs = og.quantize_rows(xr)
    xc_rows = _np(xc[torch.as_tensor(rows, device="cuda")])
    assert np.array_equal(xc_rows, rc) and np.array_equal(_np(xs)[rows].view(np.uint32), rs.view(np.uint32))
    wc_np = _np(wc)
    rwc, rws = og.quantize_tensor(_f32(w))
    assert np.array_equal(wc_np, rwc) and _np(ws).view(np.uint32)[0] == np.float32(rws).view(np.uint32)
    _check_product(_f32(y[torch.as_tensor(rows, device="cuda")])[:16], xc_rows[:16], _np(xs)[rows][:16], wc_np,
                   _np(ws)[0])


def _gemm_of_codes(xv, n=4):
    """y = xv . 1^T through the library's GEMM: xv [m, 64] values that e4m3fn holds exactly, as codes
    with scale 1; the weight rows are all 1.0 (code 0x38, scale 1), so every y[i, :] is the matrix core's
    sum of the 64 products x[i, k] * 1 (one MFMA step), rounded to bf16."""
    from oracle.numerics import e4m3fn_encode, e4m3fn_round
    assert np.array_equal(e4m3fn_round(xv), xv)
    m, k = xv.shape
    xc = torch.tensor(e4m3fn_encode(xv), dtype=torch.uint8, device="cuda")
    wc = torch.full((n, k), 0x38, dtype=torch.uint8, device="cuda")
    ones_m = torch.ones((m,), dtype=torch.float32, device="cuda")
    one = torch.ones((1,), dtype=torch.float32, device="cuda")
    y = wan.fp8_gemm(xc, ones_m, wc, one)
    torch.cuda.synchronize()
    return _f32(y), _np(xc), _np(wc)


def test_matrix_core_summation_window():
    # The premise of the product bound above, measured through the GEMM: each group of 8 consecutive
    # products is summed aligned to its largest product, bits below 2^-13 of that product's power of
    # two dropped; products in other groups are summed exactly.  Cancelling large products in two
    # groups leaves only the small ones, whose fate shows in the bf16 output.
    xv = np.zeros((4, 64))
    xv[0, 0], xv[0, 1:8], xv[0, 8] = 256.0, 2.0 ** -6, -256.0      # 2^-6 < 2^(8-13): dropped
    xv[1, 0], xv[1, 1:8], xv[1, 8] = 256.0, 2.0 ** -5, -256.0      # 2^-5 = 2^(8-13): kept
    xv[2, 0], xv[2, 8], xv[2, 16:24] = 256.0, -256.0, 2.0 ** -6    # small ones alone in group 2: exact
    xv[3, 0], xv[3, 1:8], xv[3, 8] = 1.0, 2.0 ** -9, -1.0          # 2^-9 above 2^(0-13): kept
    y, xc, wc = _gemm_of_codes(xv)
    print("  sums:", y[:, 0], flush=True)
    np.testing.assert_array_equal(y[:, 0], [0.0, 7 * 2.0 ** -5, 8 * 2.0 ** -6, 7 * 2.0 ** -9])
    assert np.all(y == y[:, :1])
    # the exact sums differ from row 0's result by the dropped products, which the bound covers
    _check_product(y, xc, np.ones(4, np.float32), wc, np.float32(1.0))


def test_summation_bound_on_adversarial_groups():
    # in every row, each group of 8 products holds one large product +-2^e and seven small ones
    # +-2^(e - gap) (random e, gap and signs); the large ones cancel in pairs of groups, so the output
    # is the sum of the small products, which the summation window can truncate.  Every output must
    # stay within the bound the parity tests use.
    rng = np.random.default_rng(77)
    m = 512
    xv = np.zeros((m, 64))
    for i in range(m):
        for pair in range(4):
            e = int(rng.integers(0, 9))
            sign = float(rng.choice([-1.0, 1.0]))
            for g, sg in ((2 * pair, sign), (2 * pair + 1, -sign)):
                gap = int(rng.integers(3, 10 + e))           # small products down to 2^-9
                xv[i, 8 * g] = sg * 2.0 ** e
                xv[i, 8 * g + 1:8 * g + 8] = rng.choice([-1.0, 1.0], 7) * 2.0 ** (e - gap)
    y, xc, wc = _gemm_of_codes(xv)
    _check_product(y, xc, np.ones(m, np.float32), wc, np.float32(1.0))


def _finite_bf16_up_to(limit):
    """Every bf16 bit pattern whose value is finite with magnitude <= limit (both zeros included),
    as float64 values."""
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    with np.errstate(invalid="ignore"):
        vals = bits.view(np.float32).astype(np.float64)
    return vals[np.isfinite(vals) & (np.abs(vals) <= limit)]


def test_every_bf16_value_converts_like_the_oracle():
    # The device's e4m3fn conversion of every bf16 value it can be asked to convert (|x| <= 448 after the
    # saturating clamp), through both quantisers: per-token activations with one 448 per row (scale 1,
    # so the code is the conversion of x itself) and the 8-bit attention's V with one 448 per channel.
    from oracle.numerics import e4m3fn_encode, e4m3fn_round
    vals = _finite_bf16_up_to(448.0)
    n = vals.size
    print(f"  {n} bf16 values", flush=True)
    cols = 1024
    rows = -(-n // (cols - 1))
    x = np.zeros((rows, cols))
    x[:, 0] = 448.0
    x.reshape(-1)[np.concatenate([np.arange(r * cols + 1, (r + 1) * cols) for r in range(rows)])[:n]] = vals
    xt = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).cuda()
    assert np.array_equal(_f32(xt).astype(np.float64), x)
    xc, xs = wan.fp8_quantize_rows(xt)
    torch.cuda.synchronize()
    assert torch.all(xs == 1.0)
    want = e4m3fn_encode(e4m3fn_round(x))
    assert np.array_equal(_np(xc), want), int((_np(xc) != want).sum())

    # V of one head: channel c holds 448 in token 0 and a slice of the values after it
    s = 1 + -(-n // 128)
    v = np.zeros((s, 128))
    v[0, :] = 448.0
    v[1:].reshape(-1)[:n] = vals
    vt = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).cuda().reshape(1, s, 1, 128)
    q = torch.zeros((1, 64, 1, 128), dtype=torch.bfloat16, device="cuda")
    z = wan.attention8_quantize(q, vt, vt)             # zero Q: smoothing factors 1
    torch.cuda.synchronize()
    assert torch.all(z["v_scale"] == 1.0)
    got = _np(z["v_codes"])[0, 0, :, :s].T                   # [s, 128]
    assert np.array_equal(got, e4m3fn_encode(e4m3fn_round(v)))
