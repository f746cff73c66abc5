"""The sustained-MFMA measurement kernel (libwan_mfma_ceiling.so) on the GPU, at a tiny size: every
instruction form launches, and its per-wave sums are finite and the same on a second launch.  (The
kernel measures the matrix core's rate for the benchmark; its arithmetic is not the attention's.)"""

import ctypes
import os

import numpy as np
import pytest
import torch

from _util import ensure_built

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", range(6))
def test_every_form_launches_and_repeats(kind):
    from video_diffusion_transformer_wan_amd import build as wan_build
    ensure_built()
    if not os.path.exists(wan_build.CEILING_LIB):
        wan_build.build()
    lib = ctypes.CDLL(wan_build.CEILING_LIB)
    f = lib.wan_mfma_ceiling_run
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    g = torch.Generator(device="cpu").manual_seed(11 + kind)
    # 64 lanes x 8 registers x 32 bytes of small integers: finite as bf16, e4m3 and int8 alike
    src = torch.randint(0, 4, (64 * 8 * 32,), generator=g, dtype=torch.uint8).to("cuda")
    n_wg = 8
    outs = []
    for _ in range(2):
        out = torch.full((n_wg * 4,), float("nan"), dtype=torch.float32, device="cuda")
        st = torch.cuda.current_stream().cuda_stream
        assert f(kind, src.data_ptr(), out.data_ptr(), n_wg, 16, st) == 0
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.all(np.isfinite(outs[0]))
    assert np.array_equal(outs[0], outs[1])
