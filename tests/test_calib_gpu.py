"""The debug build's matrix-core calibration kernel (attn_debug_calib_mfma), called through the C ABI.

It is not part of the attention path; `bench.py --mode mfma` uses it for the rate the matrix cores
sustain under the board's power limit.  These tests check that it does the arithmetic it is timed
for: zero operands give zero, every thread's result is linear in the iteration count (each
iteration adds the same 16 products to the accumulators), and bad arguments are rejected before
any launch.
"""

import ctypes

import pytest
import torch

from gpu_common import gpu_required

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gpu_required()


def _lib():
    from exact_tiled_attention_fa2_amd import debug
    return debug.debug_lib()


def _call(h, code, ops, out, blocks, iters):
    return h.attn_debug_calib_mfma(code, ctypes.c_void_p(ops.data_ptr()) if ops is not None else None,
                                   ctypes.c_void_p(out.data_ptr()) if out is not None else None, blocks, iters,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("code,tdt", [(1, torch.bfloat16), (0, torch.float16)])
def test_calib_mfma_arithmetic(code, tdt):
    print(f"[case] calib mfma dtype code {code}", flush=True)
    h = _lib()
    blocks = 8
    out1 = torch.full((blocks * 256,), float("nan"), device="cuda")
    out3 = torch.full_like(out1, float("nan"))
    zero = torch.zeros(4096, device="cuda", dtype=tdt)
    assert _call(h, code, zero, out1, blocks, 5) == 0
    torch.cuda.synchronize()
    assert torch.equal(out1, torch.zeros_like(out1))

    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    # Small integers: every product and partial sum is exact in fp32, so linearity holds bit for bit.
    ops = torch.randint(-3, 4, (4096,), device="cuda", generator=g).to(tdt)
    assert _call(h, code, ops, out1, blocks, 1) == 0
    assert _call(h, code, ops, out3, blocks, 3) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out1).all() and out1.abs().sum() > 0
    assert torch.equal(out3, 3 * out1)
    # Every workgroup computes the same thing: the result depends on the lane only.
    per_block = out1.view(blocks, 256)
    assert torch.equal(per_block, per_block[:1].expand_as(per_block))


def test_calib_mfma_rejects_bad_arguments():
    print("[case] calib mfma argument checks", flush=True)
    h = _lib()
    ops = torch.zeros(4096, device="cuda", dtype=torch.bfloat16)
    out = torch.zeros(256, device="cuda")
    assert _call(h, 1, None, out, 1, 1) == -1     # ATTN_E_NULL
    assert _call(h, 1, ops, None, 1, 1) == -1
    assert _call(h, 1, ops, out, 0, 1) == -2      # ATTN_E_SHAPE
    assert _call(h, 1, ops, out, 1, 0) == -2
    assert _call(h, 7, ops, out, 1, 1) == -4      # ATTN_E_UNSUPPORTED
    misaligned = ctypes.c_void_p(ops.data_ptr() + 2)
    assert h.attn_debug_calib_mfma(1, misaligned, ctypes.c_void_p(out.data_ptr()), 1, 1,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == -8  # ATTN_E_ALIGN
