"""The Python binding rejects tensors of the wrong dtype, shape, layout or
device before any pointer reaches the library (the kernels read raw memory:
int64 expert IDs would be misread as int32 pairs, and a short buffer would be
read past its end). Host-only: every case fails before a kernel could launch.
"""
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
from mixture_experts_ffn_align_amd import _binding as B

M, H, I, E, K = 3, 256, 128, 8, 2


def _desc():
    w = B.moe_weights(B.MOE_W_INT4_AWQ, 64, 0x10000, 0x10000, 0x10000)
    return moe.make_desc(M, H, I, E, K, 8, w, w)


def _good():
    return (torch.zeros((M, H), dtype=torch.bfloat16), torch.zeros((M, K), dtype=torch.int32),
            torch.zeros((M, K), dtype=torch.float32), torch.zeros((M, H), dtype=torch.float32),
            torch.zeros(1024, dtype=torch.uint8))


@pytest.mark.parametrize("which,bad,exc", [
    (1, torch.zeros((M, K), dtype=torch.int64), TypeError),        # torch.topk's int64 IDs
    (0, torch.zeros((M, H), dtype=torch.float16), TypeError),
    (2, torch.zeros((M, K), dtype=torch.float64), TypeError),
    (3, torch.zeros((M, H), dtype=torch.bfloat16), TypeError),
    (1, torch.zeros((M, K - 1), dtype=torch.int32), ValueError),   # fewer than k routes per token
    (0, torch.zeros((M, H + 32), dtype=torch.bfloat16), ValueError),
    (0, torch.zeros((H, M), dtype=torch.bfloat16).t(), ValueError),  # not contiguous
    (3, torch.zeros((M + 1, H), dtype=torch.float32), ValueError),
])
def test_forward_rejects_bad_tensors(which, bad, exc):
    args = list(_good())
    args[which] = bad
    with pytest.raises(exc):
        moe.moe_ffn_forward(_desc(), *args)


def test_forward_rejects_host_tensors():
    # Right dtypes and shapes, but host memory: the device pointer check fires.
    with pytest.raises(ValueError, match="GPU"):
        moe.moe_ffn_forward(_desc(), *_good())


def test_stage_calls_check_their_tensors():
    x, ids, w, y, ws = _good()
    with pytest.raises(TypeError):
        moe.moe_ffn_gate_up(_desc(), x, ids.long(), ws)
    with pytest.raises(TypeError):
        moe.moe_ffn_down_combine(_desc(), ids, w.double(), y, ws)
