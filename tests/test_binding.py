"""Argument checks of the Python binding (no GPU needed: they raise before the
library is called)."""

import pytest
import torch

import delayed_scaling_gemm_amd as dsg


def test_span_counts_addressed_elements():
    assert dsg._span(4, 5, 8) == 3 * 8 + 5
    assert dsg._span(4, 5, 8, batch=2, stride=100) == 100 + 3 * 8 + 5
    assert dsg._span(0, 5, 8) == 0 and dsg._span(4, 0, 8) == 0 and dsg._span(4, 5, 8, 0) == 0


def test_host_tensors_are_rejected():
    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    q = torch.zeros(4, 16, dtype=torch.uint8)
    s = torch.ones(1)
    with pytest.raises(ValueError, match="CUDA"):
        dsg.fp8ds_cast(x, dsg.E4M3, s, q)
    with pytest.raises(ValueError, match="CUDA"):
        dsg.fp8ds_amax(x, s)
    with pytest.raises(ValueError, match="CUDA"):
        dsg.fp8ds_gemm(dsg.OP_N, dsg.OP_T, 4, 4, 16, q, dsg.E4M3, 16, s, q, dsg.E4M3, 16, s,
                       torch.zeros(4, 4, dtype=torch.bfloat16), 4)


def test_scale_update_needs_a_format_per_tensor():
    h = torch.zeros(3, 16)
    with pytest.raises(ValueError, match="formats"):
        dsg.fp8ds_scale_update(h, torch.zeros(3, dtype=torch.int32), torch.zeros(3), [0, 0], 0, 0,
                               torch.ones(3))


def test_mx_host_tensors_and_shapes_are_rejected():
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    q = torch.zeros(4, 64, dtype=torch.uint8)
    s = torch.zeros(4, 2, dtype=torch.uint8)
    with pytest.raises(ValueError, match="CUDA"):
        dsg.fp8ds_cast_mx(x, dsg.E4M3, q, s)
    with pytest.raises(ValueError, match="2-D"):
        dsg.fp8ds_cast_mx(x.view(-1), dsg.E4M3, q, s)
    with pytest.raises(ValueError, match="CUDA"):
        dsg.fp8ds_gemm_mx(4, 4, 128, q, dsg.E4M3, 128, s, 4, q, dsg.E4M3, 128, s, 4,
                          torch.zeros(4, 4, dtype=torch.bfloat16), 4)
