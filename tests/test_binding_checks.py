"""The tensor-level binding checks every caller-supplied output and workspace
before a raw pointer reaches the C ABI (which cannot see buffer sizes).  The
checks are plain host code: they run here on CPU tensors, without a GPU."""

import pytest
import torch

from tiled_attention_forward_amd import binding

CPU = torch.device("cpu")


def _q(dtype=torch.bfloat16):
    return torch.zeros(2, 4, 33, 64, dtype=dtype)


def test_outputs_allocates_matching_buffers():
    out, lse = binding._outputs(_q(), None, None)
    assert out.shape == (2, 4, 33, 64) and out.dtype == torch.bfloat16
    assert lse.shape == (2, 4, 33) and lse.dtype == torch.float32
    out, _ = binding._outputs(_q(torch.float8_e4m3fn), None, None)
    assert out.dtype == torch.bfloat16  # FP8 inputs give a bf16 output


def test_outputs_accepts_exact_buffers():
    q = _q()
    out = torch.empty_like(q)
    lse = torch.empty(2, 4, 33, dtype=torch.float32)
    o2, l2 = binding._outputs(q, out, lse)
    assert o2 is out and l2 is lse


@pytest.mark.parametrize("bad", [
    torch.empty(2, 4, 32, 64, dtype=torch.bfloat16),           # too few rows
    torch.empty(2, 4, 33, 64, dtype=torch.float32),            # fp32 out for bf16 inputs
    torch.empty(2, 4, 64, 33, dtype=torch.bfloat16).transpose(2, 3),  # strided view
    torch.empty(2 * 4 * 33 * 64, dtype=torch.bfloat16),        # flat
])
def test_outputs_rejects_bad_out(bad):
    with pytest.raises(ValueError):
        binding._outputs(_q(), bad, None)


@pytest.mark.parametrize("bad", [
    torch.empty(2, 4, 33, dtype=torch.bfloat16),               # bf16 lse
    torch.empty(2, 4, 34, dtype=torch.float32),                # wrong size
    torch.empty(2, 33, 4, dtype=torch.float32).transpose(1, 2),  # strided
])
def test_outputs_rejects_bad_lse(bad):
    with pytest.raises(ValueError):
        binding._outputs(_q(), None, bad)


def test_fp8_out_must_be_bf16():
    q = _q(torch.float8_e4m3fn)
    with pytest.raises(ValueError):
        binding._outputs(q, torch.empty(q.shape, dtype=torch.float8_e4m3fn), None)


def test_non_tensor_rejected():
    with pytest.raises(TypeError):
        binding._check_buffer("out", [0.0], (1,), torch.float32, CPU)


def test_device_mismatch_rejected():
    t = torch.empty(3, dtype=torch.float32)
    with pytest.raises(ValueError):
        binding._check_buffer("lse", t, (3,), torch.float32, torch.device("cuda", 0))


def test_workspace_checks():
    ws = torch.empty(100, dtype=torch.uint8)
    binding._check_workspace(ws, 100, CPU)
    binding._check_workspace(torch.empty(25, dtype=torch.float32), 100, CPU)  # bytes, not elements
    with pytest.raises(ValueError):
        binding._check_workspace(ws, 101, CPU)
    with pytest.raises(ValueError):
        binding._check_workspace(torch.empty(10, 20, dtype=torch.uint8).t(), 100, CPU)
    with pytest.raises(TypeError):
        binding._check_workspace(None, 1, CPU)


def test_inputs_must_be_device_tensors():
    q = _q()
    with pytest.raises(ValueError):
        binding._check_inputs(q, q, q, None)
