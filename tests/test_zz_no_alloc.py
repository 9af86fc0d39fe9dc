"""fa_forward_split_noalloc (the key split with its partials in the library's
per-GPU scratch array, for callers that cannot allocate) against
fa_forward_split (the same kernels with a caller workspace), through the C ABI.

The calls run back to back with shrinking inputs, so each later call finds
the scratch array holding an earlier, larger call's partials: nothing in it
may be read before this call writes it.  With the same split count both entry
points run the same kernels on the same values, so their outputs must agree
bit for bit; both are also held to the oracle's bars.
"""

import pytest
import torch

from oracle import attention_forward
from tests.parity import assert_within, errors, f64
from tiled_attention_forward_amd import binding
from tiled_attention_forward_amd.workloads import custom, make_inputs

pytestmark = pytest.mark.gpu

# B, Hq, Hkv, Nq, Nk, D, dtype, causal, bias, splits -- each smaller than the one before
CASES = [
    (2, 8, 2, 1, 1000, 128, "bf16", False, False, 4),
    (1, 4, 1, 70, 300, 64, "fp16", True, True, 3),
    (1, 2, 2, 5, 130, 64, "fp32", False, False, 2),
]


def _log(*a):
    print(*a, flush=True)


def _noalloc(q, k, v, b, o, lse, w, splits):
    """One fa_forward_split_noalloc call through the C ABI on the current stream."""
    return binding.fa_forward_split_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), None if b is None else b.data_ptr(),
        o.data_ptr(), lse.data_ptr(), w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, w.scale,
        int(w.causal), binding._dtype_code(q), splits,
        torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_split_on_consecutive_calls(gpu_device):
    runs = []
    for i, case in enumerate(CASES):
        B, Hq, Hkv, Nq, Nk, D, dt, causal, bias, splits = case
        w = custom(B, Hq, Hkv, Nq, Nk, D, dt, causal, bias)
        q, k, v, b = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=60 + i))
        o = torch.full(q.shape, 7.0, dtype=q.dtype, device=gpu_device)
        lse = torch.full((B, Hq, Nq), 7.0, dtype=torch.float32, device=gpu_device)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(gpu_device)
        _log(f"noalloc call {i}: {case}")
        assert _noalloc(q, k, v, b, o, lse, w, splits) == binding.FA_OK
        assert torch.cuda.memory_allocated(gpu_device) == before
        runs.append((case, w, q, k, v, b, o, lse))
    torch.cuda.synchronize()
    for case, w, q, k, v, b, o, lse in runs:
        splits = case[9]
        o_ref, lse_ref = binding.forward_split(q, k, v, b, causal=w.causal, scale=w.scale,
                                               num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"{case}: O differs from fa_forward_split"
        assert torch.equal(lse, lse_ref), f"{case}: LSE differs from fa_forward_split"
        o64, l64 = attention_forward(f64(q), f64(k), f64(v), None if b is None else f64(b),
                                     scale=w.scale, causal=w.causal)
        st = errors(f64(o), lse.cpu().numpy(), o64, l64)
        _log(case, st)
        assert_within(st, w.dtype, str(case))


def test_noalloc_refuses_partials_beyond_the_scratch(gpu_device):
    """Partials larger than the scratch array: an error, nothing launched."""
    w = custom(1, 8, 8, 1024, 256, 64, "bf16", False, False)
    q, k, v, _ = make_inputs(w, seed=3, device=gpu_device)
    splits = 4   # 8 * 1024 rows * 64 * 4 bytes * 4 splits = 8 MiB: fits
    assert binding.fa_split_workspace_bytes(1, 8, 1024, 64, splits) <= binding.FA_SPLIT_SCRATCH_BYTES
    big = 17     # 34 MiB: does not
    assert binding.fa_split_workspace_bytes(1, 8, 1024, 64, big) > binding.FA_SPLIT_SCRATCH_BYTES
    o = torch.full(q.shape, 7.0, dtype=q.dtype, device=gpu_device)
    lse = torch.full((1, 8, 1024), 7.0, dtype=torch.float32, device=gpu_device)
    assert _noalloc(q, k, v, None, o, lse, w, big) == binding.FA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)
    assert _noalloc(q, k, v, None, o, lse, w, splits) == binding.FA_OK
    o_ref, lse_ref = binding.forward_split(q, k, v, None, causal=False, scale=w.scale,
                                           num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
