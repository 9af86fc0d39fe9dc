"""GPU parity of the FP8 (E4M3) forward against the fp64 oracle on the decoded
inputs, and the evaluation of its precision loss ("FlashAttention principles
and Triton practice", xnwp.cn/news/15505, §7: FP8 doubles the matrix-core
rate over FP16 on the hardware it discusses, at a precision cost to be
measured).

The bar is the bound the arithmetic gives (tests/parity.py, fp8_bound_check):
the probabilities are rounded to E4M3 before P.V.  Each case also runs the
bf16 kernel on the same values (every E4M3 value is a bf16 value), so the
logged pair of errors shows what the E4M3 probabilities cost.
"""

import numpy as np
import pytest
import torch

from oracle import attention_head_rows
from tests.parity import f64, fp8_bound_check, run_gpu
from tiled_attention_forward_amd import binding
from tiled_attention_forward_amd.workloads import custom, make_inputs, sample_rows

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


CASES = [
    # B, Hq, Hkv, Nq, Nk, D, causal
    (1, 2, 2, 200, 200, 64, True),
    (1, 4, 2, 333, 517, 64, False),
    (2, 4, 1, 130, 170, 128, True),
    (1, 2, 2, 1000, 1000, 128, False),
    (1, 1, 1, 1, 1, 64, False),
    (1, 2, 2, 700, 1, 128, True),       # one key
    (1, 5, 1, 64, 64, 64, True),        # group 5
    (1, 2, 2, 1000, 1000, 64, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_fp8_matches_oracle_within_bound(gpu_device, case):
    B, Hq, Hkv, Nq, Nk, D, causal = case
    w = custom(B, Hq, Hkv, Nq, Nk, D, "fp8", causal, False)
    _log(f"fp8 case {case}")
    q, k, v, _ = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=51))
    o, lse = run_gpu(q, k, v, None, w.scale, causal)
    assert o.dtype == torch.bfloat16
    mx, mean, ratio = fp8_bound_check(q, k, v, w.scale, causal, o, lse, str(case))
    # the same values through the bf16 kernel
    ob, lb = run_gpu(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16), None,
                     w.scale, causal)
    mxb, meanb, _ = fp8_bound_check(q, k, v, w.scale, causal, ob, lb, str(case) + " bf16")
    _log(f"  fp8 max {mx:.2e} mean {mean:.2e} (worst err/bound {ratio:.2f}); "
         f"bf16 on the same values max {mxb:.2e} mean {meanb:.2e}")


def test_fp8_negative_scale(gpu_device):
    w = custom(1, 2, 2, 150, 150, 64, "fp8", True, False)
    q, k, v = (t.to(gpu_device) for t in make_inputs(w, seed=52)[:3])
    o, lse = run_gpu(q, k, v, None, -0.125, True)
    fp8_bound_check(q, k, v, -0.125, True, o, lse, "negative scale")


def test_fp8_rejections(gpu_device):
    w = custom(1, 2, 2, 64, 64, 64, "fp8", False, True)
    q, k, v, b = (t.to(gpu_device) for t in make_inputs(w, seed=53))
    with pytest.raises(binding.FaError):          # no logit term with FP8
        binding.forward(q, k, v, b)
    with pytest.raises(binding.FaError):          # nor on the key-split path
        binding.forward_split(q, k, v, b, num_splits=2)
    with pytest.raises(binding.FaError):          # nor with the window
        binding.forward(q, k, v, b, causal=True, window=16)


def test_fp8_full_size_sampled(gpu_device):
    """The benchmark report shape (B2 H16 S4096 D64 causal) in FP8; sampled rows
    of two heads against the oracle, within the same bound."""
    w = custom(2, 16, 16, 4096, 4096, 64, "fp8", True, False)
    _log("full-size fp8")
    q, k, v, _ = make_inputs(w, seed=0, device=gpu_device)
    o, lse = run_gpu(q, k, v, None, w.scale, True)
    rows = np.asarray(sample_rows(w.Nq, 64, seed=4))
    rows_t = torch.as_tensor(rows, device=gpu_device)
    for b, h in ((0, 0), (1, 15)):
        qr, kh, vh = f64(q[b, h, rows_t]), f64(k[b, h]), f64(v[b, h])
        o_ref, l_ref = attention_head_rows(qr, kh, vh, rows=rows, scale=w.scale, causal=True)
        o_abs, _ = attention_head_rows(qr, kh, np.abs(vh), rows=rows, scale=w.scale, causal=True)
        m_abs, _ = attention_head_rows(0 * qr, kh, np.abs(vh), rows=rows, scale=w.scale,
                                       causal=True)
        bound = (2.0 ** -4 * o_abs + 2.0 ** -17 * m_abs * (rows + 1.0)[:, None]
                 + 2.0 ** -9 * np.abs(o_ref) + 1e-4)
        err = np.abs(f64(o[b, h, rows_t]) - o_ref)
        _log(f"  head ({b},{h}): max {err.max():.2e} mean {err.mean():.2e} "
             f"worst err/bound {(err / bound).max():.2f}")
        assert np.all(err <= bound)
        assert np.abs(lse[b, h, rows_t].cpu().numpy() - l_ref).max() <= 1e-3
    del q, k, v, o, lse
    torch.cuda.empty_cache()


SPLIT_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, causal, splits
    (1, 8, 2, 1, 1000, 128, False, 4),     # a decode step, 4 query heads per KV head
    (2, 4, 1, 1, 333, 64, False, 3),
    (1, 4, 2, 150, 333, 64, True, 3),
    (1, 2, 2, 200, 517, 128, True, 5),
    (1, 2, 2, 64, 64, 64, False, 16),      # more splits than key tiles
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_fp8_key_split_within_bound(gpu_device, case):
    """The key-split path with FP8 inputs (the decode step over an FP8 KV cache):
    each split rounds its own P to E4M3 against its own reference max, so the
    bound of the fused FP8 check applies to every split's part of the row, and
    the merge of the fp32 partials adds only float32 rounding."""
    B, Hq, Hkv, Nq, Nk, D, causal, splits = case
    w = custom(B, Hq, Hkv, Nq, Nk, D, "fp8", causal, False)
    _log(f"fp8 split case {case}")
    q, k, v, _ = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=54))
    o, lse = binding.forward_split(q, k, v, None, causal=causal, scale=w.scale,
                                   num_splits=splits)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    mx, mean, ratio = fp8_bound_check(q, k, v, w.scale, causal, o, lse, str(case))
    _log(f"  max {mx:.2e} mean {mean:.2e} worst err/bound {ratio:.2f}")
    on, ln = binding.forward_split_noalloc(q, k, v, None, causal=causal, scale=w.scale,
                                           num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(on, o) and torch.equal(ln, lse)   # same kernels, same partials


def test_fp8_decode_full_size(gpu_device):
    """The decode workload with an FP8 KV cache (B8, 20/4 heads, Nq 1, Nk 32768,
    D 128), every row against the oracle within the FP8 bound."""
    from tiled_attention_forward_amd.workloads import WORKLOADS
    w = WORKLOADS["decode_b8_hq20_hkv4_nq1_nk32768_d128_fp8"]
    _log("full-size fp8 decode")
    q, k, v, _ = make_inputs(w, seed=0, device=gpu_device)
    o, lse = binding.forward_split(q, k, v, None, causal=False, scale=w.scale)
    torch.cuda.synchronize()
    mx, mean, ratio = fp8_bound_check(q, k, v, w.scale, False, o, lse, w.name)
    _log(f"  max {mx:.2e} mean {mean:.2e} worst err/bound {ratio:.2f}")
    del q, k, v, o, lse
    torch.cuda.empty_cache()


WINDOW_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, window
    (1, 2, 2, 300, 300, 64, 37),
    (1, 4, 2, 513, 600, 128, 100),     # GQA, Nk > Nq
    (2, 2, 1, 1000, 1000, 64, 256),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "-".join(map(str, c)))
def test_fp8_window_within_bound(gpu_device, case):
    """FP8 inputs with the causal sliding window (fa_forward_window): the same
    bound over each row's visible keys."""
    B, Hq, Hkv, Nq, Nk, D, win = case
    w = custom(B, Hq, Hkv, Nq, Nk, D, "fp8", True, False)
    _log(f"fp8 window case {case}")
    q, k, v, _ = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=57))
    o, lse = binding.forward(q, k, v, None, causal=True, scale=w.scale, window=win)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    mx, mean, ratio = fp8_bound_check(q, k, v, w.scale, True, o, lse, str(case), window=win)
    _log(f"  max {mx:.2e} mean {mean:.2e} worst err/bound {ratio:.2f}")
