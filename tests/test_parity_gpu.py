"""GPU parity: fa_forward (through the C ABI) against the fp64 oracle.

Small problems are compared element by element over the whole output; the
full-size workloads run in exactly the configuration bench.py times and are
compared on sampled rows (the oracle evaluates those rows one by one) plus
properties that hold at any size.
"""

import math

import numpy as np
import pytest
import torch

from tests.parity import (f64, full_check, rounding_bound_check, run_gpu, sampled_check)
from tiled_attention_forward_amd import binding
from tiled_attention_forward_amd.workloads import WORKLOADS, custom, make_inputs, sample_rows

pytestmark = pytest.mark.gpu

SMALL = ["b1_h1_s256_d64_fp32", "b2_h16_s512_d64_fp16", "b2_h16_s512_d64_fp16_causal"]


def _log(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("name", SMALL)
def test_small_workloads_full(gpu_device, name, seed):
    w = WORKLOADS[name]
    _log(f"case {name} seed {seed}")
    q, k, v, bias = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed))
    st, _, _ = full_check(q, k, v, bias, w.scale, w.causal, w.dtype, f"{name}/{seed}")
    _log(st)


EDGE = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, bias
    (1, 1, 1, 1, 1, 64, "bf16", False, False),
    (1, 1, 1, 1, 1, 128, "bf16", True, True),
    (1, 2, 2, 1000, 1000, 64, "fp16", True, False),
    (1, 2, 2, 1000, 1000, 128, "bf16", False, True),
    (1, 2, 1, 333, 517, 64, "bf16", False, True),
    (1, 2, 1, 517, 333, 128, "fp16", True, False),
    (2, 10, 2, 200, 300, 64, "bf16", True, True),
    (1, 4, 2, 130, 70, 128, "fp32", True, True),
    (1, 3, 3, 64, 64, 64, "fp32", False, False),
    (1, 1, 1, 127, 129, 64, "bf16", True, False),
    (2, 4, 4, 128, 128, 64, "bf16", True, False),
    (1, 8, 1, 256, 256, 128, "bf16", False, False),
    (1, 2, 2, 1, 700, 64, "bf16", False, False),
    (1, 2, 2, 700, 1, 64, "bf16", True, False),
    (1, 2, 2, 70, 70, 64, "fp32", True, False),
    (1, 2, 1, 129, 131, 128, "fp16", False, True),
    (3, 2, 2, 65, 63, 64, "fp16", True, True),
    # head dims 80 and 96 (the xnwp.cn post, §5.1 and §6.4): 128-wide tiles
    (1, 2, 2, 1000, 1000, 80, "bf16", True, False),
    (1, 4, 2, 333, 517, 96, "fp16", False, True),
    (2, 10, 2, 200, 300, 80, "fp16", True, True),
    (1, 2, 1, 517, 333, 96, "bf16", True, False),
    (1, 1, 1, 1, 1, 80, "bf16", False, False),
    (1, 2, 2, 130, 70, 96, "bf16", False, False),
    # D = 128, non-causal, no bias: two 32-row query blocks per wave (256 rows
    # per workgroup) over 32-key tiles; row counts around the 32-, 64- and
    # 256-row boundaries, key counts around the 32-key tile
    (1, 2, 2, 1, 33, 128, "bf16", False, False),
    (1, 2, 1, 33, 31, 128, "fp16", False, False),
    (1, 4, 2, 65, 200, 128, "bf16", False, False),
    (2, 3, 3, 255, 257, 128, "bf16", False, False),
    (1, 2, 2, 257, 1, 128, "fp16", False, False),
    (1, 5, 1, 300, 333, 128, "bf16", False, False),
    (1, 2, 2, 513, 64, 128, "bf16", False, False),
    # head dim 256: 32-key tiles
    (1, 2, 2, 300, 300, 256, "bf16", True, False),
    (1, 4, 2, 257, 190, 256, "fp16", False, False),
    (2, 4, 1, 130, 170, 256, "bf16", True, True),
    (1, 2, 2, 1, 1, 256, "bf16", False, True),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "-".join(map(str, c)))
def test_edge_shapes(gpu_device, case):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, bias = case
    w = custom(B, Hq, Hkv, Nq, Nk, D, dt, causal, bias)
    _log(f"case {case}")
    q, k, v, b = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=7))
    st, _, _ = full_check(q, k, v, b, w.scale, causal, dt, str(case))
    _log(st)


def _check_any_scale(q, k, v, b, scale, causal, dt, what):
    """fp32: the fixed 1e-5 bar.  bf16/fp16: the fixed bars hold for the pages'
    workloads (logit std about 1-1.4); other scales widen the logit spread, so
    the derived rounding bound is checked instead."""
    if dt == "fp32":
        full_check(q, k, v, b, scale, causal, dt, what)
    else:
        o, lse = run_gpu(q, k, v, b, scale, causal)
        rounding_bound_check(q, k, v, b, scale, causal, dt, o, lse, what)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 1e-3, 0.3, -0.3])
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_scale_values(gpu_device, scale, dt):
    """Any finite scale: negative (Q sign flip), zero (uniform softmax), small, larger."""
    w = custom(1, 2, 1, 150, 150, 64, dt, True, False)
    _log(f"scale {scale} {dt}")
    q, k, v, _ = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=3))
    _check_any_scale(q, k, v, None, scale, True, dt, f"scale={scale}")
    w2 = custom(1, 2, 2, 90, 77, 128, dt, False, True)
    q, k, v, b = (t.to(gpu_device) for t in make_inputs(w2, seed=4))
    _check_any_scale(q, k, v, b, scale, False, dt, f"bias scale={scale}")


@pytest.mark.parametrize("scale", [1.0, -2.0, 2.0])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_extreme_logits_within_rounding_bound(gpu_device, scale, dt):
    """Logit spreads far beyond the workloads' (std 8-22)."""
    w = custom(1, 4, 2, 150, 170, 128, dt, True, True)
    q, k, v, b = (t.to(gpu_device) for t in make_inputs(w, seed=11))
    o, lse = run_gpu(q, k, v, b, scale, True)
    rounding_bound_check(q, k, v, b, scale, True, dt, o, lse, f"scale={scale}")


def test_no_keys(gpu_device):
    """Nk = 0: every row sees no key, O = 0 and LSE = -inf."""
    q = torch.randn(1, 2, 40, 64, device=gpu_device).to(torch.bfloat16)
    k = torch.empty(1, 2, 0, 64, device=gpu_device, dtype=torch.bfloat16)
    for causal in (False, True):
        o, lse = run_gpu(q, k, k, None, 0.125, causal)
        assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_empty_batch(gpu_device):
    q = torch.empty(0, 2, 16, 64, device=gpu_device, dtype=torch.bfloat16)
    o, lse = run_gpu(q, q, q, None, 0.125, True)
    assert o.shape == q.shape and lse.shape == (0, 2, 16)


def test_bias_minus_inf_row(gpu_device):
    """A row whose bias is -inf everywhere has no finite logit: O = 0, LSE = -inf."""
    w = custom(1, 1, 1, 70, 66, 64, "bf16", False, True)
    q, k, v, b = (t.to(gpu_device) for t in make_inputs(w, seed=5))
    b[0, 0, 3, :] = float("-inf")
    st, o, lse = full_check(q, k, v, b, w.scale, False, "bf16", "-inf bias row")
    assert torch.all(o[0, 0, 3] == 0) and torch.isneginf(lse[0, 0, 3])


def test_deterministic_and_stream(gpu_device):
    """Same inputs, same bits; a side stream gives the same result."""
    w = custom(2, 4, 2, 300, 300, 64, "bf16", True, True)
    q, k, v, b = (t.to(gpu_device) for t in make_inputs(w, seed=9))
    o1, l1 = run_gpu(q, k, v, b, w.scale, True)
    o2, l2 = run_gpu(q, k, v, b, w.scale, True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o3, l3 = binding.forward(q, k, v, b, causal=True, scale=w.scale)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


FULL = ["b2_h16_s512_d64_fp16", "b2_h16_s512_d64_fp16_causal", "b2_h16_s4096_d64_bf16_causal",
        "b8_h32_s2048_d128_bf16", "b1_hq20_hkv4_s8192_d128_bf16_causal_bias"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(gpu_device, name):
    """Full-size run as bench.py times it; oracle on sampled rows of several heads."""
    w = WORKLOADS[name]
    _log(f"full-size {name}")
    q, k, v, bias = make_inputs(w, seed=0, device=gpu_device)
    o, lse = run_gpu(q, k, v, bias, w.scale, w.causal)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    heads = sorted({(0, 0), (w.B - 1, w.Hq - 1), (0, w.Hq // 2), (w.B // 2, 1 % w.Hq)})
    rows = sample_rows(w.Nq, 40, seed=1)
    st = sampled_check(q, k, v, bias, w.scale, w.causal, w.dtype, heads, rows, o, lse, name)
    _log(st)
    if w.causal:
        # row 0 sees only key 0: O_0 = V_0 exactly in every head
        grp = w.Hq // w.Hkv
        v0 = v[:, :, 0, :].repeat_interleave(grp, dim=1)
        assert torch.equal(o[:, :, 0, :], v0)
    del q, k, v, bias, o, lse
    torch.cuda.empty_cache()


WINDOW_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, bias, window
    (1, 2, 2, 300, 300, 64, "bf16", False, 1),
    (1, 2, 2, 300, 300, 64, "bf16", False, 37),      # inside one key tile
    (1, 2, 1, 513, 513, 64, "fp16", True, 100),      # across tiles, GQA, bias
    (2, 4, 2, 1000, 1000, 128, "bf16", False, 256),
    (1, 2, 2, 700, 900, 128, "bf16", True, 129),     # Nk > Nq
    (1, 2, 2, 200, 200, 64, "fp32", False, 64),
    (1, 2, 2, 200, 200, 64, "bf16", False, 200),     # window = Nk: plain causal
    (1, 2, 2, 300, 300, 96, "bf16", False, 50),
    (1, 2, 1, 513, 513, 80, "fp16", True, 100),
    (1, 2, 2, 300, 300, 256, "bf16", False, 50),     # head size 256
    (1, 4, 2, 200, 260, 256, "fp16", True, 64),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "-".join(map(str, c)))
def test_window_forward(gpu_device, case):
    """Causal sliding window (fa_forward_window) against the oracle's window mask."""
    from oracle import attention_forward
    B, Hq, Hkv, Nq, Nk, D, dt, bias, win = case
    w = custom(B, Hq, Hkv, Nq, Nk, D, dt, True, bias)
    _log(f"window case {case}")
    q, k, v, b = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=41))
    o, lse = binding.forward(q, k, v, b, causal=True, scale=w.scale, window=win)
    torch.cuda.synchronize()
    o_ref, l_ref = attention_forward(f64(q), f64(k), f64(v), None if b is None else f64(b),
                                     scale=w.scale, causal=True, window=win)
    from tests.parity import assert_within, errors
    st = errors(f64(o), lse.cpu().numpy(), o_ref, l_ref)
    _log(st)
    assert_within(st, dt, str(case))
    if win >= Nk:
        o2, l2 = run_gpu(q, k, v, b, w.scale, True)
        assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_window_full_size_sampled(gpu_device):
    """The headline shape with a 1024-key window, sampled rows against the oracle."""
    from oracle import attention_head_rows
    w = WORKLOADS["b2_h16_s4096_d64_bf16_causal"]
    q, k, v, _ = make_inputs(w, seed=0, device=gpu_device)
    o, lse = binding.forward(q, k, v, None, causal=True, scale=w.scale, window=1024)
    torch.cuda.synchronize()
    rows = sample_rows(w.Nq, 40, seed=3)
    rt = torch.as_tensor(rows, device=gpu_device)
    from tests.parity import assert_within, errors
    for bb, h in ((0, 0), (1, 15)):
        o_ref, l_ref = attention_head_rows(f64(q[bb, h].index_select(0, rt)), f64(k[bb, h]),
                                           f64(v[bb, h]), rows=rows, scale=w.scale, causal=True,
                                           window=1024)
        st = errors(f64(o[bb, h].index_select(0, rt)), lse[bb, h].index_select(0, rt).cpu().numpy(),
                    o_ref, l_ref)
        _log(st)
        assert_within(st, "bf16", f"window 1024 b{bb} h{h}")


@pytest.mark.parametrize("D", [80, 96])
def test_narrow_head_writes_only_its_columns(gpu_device, D):
    """With D = 80 the kernel computes 96 output columns; the 16 past the row
    must not be stored (they would land on the next row, and past the last
    row outside the tensor).  The output sits at the start of a larger buffer
    whose tail is a sentinel."""
    w = custom(1, 2, 2, 129, 200, D, "bf16", True, False)
    q, k, v, _ = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=9))
    n = q.numel()
    buf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device=gpu_device)
    out = buf[:n].view(q.shape)
    o, lse = binding.forward(q, k, v, None, causal=True, scale=w.scale, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[n:] == 7.0)
    from oracle import attention_forward
    from tests.parity import assert_within, errors
    o_ref, l_ref = attention_forward(f64(q), f64(k), f64(v), None, scale=w.scale, causal=True)
    assert_within(errors(f64(o), lse.cpu().numpy(), o_ref, l_ref), "bf16", f"D={D}")


def test_head_dim_80_full_size_sampled(gpu_device):
    """The benchmark report shape (B2 H16 S4096 causal) with 80-wide heads."""
    w = custom(2, 16, 16, 4096, 4096, 80, "bf16", True, False)
    _log("full-size D=80")
    q, k, v, _ = make_inputs(w, seed=3, device=gpu_device)
    o, lse = run_gpu(q, k, v, None, w.scale, True)
    st = sampled_check(q, k, v, None, w.scale, True, "bf16", [(0, 0), (1, 15)],
                       sample_rows(w.Nq, 64, seed=3), o, lse, "D=80 full size")
    _log(st)


def test_head_dim_256_full_size_sampled(gpu_device):
    """The benchmark report shape (B2 H16 S4096 causal) with 256-wide heads."""
    w = custom(2, 16, 16, 4096, 4096, 256, "bf16", True, False)
    _log("full-size D=256")
    q, k, v, _ = make_inputs(w, seed=6, device=gpu_device)
    o, lse = run_gpu(q, k, v, None, w.scale, True)
    st = sampled_check(q, k, v, None, w.scale, True, "bf16", [(0, 0), (1, 15)],
                       sample_rows(w.Nq, 64, seed=6), o, lse, "D=256 full size")
    _log(st)
