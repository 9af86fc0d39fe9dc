"""GPU parity of the backward (fa_backward through the C ABI) against the fp64
oracle's ``attention_backward``.

The GPU forward produces O and LSE (the backward's inputs, as in training); the
oracle differentiates the definition from q, k, v, bias and dO alone.

Tolerance (the pages fix none for gradients; derived from the arithmetic):
P and dS are rounded to the input type before their products (relative
error u per term, u = 2^-8 bf16, 2^-11 fp16), D_i is formed from the rounded
O, and each gradient is rounded once more on output.  Each source moves an
element by about u relative to the gradient's own scale, so per tensor:
    bf16: max |dG - dG_ref| <= 3e-2 * max |dG_ref|,  mean <= 1e-2 * mean |dG_ref|
    fp16: max |dG - dG_ref| <= 6e-3 * max |dG_ref|,  mean <= 2e-3 * mean |dG_ref|
fp32 inputs take no rounding of P or dS: every step is an fp32 operation, the
longest sums run over Nk keys or D columns (relative error up to about
(Nk + D) 2^-24 in the worst case, 1e-6 typically), and exp2 is v_exp_f32
(about one ulp).  So
    fp32: max |dG - dG_ref| <= 1e-4 * max |dG_ref|,  mean <= 1e-5 * mean |dG_ref|
"""

import numpy as np
import pytest
import torch

from oracle import attention_backward
from tests.parity import f64
from tiled_attention_forward_amd import binding
from tiled_attention_forward_amd.workloads import WORKLOADS, custom, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": (3e-2, 1e-2), "fp16": (6e-3, 2e-3), "fp32": (1e-4, 1e-5)}


def _log(*a):
    print(*a, flush=True)


def _dout(shape, seed, dtype, device):
    g = torch.Generator(device="cpu").manual_seed(1000 + seed)
    return torch.randn(shape, generator=g).to(dtype).to(device)


def run_backward(q, k, v, bias, dout, scale, causal):
    o, lse = binding.forward(q, k, v, bias, causal=causal, scale=scale)
    dq, dk, dv = binding.backward(q, k, v, o, lse, dout, bias, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def compare(got, ref, dtype, what, atol=0.0):
    """Relative bars of the module docstring.  A gradient tensor that the
    definition makes zero by cancellation (every row sees one key: P = 1 and
    O = v, so dP - D_i = dO.v - dO.O is exactly 0 in the oracle) is instead
    held to the absolute bound ``atol``: the kernel forms dP (matrix cores) and
    D_i (from the rounded O) as two fp32 sums of D products, each off by up to
    about D 2^-24 sum_d |dO_d v_d|, and dQ and dK carry that times scale |K| or
    scale |Q|.  That applies only when the whole reference lies within atol."""
    mx_tol, mean_tol = TOL[dtype]
    out = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = f64(g)
        assert np.isfinite(g).all(), f"{what} {name}: non-finite"
        err = np.abs(g - r)
        scale_max = max(np.abs(r).max(initial=0.0), 1e-30)
        scale_mean = max(np.abs(r).mean() if r.size else 0.0, 1e-30)
        out[name] = (float(err.max(initial=0.0) / scale_max),
                     float(err.mean() / scale_mean) if r.size else 0.0)
        if np.abs(r).max(initial=0.0) <= atol:
            assert err.max(initial=0.0) <= atol, f"{what} {name} max abs {err.max()} > {atol}"
            continue
        assert err.max(initial=0.0) <= mx_tol * scale_max, f"{what} {name} max {out[name]}"
        if r.size:
            assert err.mean() <= mean_tol * scale_mean, f"{what} {name} mean {out[name]}"
    return out


def cancellation_floor(q, k, v, dout, scale):
    """The absolute floor of ``compare`` for these inputs: 2 D 2^-24 max|dO|
    max|V| D (the two sums' rounding, with |sum| <= D max|dO| max|V|) times
    scale max(|K|, |Q|)."""
    D = q.shape[-1]
    m = lambda t: float(t.abs().max()) if t.numel() else 0.0
    return 2.0 * D * 2.0 ** -24 * D * m(dout) * m(v) * abs(scale) * max(m(k), m(q))


CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, bias
    (1, 2, 2, 128, 128, 64, "bf16", False, False),
    (1, 2, 2, 200, 200, 64, "bf16", True, False),
    (2, 4, 2, 130, 170, 64, "fp16", True, True),
    (1, 4, 1, 100, 300, 128, "bf16", True, False),   # group 4: row tiles cross heads
    (1, 5, 1, 64, 64, 64, "bf16", True, False),      # group 5
    (1, 2, 1, 333, 257, 128, "bf16", False, True),
    (2, 2, 2, 257, 129, 128, "fp16", False, False),
    (1, 2, 2, 50, 300, 64, "bf16", True, False),     # keys 50.. seen by no query
    (1, 2, 2, 1, 1, 64, "bf16", False, False),
    (1, 3, 3, 65, 63, 128, "fp16", True, True),
    (1, 2, 2, 1000, 1000, 64, "bf16", True, False),
    (1, 6, 2, 7, 40, 64, "bf16", True, True),        # group 3, fewer rows than a tile
    # non-causal D = 128 without a logit term: 32-row query tiles, V in LDS
    (1, 4, 2, 97, 200, 128, "bf16", False, False),   # group 2: row tiles cross heads
    (1, 3, 1, 31, 33, 128, "bf16", False, False),    # group 3, rows < one tile, key tail
    # head sizes 80 and 96 (128-wide LDS rows, last column block partly stored)
    (1, 2, 2, 150, 170, 80, "bf16", True, False),
    (1, 4, 2, 97, 200, 96, "fp16", False, False),    # group 2
    (1, 2, 1, 130, 129, 80, "bf16", False, True),
    (1, 3, 1, 77, 64, 96, "bf16", True, True),       # group 3, bias
    # head size 256 (no logit term): 32-key dQ tiles, dK/dV in two column passes
    (1, 2, 2, 150, 170, 256, "bf16", True, False),
    (1, 4, 2, 97, 200, 256, "fp16", False, False),   # group 2: row tiles cross heads
    (1, 3, 1, 33, 31, 256, "bf16", True, False),     # group 3, rows < one tile, key tail
    (1, 2, 2, 300, 129, 256, "bf16", False, False),
    # fp32 (head sizes 64 and 128): plain fp32 arithmetic, one row or key per lane
    (1, 1, 1, 256, 256, 64, "fp32", False, False),    # the fp32 parity workload's shape
    (1, 2, 2, 200, 200, 64, "fp32", True, False),
    (2, 4, 2, 130, 170, 64, "fp32", True, True),
    (1, 4, 1, 100, 300, 128, "fp32", True, False),    # group 4
    (1, 3, 1, 97, 64, 128, "fp32", False, True),      # group 3, bias
    (1, 2, 2, 1, 1, 128, "fp32", False, False),
    (1, 5, 1, 300, 129, 64, "fp32", False, False),    # group 5, key tail
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_backward_matches_oracle(gpu_device, case):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, bias = case
    w = custom(B, Hq, Hkv, Nq, Nk, D, dt, causal, bias)
    _log(f"backward case {case}")
    q, k, v, b = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=31))
    dout = _dout(q.shape, 31, q.dtype, gpu_device)
    got = run_backward(q, k, v, b, dout, w.scale, causal)
    ref = attention_backward(f64(q), f64(k), f64(v), f64(dout),
                             None if b is None else f64(b), scale=w.scale, causal=causal)
    _log(compare(got, ref, dt, str(case)))
    if causal and Nk > Nq:
        # top-left causal: keys at positions >= Nq are seen by no query
        assert torch.all(got[1][:, :, Nq:] == 0) and torch.all(got[2][:, :, Nq:] == 0)


def test_backward_no_keys(gpu_device):
    q = torch.randn(1, 2, 40, 64, device=gpu_device).to(torch.bfloat16)
    k = torch.empty(1, 1, 0, 64, device=gpu_device, dtype=torch.bfloat16)
    o, lse = binding.forward(q, k, k, None, causal=False, scale=0.125)
    dq, dk, dv = binding.backward(q, k, k, o, lse, q.clone(), None, causal=False, scale=0.125)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0


def test_backward_no_queries_zeroes_dk_dv(gpu_device):
    q = torch.empty(1, 2, 0, 64, device=gpu_device, dtype=torch.bfloat16)
    k = torch.randn(1, 2, 70, 64, device=gpu_device).to(torch.bfloat16)
    lse = torch.empty(1, 2, 0, device=gpu_device)
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(k, 7.0)
    binding.backward(q, k, k, q, lse, q, None, causal=True, scale=0.125, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_backward_deterministic(gpu_device):
    w = custom(1, 4, 2, 300, 300, 64, "bf16", True, True)
    q, k, v, b = (t.to(gpu_device) for t in make_inputs(w, seed=32))
    dout = _dout(q.shape, 32, q.dtype, gpu_device)
    a = run_backward(q, k, v, b, dout, w.scale, True)
    c = run_backward(q, k, v, b, dout, w.scale, True)
    assert all(torch.equal(x, y) for x, y in zip(a, c))


@pytest.mark.parametrize("name", ["b2_h16_s4096_d64_bf16_causal", "b8_h32_s2048_d128_bf16",
                                  "b8_h32_s2048_d128_bf16_causal"])
def test_backward_full_size_heads(gpu_device, name):
    """Full-size run; the oracle differentiates two whole heads (MHA: a head's
    dQ, dK and dV depend only on that head's Q, K, V and dO)."""
    w = WORKLOADS[name]
    _log(f"full-size backward {name}")
    q, k, v, _ = make_inputs(w, seed=0, device=gpu_device)
    dout = _dout(q.shape, 0, q.dtype, gpu_device)
    dq, dk, dv = run_backward(q, k, v, None, dout, w.scale, w.causal)
    for bb, h in ((0, 0), (w.B - 1, w.Hq - 1)):
        sl = (slice(bb, bb + 1), slice(h, h + 1))
        ref = attention_backward(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(dout[sl]), None,
                                 scale=w.scale, causal=w.causal)
        _log(compare((dq[sl], dk[sl], dv[sl]), ref, w.dtype, f"{name} b{bb} h{h}"))
    del q, k, v, dout, dq, dk, dv
    torch.cuda.empty_cache()


WINDOW_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, bias, window
    (1, 2, 2, 300, 300, 64, "bf16", False, 37),
    (1, 4, 1, 200, 260, 128, "bf16", True, 100),     # GQA, bias, Nk > Nq
    (2, 2, 2, 513, 513, 64, "fp16", False, 129),
    (1, 5, 1, 64, 64, 64, "bf16", False, 5),          # group 5: row tiles cross heads
    (1, 3, 1, 20, 20, 128, "bf16", False, 6),         # group 3, fewer rows than a tile
    (1, 2, 2, 200, 200, 96, "bf16", False, 50),
    (1, 4, 2, 150, 180, 80, "fp16", True, 64),
    (1, 2, 2, 200, 200, 256, "bf16", False, 50),      # head size 256
    (1, 4, 2, 150, 180, 256, "fp16", False, 64),
    (1, 2, 2, 300, 300, 64, "fp32", False, 37),
    (1, 4, 1, 200, 260, 128, "fp32", True, 100),      # GQA, bias, Nk > Nq
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "-".join(map(str, c)))
def test_window_backward(gpu_device, case):
    B, Hq, Hkv, Nq, Nk, D, dt, bias, win = case
    w = custom(B, Hq, Hkv, Nq, Nk, D, dt, True, bias)
    _log(f"window backward case {case}")
    q, k, v, b = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=42))
    dout = _dout(q.shape, 42, q.dtype, gpu_device)
    o, lse = binding.forward(q, k, v, b, causal=True, scale=w.scale, window=win)
    got = binding.backward(q, k, v, o, lse, dout, b, causal=True, scale=w.scale, window=win)
    torch.cuda.synchronize()
    ref = attention_backward(f64(q), f64(k), f64(v), f64(dout), None if b is None else f64(b),
                             scale=w.scale, causal=True, window=win)
    _log(compare(got, ref, dt, str(case)))
