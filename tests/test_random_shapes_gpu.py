"""Seeded random sweep of the forward entry points (16-bit, fp32 and FP8
inputs), of the backward and of the residual chain (forward and backward),
against the oracle.

Each case draws a shape (batch, query heads, KV-head group, query and key
counts with ragged tails), an element type, a head dimension, the causal flag,
a bias, and an entry point (fused, sliding window, key split), all from one
fixed-seed generator, so the set of cases is the same on every run and a
failure names its case.  The bars are those of tests/parity.py; cases whose
logits spread wider than the pages' workloads do not occur (scale = 1/sqrt(D),
N(0, 1) inputs).  The shapes go beyond the pages' workloads, though: with few
visible keys (early causal rows, short key ranges, a logit term) an output
row is close to a single V row and reaches |O| of 2 to 5, where bf16 values
lie 0.0156 or 0.031 apart.  There an element can miss the 1e-2 max bar by its
final rounding alone, so such elements are held to one output ulp of the
exact value (tests/parity.py, ``output_spacing_check``); the mean and LSE bars
and every other element keep the stated bars.
"""

import random
import zlib

import pytest
import torch

from tests.parity import full_check, run_split
from tiled_attention_forward_amd import binding
from tiled_attention_forward_amd.workloads import custom, make_inputs

pytestmark = pytest.mark.gpu


def _cases(n=80, seed=2024):
    r = random.Random(seed)
    out = []
    while len(out) < n:
        dtype = r.choice(["bf16", "bf16", "fp16", "fp32"])
        D = r.choice([64, 128] if dtype == "fp32" else [64, 80, 96, 128, 256])
        path = r.choice(["fused", "fused", "window", "split"])
        causal = path == "window" or r.random() < 0.5
        bias = r.random() < 0.3
        hkv = r.choice([1, 2, 3])
        group = r.choice([1, 2, 5])
        nq = r.choice([1, 7, 64, 127, 200, 333])
        nk = r.choice([1, 63, 64, 65, 190, 400]) if not causal else r.choice([nq, nq + 17, 300])
        window = r.choice([1, 16, 100]) if path == "window" else None
        out.append((r.choice([1, 2]), hkv * group, hkv, nq, nk, D, dtype, causal, bias, path,
                    window))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "-".join(map(str, c)))
def test_random_case(gpu_device, case):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, bias, path, window = case
    print(f"random case {case}", flush=True)
    w = custom(B, Hq, Hkv, Nq, Nk, D, dt, causal, bias)
    seed = zlib.crc32(repr(case).encode()) % 100000   # stable across processes
    q, k, v, b = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=seed))
    if path == "split":
        full_check(q, k, v, b, w.scale, causal, dt, str(case), run=run_split(3), spacing=True)
    elif path == "window":
        from oracle import attention_forward
        from tests.parity import O_TOL, assert_within, errors, f64, output_spacing_check
        o, lse = binding.forward(q, k, v, b, causal=True, scale=w.scale, window=window)
        torch.cuda.synchronize()
        o_ref, l_ref = attention_forward(f64(q), f64(k), f64(v), None if b is None else f64(b),
                                         scale=w.scale, causal=True, window=window)
        st = errors(f64(o), lse.cpu().numpy(), o_ref, l_ref)
        if dt != "fp32" and st["max_abs"] > O_TOL[dt][0]:
            output_spacing_check(f64(o), o_ref, st, dt, str(case))
        else:
            assert_within(st, dt, str(case))
    else:
        full_check(q, k, v, b, w.scale, causal, dt, str(case), spacing=True)


# Cases of a wider sweep (other seeds) in which one element lands on the far
# bf16 neighbour of an exact value in [2, 4) (0.0104-0.0134 away, one ulp):
# they exercise the output-spacing rule.
SPACING_CASES = [
    (2, 10, 2, 127, 127, 256, "bf16", True, True, "fused", None),
    (2, 5, 1, 7, 7, 256, "bf16", True, False, "fused", None),
    (1, 6, 3, 333, 63, 256, "bf16", False, True, "fused", None),
]


@pytest.mark.parametrize("case", SPACING_CASES, ids=lambda c: "-".join(map(str, c)))
def test_output_spacing_case(gpu_device, case):
    test_random_case(gpu_device, case)


def _backward_cases(n=40, seed=4048):
    r = random.Random(seed)
    out = []
    while len(out) < n:
        dtype = r.choice(["bf16", "bf16", "fp16", "fp32"])
        D = r.choice([64, 128] if dtype == "fp32" else [64, 80, 96, 128, 256])
        # (head size 256: no logit term in the backward)
        window = r.choice([None, None, None, 1, 16, 100])
        causal = window is not None or r.random() < 0.5
        bias = D != 256 and r.random() < 0.3
        hkv = r.choice([1, 2, 3])
        group = r.choice([1, 2, 5])
        nq = r.choice([1, 7, 64, 127, 200, 333])
        nk = r.choice([1, 63, 64, 65, 190, 400]) if not causal else r.choice([nq, nq + 17, 300])
        out.append((r.choice([1, 2]), hkv * group, hkv, nq, nk, D, dtype, causal, bias, window))
    return out


@pytest.mark.parametrize("case", _backward_cases(), ids=lambda c: "-".join(map(str, c)))
def test_random_backward_case(gpu_device, case):
    """The same kind of sweep for fa_backward (and its window form): dQ, dK and
    dV against the oracle's gradients at the bars of test_backward_gpu."""
    from oracle import attention_backward
    from tests.parity import f64
    from tests.test_backward_gpu import cancellation_floor, compare
    B, Hq, Hkv, Nq, Nk, D, dt, causal, bias, window = case
    print(f"random backward case {case}", flush=True)
    w = custom(B, Hq, Hkv, Nq, Nk, D, dt, causal, bias)
    seed = zlib.crc32(repr(case).encode()) % 100000
    q, k, v, b = (None if t is None else t.to(gpu_device) for t in make_inputs(w, seed=seed))
    g = torch.Generator().manual_seed(seed + 1)
    dout = torch.randn(q.shape, generator=g).to(q.dtype).to(gpu_device)
    o, lse = binding.forward(q, k, v, b, causal=causal, scale=w.scale, window=window)
    dq, dk, dv = binding.backward(q, k, v, o, lse, dout, b, causal=causal, scale=w.scale,
                                  window=window)
    torch.cuda.synchronize()
    refs = attention_backward(f64(q), f64(k), f64(v), f64(dout), None if b is None else f64(b),
                              scale=w.scale, causal=causal, window=window)
    atol = cancellation_floor(q, k, v, dout, w.scale)
    print(compare((dq, dk, dv), refs, dt, str(case), atol=atol), flush=True)


def _chain_cases(n=24, seed=6060):
    r = random.Random(seed)
    out = []
    while len(out) < n:
        layers = r.choice([1, 2, 3, 4])
        D = r.choice([64, 80, 96, 128])
        dtype = r.choice(["bf16", "fp16"])
        causal = r.random() < 0.5
        hkv = r.choice([1, 2, 3])
        group = r.choice([1, 2, 5])
        nq = r.choice([1, 7, 64, 127, 200, 333])
        nk = r.choice([1, 63, 64, 65, 190, 400]) if not causal else r.choice([nq, nq + 17, 300])
        out.append((layers, r.choice([1, 2]), hkv * group, hkv, nq, nk, D, dtype, causal))
    return out


@pytest.mark.parametrize("case", _chain_cases(), ids=lambda c: "-".join(map(str, c)))
def test_random_chain_case(gpu_device, case):
    """The residual chain (fa_forward_chain, then fa_backward_chain) on the same
    kind of sweep: O and LSE at the forward's bars (with the output-spacing
    rule), every layer's dQ and dK and dV at the backward's."""
    from oracle import attention_chain, attention_chain_backward
    from tests.parity import O_TOL, assert_within, errors, f64, output_spacing_check
    from tests.test_backward_gpu import cancellation_floor, compare
    from tiled_attention_forward_amd.workloads import make_chain_inputs
    layers, B, Hq, Hkv, Nq, Nk, D, dt, causal = case
    print(f"random chain case {case}", flush=True)
    w = custom(B, Hq, Hkv, Nq, Nk, D, dt, causal, False)
    seed = zlib.crc32(repr(case).encode()) % 100000
    qs, ks, v = make_chain_inputs(w, layers, seed=seed)
    qs, ks, v = [t.to(gpu_device) for t in qs], [t.to(gpu_device) for t in ks], v.to(gpu_device)
    g = torch.Generator().manual_seed(seed + 1)
    dout = torch.randn(qs[-1].shape, generator=g).to(qs[-1].dtype).to(gpu_device)
    o, lse = binding.forward_chain(qs, ks, v, causal=causal, scale=w.scale)
    dqs, dks, dv = binding.backward_chain(qs, ks, v, o, lse, dout, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    hq, hk = [f64(t) for t in qs], [f64(t) for t in ks]
    o_ref, l_ref = attention_chain(hq, hk, f64(v), scale=w.scale, causal=causal)
    st = errors(f64(o), lse.cpu().numpy(), o_ref, l_ref)
    if st["max_abs"] > O_TOL[dt][0]:
        output_spacing_check(f64(o), o_ref, st, dt, str(case))
    else:
        assert_within(st, dt, str(case))
    rq, rk, rv = attention_chain_backward(hq, hk, f64(v), f64(dout), scale=w.scale,
                                          causal=causal)
    # the one-layer backward's cancellation floor (dP - D_i is a contraction
    # over D whatever the chain length), with each layer's Q and K
    atol = max(cancellation_floor(ql, kl, v, dout, w.scale) for ql, kl in zip(qs, ks))
    for l in range(layers):
        print(l, compare((dqs[l], dks[l], dv), (rq[l], rk[l], rv), dt, f"{case} layer {l}",
                         atol=atol), flush=True)


def _fp8_cases(n=16, seed=7070):
    r = random.Random(seed)
    out = []
    while len(out) < n:
        D = r.choice([64, 128])
        causal = r.random() < 0.5
        hkv = r.choice([1, 2, 3])
        group = r.choice([1, 2, 5])
        nq = r.choice([1, 7, 64, 127, 200, 333])
        nk = r.choice([1, 63, 64, 65, 190, 400]) if not causal else r.choice([nq, nq + 17, 300])
        splits = r.choice([None, None, 2, 3])
        out.append((r.choice([1, 2]), hkv * group, hkv, nq, nk, D, causal, splits))
    return out


@pytest.mark.parametrize("case", _fp8_cases(), ids=lambda c: "-".join(map(str, c)))
def test_random_fp8_case(gpu_device, case):
    """FP8 (E4M3) inputs through the fused path or the key split, at the bound
    of tests/parity.py ``fp8_bound_check``."""
    from tests.parity import fp8_bound_check
    B, Hq, Hkv, Nq, Nk, D, causal, splits = case
    print(f"random fp8 case {case}", flush=True)
    w = custom(B, Hq, Hkv, Nq, Nk, D, "fp8", causal, False)
    seed = zlib.crc32(repr(case).encode()) % 100000
    q, k, v = (t.to(gpu_device) for t in make_inputs(w, seed=seed)[:3])
    if splits is None:
        o, lse = binding.forward(q, k, v, None, causal=causal, scale=w.scale)
    else:
        o, lse = binding.forward_split(q, k, v, None, causal=causal, scale=w.scale,
                                       num_splits=splits)
    torch.cuda.synchronize()
    fp8_bound_check(q, k, v, w.scale, causal, o, lse, str(case))
