"""Seeded random sweep of the forward entry points, and of the backward,
against the oracle.

Each case draws a shape (batch, query heads, KV-head group, query and key
counts with ragged tails), an element type, a head dimension, the causal flag,
a bias, and an entry point (fused, sliding window, key split), all from one
fixed-seed generator, so the set of cases is the same on every run and a
failure names its case.  The bars are those of tests/parity.py; cases whose
logits spread wider than the pages' workloads do not occur (scale = 1/sqrt(D),
N(0, 1) inputs).
"""

import random
import zlib

import pytest
import torch

from tests.parity import full_check, run_split
from tiled_attention_forward_amd import binding
from tiled_attention_forward_amd.workloads import custom, make_inputs

pytestmark = pytest.mark.gpu


def _cases(n=40, seed=2024):
    r = random.Random(seed)
    out = []
    while len(out) < n:
        dtype = r.choice(["bf16", "bf16", "fp16", "fp32"])
        D = r.choice([64, 128] if dtype == "fp32" else [64, 80, 96, 128, 256])
        path = r.choice(["fused", "fused", "window", "split"])
        if D == 256 and path != "fused":
            path = "fused"
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
        full_check(q, k, v, b, w.scale, causal, dt, str(case), run=run_split(3))
    elif path == "window":
        from oracle import attention_forward
        from tests.parity import assert_within, errors, f64
        o, lse = binding.forward(q, k, v, b, causal=True, scale=w.scale, window=window)
        torch.cuda.synchronize()
        o_ref, l_ref = attention_forward(f64(q), f64(k), f64(v), None if b is None else f64(b),
                                         scale=w.scale, causal=True, window=window)
        assert_within(errors(f64(o), lse.cpu().numpy(), o_ref, l_ref), dt, str(case))
    else:
        full_check(q, k, v, b, w.scale, causal, dt, str(case))


def _backward_cases(n=24, seed=4048):
    r = random.Random(seed)
    out = []
    while len(out) < n:
        dtype = r.choice(["bf16", "bf16", "fp16"])
        D = r.choice([64, 80, 96, 128])
        window = r.choice([None, None, None, 1, 16, 100])
        causal = window is not None or r.random() < 0.5
        bias = r.random() < 0.3
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
