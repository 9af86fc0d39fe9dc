"""GPU parity of the chain backward (fa_backward_chain through the C ABI)
against the fp64 oracle's ``attention_chain_backward``.

The GPU chain forward produces O and LSE (the backward's inputs); the oracle
differentiates the chain's definition from the layers, V and dO alone.  The
tolerances are the backward's (relative to each gradient's own scale, see
tests/test_backward_gpu.py): the chain only lengthens the fp32-accumulated
score contraction to n_layers * D products; P and dS are rounded to the input
type as in the one-layer backward.
"""

import pytest
import torch

from oracle import attention_chain_backward
from tests.parity import f64
from tests.test_backward_gpu import _dout, compare
from tiled_attention_forward_amd import binding
from tiled_attention_forward_amd.workloads import custom, make_chain_inputs

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


CASES = [
    # layers, B, Hq, Hkv, Nq, Nk, D, dtype, causal
    (2, 1, 2, 2, 150, 150, 64, "bf16", True),
    (3, 1, 4, 2, 97, 200, 64, "fp16", False),     # group 2: query tiles cross heads
    (4, 2, 2, 1, 130, 130, 64, "bf16", True),
    (2, 1, 4, 2, 100, 170, 128, "bf16", False),
    (3, 1, 2, 2, 200, 200, 128, "bf16", True),
    (4, 1, 5, 1, 77, 64, 128, "fp16", True),      # group 5, ragged rows
    (4, 1, 2, 2, 33, 31, 128, "bf16", False),     # rows < one tile, key tail
    (1, 1, 2, 2, 64, 64, 64, "bf16", True),       # one layer: the plain backward
    (3, 1, 4, 2, 150, 200, 80, "bf16", True),     # head sizes 80 and 96
    (4, 1, 2, 1, 97, 130, 96, "fp16", False),
]


def _run(case, seed, dev):
    n, B, Hq, Hkv, Nq, Nk, D, dt, causal = case
    w = custom(B, Hq, Hkv, Nq, Nk, D, dt, causal, False)
    qs, ks, v = make_chain_inputs(w, n, seed=seed)
    qs, ks, v = [t.to(dev) for t in qs], [t.to(dev) for t in ks], v.to(dev)
    dout = _dout(qs[-1].shape, seed, qs[-1].dtype, dev)
    o, lse = binding.forward_chain(qs, ks, v, causal=causal, scale=w.scale)
    dqs, dks, dv = binding.backward_chain(qs, ks, v, o, lse, dout, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    rq, rk, rv = attention_chain_backward([f64(t) for t in qs], [f64(t) for t in ks], f64(v),
                                          f64(dout), scale=w.scale, causal=causal)
    return w, (dqs, dks, dv), (rq, rk, rv)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_chain_backward_matches_oracle(gpu_device, case):
    _log(f"chain backward case {case}")
    w, (dqs, dks, dv), (rq, rk, rv) = _run(case, 41, gpu_device)
    for l in range(case[0]):
        # each layer's dQ and dK; dV (the same for every layer) with layer 0
        st = compare((dqs[l], dks[l], dv), (rq[l], rk[l], rv), w.dtype, f"{case} layer {l}")
        _log(l, st)


def test_chain_backward_deterministic(gpu_device):
    case = (3, 1, 4, 2, 97, 200, 128, "bf16", True)
    _, a, _ = _run(case, 5, gpu_device)
    _, b, _ = _run(case, 5, gpu_device)
    for x, y in zip(a[0] + a[1] + [a[2]], b[0] + b[1] + [b[2]]):
        assert torch.equal(x, y)


def test_chain_backward_larger(gpu_device):
    """Several 128-row blocks and 128-key blocks per head at the chain
    workload's head layout (GQA group 5, D = 128, causal, four layers)."""
    case = (4, 1, 5, 1, 1024, 1024, 128, "bf16", True)
    _log(f"chain backward case {case}")
    w, (dqs, dks, dv), (rq, rk, rv) = _run(case, 9, gpu_device)
    for l in range(4):
        _log(l, compare((dqs[l], dks[l], dv), (rq[l], rk[l], rv), w.dtype, f"{case} layer {l}"))
