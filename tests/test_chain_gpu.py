"""GPU parity of the Block Attention Residual chain (fa_forward_chain through the
C ABI) against the fp64 oracle's ``attention_chain``.

Tolerances are the forward's (max |O - O_ref| <= 1e-2, mean <= 1e-3 for
bf16/fp16; LSE <= 1e-3): the chain only lengthens the fp32-accumulated score
contraction to n_layers * D products, whose rounding stays far below the
probability rounding to the input type that sets the forward's error.
"""

import numpy as np
import pytest
import torch

from oracle import attention_chain, attention_chain_head_rows
from tests.parity import assert_within, errors, f64
from tiled_attention_forward_amd import binding
from tiled_attention_forward_amd.workloads import WORKLOADS, custom, make_chain_inputs, sample_rows

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


CASES = [
    # layers, B, Hq, Hkv, Nq, Nk, D, dtype, causal
    (2, 1, 2, 2, 200, 200, 64, "bf16", True),
    (3, 1, 4, 2, 130, 170, 64, "fp16", False),
    (4, 2, 2, 1, 333, 333, 64, "bf16", True),
    (2, 1, 4, 1, 257, 129, 128, "bf16", False),
    (3, 1, 5, 1, 300, 300, 128, "fp16", True),    # group 5
    (4, 1, 2, 2, 1000, 1000, 128, "bf16", True),  # several tiles and a ragged tail
    (4, 1, 2, 2, 1, 1, 64, "bf16", False),
    (3, 1, 2, 2, 50, 300, 128, "bf16", True),     # keys 50.. seen by no query
    (2, 1, 2, 2, 77, 1, 128, "fp16", False),      # one key: O = V_0
    # head sizes 80 and 96 (128-wide tiles, the padding columns read as 0)
    (3, 1, 4, 2, 200, 333, 80, "bf16", True),
    (4, 1, 2, 1, 130, 97, 96, "fp16", False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_chain_matches_oracle(gpu_device, case):
    n, B, Hq, Hkv, Nq, Nk, D, dt, causal = case
    w = custom(B, Hq, Hkv, Nq, Nk, D, dt, causal, False)
    _log(f"chain case {case}")
    qs, ks, v = make_chain_inputs(w, n, seed=60 + n, device=gpu_device)
    o, lse = binding.forward_chain(qs, ks, v, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = attention_chain([f64(t) for t in qs], [f64(t) for t in ks], f64(v),
                                   scale=w.scale, causal=causal)
    st = errors(f64(o), lse.cpu().numpy(), o_ref, l_ref)
    _log(st)
    assert_within(st, dt, str(case))


def test_one_layer_chain_is_the_forward(gpu_device):
    w = custom(1, 4, 2, 150, 150, 64, "bf16", True, False)
    qs, ks, v = make_chain_inputs(w, 1, seed=70, device=gpu_device)
    o1, l1 = binding.forward_chain(qs, ks, v, causal=True, scale=w.scale)
    o2, l2 = binding.forward(qs[0], ks[0], v, None, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_chain_no_keys(gpu_device):
    q = torch.randn(1, 2, 40, 64, device=gpu_device).to(torch.bfloat16)
    k = torch.empty(1, 2, 0, 64, device=gpu_device, dtype=torch.bfloat16)
    o, lse = binding.forward_chain([q, q], [k, k], k, causal=False, scale=0.125)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_chain_full_size_sampled_rows(gpu_device):
    """The 20-query / 4-KV-head, S = 8192, D = 128 causal shape at the last
    layer of a 4-layer block, in the launch configuration the benchmark times;
    the oracle evaluates sampled rows of two heads."""
    w = WORKLOADS["b1_hq20_hkv4_s8192_d128_bf16_causal_chain4"]
    _log(f"full-size chain {w.name}")
    qs, ks, v = make_chain_inputs(w, w.layers, seed=0, device=gpu_device)
    o, lse = binding.forward_chain(qs, ks, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    grp = w.Hq // w.Hkv
    rows = sample_rows(w.Nq, 48, seed=5)
    rows_t = torch.as_tensor(rows, device=gpu_device)
    for h in (0, w.Hq - 1):
        hk = h // grp
        o_ref, l_ref = attention_chain_head_rows(
            [f64(t[0, h, rows_t]) for t in qs], [f64(t[0, hk]) for t in ks], f64(v[0, hk]),
            rows=np.asarray(rows), scale=w.scale, causal=True)
        st = errors(f64(o[0, h, rows_t]), lse[0, h, rows_t].cpu().numpy(), o_ref, l_ref)
        _log(h, st)
        assert_within(st, w.dtype, f"{w.name} head {h}")
    del qs, ks, v, o, lse
    torch.cuda.empty_cache()
