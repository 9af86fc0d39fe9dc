"""Ragged tails must not read past a head's rows (the zero-padding pitfall).

The xnwp.cn post (§5.2, §6.4, fifth pitfall) and the kwkr.cn tutorial (§3.3,
§4.3) pad unaligned tails with zeros and call that harmless.  It is not for K
(a zero key has logit 0 and would be counted), so the kernels mask tail keys
to -inf; the V rows of those keys, and Q rows past Nq, are read through buffer
resources that end at the head's last row, so the loads return 0 and the
masked probabilities (exactly 0) multiply zeros.  If a resource reached past
the head, the tail would read the next head's rows instead, and a NaN there
would make 0 * NaN = NaN.

Each case therefore places Q, K, V, the bias (and for the backward dO) in
device memory whose neighbours are NaN: the heads of one KV group carry real
values, every other head and the padding after the last head hold NaN, all
inside one allocation (so no access leaves it).  The checked heads must give
finite results that match the oracle, for the fused, key-split, window,
backward and residual-chain (forward and backward) paths, with Nq and Nk not
multiples of the tile sizes.
"""

import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_forward
from tests.parity import assert_within, errors, f64
from tests.test_backward_gpu import compare
from tiled_attention_forward_amd import binding
from tiled_attention_forward_amd.workloads import custom, make_inputs

pytestmark = pytest.mark.gpu

PAD = 1 << 16  # NaN elements after the last head


def _log(*a):
    print(*a, flush=True)


def _poisoned(t, keep, dev):
    """t copied to the start of a NaN-filled device allocation PAD elements
    longer; heads (dim 1) not in ``keep`` are NaN too."""
    buf = torch.full((t.numel() + PAD,), float("nan"), dtype=t.dtype, device=dev)
    view = buf[:t.numel()].view(t.shape)
    view.copy_(t.to(dev))
    drop = [h for h in range(t.shape[1]) if h not in keep]
    if drop:
        view[:, drop] = float("nan")
    return view, buf


def _setup(case, group_checked, dev, seed=5):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, bias = case[:9]
    w = custom(B, Hq, Hkv, Nq, Nk, D, dt, causal, bias)
    q, k, v, b = make_inputs(w, seed=seed)
    grp = Hq // Hkv
    heads = list(range(group_checked * grp, (group_checked + 1) * grp))
    qd, qbuf = _poisoned(q, heads, dev)
    kd, kbuf = _poisoned(k, [group_checked], dev)
    vd, vbuf = _poisoned(v, [group_checked], dev)
    bd = bbuf = None
    if b is not None:
        bd, bbuf = _poisoned(b, heads, dev)
    host = (q[:, heads], k[:, [group_checked]], v[:, [group_checked]],
            None if b is None else b[:, heads])
    return w, heads, (qd, kd, vd, bd), host, (qbuf, kbuf, vbuf, bbuf)


FWD_CASES = [
    # path, B, Hq, Hkv, Nq, Nk, D, dtype, causal, bias, extra (splits / window)
    ("fused", 1, 4, 2, 200, 333, 64, "bf16", True, True, None),
    # bias rows that allow 16-byte loads (Nk % 8 == 0) go through LDS; the last
    # key tile runs past Nk
    ("fused", 1, 4, 2, 200, 264, 64, "bf16", True, True, None),
    ("fused", 1, 4, 2, 130, 200, 128, "bf16", False, True, None),
    ("fused", 1, 4, 2, 97, 136, 96, "fp16", True, True, None),
    ("fused", 1, 4, 2, 130, 70, 128, "fp16", False, True, None),
    # two 32-row query blocks per wave (D = 128, non-causal, no bias)
    ("fused", 1, 4, 2, 300, 333, 128, "bf16", False, False, None),
    ("fused", 1, 4, 2, 65, 31, 128, "fp16", False, False, None),
    ("fused", 1, 4, 2, 97, 161, 80, "bf16", True, False, None),
    ("fused", 1, 4, 2, 75, 100, 64, "fp32", True, True, None),
    ("fused", 1, 4, 2, 100, 90, 256, "bf16", True, False, None),
    ("split", 1, 8, 2, 1, 1000, 128, "bf16", False, False, 3),
    ("split", 1, 4, 2, 150, 333, 64, "fp16", True, True, 4),
    ("split", 1, 4, 2, 70, 201, 96, "bf16", False, False, 2),
    ("window", 1, 4, 2, 300, 333, 64, "bf16", True, True, 100),
    ("window", 1, 4, 2, 300, 336, 64, "bf16", True, True, 100),
    ("window", 1, 4, 2, 200, 260, 128, "bf16", True, False, 64),
    ("window", 1, 4, 2, 200, 260, 256, "bf16", True, True, 64),
    ("split", 1, 4, 2, 150, 333, 256, "bf16", True, False, 3),
]


@pytest.mark.parametrize("group_checked", [0, 1])
@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_forward_reads_stay_in_the_head(gpu_device, case, group_checked):
    path, extra = case[0], case[10]
    _log(f"tail case {case} group {group_checked}")
    w, heads, (q, k, v, b), (hq, hk, hv, hb), bufs = _setup(case[1:10], group_checked,
                                                            gpu_device)
    if path == "fused":
        o, lse = binding.forward(q, k, v, b, causal=w.causal, scale=w.scale)
    elif path == "split":
        o, lse = binding.forward_split(q, k, v, b, causal=w.causal, scale=w.scale,
                                       num_splits=extra)
    else:
        o, lse = binding.forward(q, k, v, b, causal=True, scale=w.scale, window=extra)
    torch.cuda.synchronize()
    o_ref, l_ref = attention_forward(f64(hq), f64(hk), f64(hv), None if hb is None else f64(hb),
                                     scale=w.scale, causal=w.causal,
                                     window=extra if path == "window" else None)
    st = errors(f64(o[:, heads]), lse[:, heads].cpu().numpy(), o_ref, l_ref)
    _log(st)
    assert_within(st, w.dtype, str(case))


BWD_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, bias, window
    (1, 4, 2, 200, 333, 64, "bf16", True, False, None),
    (1, 4, 2, 130, 170, 128, "fp16", False, True, None),
    (1, 6, 2, 77, 129, 128, "bf16", True, False, None),
    (1, 4, 2, 300, 333, 64, "bf16", True, False, 100),
    (1, 4, 2, 131, 170, 128, "bf16", False, False, None),
    (1, 4, 2, 130, 170, 80, "bf16", False, False, None),
    (1, 4, 2, 77, 129, 96, "fp16", True, True, None),
    (1, 4, 2, 131, 170, 256, "bf16", True, False, None),
    (1, 4, 2, 130, 170, 64, "fp32", True, True, None),
    (1, 4, 2, 97, 161, 128, "fp32", False, False, None),
    (1, 4, 2, 300, 333, 64, "fp32", True, False, 100),
    (1, 4, 2, 200, 260, 256, "bf16", True, False, 64),
]


@pytest.mark.parametrize("group_checked", [0, 1])
@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_backward_reads_stay_in_the_head(gpu_device, case, group_checked):
    window = case[9]
    _log(f"backward tail case {case} group {group_checked}")
    w, heads, (q, k, v, b), (hq, hk, hv, hb), bufs = _setup(case[:9], group_checked, gpu_device)
    g = torch.Generator().manual_seed(77)
    dout_h = torch.randn(q.shape, generator=g).to(q.dtype)
    dout, dbuf = _poisoned(dout_h, heads, gpu_device)
    o, lse = binding.forward(q, k, v, b, causal=w.causal, scale=w.scale, window=window)
    dq, dk, dv = binding.backward(q, k, v, o, lse, dout, b, causal=w.causal, scale=w.scale,
                                  window=window)
    torch.cuda.synchronize()
    grp = w.Hq // w.Hkv
    refs = attention_backward(f64(hq), f64(hk), f64(hv), f64(dout_h[:, heads]),
                              None if hb is None else f64(hb), scale=w.scale, causal=w.causal,
                              window=window)
    got = (dq[:, heads], dk[:, [heads[0] // grp]], dv[:, [heads[0] // grp]])
    _log(compare(got, refs, w.dtype, str(case)))


CHAIN_CASES = [
    # layers, B, Hq, Hkv, Nq, Nk, D, dtype, causal
    (3, 1, 4, 2, 200, 333, 64, "bf16", True),
    (2, 1, 4, 2, 130, 70, 128, "fp16", False),
    (4, 1, 4, 2, 97, 161, 128, "bf16", True),
]


def _chain_setup(case, group_checked, dev, seed=9):
    """Every layer's Q and K, and V, in NaN-neighboured allocations; returns
    the device tensors, the checked heads' host slices and the buffers."""
    from tiled_attention_forward_amd.workloads import make_chain_inputs
    n, B, Hq, Hkv, Nq, Nk, D, dt, causal = case
    w = custom(B, Hq, Hkv, Nq, Nk, D, dt, causal, False)
    qs, ks, v = make_chain_inputs(w, n, seed=seed)
    grp = Hq // Hkv
    heads = list(range(group_checked * grp, (group_checked + 1) * grp))
    dev_q = [_poisoned(t, heads, dev) for t in qs]
    dev_k = [_poisoned(t, [group_checked], dev) for t in ks]
    vd, vbuf = _poisoned(v, [group_checked], dev)
    host = ([t[:, heads] for t in qs], [t[:, [group_checked]] for t in ks],
            v[:, [group_checked]])
    dev_t = ([t for t, _ in dev_q], [t for t, _ in dev_k], vd)
    bufs = [b for _, b in dev_q] + [b for _, b in dev_k] + [vbuf]
    return w, heads, dev_t, host, bufs


@pytest.mark.parametrize("group_checked", [0, 1])
@pytest.mark.parametrize("case", CHAIN_CASES, ids=lambda c: "-".join(map(str, c)))
def test_chain_reads_stay_in_the_head(gpu_device, case, group_checked):
    """Chain forward and backward (every layer's Q and K streamed per tile)."""
    from oracle import attention_chain, attention_chain_backward
    _log(f"chain tail case {case} group {group_checked}")
    w, heads, (qs, ks, v), (hq, hk, hv), bufs = _chain_setup(case, group_checked, gpu_device)
    o, lse = binding.forward_chain(qs, ks, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = attention_chain([f64(t) for t in hq], [f64(t) for t in hk], f64(hv),
                                   scale=w.scale, causal=w.causal)
    st = errors(f64(o[:, heads]), lse[:, heads].cpu().numpy(), o_ref, l_ref)
    _log(st)
    assert_within(st, w.dtype, str(case))

    g = torch.Generator().manual_seed(78)
    dout_h = torch.randn(qs[-1].shape, generator=g).to(qs[-1].dtype)
    dout, dbuf = _poisoned(dout_h, heads, gpu_device)
    dqs, dks, dv = binding.backward_chain(qs, ks, v, o, lse, dout, causal=w.causal,
                                          scale=w.scale)
    torch.cuda.synchronize()
    rq, rk, rv = attention_chain_backward([f64(t) for t in hq], [f64(t) for t in hk], f64(hv),
                                          f64(dout_h[:, heads]), scale=w.scale, causal=w.causal)
    hk0 = heads[0] // (w.Hq // w.Hkv)
    for l in range(case[0]):
        got = (dqs[l][:, heads], dks[l][:, [hk0]], dv[:, [hk0]])
        _log(l, compare(got, (rq[l], rk[l], rv), w.dtype, f"{case} layer {l}"))
