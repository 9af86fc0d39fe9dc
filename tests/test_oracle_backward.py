"""CPU pins of the oracle's backward (``attention_backward``).  Marker: not gpu.

What pins it, independently of its own code:
  * finite differences: the gradient of L = sum(O * dO) with respect to every
    element of q, k and v, taken by central differences of the forward
    definition (``attention_forward``, pinned elsewhere) in float64;
  * a library routine: torch's autograd in float64 on the CPU through the
    plain softmax(Q K^T * scale + bias + mask) V expression;
  * invariants that hold for any input: each row of dS sums to zero, so the
    dK rows of a KV head sum to zero; the rows of P sum to one, so the dV rows
    of a KV head sum to the dO rows of its query heads (rows that see a key).
Each pin is also run against planted mistakes, which it must catch.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_forward

SHAPES = [
    # B, Hq, Hkv, Nq, Nk, D, causal, bias
    (1, 2, 1, 5, 6, 3, False, False),
    (1, 2, 2, 6, 6, 4, True, False),
    (2, 4, 2, 4, 7, 2, False, True),
    (1, 3, 1, 7, 5, 3, True, True),
    (1, 2, 1, 6, 6, 4, True, False),   # square: catches transposed products
]


def _inputs(seed, B, Hq, Hkv, Nq, Nk, D, bias):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, Nq, D))
    k = r.standard_normal((B, Hkv, Nk, D))
    v = r.standard_normal((B, Hkv, Nk, D))
    do = r.standard_normal((B, Hq, Nq, D))
    b = r.standard_normal((B, Hq, Nq, Nk)) if bias else None
    return q, k, v, do, b


def pin_finite_differences(fn):
    h = 1e-6
    for n, (B, Hq, Hkv, Nq, Nk, D, causal, bias) in enumerate(SHAPES):
        q, k, v, do, b = _inputs(40 + n, B, Hq, Hkv, Nq, Nk, D, bias)
        scale = 0.7
        dq, dk, dv = fn(q, k, v, do, b, scale=scale, causal=causal)

        def loss(q_, k_, v_):
            o, _ = attention_forward(q_, k_, v_, b, scale=scale, causal=causal)
            return float((o * do).sum())

        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            err = np.abs(num - g).max()
            assert err <= 1e-6 * (1 + np.abs(num).max()), f"d{name} shape {n}: {err}"


def pin_torch_autograd(fn):
    for n, (B, Hq, Hkv, Nq, Nk, D, causal, bias) in enumerate(SHAPES):
        q, k, v, do, b = _inputs(60 + n, B, Hq, Hkv, Nq, Nk, D, bias)
        scale = 0.45
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        grp = Hq // Hkv
        kk = tk.repeat_interleave(grp, dim=1)
        vv = tv.repeat_interleave(grp, dim=1)
        s = torch.matmul(tq, kk.transpose(-2, -1).contiguous()) * scale
        if b is not None:
            s = s + torch.tensor(b)
        if causal:
            keep = torch.ones(Nq, Nk, dtype=torch.bool).tril()
            s = s.masked_fill(~keep, float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), vv)
        o.backward(torch.tensor(do))
        dq, dk, dv = fn(q, k, v, do, b, scale=scale, causal=causal)
        for name, got, ref in (("q", dq, tq.grad), ("k", dk, tk.grad), ("v", dv, tv.grad)):
            err = np.abs(got - ref.numpy()).max()
            assert err <= 1e-12, f"d{name} shape {n}: {err}"


def pin_invariants(fn):
    for n, (B, Hq, Hkv, Nq, Nk, D, causal, bias) in enumerate(SHAPES):
        q, k, v, do, b = _inputs(80 + n, B, Hq, Hkv, Nq, Nk, D, bias)
        dq, dk, dv = fn(q, k, v, do, b, scale=0.9, causal=causal)
        grp = Hq // Hkv
        # every row sees key 0 here (causal row i sees keys 0..i), so all rows count
        for bb in range(B):
            for hk in range(Hkv):
                assert np.abs(dk[bb, hk].sum(axis=0)).max() <= 1e-12, f"sum dK shape {n}"
                want = do[bb, hk * grp:(hk + 1) * grp].sum(axis=(0, 1))
                assert np.abs(dv[bb, hk].sum(axis=0) - want).max() <= 1e-12, f"sum dV shape {n}"


PINS = [pin_finite_differences, pin_torch_autograd, pin_invariants]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    pin(attention_backward)


def test_backward_no_keys_and_masked_rows():
    """Nk = 0: nothing to differentiate, all gradients zero and finite."""
    q = np.ones((1, 2, 3, 4))
    k = np.zeros((1, 1, 0, 4))
    dq, dk, dv = attention_backward(q, k, k, q, None, scale=1.0, causal=True)
    assert np.all(dq == 0) and dk.shape == (1, 1, 0, 4) and dv.shape == (1, 1, 0, 4)


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

def _mutant(kind):
    def fn(q, k, v, dout, bias=None, *, scale, causal):
        q, k, v, dout = (np.asarray(x, np.float64) for x in (q, k, v, dout))
        B, Hq, Nq, D = q.shape
        Hkv, Nk = k.shape[1], k.shape[2]
        grp = Hq // Hkv
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                hk = h // grp
                s = q[b, h] @ k[b, hk].T * scale
                if bias is not None:
                    s = s + bias[b, h]
                if causal and kind != "mask_dropped":
                    s = np.where(np.arange(Nk)[None, :] > np.arange(Nq)[:, None], -np.inf, s)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                p = e / e.sum(axis=1, keepdims=True)
                do = dout[b, h]
                dvh = (p @ do[:Nk] if (kind == "dv_untransposed" and Nq == Nk) else p.T @ do)
                dp = do @ v[b, hk].T
                dsum = 0.0 if kind == "no_rowsum" else (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - dsum)
                if kind == "ds_sign":
                    ds = -ds
                dq[b, h] = (ds @ k[b, hk]) * (1.0 if kind == "dq_no_scale" else scale)
                dkh = (ds @ q[b, h] if (kind == "dk_untransposed" and Nq == Nk) else ds.T @ q[b, h])
                dkh = dkh * scale
                if kind == "gqa_overwrite":
                    dk[b, hk], dv[b, hk] = dkh, dvh
                else:
                    dk[b, hk] += dkh
                    dv[b, hk] += dvh
                if kind == "dq_with_v":
                    dq[b, h] = (ds @ v[b, hk]) * scale
        return dq, dk, dv
    return fn


KINDS = ["no_rowsum", "ds_sign", "dq_no_scale", "dk_untransposed", "dv_untransposed",
         "gqa_overwrite", "mask_dropped", "dq_with_v"]


def test_unmutated_backward_harness_passes():
    for pin in PINS:
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", KINDS)
def test_backward_mutant_is_caught(kind):
    fn = _mutant(kind)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake '{kind}' passed every pin"
