"""CPU pins of the oracle's chain backward (``attention_chain_backward``).

Independent facts (marker: not gpu):
  * finite differences: the gradient of L = sum(O * dO) with respect to every
    element of every Q and K layer and of V, by central differences of the
    chain forward (``attention_chain``, pinned on its own) in float64;
  * a library routine: torch's autograd in float64 on the CPU through
    softmax(sum_l Q_l K_l^T * scale + mask) V;
  * a chain of one layer is the plain backward (``attention_backward``,
    pinned on its own);
  * invariants: each row of dS sums to zero, so the dK rows of every layer of
    a KV head sum to zero; the rows of P sum to one, so the dV rows of a KV
    head sum to the dO rows of its query heads.
Planted mistakes must trip a pin: every layer's dQ taken against the current
layer's K, the earlier layers given no gradient, dK without the scale, and
dV from the current layer's logits alone (the residual left out).
"""

import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_chain, attention_chain_backward

SHAPES = [
    # layers, B, Hq, Hkv, Nq, Nk, D, causal
    (2, 1, 2, 2, 4, 5, 3, False),
    (3, 1, 4, 2, 5, 5, 2, True),
    (4, 1, 2, 1, 4, 4, 2, True),   # square: catches transposed products
]


def _inputs(seed, n, B, Hq, Hkv, Nq, Nk, D):
    r = np.random.default_rng(seed)
    qs = [r.standard_normal((B, Hq, Nq, D)) for _ in range(n)]
    ks = [r.standard_normal((B, Hkv, Nk, D)) for _ in range(n)]
    v = r.standard_normal((B, Hkv, Nk, D))
    do = r.standard_normal((B, Hq, Nq, D))
    return qs, ks, v, do


def pin_finite_differences(fn):
    h = 1e-6
    for c, (n, B, Hq, Hkv, Nq, Nk, D, causal) in enumerate(SHAPES):
        qs, ks, v, do = _inputs(60 + c, n, B, Hq, Hkv, Nq, Nk, D)
        dqs, dks, dv = fn(qs, ks, v, do, scale=0.8, causal=causal)

        def loss(qs_, ks_, v_):
            o, _ = attention_chain(qs_, ks_, v_, scale=0.8, causal=causal)
            return float((o * do).sum())

        def numeric(which, l):
            x = {"q": qs, "k": ks}[which][l] if which != "v" else v
            g = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                if which == "v":
                    g[idx] = (loss(qs, ks, xp) - loss(qs, ks, xm)) / (2 * h)
                else:
                    lp = [a if i != l else xp for i, a in enumerate(qs if which == "q" else ks)]
                    lm = [a if i != l else xm for i, a in enumerate(qs if which == "q" else ks)]
                    if which == "q":
                        g[idx] = (loss(lp, ks, v) - loss(lm, ks, v)) / (2 * h)
                    else:
                        g[idx] = (loss(qs, lp, v) - loss(qs, lm, v)) / (2 * h)
            return g

        for l in range(n):
            assert np.abs(dqs[l] - numeric("q", l)).max() <= 1e-6, (c, "q", l)
            assert np.abs(dks[l] - numeric("k", l)).max() <= 1e-6, (c, "k", l)
        assert np.abs(dv - numeric("v", 0)).max() <= 1e-6, (c, "v")


def pin_autograd(fn):
    for c, (n, B, Hq, Hkv, Nq, Nk, D, causal) in enumerate(SHAPES):
        qs, ks, v, do = _inputs(70 + c, n, B, Hq, Hkv, Nq, Nk, D)
        dqs, dks, dv = fn(qs, ks, v, do, scale=0.6, causal=causal)
        tq = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in qs]
        tk = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in ks]
        tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
        grp = Hq // Hkv
        s = sum(q_ @ k_.repeat_interleave(grp, dim=1).transpose(-1, -2) for q_, k_ in zip(tq, tk))
        s = s * 0.6
        if causal:
            s = s.masked_fill(torch.ones(Nq, Nk, dtype=torch.bool).triu(1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv.repeat_interleave(grp, dim=1)
        (o * torch.tensor(do)).sum().backward()
        for l in range(n):
            assert np.abs(dqs[l] - tq[l].grad.numpy()).max() <= 1e-12, (c, "q", l)
            assert np.abs(dks[l] - tk[l].grad.numpy()).max() <= 1e-12, (c, "k", l)
        assert np.abs(dv - tv.grad.numpy()).max() <= 1e-12, c


def pin_one_layer_is_plain_backward(fn):
    for c, (_, B, Hq, Hkv, Nq, Nk, D, causal) in enumerate(SHAPES):
        qs, ks, v, do = _inputs(80 + c, 1, B, Hq, Hkv, Nq, Nk, D)
        dqs, dks, dv = fn(qs, ks, v, do, scale=0.5, causal=causal)
        dq, dk, dv_r = attention_backward(qs[0], ks[0], v, do, scale=0.5, causal=causal)
        assert np.abs(dqs[0] - dq).max() <= 1e-12 and np.abs(dks[0] - dk).max() <= 1e-12
        assert np.abs(dv - dv_r).max() <= 1e-12


def pin_invariants(fn):
    for c, (n, B, Hq, Hkv, Nq, Nk, D, causal) in enumerate(SHAPES):
        qs, ks, v, do = _inputs(90 + c, n, B, Hq, Hkv, Nq, Nk, D)
        dqs, dks, dv = fn(qs, ks, v, do, scale=0.9, causal=causal)
        grp = Hq // Hkv
        for l in range(n):
            assert np.abs(dks[l].sum(axis=2)).max() <= 1e-12, (c, l)
        for b in range(B):
            for hk in range(Hkv):
                want = do[b, hk * grp:(hk + 1) * grp].sum(axis=(0, 1))
                assert np.abs(dv[b, hk].sum(axis=0) - want).max() <= 1e-12, c


PINS = [pin_finite_differences, pin_autograd, pin_one_layer_is_plain_backward, pin_invariants]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_chain_backward_pin(pin):
    pin(attention_chain_backward)


def test_chain_backward_rejects_mismatched_layers():
    qs, ks, v, do = _inputs(1, 2, 1, 2, 2, 4, 4, 2)
    with pytest.raises(ValueError):
        attention_chain_backward(qs, ks[:1], v, do)
    with pytest.raises(ValueError):
        attention_chain_backward([qs[0], qs[1][:, :, :3]], ks, v, do)


def _mutant(kind):
    """attention_chain_backward with one planted mistake (one (b, hq) loop)."""
    def fn(q_layers, k_layers, v, dout, *, scale=None, causal=False):
        n = len(q_layers)
        B, Hq, Nq, D = q_layers[0].shape
        Hkv, Nk = k_layers[0].shape[1], k_layers[0].shape[2]
        grp = Hq // Hkv
        dqs = [np.zeros_like(x) for x in q_layers]
        dks = [np.zeros_like(x) for x in k_layers]
        dv = np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                hk = h // grp
                layers = range(n) if kind != "no_residual" else [n - 1]
                s = sum(q_layers[l][b, h] @ k_layers[l][b, hk].T for l in layers) * scale
                if causal:
                    s = np.where(np.arange(Nk)[None, :] > np.arange(Nq)[:, None], -np.inf, s)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                dv[b, hk] += p.T @ dout[b, h]
                dp = dout[b, h] @ v[b, hk].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                for l in range(n):
                    if kind == "last_only" and l < n - 1:
                        continue
                    kl = k_layers[n - 1 if kind == "current_k" else l][b, hk]
                    dqs[l][b, h] = scale * (ds @ kl)
                    dks[l][b, hk] += (1.0 if kind == "dk_unscaled" else scale) * (ds.T @ q_layers[l][b, h])
        return dqs, dks, dv
    return fn


def test_unmutated_harness_passes():
    for pin in (pin_autograd, pin_invariants):
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", ["current_k", "last_only", "dk_unscaled", "no_residual"])
def test_chain_backward_mutant_is_caught(kind):
    caught = 0
    for pin in (pin_autograd, pin_one_layer_is_plain_backward, pin_invariants):
        try:
            pin(_mutant(kind))
        except AssertionError:
            caught += 1
    assert caught >= 1, kind
