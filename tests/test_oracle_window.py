"""CPU pins of the oracle's sliding-window mask (``window`` with ``causal``).

Independent facts (marker: not gpu):
  * a window of at least Nk keys is the plain causal mask;
  * a window of one key leaves row i only key i: O_i = V_i, LSE_i = s_ii;
  * Q = 0, no bias: O_i is the mean of V over keys max(0, i-W+1) .. i and
    LSE_i = ln of their count (closed form);
  * brute force: scalar loops with math.exp on tiny inputs, GQA and bias;
  * the backward's window gradients match central finite differences of the
    windowed forward.
Planted mistakes (an off-by-one window edge, the window applied to the wrong
side) must trip a pin.
"""

import math

import numpy as np
import pytest

from oracle import attention_backward, attention_forward


def _in(seed, B=1, Hq=2, Hkv=1, Nq=9, Nk=9, D=3, bias=False):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, Nq, D))
    k = r.standard_normal((B, Hkv, Nk, D))
    v = r.standard_normal((B, Hkv, Nk, D))
    b = r.standard_normal((B, Hq, Nq, Nk)) if bias else None
    return q, k, v, b


def _brute(q, k, v, b, scale, window):
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    o = np.zeros(q.shape)
    lse = np.zeros((B, Hq, Nq))
    for bb in range(B):
        for h in range(Hq):
            hk = h // grp
            for i in range(Nq):
                keys = [j for j in range(Nk) if j <= i and j > i - window]
                if not keys:
                    lse[bb, h, i] = -math.inf
                    continue
                logits = []
                for j in keys:
                    s = sum(q[bb, h, i, d] * k[bb, hk, j, d] for d in range(D)) * scale
                    if b is not None:
                        s += b[bb, h, i, j]
                    logits.append(s)
                m = max(logits)
                w = [math.exp(x - m) for x in logits]
                tot = sum(w)
                lse[bb, h, i] = m + math.log(tot)
                for d in range(D):
                    o[bb, h, i, d] = sum(wi * v[bb, hk, j, d] for wi, j in zip(w, keys)) / tot
    return o, lse


def pin_wide_window_is_causal(fn):
    q, k, v, b = _in(1, Nq=8, Nk=11, bias=True)
    for w in (11, 12, 100):
        o1, l1 = fn(q, k, v, b, scale=0.6, causal=True, window=w)
        o2, l2 = attention_forward(q, k, v, b, scale=0.6, causal=True)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def pin_window_one(fn):
    q, k, v, _ = _in(2, Nq=7, Nk=7)
    o, lse = fn(q, k, v, None, scale=0.8, causal=True, window=1)
    np.testing.assert_allclose(o[0, :, :, :], np.broadcast_to(v[0, 0], o[0].shape), rtol=0,
                               atol=1e-12)
    s_ii = np.einsum("hid,id->hi", q[0], k[0, 0]) * 0.8
    np.testing.assert_allclose(lse[0], s_ii, rtol=0, atol=1e-12)


def pin_q_zero_closed_form(fn):
    _, k, v, _ = _in(3, Nq=12, Nk=12)
    q = np.zeros((1, 2, 12, 3))
    for w in (1, 3, 5, 12):
        o, lse = fn(q, k, v, None, scale=1.0, causal=True, window=w)
        for i in range(12):
            lo = max(0, i - w + 1)
            np.testing.assert_allclose(o[0, 1, i], v[0, 0, lo:i + 1].mean(axis=0), rtol=0,
                                       atol=1e-12)
            assert abs(lse[0, 1, i] - math.log(i + 1 - lo)) <= 1e-12


def pin_brute_force(fn):
    for seed, (Hq, Hkv, bias, w) in enumerate([(2, 1, False, 3), (4, 2, True, 2), (1, 1, True, 5)]):
        q, k, v, b = _in(10 + seed, B=2, Hq=Hq, Hkv=Hkv, Nq=7, Nk=6, D=3, bias=bias)
        o, lse = fn(q, k, v, b, scale=0.7, causal=True, window=w)
        o_ref, l_ref = _brute(q, k, v, b, 0.7, w)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-12)


PINS = [pin_wide_window_is_causal, pin_window_one, pin_q_zero_closed_form, pin_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_window_pin(pin):
    pin(attention_forward)


def test_window_backward_finite_differences():
    q, k, v, b = _in(20, B=1, Hq=2, Hkv=1, Nq=6, Nk=6, D=3, bias=True)
    do = np.random.default_rng(21).standard_normal(q.shape)
    dq, dk, dv = attention_backward(q, k, v, do, b, scale=0.9, causal=True, window=3)
    h = 1e-6

    def loss(q_, k_, v_):
        o, _ = attention_forward(q_, k_, v_, b, scale=0.9, causal=True, window=3)
        return float((o * do).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            am = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        assert np.abs(num - g).max() <= 1e-6 * (1 + np.abs(num).max()), name


def test_window_argument_checks():
    q, k, v, _ = _in(4)
    with pytest.raises(ValueError):
        attention_forward(q, k, v, None, scale=1.0, causal=False, window=3)
    with pytest.raises(ValueError):
        attention_forward(q, k, v, None, scale=1.0, causal=True, window=0)


def _mutant(kind):
    def fn(q, k, v, b, *, scale, causal, window):
        w = window + (1 if kind == "edge_plus_one" else 0)
        if kind == "edge_minus_one":
            w = window - 1 if window > 1 else window
        o, lse = attention_forward(q, k, v, b, scale=scale, causal=causal, window=w)
        if kind == "right_side":
            o2, l2 = attention_forward(q, k, v, b, scale=scale, causal=False)
            return o2, l2
        return o, lse
    return fn


@pytest.mark.parametrize("kind", ["edge_plus_one", "edge_minus_one", "right_side"])
def test_window_mutant_is_caught(kind):
    fn = _mutant(kind)
    caught = False
    for pin in PINS:
        try:
            pin(fn)
        except AssertionError:
            caught = True
    assert caught, kind
