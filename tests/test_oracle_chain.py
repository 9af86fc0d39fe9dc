"""CPU pins of the oracle's Block Attention Residual chain (``attention_chain``).

Independent facts (marker: not gpu):
  * linear algebra: the summed logits sum_l Q_l K_l^T * scale equal one product
    of the Q layers and the K layers concatenated along the head dimension, so
    the chain equals the plain definition evaluated on concatenated operands;
  * brute force: scalar loops with math.exp on tiny inputs, each logit formed
    as a triple sum over layers and head dimension, GQA and causal included;
  * a chain of one layer (a block's first layer) is plain attention;
  * all Q layers zero: every logit is 0, so O is the column mean of V and
    LSE = ln(number of visible keys) (closed form, causal and not);
  * the order of the earlier layers does not matter (their logits are summed).
Planted mistakes must trip a pin: the residual carrying only the previous
layer's own product (not its residual), the current layer's product dropped,
the earlier layers scaled twice, a layer's Q paired with the next layer's K,
and earlier layers read with MHA instead of GQA head mapping.
"""

import math

import numpy as np
import pytest

from oracle import attention_chain, attention_forward, attention_head_rows


def _layers(seed, n, B=1, Hq=4, Hkv=2, Nq=7, Nk=7, D=3):
    r = np.random.default_rng(seed)
    qs = [r.standard_normal((B, Hq, Nq, D)) for _ in range(n)]
    ks = [r.standard_normal((B, Hkv, Nk, D)) for _ in range(n)]
    v = r.standard_normal((B, Hkv, Nk, D))
    return qs, ks, v


SHAPES = [
    # n layers, B, Hq, Hkv, Nq, Nk, D, causal
    (2, 1, 2, 2, 5, 5, 3, False),
    (3, 1, 4, 2, 6, 6, 2, True),
    (4, 2, 3, 1, 4, 7, 3, False),
    (4, 1, 2, 1, 6, 6, 4, True),
]


def _concat(qs, ks, v, scale, causal):
    """The chain as one attention over operands concatenated along D."""
    qc, kc = np.concatenate(qs, axis=-1), np.concatenate(ks, axis=-1)
    B, Hq, Nq, _ = qc.shape
    Hkv = kc.shape[1]
    grp = Hq // Hkv
    o = np.empty((B, Hq, Nq, v.shape[-1]))
    lse = np.empty((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            o[b, h], lse[b, h] = attention_head_rows(
                qc[b, h], kc[b, h // grp], v[b, h // grp], rows=np.arange(Nq), scale=scale,
                causal=causal)
    return o, lse


def _brute(qs, ks, v, scale, causal):
    B, Hq, Nq, D = qs[0].shape
    Hkv, Nk = ks[0].shape[1], ks[0].shape[2]
    grp = Hq // Hkv
    o = np.zeros((B, Hq, Nq, v.shape[-1]))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            hk = h // grp
            for i in range(Nq):
                keys = [j for j in range(Nk) if not causal or j <= i]
                logits = [sum(qs[l][b, h, i, d] * ks[l][b, hk, j, d]
                              for l in range(len(qs)) for d in range(D)) * scale for j in keys]
                m = max(logits)
                w = [math.exp(x - m) for x in logits]
                tot = sum(w)
                lse[b, h, i] = m + math.log(tot)
                for d in range(v.shape[-1]):
                    o[b, h, i, d] = sum(wi * v[b, hk, j, d] for wi, j in zip(w, keys)) / tot
    return o, lse


def pin_concat(fn):
    for n_, (n, B, Hq, Hkv, Nq, Nk, D, causal) in enumerate(SHAPES):
        qs, ks, v = _layers(10 + n_, n, B, Hq, Hkv, Nq, Nk, D)
        o, lse = fn(qs, ks, v, scale=0.6, causal=causal)
        o_r, l_r = _concat(qs, ks, v, 0.6, causal)
        assert np.abs(o - o_r).max() <= 1e-12 and np.abs(lse - l_r).max() <= 1e-12, n_


def pin_brute(fn):
    for n_, (n, B, Hq, Hkv, Nq, Nk, D, causal) in enumerate(SHAPES):
        qs, ks, v = _layers(20 + n_, n, B, Hq, Hkv, Nq, Nk, D)
        o, lse = fn(qs, ks, v, scale=0.45, causal=causal)
        o_r, l_r = _brute(qs, ks, v, 0.45, causal)
        assert np.abs(o - o_r).max() <= 1e-12 and np.abs(lse - l_r).max() <= 1e-12, n_


def pin_q_zero(fn):
    for causal in (False, True):
        qs, ks, v = _layers(30, 3, Nq=6, Nk=6)
        qs = [np.zeros_like(q) for q in qs]
        o, lse = fn(qs, ks, v, scale=0.9, causal=causal)
        grp = qs[0].shape[1] // ks[0].shape[1]
        for h in range(qs[0].shape[1]):
            vh = v[0, h // grp]
            for i in range(6):
                cnt = i + 1 if causal else 6
                assert np.abs(o[0, h, i] - vh[:cnt].mean(axis=0)).max() <= 1e-12
                assert abs(lse[0, h, i] - math.log(cnt)) <= 1e-12


def pin_order_of_earlier_layers(fn):
    qs, ks, v = _layers(40, 4)
    o, lse = fn(qs, ks, v, scale=0.7, causal=True)
    perm = [2, 0, 1, 3]
    o2, l2 = fn([qs[i] for i in perm], [ks[i] for i in perm], v, scale=0.7, causal=True)
    assert np.abs(o - o2).max() <= 1e-12 and np.abs(lse - l2).max() <= 1e-12


PINS = [pin_concat, pin_brute, pin_q_zero, pin_order_of_earlier_layers]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_chain_pin(pin):
    pin(attention_chain)


def test_first_layer_of_a_block_is_plain_attention():
    qs, ks, v = _layers(50, 1, Nq=8, Nk=9)
    for causal in (False, True):
        o, lse = attention_chain(qs, ks, v, scale=0.5, causal=causal)
        o_r, l_r = attention_forward(qs[0], ks[0], v, scale=0.5, causal=causal)
        assert np.abs(o - o_r).max() <= 1e-14 and np.abs(lse - l_r).max() <= 1e-14


def test_chain_rejects_mismatched_layers():
    qs, ks, v = _layers(51, 2)
    with pytest.raises(ValueError):
        attention_chain(qs, ks[:1], v)
    with pytest.raises(ValueError):
        attention_chain([qs[0], qs[1][:, :, :3]], ks, v)


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

def _mutant(kind):
    def fn(qs, ks, v, *, scale, causal):
        B, Hq, Nq, D = qs[-1].shape
        Hkv, Nk = ks[-1].shape[1], ks[-1].shape[2]
        grp = Hq // Hkv
        o = np.empty((B, Hq, Nq, v.shape[-1]))
        lse = np.empty((B, Hq, Nq))
        for b in range(B):
            for h in range(Hq):
                hk = h // grp
                res = np.zeros((Nq, Nk))
                n = len(qs)
                for l in range(n - 1):
                    kl = ks[min(l + 1, n - 1)] if kind == "shifted_k" else ks[l]
                    hkl = h % Hkv if kind == "mha_mapping" else hk
                    own = qs[l][b, h] @ kl[b, hkl].T * scale
                    if kind == "scaled_twice":
                        own = own * scale
                    res = own if kind == "no_carry" else own + res
                cur = qs[-1][b, h] @ ks[-1][b, hk].T * scale
                s = res if kind == "own_dropped" and n > 1 else cur + res
                if causal:
                    s = np.where(np.arange(Nk)[None, :] > np.arange(Nq)[:, None], -np.inf, s)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                lse[b, h] = (m[:, 0] + np.log(e.sum(axis=1)))
                o[b, h] = (e / e.sum(axis=1, keepdims=True)) @ v[b, hk]
        return o, lse
    return fn


KINDS = ["no_carry", "own_dropped", "scaled_twice", "shifted_k", "mha_mapping"]


def test_unmutated_chain_harness_passes():
    for pin in PINS:
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", KINDS)
def test_chain_mutant_is_caught(kind):
    fn = _mutant(kind)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake '{kind}' passed every pin"
