"""Plant plausible mistakes in a copy of the oracle and check the pins catch each one.

Every mutant below is the oracle's definition with one deliberate error (a
dropped term, a wrong sign or index, a transposed operand, a mis-placed mask).
A pin suite that lets any of them through would not be pinning the oracle.
CPU only.
"""

import numpy as np
import pytest

from tests import oracle_pins


def _mutant(kind):
    def fn(q, k, v, bias=None, *, scale, causal):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, Hq, Nq, D = q.shape
        Hkv, Nk = k.shape[1], k.shape[2]
        grp = Hq // Hkv
        o = np.zeros((B, Hq, Nq, D))
        lse = np.zeros((B, Hq, Nq))
        for b in range(B):
            for h in range(Hq):
                hk = h % Hkv if kind == "gqa_modulo" else h // grp
                kk, vv = k[b, hk], v[b, hk]
                s = q[b, h] @ kk.T
                if kind == "sign":
                    s = -s
                if kind != "no_scale":
                    s = s * scale
                if bias is not None and kind != "bias_dropped":
                    s = s + (bias[b, h] * scale if kind == "scale_bias" else bias[b, h])
                if causal:
                    i = np.arange(Nq)[:, None]
                    j = np.arange(Nk)[None, :]
                    if kind == "causal_off_by_one":
                        hide = j >= i
                        hide[:, 0] = False
                    elif kind == "causal_reversed":
                        hide = j < i
                    else:
                        hide = j > i
                    s = np.where(hide, 0.0 if kind == "mask_as_zero" else -np.inf, s)
                m = s.max(axis=-1, keepdims=True)
                e = np.exp(s - np.where(np.isfinite(m), m, 0.0))
                if kind == "softmax_wrong_axis":
                    l_ax = e.sum(axis=-2, keepdims=True)
                    p = e / l_ax
                    l = e.sum(axis=-1, keepdims=True)
                else:
                    l = e.sum(axis=-1, keepdims=True)
                    p = e if kind == "no_normalize" else e / np.where(l > 0, l, 1.0)
                o[b, h] = p @ (kk if kind == "k_as_v" else vv)
                lv = np.where(l > 0, l, 1.0)[:, 0]
                mm = m[:, 0]
                if kind == "lse_log2":
                    lse[b, h] = mm + np.log2(lv)
                elif kind == "lse_no_max":
                    lse[b, h] = np.log(lv)
                else:
                    lse[b, h] = mm + np.log(lv)
                lse[b, h] = np.where(l[:, 0] > 0, lse[b, h], -np.inf)
        return o, lse
    return fn


MUTANTS = ["no_scale", "scale_bias", "bias_dropped", "sign", "gqa_modulo", "causal_off_by_one",
           "causal_reversed", "mask_as_zero", "softmax_wrong_axis", "no_normalize", "k_as_v",
           "lse_log2", "lse_no_max"]


def test_unmutated_copy_passes_every_pin():
    """The mutant harness with no mistake planted must pass all pins (else the test is void)."""
    fn = _mutant("none")
    for pin in oracle_pins.ALL_PINS:
        pin(fn)


@pytest.mark.parametrize("kind", MUTANTS)
def test_mutant_is_caught(kind):
    fn = _mutant(kind)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake '{kind}' passed every pin"
