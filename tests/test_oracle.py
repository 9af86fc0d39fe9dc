"""CPU pins of the fp64 oracle (marker: not gpu)."""

import math

import numpy as np
import pytest

from oracle import (attention_forward, attention_head_rows, merge_states,
                    online_attention_forward, softmax_two_pass)
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(attention_forward)


@pytest.mark.parametrize("seed", range(6))
def test_two_pass_equals_online_merge(seed):
    """The two-pass definition and the blocked online merge agree (kwkr.cn tutorial §2.1-§2.3)."""
    r = np.random.default_rng(100 + seed)
    nq, nk = int(r.integers(1, 40)), int(r.integers(1, 40))
    d = int(r.integers(1, 9))
    hkv = int(r.integers(1, 3))
    hq = hkv * int(r.integers(1, 4))
    causal = bool(seed % 2)
    q = r.standard_normal((1, hq, nq, d)) * 3.0
    k = r.standard_normal((1, hkv, nk, d))
    v = r.standard_normal((1, hkv, nk, d))
    bias = r.standard_normal((1, hq, nq, nk)) if seed % 3 == 0 else None
    bm, bn = int(r.integers(1, nq + 1)), int(r.integers(1, nk + 1))
    o1, l1 = attention_forward(q, k, v, bias, scale=0.5, causal=causal)
    o2, l2 = online_attention_forward(q, k, v, bias, scale=0.5, causal=causal, block_m=bm,
                                      block_n=bn)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_merge_states_matches_whole_row(seed):
    """Splitting a row's keys into two sets and merging the partial states gives the softmax."""
    r = np.random.default_rng(200 + seed)
    n, d = 23, 5
    s = r.standard_normal(n) * 4.0
    v = r.standard_normal((n, d))
    sel = r.random(n) < 0.4
    sel[0], sel[1] = True, False

    def state(mask):
        m = s[mask].max()
        e = np.exp(s[mask] - m)
        return m, e.sum(), e @ v[mask]

    m, l, o = merge_states(*state(sel), *state(~sel))
    p, m_ref, l_ref = softmax_two_pass(s)
    np.testing.assert_allclose(o / l, p @ v, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m + math.log(l), m_ref + math.log(l_ref), rtol=0, atol=1e-12)


def test_merge_with_empty_side():
    """A side with max -inf (no finite logit) contributes nothing and produces no NaN."""
    m, l, o = merge_states(np.array(-np.inf), np.array(0.0), np.zeros(3),
                           np.array(1.5), np.array(2.0), np.array([1.0, 2.0, 3.0]))
    assert m == 1.5 and l == 2.0 and np.all(o == [1.0, 2.0, 3.0])


def test_softmax_two_pass_all_masked_row():
    p, m, l = softmax_two_pass(np.array([[-np.inf, -np.inf], [0.0, 0.0]]))
    assert np.all(p[0] == 0) and m[0] == -np.inf and l[0] == 0
    np.testing.assert_allclose(p[1], [0.5, 0.5])


def test_row_subset_equals_full():
    """Evaluating a subset of rows gives exactly the corresponding rows of the full result."""
    r = np.random.default_rng(7)
    q = r.standard_normal((1, 2, 40, 8))
    k = r.standard_normal((1, 1, 33, 8))
    v = r.standard_normal((1, 1, 33, 8))
    b = r.standard_normal((1, 2, 40, 33))
    o, lse = attention_forward(q, k, v, b, scale=0.3, causal=True)
    rows = np.array([0, 5, 32, 33, 39])
    o_r, l_r = attention_head_rows(q[0, 1, rows], k[0, 0], v[0, 0], rows=rows, scale=0.3,
                                   causal=True, bias_rows=b[0, 1, rows])
    np.testing.assert_array_equal(o_r, o[0, 1, rows])
    np.testing.assert_array_equal(l_r, lse[0, 1, rows])


def test_large_logits_stay_finite():
    """Logits near 1e3 overflow a naive exp; the max subtraction keeps everything finite."""
    r = np.random.default_rng(8)
    q = r.standard_normal((1, 1, 6, 4)) * 300.0
    k = r.standard_normal((1, 1, 6, 4))
    v = r.standard_normal((1, 1, 6, 4))
    o, lse = attention_forward(q, k, v, None, scale=1.0, causal=False)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert np.abs(o).max() <= np.abs(v).max() + 1e-12


def test_shape_errors():
    q = np.zeros((1, 3, 4, 8))
    k = np.zeros((1, 2, 4, 8))
    with pytest.raises(ValueError):
        attention_forward(q, k, k, None, scale=1.0)
    with pytest.raises(ValueError):
        attention_forward(q, np.zeros((1, 3, 4, 4)), np.zeros((1, 3, 4, 4)), None, scale=1.0)


def test_no_keys_gives_zero_output_and_minus_inf_lse():
    """Nk = 0: no row sees a key; by the no-finite-logit reading O = 0 and LSE = -inf."""
    q = np.ones((1, 2, 3, 4))
    k = np.zeros((1, 1, 0, 4))
    for causal in (False, True):
        o, lse = attention_forward(q, k, k, None, scale=1.0, causal=causal)
        assert o.shape == (1, 2, 3, 4) and np.all(o == 0) and np.all(lse == -np.inf)
