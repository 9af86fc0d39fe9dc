"""CPU pins of the oracle's key-split functions: ``attention_partial`` (the
definition restricted to a key range) and ``merge_partials`` (the combination of
normalised partial results).  Marker: not gpu.

What pins them, independently of their own code:
  * closed form: with Q = 0 and no bias every visible logit is 0, so the
    partial over keys [a, b) is the mean of the visible V rows and its LSE is
    ln of their count (0 rows: O = 0, LSE = -inf);
  * brute force: combining normalised partials is, by definition of the
    softmax, the average of the O_s weighted by their total mass e^LSE_s, and
    the combined LSE is ln of the summed mass: written out with math.exp and
    math.log on tiny inputs;
  * consistency with the two-pass definition (itself pinned elsewhere): the
    partials of any partition of the keys, in any order and with empty ranges
    among them, merge back to attention_forward (the merge of the kwkr.cn
    tutorial, §2.2, applied to several disjoint key sets).
Each pin is also run against planted mistakes, which it must catch.
"""

import math

import numpy as np
import pytest

from oracle import attention_forward, attention_partial, merge_partials

TOL = 1e-12


def _close(a, b, tol=TOL, what=""):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(both, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(err)), f"{what}: non-finite mismatch"
    assert err.max(initial=0.0) <= tol, f"{what}: max err {err.max()}"


def _partition(r, nk, parts):
    cuts = np.sort(r.integers(0, nk + 1, size=parts - 1))
    edges = np.concatenate([[0], cuts, [nk]])
    return [(int(edges[i]), int(edges[i + 1])) for i in range(parts)]


# ---------------------------------------------------------------------------
# pins (each takes the function(s) under test)
# ---------------------------------------------------------------------------

def pin_partial_closed_form(partial):
    """Q = 0, no bias: partial over [a, b) = mean of the visible V rows, LSE = ln(count)."""
    r = np.random.default_rng(11)
    nq, nk, d = 9, 13, 3
    q = np.zeros((1, 2, nq, d))
    k = r.standard_normal((1, 1, nk, d))
    v = r.standard_normal((1, 1, nk, d))
    for causal in (False, True):
        for a, b in [(0, nk), (3, 8), (5, 5), (12, 13), (0, 1)]:
            o, lse = partial(q, k, v, None, scale=0.7, causal=causal, key_begin=a, key_end=b)
            for i in range(nq):
                hi = min(b, i + 1) if causal else b
                cnt = max(0, hi - a)
                for h in range(2):
                    if cnt == 0:
                        assert np.all(o[0, h, i] == 0) and lse[0, h, i] == -np.inf, (a, b, i)
                    else:
                        _close(o[0, h, i], v[0, 0, a:hi].mean(axis=0), what=f"O {a},{b},{i}")
                        _close(lse[0, h, i], math.log(cnt), what=f"LSE {a},{b},{i}")


def _brute_merge(o_parts, lse_parts):
    """Weighted average by the mass e^LSE_s, written out with scalar loops."""
    P = len(lse_parts)
    rows, d = o_parts.shape[1], o_parts.shape[2]
    o = np.zeros((rows, d))
    lse = np.zeros(rows)
    for i in range(rows):
        mass = 0.0
        acc = [0.0] * d
        for s in range(P):
            if lse_parts[s][i] == -math.inf:
                continue
            w = math.exp(lse_parts[s][i])
            mass += w
            for c in range(d):
                acc[c] += w * o_parts[s][i][c]
        if mass == 0.0:
            lse[i] = -math.inf
        else:
            lse[i] = math.log(mass)
            for c in range(d):
                o[i, c] = acc[c] / mass
    return o, lse


def pin_merge_brute_force(merge):
    """Tiny partials with moderate LSEs (no overflow in e^LSE), some rows empty."""
    r = np.random.default_rng(12)
    for P in (1, 2, 3, 5):
        o_parts = r.standard_normal((P, 6, 4))
        lse_parts = r.uniform(-5.0, 5.0, size=(P, 6))
        lse_parts[0, 1] = -np.inf
        if P > 1:
            lse_parts[:, 2] = -np.inf  # a row no partial saw
            o_parts[:, 2] = 0.0
        o_parts[0, 1] = 0.0
        o_ref, l_ref = _brute_merge(o_parts, lse_parts)
        o, lse = merge(o_parts, lse_parts)
        _close(o, o_ref, tol=1e-12, what=f"O P={P}")
        _close(lse, l_ref, tol=1e-12, what=f"LSE P={P}")
    o, lse = merge(np.zeros((0, 3, 2)), np.zeros((0, 3)))
    assert o.shape == (3, 2) and np.all(o == 0) and np.all(lse == -np.inf)


def pin_partition_reproduces_whole(partial, merge):
    """Partials over any partition of the keys merge back to the two-pass definition."""
    for seed in range(6):
        r = np.random.default_rng(300 + seed)
        nq, nk, d = int(r.integers(1, 20)), int(r.integers(1, 30)), int(r.integers(1, 6))
        hkv = int(r.integers(1, 3))
        hq = hkv * int(r.integers(1, 4))
        causal = bool(seed % 2)
        q = r.standard_normal((2, hq, nq, d)) * 2.0
        k = r.standard_normal((2, hkv, nk, d))
        v = r.standard_normal((2, hkv, nk, d))
        bias = r.standard_normal((2, hq, nq, nk)) if seed % 3 == 0 else None
        ranges = _partition(r, nk, int(r.integers(1, 6)))
        r.shuffle(ranges)
        parts = [partial(q, k, v, bias, scale=0.4, causal=causal, key_begin=a, key_end=b)
                 for a, b in ranges]
        o, lse = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        o_ref, l_ref = attention_forward(q, k, v, bias, scale=0.4, causal=causal)
        _close(o, o_ref, what=f"O seed {seed}")
        _close(lse, l_ref, what=f"LSE seed {seed}")


# ---------------------------------------------------------------------------
# the oracle against its pins
# ---------------------------------------------------------------------------

def test_partial_closed_form():
    pin_partial_closed_form(attention_partial)


def test_merge_brute_force():
    pin_merge_brute_force(merge_partials)


def test_partition_reproduces_whole():
    pin_partition_reproduces_whole(attention_partial, merge_partials)


def test_merge_large_lse_stays_finite():
    """LSEs near 1e3 overflow e^LSE; the max-relative merge keeps the result finite."""
    o_parts = np.array([[[1.0, 2.0]], [[3.0, 4.0]]])
    lse_parts = np.array([[1000.0], [1000.0 + math.log(3.0)]])
    o, lse = merge_partials(o_parts, lse_parts)
    _close(o, [[2.5, 3.5]], tol=1e-12)
    _close(lse, [1000.0 + math.log(4.0)], tol=1e-9)


def test_partial_range_clamped():
    """A range past the keys is clamped to them; an empty range gives O = 0, LSE = -inf."""
    r = np.random.default_rng(13)
    q = r.standard_normal((1, 1, 3, 2))
    k = r.standard_normal((1, 1, 4, 2))
    o, lse = attention_partial(q, k, k, None, scale=1.0, key_begin=2, key_end=99)
    o2, l2 = attention_partial(q, k, k, None, scale=1.0, key_begin=2, key_end=4)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)
    o, lse = attention_partial(q, k, k, None, scale=1.0, key_begin=4, key_end=4)
    assert np.all(o == 0) and np.all(lse == -np.inf)


# ---------------------------------------------------------------------------
# planted mistakes: each must trip at least one pin
# ---------------------------------------------------------------------------

def _partial_mutant(kind):
    def fn(q, k, v, bias=None, *, scale, causal, key_begin, key_end):
        nk = k.shape[2]
        a, b = key_begin, min(key_end, nk)
        if kind == "inclusive_end":
            b = min(b + 1, nk)
        if kind == "ignores_range":
            a, b = 0, nk
        if kind == "local_causal" and causal and b > a:
            # causal positions taken relative to the start of the range
            ks, vs = k[:, :, a:b], v[:, :, a:b]
            bs = None if bias is None else bias[..., a:b]
            return attention_forward(q, ks, vs, bs, scale=scale, causal=True)
        return attention_partial(q, k, v, bias, scale=scale, causal=causal, key_begin=a,
                                 key_end=b)
    return fn


def _merge_mutant(kind):
    def fn(o_parts, lse_parts):
        o_parts, lse_parts = np.asarray(o_parts, float), np.asarray(lse_parts, float)
        if len(lse_parts) == 0:
            return merge_partials(o_parts, lse_parts)
        fin = np.isfinite(lse_parts)
        m = np.where(fin, lse_parts, -np.inf).max(axis=0)
        m0 = np.where(np.isfinite(m), m, 0.0)
        w = np.where(fin, np.exp(lse_parts - m0), 0.0)
        if kind == "uniform_weights":
            w = fin.astype(float)
        if kind == "no_max_lse":
            pass
        tot = w.sum(axis=0)
        ok = tot > 0
        o = (w[..., None] * o_parts).sum(axis=0) / np.where(ok, tot, 1.0)[..., None]
        if kind == "unnormalised":
            o = (w[..., None] * o_parts).sum(axis=0)
        lse = np.where(ok, m0 + np.log(np.where(ok, tot, 1.0)), -np.inf)
        if kind == "no_max_lse":
            lse = np.where(ok, m, -np.inf)
        if kind == "drop_last" and len(lse_parts) > 1:
            return fn(o_parts[:-1], lse_parts[:-1])
        return o, lse
    return fn


def _caught(run):
    try:
        with np.errstate(all="ignore"):
            run()
    except (AssertionError, ValueError, FloatingPointError):
        return True
    return False


def test_unmutated_merge_harness_passes():
    fn = _merge_mutant("none")
    pin_merge_brute_force(fn)
    pin_partition_reproduces_whole(attention_partial, fn)
    pin_partial_closed_form(_partial_mutant("none"))
    pin_partition_reproduces_whole(_partial_mutant("none"), merge_partials)


@pytest.mark.parametrize("kind", ["inclusive_end", "ignores_range", "local_causal"])
def test_partial_mutant_is_caught(kind):
    fn = _partial_mutant(kind)
    assert (_caught(lambda: pin_partial_closed_form(fn))
            or _caught(lambda: pin_partition_reproduces_whole(fn, merge_partials))), kind


@pytest.mark.parametrize("kind", ["uniform_weights", "no_max_lse", "unnormalised", "drop_last"])
def test_merge_mutant_is_caught(kind):
    fn = _merge_mutant(kind)
    assert (_caught(lambda: pin_merge_brute_force(fn))
            or _caught(lambda: pin_partition_reproduces_whole(attention_partial, fn))), kind
