"""Pins for the fp64 attention oracle (CPU only; not collected by pytest itself).

Each ``pin_*`` function takes an attention function with the oracle's
signature ``fn(q, k, v, bias, *, scale, causal) -> (O, LSE)`` and raises
AssertionError when the function disagrees with something the pages or the
mathematics fix independently of it:

  * closed forms (Q = 0 gives the mean of the visible V rows and LSE = ln of
    their count; a single key gives O = V and LSE = the one logit);
  * the convex-combination property (identical V rows pass through);
  * a library routine (torch's scaled_dot_product_attention evaluated in fp64
    on the CPU, with its additive float mask and its GQA option);
  * brute force (pure-Python loops with math.exp on tiny inputs);
  * invariants (a per-row logit shift moves only LSE; permuting keys does not
    matter without a mask; GQA equals MHA on repeated K/V heads; the
    probabilities exp(S - LSE) sum to one; the last causal row sees every key).

``test_oracle.py`` runs them against the oracle; ``test_oracle_mutants.py``
runs them against deliberately broken copies of the oracle and checks that
every planted mistake trips at least one pin.
"""

from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(seed, B=1, Hq=2, Hkv=2, Nq=7, Nk=7, D=4, bias=False):
    r = _rng(seed)
    q = r.standard_normal((B, Hq, Nq, D))
    k = r.standard_normal((B, Hkv, Nk, D))
    v = r.standard_normal((B, Hkv, Nk, D))
    b = r.standard_normal((B, Hq, Nq, Nk)) if bias else None
    return q, k, v, b


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(both_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(err)), f"{what}: non-finite mismatch"
    assert err.max(initial=0.0) <= tol, f"{what}: max err {err.max()}"


def pin_q_zero_noncausal(fn):
    """Q = 0, no bias: every logit is 0, so O is the column mean of V and LSE = ln Nk."""
    for nq, nk in [(5, 9), (9, 5), (1, 1), (16, 16)]:
        _, k, v, _ = _inputs(1, B=2, Hq=4, Hkv=2, Nq=nq, Nk=nk, D=3)
        q = np.zeros((2, 4, nq, 3))
        o, lse = fn(q, k, v, None, scale=0.7, causal=False)
        for h in range(4):
            mean = v[:, h // 2].mean(axis=1)  # [B, D]
            _close(o[:, h], np.broadcast_to(mean[:, None, :], o[:, h].shape), what="Q=0 O")
        _close(lse, np.full(lse.shape, math.log(nk)), what="Q=0 LSE")


def pin_q_zero_causal(fn):
    """Q = 0, causal top-left: row i averages V_0..V_min(i, Nk-1); LSE_i = ln(count)."""
    for nq, nk in [(8, 8), (11, 6), (6, 11)]:
        _, k, v, _ = _inputs(2, B=1, Hq=2, Hkv=1, Nq=nq, Nk=nk, D=3)
        q = np.zeros((1, 2, nq, 3))
        o, lse = fn(q, k, v, None, scale=1.3, causal=True)
        for i in range(nq):
            n_vis = min(i + 1, nk)
            for h in range(2):
                _close(o[0, h, i], v[0, 0, :n_vis].mean(axis=0), what=f"causal Q=0 row {i}")
                _close(lse[0, h, i], math.log(n_vis), what=f"causal Q=0 LSE row {i}")


def pin_identical_v_rows(fn):
    """All V rows equal to one vector u: O = u for every query, mask and bias."""
    for causal in (False, True):
        for with_bias in (False, True):
            q, k, _, b = _inputs(3, B=1, Hq=2, Hkv=1, Nq=6, Nk=9, D=4, bias=with_bias)
            u = _rng(4).standard_normal(4)
            v = np.broadcast_to(u, (1, 1, 9, 4)).copy()
            o, _ = fn(q, k, v, b, scale=0.9, causal=causal)
            _close(o, np.broadcast_to(u, o.shape), tol=1e-12, what="identical V rows")


def pin_single_key(fn):
    """Nk = 1: softmax over one logit is 1, so O = V_0 and LSE = q.k*scale (+bias)."""
    for with_bias in (False, True):
        q, k, v, b = _inputs(5, B=2, Hq=3, Hkv=1, Nq=4, Nk=1, D=5, bias=with_bias)
        scale = 0.37
        o, lse = fn(q, k, v, b, scale=scale, causal=False)
        _close(o, np.broadcast_to(v[:, :, :1, :], o.shape), what="Nk=1 O")
        logit = np.einsum("bhid,bjd->bhij", q, k[:, 0])[..., 0] * scale
        if b is not None:
            logit = logit + b[..., 0]
        _close(lse, logit, tol=1e-12, what="Nk=1 LSE")
    # N = 1 with the causal mask: the only key is visible to the only query.
    q, k, v, _ = _inputs(6, B=1, Hq=1, Hkv=1, Nq=1, Nk=1, D=3)
    o, lse = fn(q, k, v, None, scale=2.0, causal=True)
    _close(o, v, what="N=1 causal O")
    _close(lse, (q[0, 0, 0] @ k[0, 0, 0] * 2.0).reshape(1, 1, 1), what="N=1 causal LSE")


def pin_causal_row0(fn):
    """Causal row 0 sees only key 0, so O_0 = V_0 whatever Q, K and bias are."""
    q, k, v, b = _inputs(7, B=1, Hq=4, Hkv=2, Nq=5, Nk=5, D=4, bias=True)
    o, _ = fn(q, k, v, b, scale=0.5, causal=True)
    for h in range(4):
        _close(o[0, h, 0], v[0, h // 2, 0], what="causal row 0")


def _sdpa(q, k, v, bias, scale, causal):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    mask = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias))
    gqa = tq.shape[1] != tk.shape[1]
    return F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, is_causal=causal,
                                          scale=scale, enable_gqa=gqa).numpy()


def pin_library_sdpa(fn):
    """torch's scaled_dot_product_attention in fp64 on the CPU (a library routine)."""
    cases = [
        dict(B=2, Hq=2, Hkv=2, Nq=9, Nk=13, D=8, bias=False, causal=False),
        dict(B=1, Hq=3, Hkv=3, Nq=12, Nk=12, D=4, bias=False, causal=True),
        dict(B=1, Hq=2, Hkv=2, Nq=10, Nk=10, D=4, bias=True, causal=False),
        dict(B=1, Hq=6, Hkv=2, Nq=8, Nk=11, D=4, bias=True, causal=False),
        dict(B=2, Hq=4, Hkv=1, Nq=6, Nk=6, D=4, bias=False, causal=True),
    ]
    for i, c in enumerate(cases):
        q, k, v, b = _inputs(10 + i, B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], Nq=c["Nq"], Nk=c["Nk"],
                             D=c["D"], bias=c["bias"])
        scale = 1.0 / math.sqrt(c["D"])
        o, _ = fn(q, k, v, b, scale=scale, causal=c["causal"])
        _close(o, _sdpa(q, k, v, b, scale, c["causal"]), tol=1e-12, what=f"sdpa case {i}")
    # causal plus an additive bias: torch combines them when the mask already
    # carries the -inf of the causal triangle.
    q, k, v, b = _inputs(20, B=1, Hq=2, Hkv=2, Nq=7, Nk=7, D=4, bias=True)
    tri = np.triu(np.ones((7, 7), dtype=bool), 1)
    masked = np.where(tri, -np.inf, b)
    o, _ = fn(q, k, v, b, scale=0.5, causal=True)
    _close(o, _sdpa(q, k, v, masked, 0.5, False), tol=1e-12, what="sdpa causal+bias")


def _brute(q, k, v, bias, scale, causal):
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    o = [[[[0.0] * D for _ in range(Nq)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[0.0] * Nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            hk = h // grp
            for i in range(Nq):
                logits = []
                for j in range(Nk):
                    if causal and j > i:
                        continue
                    s = 0.0
                    for d in range(D):
                        s += float(q[b, h, i, d]) * float(k[b, hk, j, d])
                    s *= scale
                    if bias is not None:
                        s += float(bias[b, h, i, j])
                    logits.append((j, s))
                mx = max(s for _, s in logits)
                ws = [(j, math.exp(s - mx)) for j, s in logits]
                tot = sum(w for _, w in ws)
                for d in range(D):
                    o[b][h][i][d] = sum(w * float(v[b, hk, j, d]) for j, w in ws) / tot
                lse[b][h][i] = mx + math.log(tot)
    return np.array(o), np.array(lse)


def pin_brute_force(fn):
    """Pure-Python loops with math.exp on shapes up to 8x8, D <= 4."""
    cases = [
        dict(B=1, Hq=1, Hkv=1, Nq=5, Nk=8, D=3, bias=False, causal=False),
        dict(B=1, Hq=2, Hkv=1, Nq=8, Nk=8, D=4, bias=True, causal=True),
        dict(B=2, Hq=4, Hkv=2, Nq=6, Nk=4, D=2, bias=True, causal=False),
        dict(B=1, Hq=3, Hkv=3, Nq=7, Nk=5, D=4, bias=False, causal=True),
        dict(B=1, Hq=4, Hkv=1, Nq=3, Nk=7, D=4, bias=False, causal=True),
    ]
    for i, c in enumerate(cases):
        q, k, v, b = _inputs(30 + i, B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], Nq=c["Nq"], Nk=c["Nk"],
                             D=c["D"], bias=c["bias"])
        scale = 0.8 + 0.1 * i
        o, lse = fn(q, k, v, b, scale=scale, causal=c["causal"])
        ob, lb = _brute(q, k, v, b, scale, c["causal"])
        _close(o, ob, tol=1e-12, what=f"brute O case {i}")
        _close(lse, lb, tol=1e-12, what=f"brute LSE case {i}")


def pin_invariants(fn):
    """Shift, permutation, GQA-as-repeat, normalisation and last-row invariants."""
    q, k, v, b = _inputs(40, B=1, Hq=4, Hkv=2, Nq=9, Nk=9, D=4, bias=True)
    scale = 0.6
    # 1. adding c_i to every logit of row i leaves O alone and moves LSE by c_i
    c = _rng(41).standard_normal((1, 4, 9))
    for causal in (False, True):
        o0, l0 = fn(q, k, v, b, scale=scale, causal=causal)
        o1, l1 = fn(q, k, v, b + c[..., None], scale=scale, causal=causal)
        _close(o1, o0, tol=1e-12, what="row shift O")
        _close(l1, l0 + c, tol=1e-12, what="row shift LSE")
    # 2. permuting keys (rows of K, V and columns of the bias) without a mask
    perm = _rng(42).permutation(9)
    o0, l0 = fn(q, k, v, b, scale=scale, causal=False)
    o1, l1 = fn(q, k[:, :, perm], v[:, :, perm], b[..., perm], scale=scale, causal=False)
    _close(o1, o0, tol=1e-12, what="key permutation O")
    _close(l1, l0, tol=1e-12, what="key permutation LSE")
    # 3. GQA equals MHA on K/V heads repeated per group (contiguous groups)
    for causal in (False, True):
        og, lg = fn(q, k, v, b, scale=scale, causal=causal)
        om, lm = fn(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), b, scale=scale,
                    causal=causal)
        _close(og, om, tol=1e-12, what="GQA as repeat O")
        _close(lg, lm, tol=1e-12, what="GQA as repeat LSE")
    # 4. probabilities recovered from LSE sum to one over the visible keys
    for causal in (False, True):
        _, lse = fn(q, k, v, b, scale=scale, causal=causal)
        s = np.einsum("bhid,bhjd->bhij", q, np.repeat(k, 2, axis=1)) * scale + b
        if causal:
            s = np.where(np.triu(np.ones((9, 9), dtype=bool), 1), -np.inf, s)
        tot = np.exp(s - lse[..., None]).sum(axis=-1)
        _close(tot, np.ones_like(tot), tol=1e-12, what="sum exp(S - LSE)")
    # 5. the last causal row (Nq = Nk) sees every key
    oc, lc = fn(q, k, v, b, scale=scale, causal=True)
    on, ln_ = fn(q, k, v, b, scale=scale, causal=False)
    _close(oc[:, :, -1], on[:, :, -1], tol=1e-12, what="last causal row O")
    _close(lc[:, :, -1], ln_[:, :, -1], tol=1e-12, what="last causal row LSE")


def pin_masked_row(fn):
    """A row whose every logit is -inf (bias) yields O = 0 and LSE = -inf, no NaN."""
    q, k, v, b = _inputs(50, B=1, Hq=1, Hkv=1, Nq=4, Nk=5, D=3, bias=True)
    b[0, 0, 2, :] = -np.inf
    o, lse = fn(q, k, v, b, scale=1.0, causal=False)
    assert np.all(o[0, 0, 2] == 0.0) and lse[0, 0, 2] == -np.inf
    assert np.all(np.isfinite(o)) and np.isfinite(lse[0, 0, [0, 1, 3]]).all()


ALL_PINS = [
    pin_q_zero_noncausal,
    pin_q_zero_causal,
    pin_identical_v_rows,
    pin_single_key,
    pin_causal_row0,
    pin_library_sdpa,
    pin_brute_force,
    pin_invariants,
    pin_masked_row,
]
