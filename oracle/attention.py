"""fp64 CPU oracle for the fused attention forward (test infrastructure only).

What it computes, per batch ``b`` and query head ``hq``::

    S   = Q[b,hq] · K[b,hk]^T · scale  (+ bias[b,hq])      logits
    S_ij = -inf  where causal and j > i                     mask
    m_i = max_j S_ij,  l_i = sum_j exp(S_ij - m_i)           two-pass softmax
    P   = exp(S - m) / l,  O = P · V[b,hk],  LSE_i = m_i + ln l_i

This is the plain, materialising definition of attention:
  * "FlashAttention principles and Triton practice" (xnwp.cn/news/15505), §2.1:
    S = Q K^T, P = softmax(S), O = P V, with S and P held whole;
  * FlashAttention forward tutorial (kwkr.cn/news/592482), §1.1 (the 1/sqrt(d)
    scale), §2.1 (softmax taken as max, then sum of exp(x - max), then divide),
    §3.4 (causal mask = strict upper triangle set to -inf);
  * Day 26 operator acceleration (blog.ans20xx.com/posts/ai/day26), the naive
    attention wrapper (scale, lower-triangular keep-mask, softmax, times V);
  * "Block Attention Residual" Triton kernel post (iqiancheng.github.io), the
    A_i formula: the additive term is added to the already-scaled logits,
    before softmax.

Readings where the pages are silent (each is listed with its reason in the
design notes of this repository):
  * causal alignment is top-left: key j is visible to query i iff j <= i;
  * the bias is not multiplied by ``scale`` and masked entries stay -inf
    whatever the bias;
  * GQA groups are contiguous: hk = hq // (Hq // Hkv);
  * the softmax statistic emitted is one natural-log LSE = m + ln l, in the
    units of the scaled-plus-bias logits;
  * a row with no finite logit yields O = 0 and LSE = -inf.

The tiled method reaches this same result in exact arithmetic (kwkr.cn
tutorial, §2.2-§2.3), so the oracle is the definition itself.  The blocked
online-softmax form below is kept only so that tests can pin the two against
each other.

Inputs are arrays of any float dtype; they are upcast to float64 exactly
(bf16/fp16/fp32 values are representable in fp64), so the oracle sees the same
rounded inputs the GPU path sees.

This module is test infrastructure.  Only ``tests/``, ``__graft_entry__.smoke``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
never does.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "softmax_two_pass",
    "attention_head_rows",
    "attention_forward",
    "online_attention_forward",
    "merge_states",
    "attention_partial",
    "merge_partials",
    "attention_backward",
    "attention_chain",
    "attention_chain_head_rows",
    "attention_chain_backward",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def softmax_two_pass(s):
    """Row-wise softmax over the last axis, two passes (kwkr.cn tutorial, §2.1).

    Pass one takes the row max m; pass two sums exp(s - m) into l and divides.
    Returns ``(p, m, l)``.  A row whose entries are all -inf has m = -inf,
    l = 0 and p = 0 (no NaN is produced).
    """
    s = _f64(s)
    if s.shape[-1] == 0:  # no key at all: the "no finite logit" case
        return s.copy(), np.full(s.shape[:-1], -np.inf), np.zeros(s.shape[:-1])
    m = s.max(axis=-1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[..., None])
    l = e.sum(axis=-1)
    l_div = np.where(l > 0, l, 1.0)
    p = np.where((l > 0)[..., None], e / l_div[..., None], 0.0)
    return p, m, l


def attention_head_rows(q_rows, k, v, *, rows, scale, causal, bias_rows=None, window=None):
    """O and LSE for selected query rows of one (batch, query head).

    q_rows    [n, D]  the query rows
    rows      [n]     their absolute query indices (used by the causal mask)
    k, v      [Nk, D] the key/value rows of the KV head these queries read
    bias_rows [n, Nk] additive logit term for those rows, or None
    window    None, or W >= 1 with causal: key j is visible to row i only if
              i - W < j <= i (a sliding window of the W most recent keys)

    Row i of the output depends only on q_i, on K, V and on bias row i, so a
    subset of rows is the same definition evaluated on fewer rows.
    """
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    nk = k.shape[0]
    s = (q_rows @ k.T) * float(scale)
    if bias_rows is not None:
        s = s + _f64(bias_rows)
    if causal:
        j = np.arange(nk, dtype=np.int64)
        s = np.where(j[None, :] > rows[:, None], -np.inf, s)
        if window is not None:
            s = np.where(j[None, :] <= rows[:, None] - int(window), -np.inf, s)
    p, m, l = softmax_two_pass(s)
    o = p @ v
    lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def _check_shapes(q, k, v, bias):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, D]")
    b, hq, nq, d = q.shape
    bk, hkv, nk, dk = k.shape
    if v.shape != k.shape or bk != b or dk != d:
        raise ValueError("k and v must be [B, Hkv, Nk, D] matching q")
    if hkv < 1 or hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if bias is not None and tuple(bias.shape) != (b, hq, nq, nk):
        raise ValueError("bias must be [B, Hq, Nq, Nk]")
    return b, hq, hkv, nq, nk, d


def attention_forward(q, k, v, bias=None, *, scale=None, causal=False, window=None):
    """Full attention forward, one (b, hq) at a time.

    q [B,Hq,Nq,D], k/v [B,Hkv,Nk,D], bias [B,Hq,Nq,Nk] or None.
    ``scale=None`` means 1/sqrt(D).  ``window`` (with ``causal``) limits each
    row i to the keys i - window < j <= i: the sliding-window attention that
    "FlashAttention principles and Triton practice", §3.1, and the kwkr.cn
    tutorial's closing remarks name as a mask variant of the same kernel.
    Returns ``(O [B,Hq,Nq,D], LSE [B,Hq,Nq])`` in float64.
    """
    if window is not None and (not causal or int(window) < 1):
        raise ValueError("window needs causal=True and window >= 1")
    b_, hq_, hkv, nq, nk, d = _check_shapes(q, k, v, bias)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    group = hq_ // hkv
    o = np.empty((b_, hq_, nq, d), dtype=np.float64)
    lse = np.empty((b_, hq_, nq), dtype=np.float64)
    rows = np.arange(nq, dtype=np.int64)
    for b in range(b_):
        for h in range(hq_):
            hk = h // group
            o[b, h], lse[b, h] = attention_head_rows(
                q[b, h], k[b, hk], v[b, hk], rows=rows, scale=scale, causal=causal,
                bias_rows=None if bias is None else bias[b, h], window=window)
    return o, lse


def merge_states(m_a, l_a, o_a, m_b, l_b, o_b):
    """Combine two partial softmax states over disjoint key sets.

    Each state is (running max m, running sum l, un-normalised output o).
    The combined max is the larger of the two; each side's sum and output are
    re-expressed against it by the factor exp(m_side - m).  This is the
    symmetric form of the merge in the kwkr.cn tutorial, §2.2.  A side whose
    max is -inf (it saw no finite logit) contributes nothing.
    """
    m_a, l_a, o_a = _f64(m_a), _f64(l_a), _f64(o_a)
    m_b, l_b, o_b = _f64(m_b), _f64(l_b), _f64(o_b)
    m = np.maximum(m_a, m_b)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    fa = np.where(np.isfinite(m_a), np.exp(m_a - m_safe), 0.0)
    fb = np.where(np.isfinite(m_b), np.exp(m_b - m_safe), 0.0)
    return m, l_a * fa + l_b * fb, o_a * fa[..., None] + o_b * fb[..., None]


def online_attention_forward(q, k, v, bias=None, *, scale=None, causal=False,
                             block_m=64, block_n=64):
    """Blocked forward with the online softmax update, in fp64.

    Follows the kwkr.cn tutorial, §2.2-§2.3: an outer loop over row blocks of
    Q and an inner loop over column blocks of K/V.  For each column block the
    running max becomes m_new = max(m_old, rowmax(S_ij)); the old sum and the
    old output are both multiplied by alpha = exp(m_old - m_new); the block's
    exp(S_ij - m_new) is added to the sum and its product with V_j to the
    output; the division by l happens once, after the last block.  While the
    running max is still -inf, alpha is taken as 0 instead of exp(-inf + inf)
    (the NaN trap of "FlashAttention principles and Triton practice", §5.1).

    Only tests use this, to pin the two-pass definition against the merge
    formula on small inputs; it is not a model of any GPU kernel.
    """
    b_, hq_, hkv, nq, nk, d = _check_shapes(q, k, v, bias)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q, k, v = _f64(q), _f64(k), _f64(v)
    bias = None if bias is None else _f64(bias)
    group = hq_ // hkv
    o = np.zeros((b_, hq_, nq, d))
    lse = np.zeros((b_, hq_, nq))
    for b in range(b_):
        for h in range(hq_):
            hk = h // group
            for r0 in range(0, nq, block_m):
                r1 = min(r0 + block_m, nq)
                rows = np.arange(r0, r1)
                m_i = np.full(r1 - r0, -np.inf)
                l_i = np.zeros(r1 - r0)
                acc = np.zeros((r1 - r0, d))
                for c0 in range(0, nk, block_n):
                    c1 = min(c0 + block_n, nk)
                    s = (q[b, h, r0:r1] @ k[b, hk, c0:c1].T) * scale
                    if bias is not None:
                        s = s + bias[b, h, r0:r1, c0:c1]
                    if causal:
                        cols = np.arange(c0, c1)
                        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
                    m_new = np.maximum(m_i, s.max(axis=1))
                    m_use = np.where(np.isfinite(m_new), m_new, 0.0)
                    alpha = np.where(np.isfinite(m_i), np.exp(m_i - m_use), 0.0)
                    p = np.exp(s - m_use[:, None])
                    l_i = l_i * alpha + p.sum(axis=1)
                    acc = acc * alpha[:, None] + p @ v[b, hk, c0:c1]
                    m_i = m_new
                ok = l_i > 0
                o[b, h, r0:r1] = np.where(ok[:, None], acc / np.where(ok, l_i, 1.0)[:, None], 0.0)
                lse[b, h, r0:r1] = np.where(ok, m_i + np.log(np.where(ok, l_i, 1.0)), -np.inf)
    return o, lse


def attention_partial(q, k, v, bias=None, *, scale=None, causal=False, key_begin=0,
                      key_end=None):
    """Attention of every query over the keys [key_begin, key_end) only.

    The definition above with every logit outside the key range set to -inf:
    the state of one disjoint key subset, normalised by its own sum.  Returns
    ``(O_part [B,Hq,Nq,D], LSE_part [B,Hq,Nq])``; rows that see no key of the
    range get O_part = 0 and LSE_part = -inf.  Causal positions stay global
    (key j is visible to query i iff j <= i), so the partials of a partition
    of the keys describe the same rows as the whole.
    """
    b_, hq_, hkv, nq, nk, d = _check_shapes(q, k, v, bias)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    key_end = nk if key_end is None else min(int(key_end), nk)
    key_begin = max(0, min(int(key_begin), key_end))
    group = hq_ // hkv
    o = np.zeros((b_, hq_, nq, d), dtype=np.float64)
    lse = np.full((b_, hq_, nq), -np.inf, dtype=np.float64)
    if key_end == key_begin:
        return o, lse
    cols = np.arange(nk)
    outside = (cols < key_begin) | (cols >= key_end)
    rows = np.arange(nq, dtype=np.int64)
    for b in range(b_):
        for h in range(hq_):
            hk = h // group
            extra = np.where(outside[None, :], -np.inf, 0.0)
            if bias is not None:
                extra = extra + _f64(bias[b, h])
            o[b, h], lse[b, h] = attention_head_rows(
                q[b, h], k[b, hk], v[b, hk], rows=rows, scale=scale, causal=causal,
                bias_rows=np.broadcast_to(extra, (nq, nk)))
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Combine normalised partial results over disjoint key sets into one.

    o_parts [P, ..., D], lse_parts [P, ...].  A normalised partial (O_s,
    LSE_s) is the state (m = LSE_s, l = 1, o = O_s): its sum times e^m is
    e^LSE_s, the same total weight.  The states are folded one after another
    with ``merge_states`` (the merge of the kwkr.cn tutorial, §2.2), and the
    result is normalised once at the end: O = o / l, LSE = m + ln l.  A
    partial with LSE = -inf (no visible key) carries l = 0 and adds nothing;
    with no partial at all, or only such ones, O = 0 and LSE = -inf.
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    if o_parts.shape[:-1] != lse_parts.shape:
        raise ValueError("o_parts must be lse_parts' shape plus a trailing D axis")
    shape = lse_parts.shape[1:]
    m = np.full(shape, -np.inf)
    l = np.zeros(shape)
    o = np.zeros(o_parts.shape[1:])
    for o_s, lse_s in zip(o_parts, lse_parts):
        l_s = np.where(np.isfinite(lse_s), 1.0, 0.0)
        m, l, o = merge_states(m, l, o, lse_s, l_s, o_s * l_s[..., None])
    ok = l > 0
    o_out = np.where(ok[..., None], o / np.where(ok, l, 1.0)[..., None], 0.0)
    lse_out = np.where(ok, m + np.log(np.where(ok, l, 1.0)), -np.inf)
    return o_out, lse_out


def attention_backward(q, k, v, dout, bias=None, *, scale=None, causal=False, window=None):
    """Gradients of the forward definition above with respect to q, k and v.

    The forward keeps only O and the per-row statistic and recomputes S and P
    in the backward ("FlashAttention principles and Triton practice", §2.3 and
    §4.3; kwkr.cn tutorial, §2.4).  What that recomputation must reproduce is
    the chain rule through the definition, per (b, hq) with hk = hq // group:

        P   = softmax(S)            (S as in the forward, masked entries -inf)
        dV  = P^T dO                (summed over the query heads of a group)
        dP  = dO V^T
        D_i = sum_j P_ij dP_ij  =  sum_d dO_id O_id     (the row sum to subtract)
        dS  = P o (dP - D)          (elementwise; masked entries have P = 0)
        dQ  = scale * dS K
        dK  = scale * dS^T Q        (summed over the query heads of a group)

    The bias term receives dS itself and is treated as a constant here (its
    gradient is not returned); LSE is an auxiliary output with no incoming
    gradient.  Rows that see no key have P = 0 and contribute nothing.
    ``window`` masks as in ``attention_forward``.
    Returns ``(dQ, dK, dV)`` in float64 with the shapes of q, k, v.
    """
    if window is not None and (not causal or int(window) < 1):
        raise ValueError("window needs causal=True and window >= 1")
    b_, hq_, hkv, nq, nk, d = _check_shapes(q, k, v, bias)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    group = hq_ // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(b_):
        for h in range(hq_):
            hk = h // group
            s = (q[b, h] @ k[b, hk].T) * float(scale)
            if bias is not None:
                s = s + _f64(bias[b, h])
            if causal:
                i = np.arange(nq)[:, None]
                j = np.arange(nk)[None, :]
                s = np.where(j > i, -np.inf, s)
                if window is not None:
                    s = np.where(j <= i - int(window), -np.inf, s)
            p, _, _ = softmax_two_pass(s)
            do = dout[b, h]
            dv[b, hk] += p.T @ do
            dp = do @ v[b, hk].T
            dsum = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - dsum)
            dq[b, h] = float(scale) * (ds @ k[b, hk])
            dk[b, hk] += float(scale) * (ds.T @ q[b, h])
    return dq, dk, dv


def attention_chain(q_layers, k_layers, v, *, scale=None, causal=False):
    """Forward of the last layer of a Block Attention Residual chain.

    "Block Attention Residual" Triton kernel post (iqiancheng.github.io), the
    A_i formula and the block diagram: consecutive layers are grouped into
    blocks of 4; inside a block, layer i adds the pre-softmax logits of layer
    i-1 to its own scaled Q_i K_i^T before the softmax, and those logits
    already carry layer i-2's, so the sum runs back to the block's first
    layer; at a block boundary the residual is zero.

    q_layers  list of the block's Q tensors up to the current layer, oldest
              first, each [B, Hq, Nq, D]
    k_layers  the matching K tensors, each [B, Hkv, Nk, D]
    v         the current layer's V, [B, Hkv, Nk, D]

    The steps follow the post's recursion, one (b, hq) at a time: the residual
    starts at zero; each earlier layer l replaces it by its own logits
    Q_l K_l^T * scale + residual; the current layer is then the forward above
    with that residual as its additive logit term (none for a block's first
    layer).  Every layer's product takes the same ``scale`` (the post divides
    each by sqrt(d)); ``scale=None`` means 1/sqrt(D).  Returns ``(O, LSE)``.
    """
    n = len(q_layers)
    if n < 1 or len(k_layers) != n:
        raise ValueError("need as many K layers as Q layers, at least one")
    q_cur, k_cur = q_layers[-1], k_layers[-1]
    b_, hq_, hkv, nq, nk, d = _check_shapes(q_cur, k_cur, v, None)
    for ql, kl in zip(q_layers, k_layers):
        if tuple(ql.shape) != tuple(q_cur.shape) or tuple(kl.shape) != tuple(k_cur.shape):
            raise ValueError("every layer of the chain has the same Q and K shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    group = hq_ // hkv
    o = np.empty((b_, hq_, nq, d), dtype=np.float64)
    lse = np.empty((b_, hq_, nq), dtype=np.float64)
    rows = np.arange(nq, dtype=np.int64)
    for b in range(b_):
        for h in range(hq_):
            hk = h // group
            o[b, h], lse[b, h] = attention_chain_head_rows(
                [ql[b, h] for ql in q_layers], [kl[b, hk] for kl in k_layers], v[b, hk],
                rows=rows, scale=scale, causal=causal)
    return o, lse


def attention_chain_head_rows(q_rows_layers, k_layers, v, *, rows, scale, causal):
    """``attention_chain`` for selected query rows of one (batch, query head).

    q_rows_layers  per layer, oldest first, the [n, D] query rows
    k_layers       per layer the [Nk, D] keys of the KV head these rows read
    v              [Nk, D] the current layer's values
    rows           [n] the rows' absolute query indices (for the causal mask)

    The residual of row i depends only on row i of each Q layer, so a subset
    of rows is the same recursion on fewer rows.
    """
    residual = None
    for ql, kl in zip(q_rows_layers[:-1], k_layers[:-1]):
        logits = (_f64(ql) @ _f64(kl).T) * float(scale)
        residual = logits if residual is None else logits + residual
    return attention_head_rows(q_rows_layers[-1], k_layers[-1], v, rows=rows, scale=scale,
                               causal=causal, bias_rows=residual)


def attention_chain_backward(q_layers, k_layers, v, dout, *, scale=None, causal=False):
    """Gradients of ``attention_chain`` with respect to every Q and K layer and V.

    The "Block Attention Residual" post trains through the fused chain: its
    first kernel version keeps the softmax statistic for the backward, which
    recomputes the logits.  The chain rule through the recursion of
    ``attention_chain``: the current layer's logits are S = sum over the
    block's layers l of Q_l K_l^T * scale (the residual is that sum over the
    earlier layers), so per (b, hq) with hk = hq // group

        P     = softmax(S)                 (causal entries -inf, as in the forward)
        dV    = P^T dO                     (summed over the query heads of a group)
        dP    = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P o (dP - D)
        dQ_l  = scale * dS K_l             for every layer l
        dK_l  = scale * dS^T Q_l           (summed over the query heads of a group)

    The earlier layers' own outputs are not part of this function: their
    gradients reach Q_l and K_l through their own attention, which the caller
    adds.  Returns ``(dq_layers, dk_layers, dv)``, lists of float64 arrays with
    the layers' shapes, and dV with v's.
    """
    n = len(q_layers)
    if n < 1 or len(k_layers) != n:
        raise ValueError("need as many K layers as Q layers, at least one")
    b_, hq_, hkv, nq, nk, d = _check_shapes(q_layers[-1], k_layers[-1], v, None)
    for ql, kl in zip(q_layers, k_layers):
        if tuple(ql.shape) != tuple(q_layers[-1].shape) or tuple(kl.shape) != tuple(k_layers[-1].shape):
            raise ValueError("every layer of the chain has the same Q and K shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qs = [_f64(x) for x in q_layers]
    ks = [_f64(x) for x in k_layers]
    v, dout = _f64(v), _f64(dout)
    if dout.shape != qs[-1].shape:
        raise ValueError("dout must have the Q layers' shape")
    group = hq_ // hkv
    dqs = [np.zeros_like(x) for x in qs]
    dks = [np.zeros_like(x) for x in ks]
    dv = np.zeros_like(v)
    for b in range(b_):
        for h in range(hq_):
            hk = h // group
            s = sum(qs[l][b, h] @ ks[l][b, hk].T for l in range(n)) * float(scale)
            if causal:
                i = np.arange(nq)[:, None]
                j = np.arange(nk)[None, :]
                s = np.where(j > i, -np.inf, s)
            p, _, _ = softmax_two_pass(s)
            do = dout[b, h]
            dv[b, hk] += p.T @ do
            dp = do @ v[b, hk].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            for l in range(n):
                dqs[l][b, h] = float(scale) * (ds @ ks[l][b, hk])
                dks[l][b, hk] += float(scale) * (ds.T @ qs[l][b, h])
    return dqs, dks, dv
