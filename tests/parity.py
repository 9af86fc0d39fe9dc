"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on
the same input bits, compare against the stated tolerances.

Tolerances (absolute, on O upcast to float64, and on LSE):
  bf16 / fp16 inputs: max |O - O_ref| <= 1e-2 and mean |O - O_ref| <= 1e-3
  fp32 inputs:        max |O - O_ref| <= 1e-5
  LSE (all dtypes):   max |LSE - LSE_ref| <= 1e-3
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import attention_forward, attention_head_rows
from tiled_attention_forward_amd import binding

O_TOL = {"bf16": (1e-2, 1e-3), "fp16": (1e-2, 1e-3), "fp32": (1e-5, 1e-5)}
LSE_TOL = 1e-3


def f64(t: torch.Tensor) -> np.ndarray:
    # (to the host first: the host converts every dtype, FP8 included, exactly)
    return t.detach().cpu().to(torch.float32).numpy().astype(np.float64)


def errors(o, lse, o_ref, lse_ref):
    o, lse = np.asarray(o, np.float64), np.asarray(lse, np.float64)
    assert np.isfinite(o).all(), "non-finite output"
    d = np.abs(o - o_ref)
    both = np.isinf(lse) & np.isinf(lse_ref) & (np.sign(lse) == np.sign(lse_ref))
    dl = np.where(both, 0.0, np.abs(lse - lse_ref))
    return {"max_abs": float(d.max(initial=0.0)), "mean_abs": float(d.mean()) if d.size else 0.0,
            "lse_max": float(dl.max(initial=0.0)), "n": int(d.size)}


def assert_within(stats, dtype, what=""):
    mx, mean = O_TOL[dtype]
    assert np.isfinite(stats["lse_max"]), f"{what}: LSE mismatch in infinities {stats}"
    assert stats["max_abs"] <= mx, f"{what}: max abs {stats}"
    assert stats["mean_abs"] <= mean, f"{what}: mean abs {stats}"
    assert stats["lse_max"] <= LSE_TOL, f"{what}: LSE {stats}"


def run_gpu(q, k, v, bias, scale, causal):
    o, lse = binding.forward(q, k, v, bias, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def run_split(num_splits=None):
    """fa_forward_split with a given split count (None: the library's suggestion)."""
    def run(q, k, v, bias, scale, causal):
        o, lse = binding.forward_split(q, k, v, bias, causal=causal, scale=scale,
                                       num_splits=num_splits)
        torch.cuda.synchronize()
        return o, lse
    return run


def output_spacing_check(o, o_ref, stats, dtype, what=""):
    """For shapes beyond the pages' workloads: where an element of a 16-bit
    output misses the 1e-2 max bar, the miss must come from the output's own
    spacing.  In [2, 4) consecutive bf16 values are 2^-6 = 0.0156 apart, so
    an fp32 result off by a few thousandths before its final rounding can
    land on the far neighbour of the exact value, 0.0104 or more away.  Each
    such element must be at most one output ulp from the exact value rounded
    to the output type (for fp16 below |O| = 8 that is tighter than the bar
    itself) and have |O_ref| >= 1; the mean and LSE bars stay as stated.
    Returns the number of elements held to this rule instead."""
    mx, mean = O_TOL[dtype]
    assert np.isfinite(stats["lse_max"]), f"{what}: LSE mismatch in infinities {stats}"
    assert stats["mean_abs"] <= mean, f"{what}: mean abs {stats}"
    assert stats["lse_max"] <= LSE_TOL, f"{what}: LSE {stats}"
    og = np.asarray(o, np.float64)
    err = np.abs(og - o_ref)
    over = err > mx
    if not over.any():
        return 0
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    mant = {"bf16": 7, "fp16": 10}[dtype]
    ref = o_ref[over]
    assert np.all(np.abs(ref) >= 1.0), f"{what}: max bar missed below |O| = 1 {stats}"
    rne = torch.from_numpy(ref).to(tdt).to(torch.float64).numpy()
    ulp = 2.0 ** (np.floor(np.log2(np.abs(rne))) - mant)
    assert np.all(np.abs(og[over] - rne) <= ulp), f"{what}: more than one output ulp {stats}"
    return int(over.sum())


def full_check(q, k, v, bias, scale, causal, dtype, what="", run=None, spacing=False):
    """Whole-tensor comparison with the oracle (small problems).  ``run`` is the
    GPU entry point to test (default: fa_forward through ``run_gpu``).  With
    ``spacing`` (shapes beyond the pages' workloads, 16-bit outputs), elements
    that miss the max bar are held to ``output_spacing_check`` instead."""
    o, lse = (run or run_gpu)(q, k, v, bias, scale, causal)
    o_ref, lse_ref = attention_forward(f64(q), f64(k), f64(v),
                                       None if bias is None else f64(bias),
                                       scale=scale, causal=causal)
    st = errors(f64(o), lse.cpu().numpy(), o_ref, lse_ref)
    if spacing and dtype in ("bf16", "fp16") and st["max_abs"] > O_TOL[dtype][0]:
        n = output_spacing_check(f64(o), o_ref, st, dtype, what)
        print(f"{what}: {n} element(s) past the max bar, each within one output ulp", flush=True)
    else:
        assert_within(st, dtype, what)
    return st, o, lse


def sampled_check(q, k, v, bias, scale, causal, dtype, heads, rows, o, lse, what=""):
    """Compare selected (b, hq, rows) of a full-size GPU result with the oracle,
    which evaluates exactly those rows (each row depends only on its own query,
    its bias row and the whole K/V of its KV head)."""
    B, Hq, Nq, D = q.shape
    grp = Hq // k.shape[1]
    rows_t = torch.as_tensor(rows, device=q.device)
    worst = {"max_abs": 0.0, "mean_abs": 0.0, "lse_max": 0.0, "n": 0}
    sum_abs = 0.0
    for b, h in heads:
        hk = h // grp
        o_ref, l_ref = attention_head_rows(
            f64(q[b, h].index_select(0, rows_t)), f64(k[b, hk]), f64(v[b, hk]), rows=rows,
            scale=scale, causal=causal,
            bias_rows=None if bias is None else f64(bias[b, h].index_select(0, rows_t)))
        st = errors(f64(o[b, h].index_select(0, rows_t)),
                    lse[b, h].index_select(0, rows_t).cpu().numpy(), o_ref, l_ref)
        worst["max_abs"] = max(worst["max_abs"], st["max_abs"])
        worst["lse_max"] = max(worst["lse_max"], st["lse_max"])
        sum_abs += st["mean_abs"] * st["n"]
        worst["n"] += st["n"]
    worst["mean_abs"] = sum_abs / max(worst["n"], 1)
    assert_within(worst, dtype, what)
    return worst


def rounding_bound_check(q, k, v, bias, scale, causal, dtype, o, lse, what=""):
    """For logit spreads wider than the pages' workloads, check the bound the
    arithmetic gives instead of the fixed bar.  With u the unit roundoff of the
    input type (2^-8 bf16, 2^-11 fp16), each probability is rounded before P.V
    (relative error <= u per term) and O is rounded once (<= u relative), so
    elementwise |dO| <= u * (P.|V|) + u * |O| + 1e-4, the last term covering fp32
    accumulation and the exp2 approximation.  The mean of |dO| keeps the
    stated mean bar (1e-3), and LSE its 1e-3 bar."""
    u = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}[dtype]
    bq, bk, bv = f64(q), f64(k), f64(v)
    bb = None if bias is None else f64(bias)
    o_ref, l_ref = attention_forward(bq, bk, bv, bb, scale=scale, causal=causal)
    o_abs, _ = attention_forward(bq, bk, np.abs(bv), bb, scale=scale, causal=causal)
    bound = u * o_abs + u * np.abs(o_ref) + 1e-4
    err = np.abs(f64(o) - o_ref)
    assert np.all(err <= bound), f"{what}: worst err/bound {float((err / bound).max())}"
    assert err.mean() <= O_TOL[dtype][1], f"{what}: mean abs {float(err.mean())}"
    assert np.abs(lse.cpu().numpy() - l_ref).max() <= LSE_TOL, f"{what}: LSE"


def fp8_bound_check(q, k, v, scale, causal, o, lse, what="", window=None):
    """FP8 (E4M3) inputs: the kernel rounds each probability to E4M3 before P.V,
    as p' = p * 2^7 relative to its running max reference (p' in (0, 2^8]):
    relative error <= 2^-4 for normal values, absolute <= 2^-10 below E4M3's
    smallest normal 2^-6, in units where the row's sum is >= 2^7.  O is rounded
    once to bf16.  So elementwise
        |dO_i| <= 2^-4 (P.|V|)_i + 2^-17 sum_{visible j} |v_j| + 2^-9 |O_i| + 1e-4,
    with the sum over row i's visible keys (the oracle with Q = 0 and |V| gives
    its mean).  The inputs are decoded exactly, so the scores carry no input
    rounding; LSE is formed from the unrounded p and keeps its 1e-3 bar.
    Returns (max |dO|, mean |dO|, worst err / bound)."""
    bq, bk, bv = f64(q), f64(k), f64(v)
    o_ref, l_ref = attention_forward(bq, bk, bv, None, scale=scale, causal=causal, window=window)
    o_abs, _ = attention_forward(bq, bk, np.abs(bv), None, scale=scale, causal=causal,
                                 window=window)
    m_abs, _ = attention_forward(np.zeros_like(bq), bk, np.abs(bv), None, scale=scale,
                                 causal=causal, window=window)
    nq, nk = bq.shape[2], bk.shape[2]
    count = (np.minimum(np.arange(nq) + 1, nk) if causal else np.full(nq, nk)).astype(np.float64)
    if window is not None:
        count = np.minimum(count, float(window))
    bound = (2.0 ** -4 * o_abs + 2.0 ** -17 * m_abs * count[None, None, :, None]
             + 2.0 ** -9 * np.abs(o_ref) + 1e-4)
    err = np.abs(f64(o) - o_ref)
    ratio = float((err / bound).max(initial=0.0))
    assert np.all(err <= bound), f"{what}: worst err/bound {ratio}"
    dl = np.abs(lse.cpu().numpy().astype(np.float64) - l_ref)
    assert dl.max(initial=0.0) <= LSE_TOL, f"{what}: LSE {dl.max()}"
    return float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0, ratio
