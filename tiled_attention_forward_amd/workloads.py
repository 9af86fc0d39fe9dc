"""Seeded synthetic workloads for the attention forward.

This module only describes shapes and draws random inputs.  It holds none of
the attention arithmetic, so both the HIP path's tests/bench and the fp64
oracle can take their inputs from it without sharing any method code.

Every tensor is drawn i.i.d. N(0, 1) in float32 from a seeded
``torch.Generator`` on the requested device and then rounded (round to
nearest even) to the workload's dtype, in the order Q, K, V, then the bias one
(b, head) slice at a time.  The same seed gives different values on the CPU
and on the GPU (different generators); a test that compares with the oracle
copies the exact device tensors to the host.

The shapes are those the pages discuss: the numeric-alignment check of the
Day 26 post (B=2, H=16, S=512, D=64 fp16), its benchmark report shape (B=2,
H=16, S=4096, D=64 bf16 causal), the S/P size example of the kwkr.cn tutorial
(B=8, H=32, N=2048, D=128), and the GQA 20 query / 4 KV head setup of the Block
Attention Residual post with a dense pre-softmax logit term.

Two more shapes exercise the key-split path, where row blocks alone leave most
of the 256 compute units idle; the pages give no such benchmark, so they are
synthetic choices: one decode step (Nq = 1) of the same 20/4-head, D = 128
setup for 8 sequences over a 32768-entry KV cache, and a long sequence with
only two heads (B = 1, H = 2, S = 16384, D = 64, 256 row blocks).  The
sliding-window shape is the benchmark report shape with each row limited to
its 1024 most recent keys.  The chain shape is the same GQA setup at the last
layer of a 4-layer Block Attention Residual block, whose logits sum the Q K^T
products of all four layers (in place of the dense logit tensor); its Q and K
are drawn layer by layer (Q_l, then K_l, oldest layer first), then V.  The
FP8 shape is the benchmark report shape with Q, K and V rounded to E4M3.  The
report shape with a dense logit term (D = 64) measures the bias path at the
head size where the softmax, not the matrix products, bounds the kernel.  The
decode shape also runs with an FP8 (E4M3) KV cache: half the bytes to stream.  The
causal variant of the tutorial's shape is the common training case at D = 128
(causal, no logit term), timed for the backward.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

_DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16,
           "fp8": torch.float8_e4m3fn}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    D: int
    dtype: str
    causal: bool
    bias: bool
    path: str = "fused"   # "fused": fa_forward; "split": fa_forward_split
    window: int = 0       # causal sliding window (fa_forward_window), 0 = none
    layers: int = 0       # Block Attention Residual chain length (fa_forward_chain), 0 = none

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def metric_flops(self) -> float:
        """4*B*H*Nq*Nk*D: the attention-TFLOPS numerator, not halved for causal."""
        return 4.0 * self.B * self.Hq * self.Nq * self.Nk * self.D

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the mask leaves visible (top-left causal,
        with the sliding window when there is one)."""
        if not self.causal:
            return self.B * self.Hq * self.Nq * self.Nk
        if self.window:
            per_head = sum(max(0, min(i, self.Nk - 1) - max(0, i - self.window + 1) + 1)
                           for i in range(self.Nq))
            return self.B * self.Hq * per_head
        per_head = 0
        # rows 0..Nq-1 see min(i+1, Nk) keys
        full = max(0, self.Nq - self.Nk)          # rows i >= Nk see all Nk keys
        tri_rows = self.Nq - full                 # rows 0..min(Nq,Nk)-1
        per_head = tri_rows * (tri_rows + 1) // 2 + full * self.Nk
        return self.B * self.Hq * per_head

    def useful_flops(self) -> float:
        """2 flops x D per visible (query, key) pair for each product: Q K^T
        (one per chain layer) and P V."""
        return 2.0 * self.D * (max(1, self.layers) + 1) * self.visible_pairs()

    def io_bytes(self) -> int:
        """Algorithmic HBM bytes: read Q, K, V (every layer's Q and K for a
        chain; the visible bias entries), write O and LSE."""
        esz = torch.tensor([], dtype=self.torch_dtype).element_size()
        oesz = 2 if self.dtype == "fp8" else esz   # FP8 inputs give a bf16 output
        nl = max(1, self.layers)
        qo = self.B * self.Hq * self.Nq * self.D * (nl * esz + oesz)
        kv = (nl + 1) * self.B * self.Hkv * self.Nk * self.D * esz
        lse = self.B * self.Hq * self.Nq * 4
        bias = self.visible_pairs() * esz if self.bias else 0
        return qo + kv + lse + bias


WORKLOADS = {
    w.name: w
    for w in [
        Workload("b1_h1_s256_d64_fp32", 1, 1, 1, 256, 256, 64, "fp32", False, False),
        Workload("b2_h16_s512_d64_fp16", 2, 16, 16, 512, 512, 64, "fp16", False, False),
        Workload("b2_h16_s512_d64_fp16_causal", 2, 16, 16, 512, 512, 64, "fp16", True, False),
        Workload("b2_h16_s4096_d64_bf16_causal", 2, 16, 16, 4096, 4096, 64, "bf16", True, False),
        Workload("b8_h32_s2048_d128_bf16", 8, 32, 32, 2048, 2048, 128, "bf16", False, False),
        Workload("b8_h32_s2048_d128_bf16_causal", 8, 32, 32, 2048, 2048, 128, "bf16", True, False),
        Workload("b1_hq20_hkv4_s8192_d128_bf16_causal_bias", 1, 20, 4, 8192, 8192, 128, "bf16",
                 True, True),
        Workload("b2_h16_s4096_d64_bf16_causal_bias", 2, 16, 16, 4096, 4096, 64, "bf16", True,
                 True),
        Workload("decode_b8_hq20_hkv4_nq1_nk32768_d128_bf16", 8, 20, 4, 1, 32768, 128, "bf16",
                 False, False, "split"),
        Workload("decode_b8_hq20_hkv4_nq1_nk32768_d128_fp8", 8, 20, 4, 1, 32768, 128, "fp8",
                 False, False, "split"),
        Workload("b1_h2_s16384_d64_bf16", 1, 2, 2, 16384, 16384, 64, "bf16", False, False,
                 "split"),
        Workload("b2_h16_s4096_d64_bf16_swa1024", 2, 16, 16, 4096, 4096, 64, "bf16", True, False,
                 window=1024),
        Workload("b2_h16_s4096_d64_fp8_causal", 2, 16, 16, 4096, 4096, 64, "fp8", True, False),
        Workload("b1_hq20_hkv4_s8192_d128_bf16_causal_chain4", 1, 20, 4, 8192, 8192, 128, "bf16",
                 True, False, layers=4),
    ]
}

HEADLINE = "b2_h16_s4096_d64_bf16_causal"


def custom(B, Hq, Hkv, Nq, Nk, D, dtype, causal, bias, name="custom") -> Workload:
    return Workload(name, B, Hq, Hkv, Nq, Nk, D, dtype, bool(causal), bool(bias))


def make_inputs(w: Workload, seed: int = 0, device="cpu"):
    """Draw (q, k, v, bias) for workload ``w``; bias is None when w.bias is False.

    q [B,Hq,Nq,D], k/v [B,Hkv,Nk,D], bias [B,Hq,Nq,Nk], all contiguous, dtype
    ``w.torch_dtype``, on ``device``.
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    dt = w.torch_dtype

    def draw(shape):
        return torch.randn(shape, generator=g, dtype=torch.float32, device=dev).to(dt)

    q = draw((w.B, w.Hq, w.Nq, w.D))
    k = draw((w.B, w.Hkv, w.Nk, w.D))
    v = draw((w.B, w.Hkv, w.Nk, w.D))
    bias = None
    if w.bias:
        bias = torch.empty((w.B, w.Hq, w.Nq, w.Nk), dtype=dt, device=dev)
        for b in range(w.B):
            for h in range(w.Hq):
                bias[b, h] = draw((w.Nq, w.Nk))
    return q, k, v, bias


def make_chain_inputs(w: Workload, n_layers: int, seed: int = 0, device="cpu"):
    """Draw (q_layers, k_layers, v) for an n_layers chain of workload ``w``:
    Q_0, K_0, Q_1, K_1, ... in that order from one seeded generator, then V,
    each as ``make_inputs`` draws Q, K and V."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    dt = w.torch_dtype

    def draw(shape):
        return torch.randn(shape, generator=g, dtype=torch.float32, device=dev).to(dt)

    qs, ks = [], []
    for _ in range(n_layers):
        qs.append(draw((w.B, w.Hq, w.Nq, w.D)))
        ks.append(draw((w.B, w.Hkv, w.Nk, w.D)))
    v = draw((w.B, w.Hkv, w.Nk, w.D))
    return qs, ks, v


def sample_rows(n: int, count: int, seed: int = 0, tile: int = 64):
    """Deterministic row sample: the first and last rows, rows on both sides of
    tile boundaries, and random rows, sorted and unique (all < n)."""
    picks = {0, 1, 2, n - 1, n - 2}
    for t in range(tile, n, tile * max(1, n // (tile * 8))):
        picks.update({t - 1, t})
    gen = torch.Generator().manual_seed(int(seed) + 12345)
    extra = torch.randint(0, n, (count,), generator=gen).tolist()
    picks.update(extra)
    return sorted(p for p in picks if 0 <= p < n)
