"""Host-side accounting for the attention forward: flop and byte counts, rates.

Nothing here runs on the GPU or touches the attention arithmetic itself.
"""

from __future__ import annotations

# MI355X published dense peaks (bf16/fp16 MFMA, FP8 MFMA at twice the 16-bit
# rate, fp32 MFMA) and HBM3E bandwidth.
MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp8": 5033.2, "fp32": 157.3}
HBM_PEAK_GBS = 8000.0


def attention_tflops(batch: int, heads: int, seq: int, head_dim: int, seconds: float) -> float:
    """4*B*H*S^2*D / t in TFLOP/s: the formula of the Day 26 post's CUDA-event
    timing section (blog.ans20xx.com/posts/ai/day26); not halved for causal."""
    return 4.0 * batch * heads * seq * seq * head_dim / seconds / 1e12


def score_matrix_elems(batch: int, heads: int, n: int) -> int:
    """Elements of one materialised N x N score (or probability) matrix per
    batch and head, as counted in the kwkr.cn tutorial §1.2."""
    return batch * heads * n * n


def qkvo_bytes(batch: int, heads: int, n: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of Q, K, V and O together ([B,H,N,D] each)."""
    return 4 * batch * heads * n * head_dim * elem_bytes
