"""Host logic checked against numbers the pages print (fixtures in tests/golden/)."""

import os

import pytest

from tiled_attention_forward_amd import metrics
from tiled_attention_forward_amd.workloads import WORKLOADS, Workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def test_day26_report_tflops_formula():
    """Each printed TFLOPS equals 4*B*H*S^2*D over the printed median time (within print rounding)."""
    rows = list(_rows("day26_h100_report.txt"))
    assert len(rows) == 4
    for backend, median_ms, _p90, _mem, tflops in rows:
        got = metrics.attention_tflops(2, 16, 4096, 64, float(median_ms) / 1e3)
        assert got == pytest.approx(float(tflops), rel=5e-3), backend


def test_headline_workload_metric_flops():
    w = WORKLOADS["b2_h16_s4096_d64_bf16_causal"]
    assert w.metric_flops() == 4 * 2 * 16 * 4096 * 4096 * 64
    # the 11.9 ms flash-attn v2 line of the report
    assert w.metric_flops() / 11.9e-3 / 1e12 == pytest.approx(11.57, rel=5e-3)
    # causal top-left: S(S+1)/2 visible pairs per head
    assert w.visible_pairs() == 2 * 16 * 4096 * 4097 // 2


@pytest.mark.parametrize("row", list(_rows("materialised_sizes.txt")), ids=lambda r: r[0])
def test_materialised_sizes(row):
    name, B, H, N, D, esz, qty, printed = row[:8]
    B, H, N, D, esz, printed = int(B), int(H), int(N), int(D), int(esz), float(printed)
    if qty == "elems_per_tensor":
        got = B * H * N * D
    elif qty == "bytes_qkvo":
        got = metrics.qkvo_bytes(B, H, N, D, esz)
    elif qty == "elems_S":
        got = metrics.score_matrix_elems(B, H, N)
    elif qty == "bytes_S":
        got = metrics.score_matrix_elems(B, H, N) * esz
    elif qty == "bytes_SP":
        got = 2 * metrics.score_matrix_elems(B, H, N) * esz
    elif qty == "tile5_bytes":
        got = 5 * N * D * esz  # Q, K, V, S, O tiles of 64 x 64
    else:
        raise AssertionError(qty)
    # the pages round to two or three significant figures and mix 1e9 with 2^30
    assert got == pytest.approx(printed, rel=0.08), (name, got, printed)


def test_wide_head_workload_is_the_size_example():
    """The B8 H32 S2048 D128 workload is the shape whose S and P need about 4.2 GB (kwkr §1.2)."""
    w = WORKLOADS["b8_h32_s2048_d128_bf16"]
    assert 2 * metrics.score_matrix_elems(w.B, w.Hq, w.Nq) * 2 == pytest.approx(4.2e9, rel=0.03)


def test_io_bytes_counts():
    w = Workload("t", 1, 2, 1, 10, 12, 64, "bf16", True, True)
    # q,o: 2*1*2*10*64*2; k,v: 2*1*1*12*64*2; lse: 1*2*10*4; bias: visible pairs * 2
    vis = 2 * (10 * 11 // 2)
    assert w.visible_pairs() == vis
    assert w.io_bytes() == 2 * 2 * 10 * 64 * 2 + 2 * 12 * 64 * 2 + 2 * 10 * 4 + vis * 2
