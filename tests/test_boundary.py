"""The C-ABI boundary on the CPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before anything is launched.

Nothing here launches a kernel: fa_check_args is pure host code, and
fa_forward returns its validation status before it reaches HIP.
"""

import ctypes
import math
import os
import re
import subprocess

import pytest

from tiled_attention_forward_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# Fake, well-separated, 256-byte-aligned device addresses (never dereferenced).
Q, K, V, BIAS, O, L = (0x100000000 * (i + 1) for i in range(6))
OK_ARGS = dict(q=Q, k=K, v=V, bias=None, o=O, lse=L, B=2, Hq=4, Hkv=2, Nq=100, Nk=77, D=64,
               scale=0.125, causal=1, dtype=binding.FA_DTYPE_BF16)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fa_\w+)\s*\(", text, re.M)))


def check(**over):
    a = dict(OK_ARGS, **over)
    return binding.fa_check_args(a["q"], a["k"], a["v"], a["bias"], a["o"], a["lse"], a["B"],
                                 a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["D"], a["scale"],
                                 a["causal"], a["dtype"])


def forward_status(**over):
    a = dict(OK_ARGS, **over)
    return binding.fa_forward(a["q"], a["k"], a["v"], a["bias"], a["o"], a["lse"], a["B"],
                              a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["D"], a["scale"],
                              a["causal"], a["dtype"], None)


def test_library_loads_and_exports_every_declared_symbol():
    lib = binding.load_library()
    names = declared_functions()
    assert set(names) == {"fa_check_args", "fa_forward", "fa_forward_split",
                          "fa_forward_split_noalloc", "fa_merge",
                          "fa_split_count", "fa_split_workspace_bytes", "fa_backward",
                          "fa_backward_workspace_bytes", "fa_forward_window",
                          "fa_backward_window", "fa_forward_chain", "fa_backward_chain",
                          "fa_status_string", "fa_version"}
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(fa_\w+)$", out, re.M))
    assert set(names) <= exported, set(names) - exported


def test_library_imports_no_allocator():
    """O(N) memory (xnwp.cn post, §2.2; kwkr.cn tutorial, §1.3): the library
    never materialises S or P, and more than that allocates nothing at all.  It
    imports no HIP (or C) allocation routine, so no call can hide an N x N
    buffer behind a pointer the caller never sees."""
    out = subprocess.run(["nm", "-D", "--undefined-only", binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    imported = set(re.findall(r"\bU\s+(\w+)", out))
    alloc = {n for n in imported
             if re.match(r"(hip\w*Malloc\w*|hip\w*Alloc\w*|hipMemCreate|hipMemPool\w*|"
                         r"malloc|calloc|realloc|_Zn[wa]m\w*)$", n)}
    assert not alloc, alloc
    assert "hipLaunchKernel" in imported  # the scan itself sees the HIP imports


def test_version_and_status_strings():
    assert binding.fa_version().startswith("fa ") and "gfx950" in binding.fa_version()
    for code in range(0, 13):
        s = binding.fa_status_string(code)
        assert s and s != "unknown status", code
    assert binding.fa_status_string(99) == "unknown status"


def test_valid_arguments_pass():
    assert check() == 0
    assert check(bias=BIAS) == 0
    assert check(D=128, dtype=binding.FA_DTYPE_FP32, causal=0) == 0
    assert check(dtype=binding.FA_DTYPE_FP16, Hq=20, Hkv=4) == 0
    assert check(scale=0.0) == 0 and check(scale=-1.0) == 0
    assert check(Nk=0) == 0   # rows with no key: O = 0, LSE = -inf
    assert check(Nk=0, k=None, v=None) == 0   # K and V are not read when Nk = 0


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_null_pointer(field):
    assert check(**{field: None}) == 1
    assert forward_status(**{field: None}) == 1


def test_empty_problem_needs_no_pointers_and_launches_nothing():
    for over in (dict(B=0), dict(Hq=0, Hkv=0), dict(Nq=0)):
        assert check(q=None, k=None, v=None, o=None, lse=None, **over) == 0
        assert forward_status(q=None, k=None, v=None, o=None, lse=None, **over) == 0


@pytest.mark.parametrize("over,code", [
    (dict(B=-1), 2), (dict(Nq=-5), 2), (dict(Nk=-1), 2), (dict(Hkv=0), 2),
    (dict(Hq=5, Hkv=2), 3), (dict(Hq=4, Hkv=3), 3),
    (dict(D=72), 4), (dict(D=112), 4), (dict(D=32), 4), (dict(D=512), 4), (dict(D=0), 4),
    (dict(D=256, dtype=binding.FA_DTYPE_FP32), 4),
    (dict(D=96, dtype=binding.FA_DTYPE_FP32), 4),
    (dict(dtype=4), 5), (dict(dtype=-1), 5),
    (dict(dtype=binding.FA_DTYPE_FP8_E4M3, bias=BIAS), 5),   # FP8 takes no logit term
    (dict(dtype=binding.FA_DTYPE_FP8_E4M3, D=80), 4),
    (dict(scale=math.nan), 6), (dict(scale=math.inf), 6), (dict(scale=-math.inf), 6),
    (dict(q=Q + 8), 7), (dict(k=K + 4), 7), (dict(v=V + 2), 7), (dict(o=O + 8), 7),
    (dict(bias=BIAS + 8), 7), (dict(lse=L + 2), 7),
    (dict(o=Q), 8), (dict(o=K + 64), 8), (dict(lse=V), 8), (dict(lse=O + 256), 8),
    (dict(bias=BIAS, o=BIAS + 1024), 8), (dict(lse=Q + 1024), 8),
    (dict(Nq=1 << 30), 9), (dict(Nk=1 << 30), 9), (dict(B=1 << 22, Hq=1 << 10, Hkv=1), 9),
])
def test_rejections(over, code):
    assert check(**over) == code
    assert forward_status(**over) == code  # returned before any launch


def test_head_dim_pitfall_is_an_error_not_a_truncation():
    """A 96-wide head with a 64-wide kernel block silently drops columns, and an
    80-wide one reads past the row, in the kernel of the xnwp.cn post (§5.1,
    §6.4); here 80 and 96 run in a 128-wide tile (bf16/fp16) and every other
    unsupported D is refused."""
    for d in (1, 16, 63, 65, 72, 88, 112, 127, 129, 192):
        assert check(D=d) == 4
    for d in (64, 80, 96, 128, 256):
        assert check(D=d) == 0
        assert check(D=d, dtype=binding.FA_DTYPE_FP16) == 0
    assert check(D=80, dtype=binding.FA_DTYPE_FP32) == 4
    assert check(D=96, dtype=binding.FA_DTYPE_FP32) == 4


def test_forward_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.forward(q, q, q)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setenv("FA_LIBRARY", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library()
    monkeypatch.setattr(binding, "_lib", None)


# ---------------------------------------------------------------------------
# key-split path and merge: validation only (no launch on the CPU)
# ---------------------------------------------------------------------------

WS = 0x100000000 * 8   # fake workspace address, far from the tensors above


def split_status(num_splits=4, workspace=WS, workspace_bytes=1 << 40, **over):
    a = dict(OK_ARGS, **over)
    return binding.fa_forward_split(a["q"], a["k"], a["v"], a["bias"], a["o"], a["lse"], a["B"],
                                    a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["D"], a["scale"],
                                    a["causal"], a["dtype"], num_splits, workspace,
                                    workspace_bytes, None)


def test_split_workspace_bytes_layout():
    # partial O fp32 [S][B*Hq*Nq][D], then partial LSE fp32 [S][B*Hq*Nq] from a 256-byte boundary
    rows = 2 * 4 * 100
    for s in (1, 3, 32):
        o_bytes = s * rows * 64 * 4
        o_pad = (o_bytes + 255) // 256 * 256
        assert binding.fa_split_workspace_bytes(2, 4, 100, 64, s) == o_pad + s * rows * 4
    assert binding.fa_split_workspace_bytes(1, 1, 1, 128, 1) == 512 + 4
    assert binding.fa_split_workspace_bytes(1, 1, 1, 256, 1) == 1024 + 4   # head size 256
    assert binding.fa_split_workspace_bytes(0, 4, 100, 64, 2) == 0
    for bad, code in ((dict(num_splits=0), 2), (dict(num_splits=1025), 2), (dict(D=72), 4),
                      (dict(B=-1), 2)):
        a = {**dict(B=2, Hq=4, Nq=100, D=64, num_splits=2), **bad}
        with pytest.raises(binding.FaError) as e:
            binding.fa_split_workspace_bytes(a["B"], a["Hq"], a["Nq"], a["D"], a["num_splits"])
        assert e.value.status == code


def test_split_count_heuristic():
    # decode step: 8 batches x 4 KV heads, 5 query heads per group, Nq = 1, 32768 keys:
    # 32 row blocks -> 16 splits of 32 tiles each (512 workgroups)
    assert binding.fa_split_count(8, 20, 4, 1, 32768, 128) == 16
    # two heads of 16384 rows: 256 row blocks -> 2 splits
    assert binding.fa_split_count(1, 2, 2, 16384, 16384, 64) == 2
    # enough row blocks already: 2 x 16 heads x 32 blocks of 128 rows
    assert binding.fa_split_count(2, 16, 16, 4096, 4096, 64) == 1
    # few keys: at least 4 tiles per split
    assert binding.fa_split_count(1, 1, 1, 1, 64 * 8, 64) == 2
    assert binding.fa_split_count(1, 1, 1, 1, 10, 64) == 1
    assert binding.fa_split_count(1, 1, 1, 1, 1 << 24, 64) == 512
    assert binding.fa_split_count(0, 1, 1, 1, 100, 64) == 1
    with pytest.raises(binding.FaError):
        binding.fa_split_count(1, 5, 2, 1, 100, 64)


def test_split_rejections_before_launch():
    need = binding.fa_split_workspace_bytes(2, 4, 100, 64, 4)
    assert split_status(num_splits=0) == 2
    assert split_status(num_splits=1025) == 2
    assert split_status(workspace=None) == 11
    assert split_status(workspace=WS + 8) == 11
    assert split_status(workspace_bytes=need - 1) == 11
    assert split_status(workspace=O) == 8            # workspace over the output
    assert split_status(workspace=Q - 256) == 8      # runs into q
    assert split_status(D=72) == 4 and split_status(q=None) == 1   # the common checks first
    assert split_status(D=256, workspace=None) == 11   # 256 passes the head check
    # packed rows of one KV head: (Hq/Hkv) * Nq * D * 2 bytes must stay below 2^31
    assert split_status(Hq=64, Hkv=1, Nq=1 << 18, B=1, workspace_bytes=1 << 62) == 9
    # empty problem: nothing launched, no workspace needed
    assert split_status(B=0, workspace=None, workspace_bytes=0) == 0


def noalloc_status(num_splits=4, **over):
    a = dict(OK_ARGS, **over)
    return binding.fa_forward_split_noalloc(a["q"], a["k"], a["v"], a["bias"], a["o"], a["lse"],
                                            a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["D"],
                                            a["scale"], a["causal"], a["dtype"], num_splits, None)


def test_split_noalloc_rejections_before_launch():
    """The allocation-free key split checks what fa_forward_split checks (except
    the workspace), and refuses partials larger than its scratch array before
    touching the GPU."""
    assert noalloc_status(num_splits=0) == 2 and noalloc_status(num_splits=1025) == 2
    assert noalloc_status(D=72) == 4 and noalloc_status(D=256, o=Q) == 8   # 256 passes
    assert noalloc_status(q=None) == 1 and noalloc_status(o=O + 8) == 7
    assert noalloc_status(o=Q) == 8
    # FP8 is accepted (the decode step over an FP8 KV cache): the scratch
    # limit is what stops this call, not the type; FP8 with a bias is refused
    fp8 = binding.FA_DTYPE_FP8_E4M3
    assert noalloc_status(dtype=fp8, bias=BIAS) == 5 and noalloc_status(dtype=fp8, D=80) == 4
    # just over the limit: rows * D * 4 * splits (plus the LSE part) > 32 MiB
    limit = binding.FA_SPLIT_SCRATCH_BYTES
    rows = 2 * 4 * 100
    over = limit // (rows * 64 * 4) + 1
    assert binding.fa_split_workspace_bytes(2, 4, 100, 64, over) > limit
    assert noalloc_status(num_splits=over) == binding.FA_ERR_SCRATCH_LIMIT
    assert noalloc_status(num_splits=over, dtype=fp8) == binding.FA_ERR_SCRATCH_LIMIT
    assert noalloc_status(B=64, Hq=32, Hkv=32, Nq=4096, num_splits=1) == 12
    assert "scratch" in binding.fa_status_string(12)
    # empty problem: nothing launched
    assert noalloc_status(B=0, q=None, o=None, lse=None) == 0


def merge_status(part_o=WS, part_lse=WS + (1 << 30), num_parts=3, rows=10, D=64, o=O, lse=L,
                 dtype=binding.FA_DTYPE_BF16):
    return binding.fa_merge(part_o, part_lse, num_parts, rows, D, o, lse, dtype, None)


def test_merge_rejections_before_launch():
    assert merge_status(rows=0) == 0 and merge_status(rows=0, o=None, lse=None) == 0
    assert merge_status(dtype=7) == 5
    assert merge_status(num_parts=-1) == 2 and merge_status(rows=-1) == 2
    assert merge_status(D=6) == 4 and merge_status(D=0) == 4 and merge_status(D=65540) == 4
    assert merge_status(o=None) == 1 and merge_status(part_lse=None) == 1
    assert merge_status(part_o=WS + 4) == 7 and merge_status(lse=L + 2) == 7
    assert merge_status(o=WS + 64) == 8 and merge_status(lse=WS + (1 << 30) + 8) == 8
    assert merge_status(num_parts=1 << 31) == 9


# ---------------------------------------------------------------------------
# backward: validation only (no launch on the CPU)
# ---------------------------------------------------------------------------

GO, DQ, DK, DV = (0x100000000 * (i + 10) for i in range(4))


def bwd_status(workspace=WS, workspace_bytes=1 << 40, dout=GO, dq=DQ, dk=DK, dv=DV, **over):
    a = dict(OK_ARGS, **over)
    return binding.fa_backward(a["q"], a["k"], a["v"], a["bias"], a["o"], a["lse"], dout, dq, dk,
                               dv, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["D"],
                               a["scale"], a["causal"], a["dtype"], workspace, workspace_bytes,
                               None)


def test_backward_workspace_bytes():
    rows = 2 * 4 * 100
    assert binding.fa_backward_workspace_bytes(2, 4, 100) == ((rows + 63) // 64 * 64 + rows) * 4
    assert binding.fa_backward_workspace_bytes(0, 4, 100) == 0
    with pytest.raises(binding.FaError):
        binding.fa_backward_workspace_bytes(-1, 4, 100)


def test_backward_rejections_before_launch():
    assert bwd_status(dtype=binding.FA_DTYPE_FP8_E4M3) == 5   # no FP8 backward
    # fp32: head sizes 64 and 128 (as its forward); those pass to the workspace check
    assert bwd_status(dtype=binding.FA_DTYPE_FP32, D=96) == 4
    assert bwd_status(dtype=binding.FA_DTYPE_FP32, D=256) == 4
    assert bwd_status(dtype=binding.FA_DTYPE_FP32, workspace=None) == 11
    assert bwd_status(dtype=binding.FA_DTYPE_FP32, D=128, workspace=None) == 11
    assert bwd_status(D=72) == 4 and bwd_status(q=None) == 1   # the forward's checks first
    assert bwd_status(D=256, bias=BIAS) == 4                   # D = 256 takes no logit term
    assert bwd_status(D=256, workspace=None) == 11             # D = 256 passes the head check
    # 80 and 96 pass the head-size check (the workspace check after it fails)
    assert bwd_status(D=96, workspace=None) == 11 and bwd_status(D=80, workspace=None) == 11
    assert bwd_status(dout=None) == 1 and bwd_status(dq=None) == 1
    assert bwd_status(dk=None) == 1 and bwd_status(dv=None) == 1
    assert bwd_status(dq=DQ + 8) == 7 and bwd_status(dout=GO + 4) == 7
    need = binding.fa_backward_workspace_bytes(2, 4, 100)
    assert bwd_status(workspace=None) == 11 and bwd_status(workspace_bytes=need - 4) == 11
    assert bwd_status(workspace=WS + 8) == 11
    assert bwd_status(dq=Q) == 8 and bwd_status(dk=V + 64) == 8 and bwd_status(dv=DK) == 8
    assert bwd_status(workspace=GO) == 8
    # no rows and no keys: nothing to do, nothing needed
    assert bwd_status(B=0, q=None, k=None, v=None, o=None, lse=None, dout=None, dq=None, dk=None,
                      dv=None, workspace=None) == 0
    # no query rows but keys present: dk and dv are still written (zeros), so needed
    assert bwd_status(Nq=0, dk=None) == 1


def test_window_rejections_before_launch():
    lib = binding.load_library()
    a = dict(OK_ARGS)
    args = (a["q"], a["k"], a["v"], a["bias"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
            a["Nq"], a["Nk"], a["D"], a["scale"])
    assert lib.fa_forward_window(*args, 0, a["dtype"], None) == 2
    assert lib.fa_forward_window(*args, -3, a["dtype"], None) == 2
    assert lib.fa_forward_window(*args, 1 << 30, a["dtype"], None) == 9
    assert lib.fa_forward_window(*args[:11], 72, a["scale"], 16, a["dtype"], None) == 4
    # 256 passes the head check (the overlap check after it fails)
    args_o = (a["q"], a["k"], a["v"], a["bias"], a["q"]) + args[5:11]
    assert lib.fa_forward_window(*args_o, 256, a["scale"], 16, a["dtype"], None) == 8
    bargs = (a["q"], a["k"], a["v"], None, a["o"], a["lse"], GO, DQ, DK, DV, a["B"], a["Hq"],
             a["Hkv"], a["Nq"], a["Nk"], a["D"], a["scale"])
    assert lib.fa_backward_window(*bargs, 0, a["dtype"], WS, 1 << 40, None) == 2
    assert lib.fa_backward_window(*bargs, 8, binding.FA_DTYPE_FP8_E4M3, WS, 1 << 40, None) == 5
    assert lib.fa_backward_window(*bargs, 8, binding.FA_DTYPE_FP32, None, 0, None) == 11
    assert lib.fa_backward_window(*bargs[:15], 256, a["scale"], 8, a["dtype"], None, 0,
                                  None) == 11   # 256 passes the head check


def test_chain_rejections_before_launch():
    Q0, K0 = 0x1000000000, 0x1100000000
    a = dict(OK_ARGS)

    def chain(qs, ks, n=None, **over):
        b = dict(a, **over)
        return binding.fa_forward_chain(qs, ks, b["v"], b["o"], b["lse"], b["B"], b["Hq"],
                                        b["Hkv"], b["Nq"], b["Nk"], b["D"], b["scale"],
                                        b["causal"], b["dtype"], None) if n is None else \
            binding.load_library().fa_forward_chain(None, None, n, b["v"], b["o"], b["lse"],
                                                    b["B"], b["Hq"], b["Hkv"], b["Nq"], b["Nk"],
                                                    b["D"], b["scale"], b["causal"], b["dtype"],
                                                    None)
    assert chain(None, None, n=2) == 1                        # no layer arrays
    assert chain([], []) == 2                                 # no layer
    assert chain([Q0, Q] * 2 + [Q], [K0, K] * 2 + [K]) == 2   # five layers
    assert chain([Q0, Q], [K0, K], dtype=binding.FA_DTYPE_FP32) == 5
    assert chain([Q0, Q], [K0, K], D=72) == 4 and chain([Q0, Q], [K0, K], D=256) == 4
    assert chain([Q0, Q], [K0, K], D=96, o=Q0) == 8           # 80 and 96 pass the head check
    assert chain([Q0, Q], [K0, K], Hq=3) == 3
    assert chain([None, Q], [K0, K]) == 1                     # a layer's Q missing
    assert chain([Q0, Q], [K0 + 8, K]) == 7                   # a layer's K misaligned
    assert chain([Q0, Q], [K0, K], o=Q0) == 8                 # output over an earlier Q
    assert chain([Q0, Q], [K0, K], B=0) == 0                  # empty: nothing launched


def test_chain_backward_rejections_before_launch():
    Q0, K0, DQ0, DK0 = 0x1000000000, 0x1100000000, 0x1200000000, 0x1300000000
    a = dict(OK_ARGS)

    def bchain(qs, ks, dqs, dks, workspace=WS, dv=DV, dout=GO, **over):
        b = dict(a, **over)
        return binding.fa_backward_chain(qs, ks, b["v"], b["o"], b["lse"], dout, dqs, dks, dv,
                                         b["B"], b["Hq"], b["Hkv"], b["Nq"], b["Nk"], b["D"],
                                         b["scale"], b["causal"], b["dtype"], workspace, 1 << 40,
                                         None)
    lib = binding.load_library()
    assert lib.fa_backward_chain(None, None, 2, V, O, L, GO, None, None, DV, 2, 4, 2, 100, 77,
                                 64, 0.125, 1, a["dtype"], WS, 1 << 40, None) == 1
    ok = ([Q0, Q], [K0, K], [DQ0, DQ], [DK0, DK])
    assert bchain([], [], [], []) == 2                                     # no layer
    assert bchain([Q0, Q] * 2 + [Q], [K0, K] * 2 + [K], [DQ0, DQ] * 2 + [DQ],
                  [DK0, DK] * 2 + [DK]) == 2                               # five layers
    assert bchain(*ok, dtype=binding.FA_DTYPE_FP32) == 5                   # 16-bit only
    assert bchain(*ok, D=72) == 4 and bchain(*ok, D=256) == 4              # no 256 chain
    assert bchain(*ok, D=96, workspace=None) == 11                         # 80, 96 pass
    assert bchain(*ok, Hq=3) == 3
    assert bchain([None, Q], [K0, K], [DQ0, DQ], [DK0, DK]) == 1           # a layer's Q missing
    assert bchain([Q0, Q], [K0, K], [None, DQ], [DK0, DK]) == 1            # a layer's dQ missing
    assert bchain([Q0, Q], [K0 + 8, K], [DQ0, DQ], [DK0, DK]) == 7         # a layer's K misaligned
    assert bchain(*ok, workspace=None) == 11
    assert bchain([Q0, Q], [K0, K], [Q, DQ], [DK0, DK]) == 8               # dQ_0 over the last Q
    assert bchain([Q0, Q], [K0, K], [DQ0, DQ], [DK0, K0]) == 8             # dK_1 over K_0
    assert bchain([Q0, Q], [K0, K], [DQ0, DQ0], [DK0, DK]) == 8            # two dQ on one buffer
    assert bchain(*ok, dv=DK0) == 8                                        # dV over dK_0
    assert bchain(*ok, B=0) == 0                                           # empty: nothing launched


def test_fp8_rejections_before_launch():
    fp8 = binding.FA_DTYPE_FP8_E4M3
    assert check(dtype=fp8) == 0 and check(dtype=fp8, D=128) == 0
    # the bf16 output is twice the size of the FP8 q: [O, O + 2*|q|) must be clear
    nq_fp8 = 2 * 4 * 100 * 64
    assert check(dtype=fp8, o=O, lse=O + nq_fp8 + 256) == 8
    assert check(dtype=fp8, o=O, lse=O + 2 * nq_fp8) == 0
    lib = binding.load_library()
    a = dict(OK_ARGS)
    args = (a["q"], a["k"], a["v"], None, a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
            a["Nq"], a["Nk"], a["D"], a["scale"])
    # the window takes FP8 (no bias): past the type check, an overlap is what fails
    o_over = args[:4] + (a["q"],) + args[5:]
    assert lib.fa_forward_window(*o_over, 16, fp8, None) == 8
    bias_w = args[:3] + (BIAS,) + args[4:]
    assert lib.fa_forward_window(*bias_w, 16, fp8, None) == 5
    # the key split takes FP8 (no bias): past the type check, a missing
    # workspace is what fails
    assert lib.fa_forward_split(*args, 1, fp8, 2, None, 0, None) == 11
    bias_args = args[:3] + (BIAS,) + args[4:]
    assert lib.fa_forward_split(*bias_args, 1, fp8, 2, WS, 1 << 40, None) == 5
    bargs = (a["q"], a["k"], a["v"], None, a["o"], a["lse"], GO, DQ, DK, DV, a["B"], a["Hq"],
             a["Hkv"], a["Nq"], a["Nk"], a["D"], a["scale"])
    assert lib.fa_backward(*bargs, 1, fp8, WS, 1 << 40, None) == 5
    assert binding.fa_merge(WS, WS + 4096, 2, 10, 64, O, L, fp8, None) == 5
