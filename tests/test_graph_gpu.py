"""HIP graph capture of the entry points (torch.cuda.CUDAGraph over the C ABI).

The library allocates nothing, never synchronises and issues no memset, so its
launches can be captured and replayed: a serving or training loop can put the
attention step in a graph to drop the per-launch host cost.  Each test
captures one entry point on fixed buffers, then replays it several times with
new values copied into the inputs, eager work and synchronisations between
the replays, and compares every replay bit for bit with an eager call on the
same inputs (the kernels are deterministic).
"""

import pytest
import torch

from tiled_attention_forward_amd import binding
from tiled_attention_forward_amd.workloads import custom, make_inputs

pytestmark = pytest.mark.gpu


def _fresh(w, seed, dev):
    return [t.to(dev) for t in make_inputs(w, seed=seed) if t is not None]


def test_forward_replays_match_eager(gpu_device):
    w = custom(2, 8, 2, 700, 700, 64, "bf16", True, True)
    q, k, v, b = _fresh(w, 80, gpu_device)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.Nq, device=gpu_device)
    binding.forward(q, k, v, b, causal=True, scale=w.scale, out=o, lse=lse)  # warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.forward(q, k, v, b, causal=True, scale=w.scale, out=o, lse=lse)
    for rep in range(3):
        for dst, src in zip((q, k, v, b), _fresh(w, 81 + rep, gpu_device)):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        o_ref, l_ref = binding.forward(q, k, v, b, causal=True, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"replay {rep}"


def test_split_forward_replays_match_eager(gpu_device):
    w = custom(2, 8, 2, 1, 3000, 128, "bf16", False, False)
    q, k, v = _fresh(w, 90, gpu_device)
    splits = 6
    ws = torch.empty(binding.fa_split_workspace_bytes(w.B, w.Hq, w.Nq, w.D, splits),
                     dtype=torch.uint8, device=gpu_device)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.Nq, device=gpu_device)
    st = torch.cuda.current_stream()

    def call(stream):
        rc = binding.fa_forward_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), None,
                                      o.data_ptr(), lse.data_ptr(), w.B, w.Hq, w.Hkv, w.Nq,
                                      w.Nk, w.D, w.scale, 0, binding.FA_DTYPE_BF16, splits,
                                      ws.data_ptr(), ws.numel(), stream.cuda_stream)
        assert rc == 0

    call(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
    for rep in range(3):
        for dst, src in zip((q, k, v), _fresh(w, 91 + rep, gpu_device)):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        o_g, l_g = o.clone(), lse.clone()
        call(st)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o) and torch.equal(l_g, lse), f"replay {rep}"


def test_backward_replays_match_eager(gpu_device):
    w = custom(1, 4, 2, 300, 300, 128, "bf16", True, False)
    q, k, v = _fresh(w, 100, gpu_device)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(5)).to(q.dtype).to(
        gpu_device)
    o, lse = binding.forward(q, k, v, None, causal=True, scale=w.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(binding.fa_backward_workspace_bytes(w.B, w.Hq, w.Nq), dtype=torch.uint8,
                     device=gpu_device)
    binding.backward(q, k, v, o, lse, dout, None, causal=True, scale=w.scale, dq=dq, dk=dk, dv=dv,
                     workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.backward(q, k, v, o, lse, dout, None, causal=True, scale=w.scale,
                         dq=dq, dk=dk, dv=dv, workspace=ws)
    for rep in range(3):
        dout.copy_(torch.randn(q.shape, generator=torch.Generator().manual_seed(6 + rep))
                   .to(q.dtype).to(gpu_device))
        g.replay()
        torch.cuda.synchronize()
        ref = binding.backward(q, k, v, o, lse, dout, None, causal=True, scale=w.scale)
        torch.cuda.synchronize()
        assert all(torch.equal(a, r) for a, r in zip((dq, dk, dv), ref)), f"replay {rep}"
