"""ctypes binding of libfa.so (argument marshalling only).

``fa_forward``, ``fa_forward_split``, ``fa_forward_split_noalloc``, ``fa_merge``,
``fa_backward``, ``fa_split_count``, ``fa_split_workspace_bytes``,
``fa_backward_workspace_bytes``, ``fa_check_args``, ``fa_status_string`` and
``fa_version`` take the same arguments as the C functions of
``include/fa.h`` (device pointers as Python ints; the size queries return
their value).  ``forward``, ``forward_split``, ``forward_split_noalloc``,
``forward_chain``, ``merge`` and ``backward`` are the tensor-level
conveniences: they check the torch tensors, allocate outputs (and the
key-split workspace) with torch unless given, and call the library on the
current stream.  Every step of the attention runs in the library's kernels;
if the library is missing or does not load, the call raises instead of
computing anything some other way.
"""

from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))

FA_DTYPE_BF16, FA_DTYPE_FP16, FA_DTYPE_FP32, FA_DTYPE_FP8_E4M3 = 0, 1, 2, 3
FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL_POINTER", 2: "FA_ERR_BAD_SIZE", 3: "FA_ERR_HEAD_GROUPS",
    4: "FA_ERR_HEAD_DIM", 5: "FA_ERR_DTYPE", 6: "FA_ERR_SCALE", 7: "FA_ERR_ALIGNMENT",
    8: "FA_ERR_OVERLAP", 9: "FA_ERR_TOO_LARGE", 10: "FA_ERR_HIP", 11: "FA_ERR_WORKSPACE",
    12: "FA_ERR_SCRATCH_LIMIT",
}
FA_ERR_SCRATCH_LIMIT = 12
# bytes of the library's per-GPU scratch array (fa_forward_split_noalloc)
FA_SPLIT_SCRATCH_BYTES = 32 << 20

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return os.environ.get("FA_LIBRARY", os.path.join(PKG, "libfa.so"))


def load_library():
    """Load libfa.so once; raise FaError-like RuntimeError if it is absent or broken."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m tiled_attention_forward_amd.build`")
    lib = ctypes.CDLL(path)
    p, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.fa_check_args.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, f32, i32, i32]
    lib.fa_check_args.restype = i32
    lib.fa_forward.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, f32, i32, i32, p]
    lib.fa_forward.restype = i32
    lib.fa_forward_window.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, f32, i64,
                                      i32, p]
    lib.fa_forward_window.restype = i32
    lib.fa_backward_window.argtypes = [p, p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64,
                                       f32, i64, i32, p, i64, p]
    lib.fa_backward_window.restype = i32
    lib.fa_forward_chain.argtypes = [ctypes.POINTER(p), ctypes.POINTER(p), i64, p, p, p, i64,
                                     i64, i64, i64, i64, i64, f32, i32, i32, p]
    lib.fa_forward_chain.restype = i32
    lib.fa_forward_split.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, f32, i32,
                                     i32, i64, p, i64, p]
    lib.fa_forward_split.restype = i32
    lib.fa_forward_split_noalloc.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, f32,
                                             i32, i32, i64, p]
    lib.fa_forward_split_noalloc.restype = i32
    lib.fa_split_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ctypes.POINTER(i64)]
    lib.fa_split_workspace_bytes.restype = i32
    lib.fa_split_count.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.POINTER(i64)]
    lib.fa_split_count.restype = i32
    lib.fa_merge.argtypes = [p, p, i64, i64, i64, p, p, i32, p]
    lib.fa_merge.restype = i32
    lib.fa_backward.argtypes = [p, p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, f32,
                                i32, i32, p, i64, p]
    lib.fa_backward.restype = i32
    lib.fa_backward_chain.argtypes = [ctypes.POINTER(p), ctypes.POINTER(p), i64, p, p, p, p,
                                      ctypes.POINTER(p), ctypes.POINTER(p), p, i64, i64, i64,
                                      i64, i64, i64, f32, i32, i32, p, i64, p]
    lib.fa_backward_chain.restype = i32
    lib.fa_backward_workspace_bytes.argtypes = [i64, i64, i64, ctypes.POINTER(i64)]
    lib.fa_backward_workspace_bytes.restype = i32
    lib.fa_status_string.argtypes = [i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_check_args(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, dtype) -> int:
    return load_library().fa_check_args(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D,
                                        float(scale), int(causal), int(dtype))


def fa_forward(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, dtype,
               stream) -> int:
    return load_library().fa_forward(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D,
                                     float(scale), int(causal), int(dtype), stream)


def fa_forward_split(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, dtype,
                     num_splits, workspace, workspace_bytes, stream) -> int:
    return load_library().fa_forward_split(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D,
                                           float(scale), int(causal), int(dtype),
                                           int(num_splits), workspace, int(workspace_bytes),
                                           stream)


def fa_forward_split_noalloc(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, dtype,
                             num_splits, stream) -> int:
    return load_library().fa_forward_split_noalloc(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D,
                                                   float(scale), int(causal), int(dtype),
                                                   int(num_splits), stream)


def fa_merge(part_o, part_lse, num_parts, rows, D, o, lse, dtype, stream) -> int:
    return load_library().fa_merge(part_o, part_lse, int(num_parts), int(rows), int(D), o, lse,
                                   int(dtype), stream)


def fa_split_workspace_bytes(B, Hq, Nq, D, num_splits) -> int:
    """Workspace bytes of fa_forward_split; raises FaError on invalid sizes."""
    out = ctypes.c_int64(0)
    st = load_library().fa_split_workspace_bytes(B, Hq, Nq, D, num_splits, ctypes.byref(out))
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))
    return out.value


def fa_split_count(B, Hq, Hkv, Nq, Nk, D) -> int:
    """The library's suggested key-split count; raises FaError on invalid sizes."""
    out = ctypes.c_int64(0)
    st = load_library().fa_split_count(B, Hq, Hkv, Nq, Nk, D, ctypes.byref(out))
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))
    return out.value


def fa_backward(q, k, v, bias, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, D, scale, causal,
                dtype, workspace, workspace_bytes, stream) -> int:
    return load_library().fa_backward(q, k, v, bias, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk,
                                      D, float(scale), int(causal), int(dtype), workspace,
                                      int(workspace_bytes), stream)


def fa_backward_workspace_bytes(B, Hq, Nq) -> int:
    """Workspace bytes of fa_backward; raises FaError on invalid sizes."""
    out = ctypes.c_int64(0)
    st = load_library().fa_backward_workspace_bytes(B, Hq, Nq, ctypes.byref(out))
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))
    return out.value


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_version() -> str:
    return load_library().fa_version().decode()


def _dtype_code(t) -> int:
    import torch
    codes = {torch.bfloat16: FA_DTYPE_BF16, torch.float16: FA_DTYPE_FP16,
             torch.float32: FA_DTYPE_FP32, torch.float8_e4m3fn: FA_DTYPE_FP8_E4M3}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check_inputs(q, k, v, bias):
    for name, t in (("q", q), ("k", k), ("v", v)) + ((("bias", bias),) if bias is not None else ()):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA tensor")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D, got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Hkv, Nk, D] matching q")
    if bias is not None and tuple(bias.shape) != (B, Hq, Nq, Nk):
        raise ValueError("bias must be [B, Hq, Nq, Nk]")
    return B, Hq, Hkv, Nq, Nk, D


def _check_buffer(name, t, shape, dtype, device):
    """A caller-supplied output or workspace tensor must be exactly what the
    kernels will write through a raw pointer: the C ABI cannot see a tensor's
    size, so a wrong shape, dtype, stride or device would send the kernels
    past the allocation.  Raises ValueError (TypeError for a non-tensor)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, not {type(t).__name__}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(t, need, device):
    """A caller-supplied workspace: a contiguous tensor on ``device`` of at least
    ``need`` bytes (the C ABI checks the byte count it is given; this makes
    sure that count describes memory the tensor really owns)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"workspace must be a torch.Tensor, not {type(t).__name__}")
    if t.device != device or not t.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if t.numel() * t.element_size() < need:
        raise ValueError(f"workspace holds {t.numel() * t.element_size()} bytes, "
                         f"{need} needed")


def _out_dtype(q):
    import torch
    # FP8 (E4M3) inputs give a bf16 output
    return torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype


def _outputs(q, out, lse):
    """Allocate O [B,Hq,Nq,D] and LSE [B,Hq,Nq] float32 on q's device, or check
    the caller's."""
    import torch
    B, Hq, Nq, _ = q.shape
    odt = _out_dtype(q)
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    else:
        _check_buffer("out", out, q.shape, odt, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    else:
        _check_buffer("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    return out, lse


def forward(q, k, v, bias=None, *, causal=False, scale=None, out=None, lse=None, stream=None,
            window=None):
    """O, LSE = attention(q, k, v [, bias]) on the GPU through fa_forward.

    q [B,Hq,Nq,D], k/v [B,Hkv,Nk,D], bias [B,Hq,Nq,Nk] or None: contiguous
    CUDA tensors of one dtype (bf16, fp16 or fp32).  ``scale=None`` means
    1/sqrt(D).  ``out``/``lse`` may be preallocated ([B,Hq,Nq,D] dtype and
    [B,Hq,Nq] float32).  Runs on ``stream`` (a torch.cuda.Stream) or the
    current stream.  ``window`` (requires ``causal``) calls
    fa_forward_window: row i sees keys i - window < j <= i.
    """
    import torch
    lib = load_library()
    B, Hq, Hkv, Nq, Nk, D = _check_inputs(q, k, v, bias)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out, lse = _outputs(q, out, lse)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if window is not None:
        if not causal:
            raise ValueError("window requires causal=True")
        st = lib.fa_forward_window(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   bias.data_ptr() if bias is not None else None,
                                   out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, D,
                                   float(scale), int(window), _dtype_code(q), stream.cuda_stream)
    else:
        st = lib.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            bias.data_ptr() if bias is not None else None,
                            out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, D, float(scale),
                            int(bool(causal)), _dtype_code(q), stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))
    return out, lse


def fa_forward_chain(q_ptrs, k_ptrs, v, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, dtype,
                     stream) -> int:
    """fa_forward_chain with Python lists of device addresses for the layers."""
    n = len(q_ptrs)
    qa = (ctypes.c_void_p * max(n, 1))(*q_ptrs)
    ka = (ctypes.c_void_p * max(len(k_ptrs), 1))(*k_ptrs)
    return load_library().fa_forward_chain(qa, ka, n, v, o, lse, B, Hq, Hkv, Nq, Nk, D, scale,
                                           causal, dtype, stream)


def forward_chain(q_layers, k_layers, v, *, causal=False, scale=None, out=None, lse=None,
                  stream=None):
    """O, LSE of the last layer of a Block Attention Residual chain (fa_forward_chain).

    q_layers / k_layers: the block's Q and K tensors up to the current layer,
    oldest first (1 to 4 layers), each shaped like q / k of ``forward``; v is
    the current layer's V.  The logits are sum_l Q_l K_l^T * scale.
    """
    import torch
    lib = load_library()
    if len(q_layers) != len(k_layers) or not q_layers:
        raise ValueError("need as many K layers as Q layers, at least one")
    B, Hq, Hkv, Nq, Nk, D = _check_inputs(q_layers[-1], k_layers[-1], v, None)
    for ql, kl in zip(q_layers, k_layers):
        _check_inputs(ql, kl, v, None)
        if ql.shape != q_layers[-1].shape or ql.dtype != v.dtype or kl.dtype != v.dtype:
            raise ValueError("every layer needs the shapes and dtype of the last one")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out, lse = _outputs(q_layers[-1], out, lse)
    if stream is None:
        stream = torch.cuda.current_stream(v.device)
    st = fa_forward_chain([t.data_ptr() for t in q_layers], [t.data_ptr() for t in k_layers],
                          v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, D,
                          float(scale), int(bool(causal)), _dtype_code(v), stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))
    return out, lse


def forward_split(q, k, v, bias=None, *, causal=False, scale=None, num_splits=None,
                  workspace=None, out=None, lse=None, stream=None):
    """The same result as ``forward`` through the key-split path (fa_forward_split).

    ``num_splits=None`` takes the library's suggestion (fa_split_count).
    ``workspace`` may be a preallocated CUDA uint8 tensor of at least
    fa_split_workspace_bytes(...) bytes; otherwise one is allocated with torch.
    """
    import torch
    lib = load_library()
    B, Hq, Hkv, Nq, Nk, D = _check_inputs(q, k, v, bias)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if num_splits is None:
        num_splits = fa_split_count(B, Hq, Hkv, Nq, Nk, D)
    need = fa_split_workspace_bytes(B, Hq, Nq, D, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, need, q.device)
    out, lse = _outputs(q, out, lse)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = lib.fa_forward_split(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              bias.data_ptr() if bias is not None else None,
                              out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, D,
                              float(scale), int(bool(causal)), _dtype_code(q), int(num_splits),
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))
    return out, lse


def forward_split_noalloc(q, k, v, bias=None, *, causal=False, scale=None, num_splits=None,
                          out=None, lse=None, stream=None):
    """``forward_split`` through fa_forward_split_noalloc: the partials go to
    the library's per-GPU scratch array instead of a workspace, so with ``out``
    and ``lse`` given nothing is allocated.  Calls that can overlap on one GPU
    race on that array."""
    import torch
    lib = load_library()
    B, Hq, Hkv, Nq, Nk, D = _check_inputs(q, k, v, bias)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if num_splits is None:
        num_splits = fa_split_count(B, Hq, Hkv, Nq, Nk, D)
    out, lse = _outputs(q, out, lse)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = lib.fa_forward_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      bias.data_ptr() if bias is not None else None,
                                      out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, D,
                                      float(scale), int(bool(causal)), _dtype_code(q),
                                      int(num_splits), stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))
    return out, lse


def merge(part_o, part_lse, dtype, *, out=None, lse=None, stream=None):
    """O, LSE from normalised partials through fa_merge.

    part_o float32 [P, ..., D], part_lse float32 [P, ...] (contiguous CUDA
    tensors); the result has shape [..., D] in ``dtype`` and [...] float32.
    """
    import torch
    lib = load_library()
    if part_o.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise TypeError("partials must be float32")
    if not (part_o.is_cuda and part_lse.is_cuda and part_o.is_contiguous()
            and part_lse.is_contiguous()):
        raise ValueError("partials must be contiguous CUDA tensors")
    if tuple(part_o.shape[:-1]) != tuple(part_lse.shape):
        raise ValueError("part_o must be part_lse's shape plus a trailing D axis")
    P, D = part_o.shape[0], part_o.shape[-1]
    rows = part_lse[0].numel() if P > 0 else math.prod(part_lse.shape[1:])
    if part_lse.device != part_o.device:
        raise ValueError("part_o and part_lse must be on one device")
    if out is None:
        out = torch.empty(tuple(part_o.shape[1:]), dtype=dtype, device=part_o.device)
    else:
        _check_buffer("out", out, part_o.shape[1:], dtype, part_o.device)
    if lse is None:
        lse = torch.empty(tuple(part_lse.shape[1:]), dtype=torch.float32, device=part_o.device)
    else:
        _check_buffer("lse", lse, part_lse.shape[1:], torch.float32, part_o.device)
    if stream is None:
        stream = torch.cuda.current_stream(part_o.device)
    st = lib.fa_merge(part_o.data_ptr() if P > 0 else None,
                      part_lse.data_ptr() if P > 0 else None, P, rows, D, out.data_ptr(),
                      lse.data_ptr(), _dtype_code(out), stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))
    return out, lse


def backward(q, k, v, o, lse, dout, bias=None, *, causal=False, scale=None, dq=None, dk=None,
             dv=None, workspace=None, stream=None, window=None):
    """dQ, dK, dV of attention(q, k, v [, bias]) through fa_backward.

    ``o`` and ``lse`` are the outputs of ``forward`` on the same arguments and
    ``dout`` the gradient with respect to ``o``.  bf16/fp16 tensors, or fp32
    at head sizes 64 and 128; outputs and the workspace are allocated with
    torch unless given.  ``window`` (requires ``causal``) calls
    fa_backward_window.
    """
    import torch
    lib = load_library()
    B, Hq, Hkv, Nq, Nk, D = _check_inputs(q, k, v, bias)
    for name, t in (("o", o), ("dout", dout)):
        _check_buffer(name, t, q.shape, q.dtype, q.device)
    _check_buffer("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is not None:
            _check_buffer(name, t, like.shape, like.dtype, like.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = fa_backward_workspace_bytes(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, need, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(),
            bias.data_ptr() if bias is not None else None, o.data_ptr(), lse.data_ptr(),
            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nk, D,
            float(scale))
    tail = (_dtype_code(q), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            stream.cuda_stream)
    if window is not None:
        if not causal:
            raise ValueError("window requires causal=True")
        st = lib.fa_backward_window(*ptrs, int(window), *tail)
    else:
        st = lib.fa_backward(*ptrs, int(bool(causal)), *tail)
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))
    return dq, dk, dv


def fa_backward_chain(q_ptrs, k_ptrs, v, o, lse, dout, dq_ptrs, dk_ptrs, dv, B, Hq, Hkv, Nq,
                      Nk, D, scale, causal, dtype, workspace, workspace_bytes, stream) -> int:
    """fa_backward_chain with Python lists of device addresses for the layers."""
    arr = lambda xs: (ctypes.c_void_p * max(len(xs), 1))(*xs)
    return load_library().fa_backward_chain(arr(q_ptrs), arr(k_ptrs), len(q_ptrs), v, o, lse,
                                            dout, arr(dq_ptrs), arr(dk_ptrs), dv, B, Hq, Hkv, Nq,
                                            Nk, D, scale, causal, dtype, workspace,
                                            workspace_bytes, stream)


def backward_chain(q_layers, k_layers, v, o, lse, dout, *, causal=False, scale=None,
                   dq_layers=None, dk_layers=None, dv=None, workspace=None, stream=None):
    """Gradients of ``forward_chain`` through fa_backward_chain.

    Returns ``(dq_layers, dk_layers, dv)``: the gradients of every Q and K
    layer of the chain (oldest first) and of v, for ``o`` and ``lse`` from
    ``forward_chain`` on the same arguments and ``dout`` the gradient with
    respect to ``o``.  bf16/fp16, D = 64 or 128; outputs and the workspace are
    allocated with torch unless given.
    """
    import torch
    lib = load_library()
    if len(q_layers) != len(k_layers) or not q_layers:
        raise ValueError("need as many K layers as Q layers, at least one")
    B, Hq, Hkv, Nq, Nk, D = _check_inputs(q_layers[-1], k_layers[-1], v, None)
    for ql, kl in zip(q_layers, k_layers):
        _check_inputs(ql, kl, v, None)
        if ql.shape != q_layers[-1].shape or ql.dtype != v.dtype or kl.dtype != v.dtype:
            raise ValueError("every layer needs the shapes and dtype of the last one")
    q = q_layers[-1]
    for name, t in (("o", o), ("dout", dout)):
        _check_buffer(name, t, q.shape, q.dtype, q.device)
    _check_buffer("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    n = len(q_layers)
    if dq_layers is None:
        dq_layers = [torch.empty_like(t) for t in q_layers]
    if dk_layers is None:
        dk_layers = [torch.empty_like(t) for t in k_layers]
    if len(dq_layers) != n or len(dk_layers) != n:
        raise ValueError("need one dQ and one dK buffer per layer")
    for t in dq_layers:
        _check_buffer("dq", t, q.shape, q.dtype, q.device)
    for t in dk_layers:
        _check_buffer("dk", t, v.shape, v.dtype, v.device)
    if dv is None:
        dv = torch.empty_like(v)
    else:
        _check_buffer("dv", dv, v.shape, v.dtype, v.device)
    need = fa_backward_workspace_bytes(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, need, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_backward_chain([t.data_ptr() for t in q_layers], [t.data_ptr() for t in k_layers],
                           v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                           [t.data_ptr() for t in dq_layers], [t.data_ptr() for t in dk_layers],
                           dv.data_ptr(), B, Hq, Hkv, Nq, Nk, D, float(scale), int(bool(causal)),
                           _dtype_code(v), workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))
    return dq_layers, dk_layers, dv
