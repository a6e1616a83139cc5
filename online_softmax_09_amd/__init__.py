"""MI355X (gfx950) tiled attention forward and row-wise online softmax.

A thin binding over the C ABI of ``libmi355attn.so`` (``include/mi355attn.h``): it
checks tensor dtypes, devices and shapes, allocates outputs with torch, and passes raw
device pointers and torch's current HIP stream.  Every step of the computation runs
in the library's HIP kernels; there is no CPU or PyTorch fallback, and a missing
library raises.

Functions carry the names of the C entry points:

* ``fa_fwd(q, k, v, scale, causal)``      bf16 [B, H, N, d] -> (o bf16, lse float32 [B, H, N])
* ``fa_fwd_f32(q, k, v, scale, causal)``  the same in float32
* ``online_softmax_rows(x)``              float32 [rows, cols] -> softmax of every row
* ``fa_bwd(q, k, v, o, lse, dout, scale, causal)``  bf16 -> (dq, dk, dv), the gradients
  of ``fa_fwd`` for the upstream gradient ``dout``
"""

import math

from . import _lib

__all__ = ["fa_fwd", "fa_fwd_f32", "fa_bwd", "online_softmax_rows", "library_path", "version"]


def library_path():
    return _lib.LIB_PATH


def version():
    return _lib.load().mi355attn_version()


def _torch():
    import torch

    return torch


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _attention_args(q, k, v, dtype, out, lse):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU device")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on the same device")
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if (lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    return out, lse


def _attention(entry, q, k, v, scale, causal, out, lse, stream, dtype):
    torch = _torch()
    out, lse = _attention_args(q, k, v, dtype, out, lse)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(q.device):
        rc = getattr(_lib.load(), entry)(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            B, H, N, d, float(scale), 1 if causal else 0, _stream_handle(stream, q.device))
    _lib.check(rc, entry)
    return out, lse


def fa_fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """bf16 attention forward on the GPU; returns (o, lse).  scale defaults to 1/sqrt(d)."""
    return _attention("fa_fwd", q, k, v, scale, causal, out, lse, stream, _torch().bfloat16)


def fa_fwd_f32(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """float32 attention forward on the GPU; returns (o, lse).  scale defaults to 1/sqrt(d)."""
    return _attention("fa_fwd_f32", q, k, v, scale, causal, out, lse, stream, _torch().float32)


def fa_bwd(q, k, v, o, lse, dout, scale=None, causal=False, dq=None, dk=None, dv=None, workspace=None,
           stream=None):
    """Gradients (dq, dk, dv) of the bf16 attention forward for the upstream gradient dout.

    o and lse are fa_fwd's outputs for the same q, k, v, scale and causal.  The float32
    workspace the library needs (8 bytes per row) is allocated here unless given.
    """
    torch = _torch()
    _attention_args(q, k, v, torch.bfloat16, o, lse)
    _attention_args(q, k, dout, torch.bfloat16, None, lse)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    grads = []
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        if g is None:
            g = torch.empty_like(q)
        if g.shape != q.shape or g.dtype != torch.bfloat16 or not g.is_contiguous() or g.device != q.device:
            raise ValueError(f"{name} must be a contiguous bf16 tensor like q")
        grads.append(g)
    lib = _lib.load()
    need = lib.fa_bwd_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
    if (workspace.dtype != torch.float32 or not workspace.is_contiguous() or workspace.device != q.device
            or workspace.numel() * 4 < need):
        raise ValueError(f"workspace must be a contiguous float32 tensor of at least {need} bytes on q's device")
    with torch.cuda.device(q.device):
        rc = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                        grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(), workspace.data_ptr(),
                        B, H, N, d, float(scale), 1 if causal else 0, _stream_handle(stream, q.device))
    _lib.check(rc, "fa_bwd")
    return tuple(grads)


def online_softmax_rows(x, out=None, stream=None):
    """Softmax of every row of a contiguous float32 [rows, cols] GPU tensor.

    ``out`` may be ``x`` itself (in place).
    """
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or not x.is_cuda:
        raise TypeError("x must be a float32 GPU tensor")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [rows, cols] tensor")
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous tensor like x")
    rows, cols = x.shape
    with torch.cuda.device(x.device):
        rc = _lib.load().online_softmax_rows(x.data_ptr(), out.data_ptr(), rows, cols,
                                             _stream_handle(stream, x.device))
    _lib.check(rc, "online_softmax_rows")
    return out
