"""MI355X (gfx950) tiled attention forward and row-wise online softmax.

A thin binding over the C ABI of ``libmi355attn.so`` (``include/mi355attn.h``): it
checks tensor dtypes, devices and shapes, allocates outputs with torch, and passes raw
device pointers and torch's current HIP stream.  Every step of the computation runs
in the library's HIP kernels; there is no CPU or PyTorch fallback, and a missing
library raises.

Functions carry the names of the C entry points:

* ``fa_fwd(q, k, v, scale, causal)``      bf16 [B, H, N, d] -> (o bf16, lse float32 [B, H, N])
* ``fa_fwd_f16(q, k, v, scale, causal)``  the same in fp16
* ``fa_fwd_f32(q, k, v, scale, causal)``  the same in float32
* ``online_softmax_rows(x)``              float32 [rows, cols] -> softmax of every row
* ``fa_bwd(q, k, v, o, lse, dout, scale, causal)``  bf16 -> (dq, dk, dv), the gradients
  of ``fa_fwd`` for the upstream gradient ``dout``
* ``fa_fwd_splitkv(q, k, v, scale, causal, n_splits)``  bf16 q [B, H, Nq, d] against
  k, v [B, H, Nk, d] -> (o, lse), keys cut into parts merged in the log domain
* ``fa_fwd_splitkv_noalloc(q, k, v, scale, causal, n_splits)``  the same with the partial
  results in the library's own per-device scratch (no workspace, nothing allocated)
* ``attn_merge_states(o_parts, lse_parts)``  float32 partial results -> (o bf16, lse)
* ``fused_add_rmsnorm(x, residual, gamma, eps)`` / ``fused_add_layernorm(x, residual, gamma,
  beta, eps)``  bf16 [rows, cols] -> (y, h = x + residual)
"""

import math

from . import _lib

__all__ = ["fa_fwd", "fa_fwd_f16", "fa_fwd_f32", "fa_bwd", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc",
           "attn_merge_states", "online_softmax_rows",
           "fused_add_rmsnorm", "fused_add_layernorm", "library_path", "version"]


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


def fa_fwd_f16(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """fp16 attention forward on the GPU; returns (o, lse).  scale defaults to 1/sqrt(d)."""
    return _attention("fa_fwd_f16", q, k, v, scale, causal, out, lse, stream, _torch().float16)


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


def _check_gpu_tensor(name, t, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name} must be a {dtype} GPU tensor")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def _splitkv_args(q, k, v, scale, out, lse):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_gpu_tensor(name, t, torch.bfloat16, 4)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape or k.device != q.device or v.device != q.device:
        raise ValueError("k and v must be [B, H, Nk, d] on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_gpu_tensor("out", out, torch.bfloat16, 4)
    _check_gpu_tensor("lse", lse, torch.float32, 3)
    if out.shape != q.shape or lse.shape != (B, H, Nq):
        raise ValueError("out must be like q and lse [B, H, Nq]")
    return B, H, Nq, Nk, d, float(scale), out, lse


def fa_fwd_splitkv(q, k, v, scale=None, causal=False, n_splits=1, out=None, lse=None, workspace=None,
                   stream=None):
    """bf16 attention of q [B, H, Nq, d] against k, v [B, H, Nk, d] with the keys cut into
    n_splits parts merged in the log domain; returns (o, lse).  Causal masks are
    bottom-right aligned (query i sees keys j <= Nk - Nq + i)."""
    torch = _torch()
    B, H, Nq, Nk, d, scale, out, lse = _splitkv_args(q, k, v, scale, out, lse)
    lib = _lib.load()
    need = lib.fa_fwd_splitkv_workspace_bytes(B, H, Nq, d, int(n_splits))
    if need < 0:
        raise ValueError("bad sizes")
    if workspace is None:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
    if workspace.dtype != torch.float32 or not workspace.is_contiguous() or workspace.numel() * 4 < need:
        raise ValueError(f"workspace must be a contiguous float32 tensor of at least {need} bytes")
    with torch.cuda.device(q.device):
        rc = lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                workspace.data_ptr(), B, H, Nq, Nk, d, scale, 1 if causal else 0,
                                int(n_splits), _stream_handle(stream, q.device))
    _lib.check(rc, "fa_fwd_splitkv")
    return out, lse


def fa_fwd_splitkv_noalloc(q, k, v, scale=None, causal=False, n_splits=1, out=None, lse=None, stream=None):
    """fa_fwd_splitkv with the partial results in the library's per-device scratch instead
    of a workspace (the C entry point allocates nothing; pass out and lse to keep this
    wrapper from allocating them).  Calls that overlap on one device race."""
    torch = _torch()
    B, H, Nq, Nk, d, scale, out, lse = _splitkv_args(q, k, v, scale, out, lse)
    with torch.cuda.device(q.device):
        rc = _lib.load().fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                lse.data_ptr(), B, H, Nq, Nk, d, scale, 1 if causal else 0,
                                                int(n_splits), _stream_handle(stream, q.device))
    _lib.check(rc, "fa_fwd_splitkv_noalloc")
    return out, lse


def attn_merge_states(o_parts, lse_parts, out=None, lse=None, stream=None):
    """Merge float32 partial results o_parts [P, rows, d], lse_parts [P, rows] (natural
    log, -inf = empty part) into (o bf16 [rows, d], lse float32 [rows])."""
    torch = _torch()
    _check_gpu_tensor("o_parts", o_parts, torch.float32, 3)
    _check_gpu_tensor("lse_parts", lse_parts, torch.float32, 2)
    P, rows, d = o_parts.shape
    if lse_parts.shape != (P, rows) or lse_parts.device != o_parts.device:
        raise ValueError("lse_parts must be [P, rows] on o_parts' device")
    if out is None:
        out = torch.empty((rows, d), dtype=torch.bfloat16, device=o_parts.device)
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=o_parts.device)
    _check_gpu_tensor("out", out, torch.bfloat16, 2)
    _check_gpu_tensor("lse", lse, torch.float32, 1)
    if out.shape != (rows, d) or lse.shape != (rows,):
        raise ValueError("out must be [rows, d] and lse [rows]")
    with torch.cuda.device(o_parts.device):
        rc = _lib.load().attn_merge_states(o_parts.data_ptr(), lse_parts.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                           P, rows, d, _stream_handle(stream, o_parts.device))
    _lib.check(rc, "attn_merge_states")
    return out, lse


def _norm(layer, x, residual, gamma, beta, eps, out, residual_out, stream):
    torch = _torch()
    _check_gpu_tensor("x", x, torch.bfloat16, 2)
    rows, cols = x.shape
    if residual is not None:
        _check_gpu_tensor("residual", residual, torch.bfloat16, 2)
        if residual.shape != x.shape or residual.device != x.device:
            raise ValueError("residual must be like x")
    for name, t in (("gamma", gamma), ("beta", beta if layer else None)):
        if t is None and name == "beta":
            continue
        _check_gpu_tensor(name, t, torch.bfloat16, 1)
        if t.shape != (cols,) or t.device != x.device:
            raise ValueError(f"{name} must be [cols] on x's device")
    if out is None:
        out = torch.empty_like(x)
    if residual_out is None:
        residual_out = torch.empty_like(x)
    for name, t in (("out", out), ("residual_out", residual_out)):
        _check_gpu_tensor(name, t, torch.bfloat16, 2)
        if t.shape != x.shape or t.device != x.device:
            raise ValueError(f"{name} must be like x")
    lib = _lib.load()
    rp = residual.data_ptr() if residual is not None else None
    with torch.cuda.device(x.device):
        if layer:
            rc = lib.fused_add_layernorm(x.data_ptr(), rp, gamma.data_ptr(), beta.data_ptr(), out.data_ptr(),
                                         residual_out.data_ptr(), rows, cols, float(eps),
                                         _stream_handle(stream, x.device))
        else:
            rc = lib.fused_add_rmsnorm(x.data_ptr(), rp, gamma.data_ptr(), out.data_ptr(), residual_out.data_ptr(),
                                       rows, cols, float(eps), _stream_handle(stream, x.device))
    _lib.check(rc, "fused_add_layernorm" if layer else "fused_add_rmsnorm")
    return out, residual_out


def fused_add_rmsnorm(x, residual, gamma, eps=1e-6, out=None, residual_out=None, stream=None):
    """RMSNorm of h = x + residual (residual may be None) over the rows of a bf16 [rows, cols]
    tensor; returns (y, h) in bf16.  out / residual_out may be x or residual (in place)."""
    return _norm(False, x, residual, gamma, None, eps, out, residual_out, stream)


def fused_add_layernorm(x, residual, gamma, beta, eps=1e-5, out=None, residual_out=None, stream=None):
    """LayerNorm of h = x + residual (residual may be None); returns (y, h) in bf16."""
    return _norm(True, x, residual, gamma, beta, eps, out, residual_out, stream)


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
