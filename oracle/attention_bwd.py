"""Gradients of standard attention with the score and probability matrices materialised,
in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests and the bench's
cpu_baseline leg, never by the GPU library.

What the pages fix: the backward pass of the tiled method produces the gradients of the
same exact attention, but instead of keeping the N x N probability matrix from the
forward it recomputes the local scores from a few saved row statistics ([SNS] section
7.2 and question 4; [WHY] section "floating-point addition is not associative"; [INT]
standard answer, point 2 on recomputation).  The pages do not write
the gradient formulas, so the oracle takes the plainest reading: the derivative of the
definition

    S = scale * Q K^T,   P = softmax(S) row by row (visible keys only),   O = P V

with respect to Q, K and V, for an upstream gradient dO = dL/dO, by the chain rule:

    dV   = P^T dO
    dP   = dO V^T
    dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik)     (Jacobian of a row softmax)
    dQ   = scale * dS K
    dK   = scale * dS^T Q

Hidden (causal) entries have P_ij = 0 and therefore dS_ij = 0.  Everything here is the
materialised definition: S, P, dP and dS exist in full for each block of query rows.
Rows are processed one block at a time only to bound host memory; dK and dV add the
blocks' contributions, which reorders a sum over query rows and changes nothing else.
"""

import numpy as np

from .attention import _as_f64


def _head_backward(q, k, v, do, scale, causal, block_rows):
    """dQ, dK, dV [N, d] of one (batch, head) slice; all inputs float64 [N, d]."""
    N = q.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    keys = np.arange(N)
    for r0 in range(0, N, block_rows):
        rows = np.arange(r0, min(N, r0 + block_rows))
        s = scale * (q[rows] @ k.T)                              # [R, N]
        if causal:
            s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
        m = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / np.sum(e, axis=1, keepdims=True)                 # softmax rows
        dp = do[rows] @ v.T                                      # dL/dP
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))    # through the softmax
        dq[rows] = scale * (ds @ k)
        dk += scale * (ds.T @ q[rows])
        dv += p.T @ do[rows]
    return dq, dk, dv


def attention_backward(q, k, v, do, scale, causal, heads=None, block_rows=512):
    """Gradients (dQ, dK, dV) of O = softmax(scale Q K^T) V for the upstream gradient dO.

    q, k, v, do: [B, H, N, d] (NumPy arrays or CPU torch tensors of any float dtype).
    heads: None for every (b, h), else a list of (b, h) pairs; the results are then
    [len(heads), N, d] in that order.
    Returns float64 NumPy arrays ([B, H, N, d] each when heads is None).
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    if q.ndim != 4 or any(t.shape != q.shape for t in (k, v, do)):
        raise ValueError("q, k, v, do must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    scale = float(scale)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in pairs:
        if not (0 <= b < B and 0 <= h < H):
            raise ValueError("head index out of range")
    out = [np.empty((len(pairs), N, d)) for _ in range(3)]
    for n, (b, h) in enumerate(pairs):
        grads = _head_backward(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, block_rows)
        for t in range(3):
            out[t][n] = grads[t]
    if heads is None:
        return tuple(t.reshape(B, H, N, d) for t in out)
    return tuple(out)
