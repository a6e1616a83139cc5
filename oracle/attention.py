"""Standard attention with the score matrix materialised, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, smoke and
the bench's cpu_baseline leg, never by the GPU library.

Definition followed ([FAM] "the problem starts with the intermediate matrix" and
[SNS] section 7 write the same operation; [WHY] states it with the 1/sqrt(d) factor):

    S = scale * Q K^T            (N x N per (batch, head), materialised here)
    P = softmax(S) row by row    (the three scans of [SNS] section 3)
    O = P V
    LSE_i = m_i + ln l_i         (natural log of sum_j exp(S_ij))

Readings taken where the pages are silent:

* ``scale`` is applied to the scores before the softmax; callers pass 1/sqrt(d).
* Layout is [B, H, N, d] for Q, K, V and O, [B, H, N] for LSE.
* Causal masking is top-left aligned self-attention: query i sees keys j <= i, so
  no row is ever empty.
* LSE is the natural logarithm of the sum over visible keys of exp(scaled score).

Rows are evaluated one block of query rows at a time only to bound host memory;
every row is an independent instance of the definition, so this is not a change
of algorithm.  ``attention_rows`` evaluates a chosen subset of query rows in the
same way.
"""

import numpy as np


def _as_f64(t):
    """Exact float64 copy of a NumPy array or a CPU torch tensor (fp32 or bf16)."""
    if hasattr(t, "detach"):  # torch tensor: upcast in torch, then hand to NumPy
        import torch

        return t.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def _rows_one_head(q, k, v, scale, causal, rows):
    """O and LSE for query rows ``rows`` of one (batch, head) slice.

    q, k, v: float64 [N, d]; rows: int64 [R].  Returns O [R, d], LSE [R].
    """
    s = scale * (q[rows] @ k.T)                      # scores, [R, N]
    if causal:
        keys = np.arange(k.shape[0])
        s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
    m = np.max(s, axis=1, keepdims=True)             # scan 1: row maximum
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key")
    e = np.exp(s - m)                                # masked entries give exp(-inf) = 0
    l = np.sum(e, axis=1, keepdims=True)             # scan 2: row sum
    p = e / l                                        # scan 3: normalised weights
    o = p @ v
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def attention_rows(q, k, v, scale, causal, rows=None, block_rows=256):
    """Attention output and LSE for selected query rows, in float64.

    q, k, v: [B, H, N, d] (NumPy arrays or CPU torch tensors of any float dtype).
    rows:    None (all N rows), an int array [R] (the same rows in every head) or
             an int array [B, H, R] (rows chosen per head).
    Returns (O [B, H, R, d], LSE [B, H, R]) as float64 NumPy arrays.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    scale = float(scale)
    if rows is None:
        rows = np.arange(N, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    if rows.ndim == 1:
        rows = np.broadcast_to(rows, (B, H, rows.shape[0]))
    if rows.shape[:2] != (B, H):
        raise ValueError("rows must be [R] or [B, H, R]")
    if rows.size and (rows.min() < 0 or rows.max() >= N):
        raise ValueError("row index out of range")
    R = rows.shape[2]
    o = np.empty((B, H, R, d), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, R, block_rows):
                sel = rows[b, h, r0:r0 + block_rows]
                o[b, h, r0:r0 + len(sel)], lse[b, h, r0:r0 + len(sel)] = _rows_one_head(
                    q[b, h], k[b, h], v[b, h], scale, causal, sel)
    return o, lse


def attention(q, k, v, scale, causal):
    """Full attention forward: (O [B, H, N, d], LSE [B, H, N]) in float64."""
    return attention_rows(q, k, v, scale, causal, rows=None)
