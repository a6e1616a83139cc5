"""Attention with separate query and key lengths, and the log-domain merge of partial
attention results, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests and the bench's
cpu_baseline leg, never by the GPU library.

``attention_rect`` is the definition of ``attention`` in oracle/attention.py for N_q
queries against N_k keys.  Reading taken where the pages are silent: with causal
masking the queries are the last N_q positions of the key
sequence (bottom-right alignment, the shape of inference with a key/value cache, which
[INT] follow-up 3 mentions), so query i sees keys j <= N_k - N_q + i.  With
N_q = N_k this is the top-left alignment of ``attention``.

``merge_attention_states`` combines results computed over disjoint parts of the key
sequence.  [SNS] section 4.1 merges two online-softmax states (m_a, l_a) and (m_b, l_b)
as m = max(m_a, m_b), l = l_a exp(m_a - m) + l_b exp(m_b - m); [INT] follow-up 1 applies
the same rescaling to the per-block weighted sums.  For a part p holding the normalised
output O_p = (sum_j e^{s_j} v_j) / (sum_j e^{s_j}) and LSE_p = ln sum_j e^{s_j} over its
keys, the unnormalised sum is e^{LSE_p} O_p, so the whole sequence has

    LSE = ln sum_p e^{LSE_p},        O = sum_p e^{LSE_p - LSE} O_p .

The oracle evaluates exactly that, with the maximum over parts subtracted before the
exponentials ([SNS] section 2.1).  A part with no keys is (O_p, LSE_p) = (anything, -inf)
and contributes nothing.
"""

import numpy as np

from .attention import _as_f64


def attention_rect(q, k, v, scale, causal):
    """(O [B, H, Nq, d], LSE [B, H, Nq]) for q [B, H, Nq, d] and k, v [B, H, Nk, d].

    Causal masking is bottom-right aligned: query i sees keys j <= Nk - Nq + i (Nq <= Nk
    required).  A query row with no visible key raises.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    Nq, Nk = q.shape[2], k.shape[2]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    s = float(scale) * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        s = np.where(j > Nk - Nq + i, -np.inf, s)
    m = np.max(s, axis=-1, keepdims=True)                # scan 1
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key")
    e = np.exp(s - m)
    l = np.sum(e, axis=-1, keepdims=True)                # scan 2
    o = (e / l) @ v                                      # scan 3, then P V
    return o, m[..., 0] + np.log(l[..., 0])


def merge_attention_states(o_parts, lse_parts):
    """Merge P partial results over disjoint key sets.

    o_parts: [P, ..., d] normalised partial outputs; lse_parts: [P, ...] their LSE
    (natural log; -inf marks a part with no keys).  Returns (O [..., d], LSE [...]).
    A row whose parts are all empty has no defined result and raises.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    if o_parts.shape[:-1] != lse_parts.shape or o_parts.shape[0] < 1:
        raise ValueError("o_parts must be [P, ..., d] and lse_parts [P, ...]")
    m = np.max(lse_parts, axis=0)
    if not np.all(np.isfinite(m)):
        raise ValueError("a row has no keys in any part")
    w = np.exp(lse_parts - m)                            # 0 for empty parts
    tot = np.sum(w, axis=0)
    lse = m + np.log(tot)
    o = np.sum((w / tot)[..., None] * np.where(np.isfinite(lse_parts)[..., None], o_parts, 0.0), axis=0)
    return o, lse

