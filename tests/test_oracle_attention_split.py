"""Pins for the rectangular-attention and merge oracles (float64).

Each check takes the implementation under test, so it also runs on copies with a planted
mistake (top-left instead of bottom-right causal alignment, merge without the maximum
subtracted, merge weights left unnormalised, parts averaged, LSE of the largest part
only) and must fail there.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads


def _rand(shape, seed, sd=1.0):
    return workloads.generator(seed).normal(0.0, sd, size=shape)


# --------------------------------------------------------------------------
# attention_rect
# --------------------------------------------------------------------------

def check_rect_square(rect):
    """Nq = Nk is the square oracle (already pinned) with both masks."""
    q, k, v = (_rand((2, 2, 33, 8), s) for s in (1, 2, 3))
    for causal in (False, True):
        o, l = rect(q, k, v, 0.3, causal)
        o2, l2 = oracle.attention(q, k, v, 0.3, causal)
        if not (np.allclose(o, o2, rtol=1e-13, atol=1e-14) and np.allclose(l, l2, rtol=1e-13, atol=1e-14)):
            return False
    return True


def check_rect_sdpa(rect):
    """CPU float64 scaled_dot_product_attention with an explicit bottom-right mask."""
    for Nq, Nk, causal in ((1, 70, True), (5, 70, True), (16, 300, False), (40, 129, True)):
        q, k, v = _rand((1, 3, Nq, 16), 10 + Nq), _rand((1, 3, Nk, 16), 20 + Nk), _rand((1, 3, Nk, 16), 30)
        mask = None
        if causal:
            i = np.arange(Nq)[:, None]
            j = np.arange(Nk)[None, :]
            mask = torch.from_numpy(j <= Nk - Nq + i)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                             attn_mask=mask, scale=0.25)
        o, _ = rect(q, k, v, 0.25, causal)
        if not np.allclose(o, ref.numpy(), rtol=1e-11, atol=1e-12):
            return False
    return True


def check_rect_last_row(rect):
    """The last query of a causal call sees every key: it equals the non-causal row, and
    with K = 0 every row is the mean of its visible values (LSE = ln count)."""
    Nq, Nk = 6, 50
    q, k, v = _rand((1, 1, Nq, 4), 41), _rand((1, 1, Nk, 4), 42), _rand((1, 1, Nk, 4), 43)
    oc, lc = rect(q, k, v, 0.7, True)
    on, ln = rect(q, k, v, 0.7, False)
    if not (np.allclose(oc[:, :, -1], on[:, :, -1], rtol=1e-13) and np.allclose(lc[:, :, -1], ln[:, :, -1])):
        return False
    o0, l0 = rect(q, np.zeros_like(k), v, 0.7, True)
    for i in range(Nq):
        n = Nk - Nq + i + 1
        if not (np.allclose(o0[0, 0, i], v[0, 0, :n].mean(axis=0), rtol=1e-12, atol=1e-13)
                and math.isclose(l0[0, 0, i], math.log(n), rel_tol=1e-13)):
            return False
    return True


# --------------------------------------------------------------------------
# merge_attention_states
# --------------------------------------------------------------------------

def check_merge_recovers_full(merge):
    """Attention over key slices, merged, is attention over all keys (any split points)."""
    g = workloads.generator(51)
    q, k, v = _rand((1, 2, 3, 8), 52), _rand((1, 2, 90, 8), 53), _rand((1, 2, 90, 8), 54)
    full_o, full_l = oracle.attention_rect(q, k, v, 0.5, False)
    for _ in range(5):
        cuts = np.sort(g.choice(np.arange(1, 90), size=int(g.integers(1, 6)), replace=False))
        bounds = list(zip(np.r_[0, cuts], np.r_[cuts, 90]))
        parts = [oracle.attention_rect(q, k[:, :, a:b], v[:, :, a:b], 0.5, False) for a, b in bounds]
        o, l = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        if not (np.allclose(o, full_o, rtol=1e-12, atol=1e-13) and np.allclose(l, full_l, rtol=1e-13)):
            return False
    return True


def check_merge_closed_forms(merge):
    o1 = _rand((3, 4), 61)
    l1 = np.array([0.3, -2.0, 1000.0])
    # two identical parts: O unchanged, LSE + ln 2
    o, l = merge(np.stack([o1, o1]), np.stack([l1, l1]))
    if not (np.allclose(o, o1, rtol=1e-14) and np.allclose(l, l1 + math.log(2.0), rtol=1e-14)):
        return False
    # an empty part (LSE = -inf, O arbitrary) changes nothing
    o, l = merge(np.stack([o1, np.full_like(o1, 123.0)]), np.stack([l1, np.full(3, -np.inf)]))
    if not (np.allclose(o, o1, rtol=1e-14) and np.allclose(l, l1, rtol=1e-14)):
        return False
    # two parts: weights e^{l1}, e^{l2} normalised; part order does not matter
    o2 = _rand((3, 4), 62)
    l2 = np.array([1.3, -2.5, 999.0])
    o, l = merge(np.stack([o1, o2]), np.stack([l1, l2]))
    ob, lb = merge(np.stack([o2, o1]), np.stack([l2, l1]))
    w1 = 1.0 / (1.0 + np.exp(l2 - l1))
    ref = w1[:, None] * o1 + (1.0 - w1)[:, None] * o2
    return (np.allclose(o, ref, rtol=1e-12, atol=1e-14) and np.allclose(o, ob, rtol=1e-14)
            and np.allclose(l, np.logaddexp(l1, l2), rtol=1e-14) and np.allclose(l, lb, rtol=1e-15))


def test_rect_square():
    assert check_rect_square(oracle.attention_rect)


def test_rect_sdpa_fp64():
    assert check_rect_sdpa(oracle.attention_rect)


def test_rect_last_row_and_zero_keys():
    assert check_rect_last_row(oracle.attention_rect)


def test_merge_recovers_full_attention():
    assert check_merge_recovers_full(oracle.merge_attention_states)


def test_merge_closed_forms():
    assert check_merge_closed_forms(oracle.merge_attention_states)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.attention_rect(np.zeros((1, 1, 5, 4)), np.zeros((1, 1, 3, 4)), np.zeros((1, 1, 3, 4)), 1.0, True)
    with pytest.raises(ValueError):
        oracle.merge_attention_states(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))


# --------------------------------------------------------------------------
# Planted mistakes
# --------------------------------------------------------------------------

def _mut_top_left(q, k, v, scale, causal):
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        i = np.arange(q.shape[2])[:, None]
        j = np.arange(k.shape[2])[None, :]
        s = np.where(j > i, -np.inf, s)          # mistake: top-left alignment
    m = s.max(-1, keepdims=True)
    e = np.exp(s - m)
    return (e / e.sum(-1, keepdims=True)) @ v, m[..., 0] + np.log(e.sum(-1))


def _mut_merge_no_max(o_parts, lse_parts):
    w = np.exp(np.asarray(lse_parts, dtype=np.float64))      # mistake: overflows at LSE ~ 1000
    tot = w.sum(0)
    return (w[..., None] * np.asarray(o_parts)).sum(0) / tot[..., None], np.log(tot)


def _mut_merge_unnormalised(o_parts, lse_parts):
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(0)
    w = np.exp(lse_parts - m)
    return (w[..., None] * np.asarray(o_parts)).sum(0), m + np.log(w.sum(0))   # mistake: no / sum


def _mut_merge_average(o_parts, lse_parts):
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    return np.asarray(o_parts).mean(0), np.logaddexp.reduce(lse_parts, axis=0)   # mistake: plain mean


def _mut_merge_max_lse(o_parts, lse_parts):
    o, _ = oracle.merge_attention_states(o_parts, lse_parts)
    return o, np.asarray(lse_parts, dtype=np.float64).max(0)   # mistake: LSE of the largest part


RECT_CHECKS = (check_rect_square, check_rect_sdpa, check_rect_last_row)
MERGE_CHECKS = (check_merge_recovers_full, check_merge_closed_forms)


def _all_pass(checks, impl):
    with np.errstate(all="ignore"):
        res = []
        for c in checks:
            try:
                res.append(c(impl))
            except Exception:
                res.append(False)
    return all(res)


def test_pins_catch_rect_mutants():
    assert not _all_pass(RECT_CHECKS, _mut_top_left)


@pytest.mark.parametrize("mutant", [_mut_merge_no_max, _mut_merge_unnormalised, _mut_merge_average,
                                    _mut_merge_max_lse])
def test_pins_catch_merge_mutants(mutant):
    assert not _all_pass(MERGE_CHECKS, mutant)
