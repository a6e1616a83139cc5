"""Pins for the attention oracle (float64, S materialised).

As for the softmax pins, each check takes the implementation under test, so the same
checks also run on copies of the oracle with a planted mistake (wrong mask index,
scale dropped, K used untransposed, softmax over the wrong axis, V rows permuted)
and must fail there.
"""

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads


def _rand(shape, seed, sd=1.0):
    return workloads.generator(seed).normal(0.0, sd, size=shape)


# --------------------------------------------------------------------------
# Independent brute force: Python loops, math.fsum, 50-digit decimal LSE.
# --------------------------------------------------------------------------

def _brute(q, k, v, scale, causal):
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    getcontext().prec = 50
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                s = [scale * math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t]) for t in range(d))
                     for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for t in range(d):
                    o[b, h, i, t] = math.fsum(wj * float(v[b, h, j, t]) for wj, j in zip(w, keys)) / tot
                lse[b, h, i] = float(sum(Decimal(x).exp() for x in s).ln())
    return o, lse


# --------------------------------------------------------------------------
# Pins as functions of the implementation attention(q, k, v, scale, causal).
# --------------------------------------------------------------------------

def check_brute_force(attn):
    q, k, v = _rand((1, 2, 6, 3), 1), _rand((1, 2, 6, 3), 2), _rand((1, 2, 6, 3), 3)
    for causal in (False, True):
        o, lse = attn(q, k, v, 0.7, causal)
        ob, lb = _brute(q, k, v, 0.7, causal)
        if not (np.allclose(o, ob, rtol=1e-12, atol=1e-13) and np.allclose(lse, lb, rtol=1e-12, atol=1e-13)):
            return False
    return True


def check_sdpa(attn):
    """CPU float64 scaled_dot_product_attention is the library routine for O."""
    for (B, H, N, d), causal, seed in (((2, 3, 37, 16), False, 4), ((2, 3, 37, 16), True, 5),
                                        ((1, 2, 129, 64), True, 6)):
        q, k, v = (_rand((B, H, N, d), seed + 10 * t) for t in range(3))
        scale = 1.0 / math.sqrt(d)
        o, _ = attn(q, k, v, scale, causal)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                             torch.from_numpy(v), is_causal=causal, scale=scale)
        if not np.allclose(o, ref.numpy(), rtol=1e-11, atol=1e-12):
            return False
    return True


def check_closed_forms(attn):
    B, H, N, d = 1, 2, 50, 8
    q, k, v = _rand((B, H, N, d), 21), _rand((B, H, N, d), 22), _rand((B, H, N, d), 23)
    # V identical rows: every output row equals that row
    vc = np.broadcast_to(v[:, :, :1, :], v.shape).copy()
    for causal in (False, True):
        o, _ = attn(q, k, vc, 0.3, causal)
        if not np.allclose(o, vc, rtol=1e-13, atol=1e-13):
            return False
    # K = 0: uniform weights -> O_i is the mean of the visible V rows, LSE = ln |A_i|
    kz = np.zeros_like(k)
    o, lse = attn(q, kz, v, 0.3, True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    if not (np.allclose(o, prefix, rtol=1e-12, atol=1e-13)
            and np.allclose(lse, np.log(np.arange(1, N + 1))[None, None, :], rtol=1e-13, atol=1e-13)):
        return False
    o, lse = attn(q, kz, v, 0.3, False)
    if not (np.allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-13)
            and np.allclose(lse, math.log(N), rtol=1e-14)):
        return False
    # causal row 0 sees only key 0: O_0 = V_0 and LSE_0 = scale * q_0 . k_0
    o, lse = attn(q, k, v, 0.3, True)
    if not (np.array_equal(o[:, :, 0], v[:, :, 0])
            and np.allclose(lse[:, :, 0], 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                            rtol=1e-14, atol=1e-15)):
        return False
    # non-causal: permuting key/value rows together changes nothing
    perm = workloads.generator(24).permutation(N)
    o1, l1 = attn(q, k, v, 0.3, False)
    o2, l2 = attn(q, k[:, :, perm], v[:, :, perm], 0.3, False)
    return np.allclose(o1, o2, rtol=1e-12, atol=1e-13) and np.allclose(l1, l2, rtol=1e-13)


def worked_example_inputs(d=64, shift=False):
    """The pages' worked row embedded in attention: N = 3, scale = 1.

    q_i = e_1 (+ e_2 when shifted), k_j = j e_1 (+ 1000 e_2), v_j = 10 (j + 1) e_1, so
    row i has scores [0, 1, 2] (+1000) and values [10, 20, 30] in column 0.
    """
    q = np.zeros((1, 1, 3, d))
    k = np.zeros((1, 1, 3, d))
    v = np.zeros((1, 1, 3, d))
    q[..., 0] = 1.0
    for j in range(3):
        k[0, 0, j, 0] = j
        v[0, 0, j, 0] = 10.0 * (j + 1)
    if shift:
        q[..., 1] = 1.0
        k[..., 1] = 1000.0
    return q, k, v


def check_worked_example(attn):
    getcontext().prec = 50
    e = [Decimal(j).exp() for j in range(3)]
    o_exact = float(sum(ej * 10 * (j + 1) for j, ej in enumerate(e)) / sum(e))
    lse_exact = float(sum(e).ln())
    for shift in (False, True):
        o, lse = attn(*worked_example_inputs(shift=shift), 1.0, False)
        if round(float(o[0, 0, 0, 0]), 6) != 25.752104:
            return False
        if not np.allclose(o[0, 0, :, 0], o_exact, rtol=1e-12):
            return False
        if not np.all(o[0, 0, :, 1:] == 0.0):
            return False
        if not np.allclose(lse[0, 0], lse_exact + (1000.0 if shift else 0.0), rtol=1e-13):
            return False
    return True


def test_brute_force():
    assert check_brute_force(oracle.attention)


def test_sdpa_fp64():
    assert check_sdpa(oracle.attention)


def test_closed_forms():
    assert check_closed_forms(oracle.attention)


def test_worked_example_embedded():
    assert check_worked_example(oracle.attention)


def test_rows_subset_matches_full():
    B, H, N, d = 2, 3, 70, 16
    q, k, v = _rand((B, H, N, d), 31), _rand((B, H, N, d), 32), _rand((B, H, N, d), 33)
    o, lse = oracle.attention(q, k, v, 0.25, True)
    rows = workloads.sampled_query_rows(B, H, N, 10, seed=3)
    os_, ls_ = oracle.attention_rows(q, k, v, 0.25, True, rows=rows, block_rows=4)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(os_[b, h], o[b, h, rows[b, h]])
            assert np.array_equal(ls_[b, h], lse[b, h, rows[b, h]])
    r1 = np.array([0, 5, 69])
    o1, l1 = oracle.attention_rows(q, k, v, 0.25, True, rows=r1)
    assert np.array_equal(o1, o[:, :, r1]) and np.array_equal(l1, lse[:, :, r1])


def test_accepts_bf16_torch_exactly():
    q, k, v = workloads.attention_inputs(1, 1, 40, 64, seed=9, dtype="bf16")
    o_t, l_t = oracle.attention(q, k, v, 0.125, True)
    o_n, l_n = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), 0.125, True)
    assert np.array_equal(o_t, o_n) and np.array_equal(l_t, l_n)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((1, 1, 4, 8)), np.zeros((1, 1, 5, 8)), np.zeros((1, 1, 4, 8)), 1.0, False)
    with pytest.raises(ValueError):
        oracle.attention_rows(np.zeros((1, 1, 4, 8)), np.zeros((1, 1, 4, 8)), np.zeros((1, 1, 4, 8)),
                              1.0, False, rows=[4])


# --------------------------------------------------------------------------
# Planted mistakes: each must fail at least one pin.
# --------------------------------------------------------------------------

def _mut_mask_off_by_one(q, k, v, scale, causal):
    # mistake: query i also sees key i + 1
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    N = q.shape[2]
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        j = np.arange(N)
        s = np.where(j[None, :] > j[:, None] + 1, -np.inf, s)
    m = s.max(-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(-1, keepdims=True)
    return (e / l) @ v, m[..., 0] + np.log(l[..., 0])


def _mut_no_scale(q, k, v, scale, causal):
    return oracle.attention(q, k, v, 1.0, causal)


def _mut_k_untransposed(q, k, v, scale, causal):
    # mistake: contracts q with k's columns as if k were stored [d, N] (square case)
    k = np.asarray(k, dtype=np.float64)
    if k.shape[2] == k.shape[3]:
        k = np.swapaxes(k, 2, 3)
    else:
        k = k[:, :, ::-1]
    return oracle.attention(q, k, v, scale, causal)


def _mut_wrong_axis(q, k, v, scale, causal):
    # mistake: softmax normalised over queries instead of keys
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    N = q.shape[2]
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        j = np.arange(N)
        s = np.where(j[None, :] > j[:, None], -np.inf, s)
    m = s.max(-2, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(-2, keepdims=True)
    mm = s.max(-1)
    return (e / l) @ v, mm + np.log(np.exp(s - mm[..., None]).sum(-1))


def _mut_lse_log2(q, k, v, scale, causal):
    o, lse = oracle.attention(q, k, v, scale, causal)
    return o, lse / math.log(2.0)


def _mut_v_shifted(q, k, v, scale, causal):
    # mistake: the value rows are taken one position late (wrong index)
    v = np.asarray(v, dtype=np.float64)
    return oracle.attention(q, k, np.roll(v, 1, axis=2), scale, causal)


ALL_CHECKS = (check_brute_force, check_sdpa, check_closed_forms, check_worked_example)


@pytest.mark.parametrize("mutant", [_mut_mask_off_by_one, _mut_no_scale, _mut_k_untransposed,
                                    _mut_wrong_axis, _mut_lse_log2, _mut_v_shifted])
def test_pins_catch_attention_mutants(mutant):
    with np.errstate(all="ignore"):
        results = []
        for chk in ALL_CHECKS:
            try:
                results.append(chk(mutant))
            except Exception:
                results.append(False)
    assert not all(results)
