"""Pins for the attention-gradient oracle (float64, S and P materialised).

Each check takes the implementation under test, so the same checks also run on copies
of the oracle with a planted mistake (softmax Jacobian without its row term, dS used
untransposed for dK, scale dropped from dQ, P used untransposed for dV, causal mask one
key too wide) and must fail there.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def _rand(shape, seed, sd=1.0):
    return workloads.generator(seed).normal(0.0, sd, size=shape)


def _inputs(B, H, N, d, seed):
    return tuple(_rand((B, H, N, d), seed + 10 * t) for t in range(4))


def _forward_sum(q, k, v, do, scale, causal):
    """L = sum(O * dO) for the definition, in plain float64 loops over heads."""
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        N = q.shape[2]
        j = np.arange(N)
        s = np.where(j[None, :] > j[:, None], -np.inf, s)
    m = s.max(-1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(-1, keepdims=True)
    return float(np.sum((p @ v) * do))


# --------------------------------------------------------------------------
# Pins as functions of the implementation bwd(q, k, v, do, scale, causal).
# --------------------------------------------------------------------------

def check_finite_differences(bwd):
    """Central differences of L = sum(O * dO) on a tiny case: brute force."""
    q, k, v, do = _inputs(1, 2, 5, 3, 1)
    eps = 1e-6
    for causal in (False, True):
        grads = bwd(q, k, v, do, 0.8, causal)
        for t, arr in enumerate((q, k, v)):
            num = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                plus = [x.copy() for x in (q, k, v)]
                minus = [x.copy() for x in (q, k, v)]
                plus[t][idx] += eps
                minus[t][idx] -= eps
                num[idx] = (_forward_sum(*plus, do, 0.8, causal) - _forward_sum(*minus, do, 0.8, causal)) / (2 * eps)
            if not np.allclose(grads[t], num, rtol=1e-6, atol=1e-8):
                return False
    return True


def check_autograd(bwd):
    """torch.autograd through CPU float64 scaled_dot_product_attention (library routine)."""
    for (B, H, N, d), causal, seed in (((2, 2, 33, 16), False, 4), ((2, 2, 33, 16), True, 5),
                                        ((1, 1, 130, 64), True, 6)):
        q, k, v, do = _inputs(B, H, N, d, seed)
        scale = 1.0 / math.sqrt(d)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        out.backward(torch.from_numpy(do))
        grads = bwd(q, k, v, do, scale, causal)
        for g, ref in zip(grads, (tq.grad, tk.grad, tv.grad)):
            if not np.allclose(g, ref.numpy(), rtol=1e-10, atol=1e-12):
                return False
    return True


def check_closed_forms(bwd):
    B, H, N, d = 1, 2, 40, 8
    q, k, v, do = _inputs(B, H, N, d, 21)
    scale = 0.4
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        # every row of dS sums to zero, so the key-gradients sum to zero over keys
        if not np.allclose(dk.sum(axis=2), 0.0, atol=1e-11):
            return False
        # every row of P sums to one, so the value-gradients sum to the sum of dO
        if not np.allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-12, atol=1e-12):
            return False
        # V with identical rows: O does not depend on Q or K
        vc = np.broadcast_to(v[:, :, :1, :], v.shape).copy()
        dq0, dk0, _ = bwd(q, k, vc, do, scale, causal)
        if not (np.allclose(dq0, 0.0, atol=1e-12) and np.allclose(dk0, 0.0, atol=1e-12)):
            return False
    # causal row 0 sees only key 0, so its query gradient is zero; only the last row sees
    # the last key, so that key's value gradient is P[N-1, N-1] dO_{N-1}
    dq, dk, dv = bwd(q, k, v, do, scale, True)
    if not np.allclose(dq[:, :, 0], 0.0, atol=1e-14):
        return False
    s_last = scale * np.einsum("bhjd,bhd->bhj", k, q[:, :, -1])
    p_last = np.exp(s_last - s_last.max(-1, keepdims=True))
    p_last /= p_last.sum(-1, keepdims=True)
    if not np.allclose(dv[:, :, -1], p_last[:, :, -1:] * do[:, :, -1], rtol=1e-12, atol=1e-14):
        return False
    # K = 0: uniform weights over the visible keys, dQ = 0 and dV_j = sum over the rows
    # that see key j of dO_i / |A_i|
    kz = np.zeros_like(k)
    dq, _, dv = bwd(q, kz, v, do, scale, True)
    counts = np.arange(1, N + 1)[None, None, :, None]
    ref = np.cumsum((do / counts)[:, :, ::-1], axis=2)[:, :, ::-1]
    if not (np.allclose(dq, 0.0, atol=1e-13) and np.allclose(dv, ref, rtol=1e-12, atol=1e-13)):
        return False
    return True


def check_linear_in_do(bwd):
    """Gradients are linear in the upstream gradient dO."""
    q, k, v, do = _inputs(1, 1, 17, 4, 31)
    do2 = _rand(do.shape, 77)
    a = bwd(q, k, v, do, 0.5, True)
    b = bwd(q, k, v, do2, 0.5, True)
    c = bwd(q, k, v, 2.0 * do - 3.0 * do2, 0.5, True)
    return all(np.allclose(z, 2.0 * x - 3.0 * y, rtol=1e-11, atol=1e-12) for x, y, z in zip(a, b, c))


def test_finite_differences():
    assert check_finite_differences(oracle.attention_backward)


def test_autograd_fp64():
    assert check_autograd(oracle.attention_backward)


def test_closed_forms_and_invariants():
    assert check_closed_forms(oracle.attention_backward)


def test_linear_in_upstream_gradient():
    assert check_linear_in_do(oracle.attention_backward)


def test_head_subset_and_blocking():
    q, k, v, do = _inputs(2, 3, 70, 16, 41)
    full = oracle.attention_backward(q, k, v, do, 0.25, True, block_rows=512)
    sub = oracle.attention_backward(q, k, v, do, 0.25, True, heads=[(1, 2), (0, 1)], block_rows=16)
    for g, s in zip(full, sub):
        assert np.allclose(s[0], g[1, 2], rtol=1e-13, atol=1e-14)
        assert np.allclose(s[1], g[0, 1], rtol=1e-13, atol=1e-14)


def test_accepts_bf16_torch_exactly():
    q, k, v = workloads.attention_inputs(1, 1, 40, 64, seed=9, dtype="bf16")
    do = workloads.attention_inputs(1, 1, 40, 64, seed=10, dtype="bf16")[0]
    a = oracle.attention_backward(q, k, v, do, 0.125, True)
    b = oracle.attention_backward(*(t.float().numpy() for t in (q, k, v, do)), 0.125, True)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_rejects_bad_shapes():
    z = np.zeros((1, 1, 4, 8))
    with pytest.raises(ValueError):
        oracle.attention_backward(z, z, z, np.zeros((1, 1, 5, 8)), 1.0, False)
    with pytest.raises(ValueError):
        oracle.attention_backward(z, z, z, z, 1.0, False, heads=[(0, 1)])


# --------------------------------------------------------------------------
# Planted mistakes: each must fail at least one pin.
# --------------------------------------------------------------------------

def _materialised(q, k, v, do, scale, causal, mask_shift=0):
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        j = np.arange(q.shape[2])
        s = np.where(j[None, :] > j[:, None] + mask_shift, -np.inf, s)
    m = s.max(-1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(-1, keepdims=True)
    dp = do @ np.swapaxes(v, 2, 3)
    return q, k, v, do, p, dp


def _mut_no_row_term(q, k, v, do, scale, causal):
    q, k, v, do, p, dp = _materialised(q, k, v, do, scale, causal)
    ds = p * dp                                   # mistake: Jacobian row term dropped
    return scale * ds @ k, scale * np.swapaxes(ds, 2, 3) @ q, np.swapaxes(p, 2, 3) @ do


def _mut_dk_untransposed(q, k, v, do, scale, causal):
    q, k, v, do, p, dp = _materialised(q, k, v, do, scale, causal)
    ds = p * (dp - np.sum(p * dp, -1, keepdims=True))
    return scale * ds @ k, scale * ds @ q, np.swapaxes(p, 2, 3) @ do   # mistake: ds not transposed


def _mut_dq_no_scale(q, k, v, do, scale, causal):
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal)
    return dq / scale, dk, dv


def _mut_dv_untransposed(q, k, v, do, scale, causal):
    dq, dk, _ = oracle.attention_backward(q, k, v, do, scale, causal)
    _, _, _, do_, p, _ = _materialised(q, k, v, do, scale, causal)
    return dq, dk, p @ do_                        # mistake: P instead of P^T


def _mut_mask_wide(q, k, v, do, scale, causal):
    q, k, v, do, p, dp = _materialised(q, k, v, do, scale, causal, mask_shift=1)
    ds = p * (dp - np.sum(p * dp, -1, keepdims=True))
    return scale * ds @ k, scale * np.swapaxes(ds, 2, 3) @ q, np.swapaxes(p, 2, 3) @ do


ALL_CHECKS = (check_finite_differences, check_autograd, check_closed_forms, check_linear_in_do)


@pytest.mark.parametrize("mutant", [_mut_no_row_term, _mut_dk_untransposed, _mut_dq_no_scale,
                                    _mut_dv_untransposed, _mut_mask_wide])
def test_pins_catch_backward_mutants(mutant):
    with np.errstate(all="ignore"):
        results = []
        for chk in ALL_CHECKS:
            try:
                results.append(chk(mutant))
            except Exception:
                results.append(False)
    assert not all(results)
