"""Pins for the row-softmax oracle and the scalar online-normaliser instruments.

Each pin is a ``check_*`` function taking the implementation under test, so the
same check runs on the oracle (must pass) and on copies with a planted mistake
(must fail): this shows the pins catch a dropped term, a wrong sign or a missing
rescale, not only that the oracle agrees with itself.
"""

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Independent high-precision brute force (50-digit decimal), tiny inputs only.
# --------------------------------------------------------------------------

def _dec_exp(x):
    return Decimal(x).exp()


def _dec_softmax(row):
    getcontext().prec = 50
    m = max(Decimal(float(a)) for a in row)
    e = [(Decimal(float(a)) - m).exp() for a in row]
    tot = sum(e)
    return [float(t / tot) for t in e], float(m + tot.ln())


def _dec_weighted(scores, values):
    getcontext().prec = 50
    w = [Decimal(float(s)).exp() for s in scores]
    return float(sum(wi * Decimal(float(v)) for wi, v in zip(w, values)) / sum(w))


# --------------------------------------------------------------------------
# Pins as functions of the implementation.
# --------------------------------------------------------------------------

def check_worked_row(weighted):
    """The pages' worked row prints 25.752104 and survives a +1000 shift."""
    g = _golden("worked_row.json")
    a = weighted(g["scores"], g["values"])
    if round(a, g["printed_decimals"]) != g["printed"]:
        return False
    exact = _dec_weighted(g["scores"], g["values"])
    if not math.isclose(a, exact, rel_tol=g["rel_tol"]):
        return False
    for shift in (g["shift"], -g["shift"]):
        b = weighted([s + shift for s in g["scores"]], g["values"])
        if not math.isclose(b, a, rel_tol=g["rel_tol"]):
            return False
    return True


def check_random_rows(weighted):
    """Online vs all-weights-first on the 390 random rows, rel 1e-12."""
    g = _golden("random_rows.json")
    rows = [r for r in workloads.scalar_rows() if r[0].startswith("len")]
    assert len(rows) == g["count"]
    lengths = {len(s) for _, s, _ in rows}
    assert min(lengths) == g["min_length"] and max(lengths) == g["max_length"]
    for _, s, v in rows:
        if not math.isclose(weighted(s, v), oracle.weighted_full(s, v),
                            rel_tol=g["rel_tol"], abs_tol=1e-12):
            return False
    return True


def check_softmax_rows(softmax_rows):
    """Tiny rows vs 50-digit brute force; all-equal and single-element exact."""
    g = workloads.generator(11)
    for n in (1, 2, 3, 5, 8):
        for _ in range(5):
            row = g.normal(0.0, 3.0, size=n)
            y, m, l = softmax_rows(row[None, :])
            ref, lse = _dec_softmax(row)
            if not np.allclose(y[0], ref, rtol=1e-14, atol=1e-300):
                return False
            if not math.isclose(m[0] + math.log(l[0]), lse, rel_tol=1e-14, abs_tol=1e-14):
                return False
    y, _, _ = softmax_rows(np.full((2, 4096), 7.25))
    if not np.all(y == 1.0 / 4096):
        return False
    y, _, _ = softmax_rows(np.array([[-3.5], [1000.0]]))
    if not np.all(y == 1.0):
        return False
    # very large positive / negative entries: finite and shift-invariant
    row = g.normal(0.0, 3.0, size=64)
    y0, _, _ = softmax_rows(row[None, :])
    for sh in (1000.0, -1000.0, 1e6):
        y1, _, _ = softmax_rows((row + sh)[None, :])
        if not np.all(np.isfinite(y1)) or not np.allclose(y1, y0, rtol=1e-9, atol=1e-15):
            return False
    return True


def _random_chunks(g, n, k):
    cuts = np.sort(g.choice(np.arange(1, n), size=k - 1, replace=False)) if k > 1 else []
    return np.split(np.arange(n), cuts)


def check_merge_order(online_state, merge_state):
    """Chunk a row, merge in four orders; all match the whole-row (m, l)."""
    g = workloads.generator(12)
    ident = (-math.inf, 0.0)
    for trial in range(60):
        n = int(g.integers(2, 200))
        x = g.normal(0.0, 3.0, size=n)
        if trial % 3 == 0:
            x[g.integers(0, n)] += 1000.0
        _, m_ref, l_ref = oracle.softmax_rows(x[None, :])
        k = int(g.integers(1, min(n, 12) + 1))
        states = [online_state(x[c]) for c in _random_chunks(g, n, k)]
        left = ident
        for s in states:
            left = merge_state(left, s)
        right = ident
        for s in reversed(states):
            right = merge_state(s, right)
        level = list(states)
        while len(level) > 1:
            nxt = [merge_state(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
            if len(level) % 2:
                nxt.append(level[-1])
            level = nxt
        tree = level[0]
        pool = list(states)
        while len(pool) > 1:
            i, j = sorted(g.choice(len(pool), size=2, replace=False))
            b = pool.pop(j)
            a = pool.pop(i)
            pool.append(merge_state(a, b) if g.random() < 0.5 else merge_state(b, a))
        rnd = pool[0]
        for m, l in (left, right, tree, rnd):
            if m != m_ref[0] or not math.isclose(l, l_ref[0], rel_tol=1e-12):
                return False
    # identity on both sides, and of two empty states
    s = online_state([0.5, -1.0])
    if merge_state(ident, s) != s or merge_state(s, ident) != s:
        return False
    m, l = merge_state(ident, ident)
    return m == -math.inf and l == 0.0


# --------------------------------------------------------------------------
# The oracle passes every pin.
# --------------------------------------------------------------------------

def test_worked_row_online():
    assert check_worked_row(lambda s, v: oracle.online_weighted(s, v)[0])


def test_worked_row_full_weights():
    assert check_worked_row(oracle.weighted_full)


def test_worked_row_lse_and_probabilities():
    # softmax of [0, 1, 2]: closed form probabilities e^i / (1 + e + e^2) via decimal
    y, m, l = oracle.softmax_rows(np.array([[0.0, 1.0, 2.0]]))
    ref, lse = _dec_softmax([0.0, 1.0, 2.0])
    assert np.allclose(y[0], ref, rtol=1e-15)
    assert math.isclose(m[0] + math.log(l[0]), lse, rel_tol=1e-15)
    assert math.isclose(lse, 2.40760596444438, rel_tol=1e-13)


def test_random_rows_online_vs_full():
    assert check_random_rows(lambda s, v: oracle.online_weighted(s, v)[0])


def test_online_weighted_state_matches_three_scans():
    for _, s, _v in workloads.scalar_rows():
        _, m, l = oracle.online_weighted(s, _v)
        _, m3, l3 = oracle.softmax_rows(np.array(s)[None, :])
        assert m == m3[0]
        assert math.isclose(l, l3[0], rel_tol=1e-12)


def test_softmax_rows_pins():
    assert check_softmax_rows(oracle.softmax_rows)


def test_softmax_rows_vs_torch_fp64():
    x = torch.from_numpy(workloads.generator(5).normal(0.0, 3.0, size=(40, 333)))
    y, m, l = oracle.softmax_rows(x.numpy())
    assert np.allclose(y, torch.softmax(x, dim=-1).numpy(), rtol=1e-13, atol=1e-300)
    assert np.allclose(m + np.log(l), torch.logsumexp(x, dim=-1).numpy(), rtol=1e-14)
    assert np.allclose(oracle.logsumexp_rows(x.numpy()), torch.logsumexp(x, dim=-1).numpy(),
                       rtol=1e-14)


def test_softmax_rows_empty_row_rejected():
    with pytest.raises(ValueError):
        oracle.softmax_rows(np.zeros((3, 0)))


def test_online_state_matches_three_scans():
    g = workloads.generator(13)
    for n in (1, 2, 7, 64, 1000):
        x = g.normal(0.0, 3.0, size=n)
        m, l = oracle.online_state(x)
        _, m3, l3 = oracle.softmax_rows(x[None, :])
        assert m == m3[0] and math.isclose(l, l3[0], rel_tol=1e-12)
    assert oracle.online_state([]) == (-math.inf, 0.0)


def test_merge_state_order_independence():
    assert check_merge_order(oracle.online_state, oracle.merge_state)


def test_rescale_factor_printed():
    g = _golden("rescale_factor.json")
    # the factor that moves a sum from base m_old to base m_new: state (m_old, 1)
    # merged with an empty-valued state at m_new has l = exp(m_old - m_new)
    m, l = oracle.merge_state((g["m_old"], 1.0), (g["m_new"], 0.0))
    assert m == g["m_new"]
    assert round(l, g["printed_decimals"]) == g["printed"]
    getcontext().prec = 50
    assert math.isclose(l, float((Decimal(g["m_old"]) - Decimal(g["m_new"])).exp()),
                        rel_tol=1e-15)


def test_averaging_block_softmaxes_is_not_the_softmax():
    # lihaoran.work note, "why per-block softmaxes cannot be averaged": per-block
    # normalised results cannot simply be averaged; merging the states is right.
    g = workloads.generator(14)
    x = g.normal(0.0, 3.0, size=40)
    v = g.uniform(-10, 10, size=40)
    a, b = slice(0, 15), slice(15, 40)
    wa, _, _ = oracle.softmax_rows(x[a][None, :])
    wb, _, _ = oracle.softmax_rows(x[b][None, :])
    averaged = 0.5 * (wa[0] @ v[a] + wb[0] @ v[b])
    truth = oracle.weighted_full(x, v)
    assert abs(averaged - truth) > 1e-3
    # the merged states reproduce the truth
    sa, sb = oracle.online_state(x[a]), oracle.online_state(x[b])
    m, l = oracle.merge_state(sa, sb)
    ua = math.fsum(math.exp(t - m) * vv for t, vv in zip(x[a], v[a]))
    ub = math.fsum(math.exp(t - m) * vv for t, vv in zip(x[b], v[b]))
    assert math.isclose((ua + ub) / l, truth, rel_tol=1e-12)


# --------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle fails at least one pin.
# --------------------------------------------------------------------------

def _weighted_no_u_rescale(scores, values):
    # mistake: l is rescaled when the maximum moves but u is not
    m, l, u = -math.inf, 0.0, 0.0
    for a, v in zip(scores, values):
        mn = max(m, a)
        c = 0.0 if m == -math.inf else math.exp(m - mn)
        w = math.exp(a - mn)
        l, u, m = c * l + w, u + w * v, mn
    return u / l


def _weighted_sign_flip(scores, values):
    # mistake: exp(m' - m) instead of exp(m - m')
    m, l, u = -math.inf, 0.0, 0.0
    for a, v in zip(scores, values):
        mn = max(m, a)
        c = 0.0 if m == -math.inf else math.exp(mn - m)
        w = math.exp(a - mn)
        l, u, m = c * l + w, c * u + w * v, mn
    return u / l


def _weighted_no_max(scores, values):
    # mistake: no max subtraction (overflows for large scores)
    try:
        w = [math.exp(a) for a in scores]
    except OverflowError:
        return float("nan")
    return math.fsum(x * v for x, v in zip(w, values)) / math.fsum(w)


def _softmax_no_max(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(x)
        l = e.sum(axis=-1, keepdims=True)
        return e / l, np.zeros(x.shape[:-1]), l[..., 0]


def _softmax_drop_last(x):
    # mistake: the sum skips the last element (an off-by-one)
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    l = np.exp(x[..., :-1] - m).sum(axis=-1, keepdims=True)
    l = np.where(l == 0, 1.0, l)
    return np.exp(x - m) / l, m[..., 0], l[..., 0]


def _merge_one_sided(a, b):
    # mistake: only the first state is moved to the new base
    m = max(a[0], b[0])
    if m == -math.inf:
        return m, 0.0
    da = 0.0 if a[0] == -math.inf else math.exp(a[0] - m)
    return m, a[1] * da + b[1]


@pytest.mark.parametrize("mutant", [_weighted_no_u_rescale, _weighted_sign_flip, _weighted_no_max])
def test_pins_catch_weighted_mutants(mutant):
    assert not (check_worked_row(mutant) and check_random_rows(mutant))


@pytest.mark.parametrize("mutant", [_softmax_no_max, _softmax_drop_last])
def test_pins_catch_softmax_mutants(mutant):
    assert not check_softmax_rows(mutant)


def test_pins_catch_merge_mutant():
    assert not check_merge_order(oracle.online_state, _merge_one_sided)


def test_masked_entries():
    """Entries of -inf (masked) get probability exactly 0, and the others equal the softmax
    of the finite entries alone (e^-inf = 0 adds nothing to the normaliser); a row with one
    finite entry is one-hot; a row of -inf only has normaliser 0 and gives NaN."""
    g = np.random.default_rng(workloads.SEED_BASE + 4700)
    x = g.normal(0.0, 3.0, size=(6, 50))
    mask = g.random(size=x.shape) < 0.5
    mask[:, 7] = False  # every row keeps a finite entry
    xm = np.where(mask, -np.inf, x)
    y, m, l = oracle.softmax_rows(xm)
    assert np.all(y[mask] == 0.0)
    for r in range(x.shape[0]):
        keep = ~mask[r]
        ref, _, _ = oracle.softmax_rows(x[r, keep])
        np.testing.assert_allclose(y[r, keep], ref, rtol=1e-15, atol=0)
        ref_t = torch.softmax(torch.from_numpy(xm[r]), dim=0).numpy()
        np.testing.assert_allclose(y[r], ref_t, rtol=1e-13, atol=1e-300)
    one = np.full((1, 9), -np.inf)
    one[0, 4] = 2.5
    y1, _, _ = oracle.softmax_rows(one)
    assert y1[0, 4] == 1.0 and np.all(np.delete(y1[0], 4) == 0.0)
    with np.errstate(invalid="ignore"):
        yn, _, ln = oracle.softmax_rows(np.full((1, 5), -np.inf))
    assert np.all(np.isnan(yn))
