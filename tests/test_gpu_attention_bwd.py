"""GPU parity of fa_bwd (bf16 gradients, through the C ABI) against the float64 oracle.

The GPU path takes O and LSE from fa_fwd on the same inputs, as a caller would; the
oracle differentiates the definition directly from Q, K, V and dO.

Gate (derived from the bf16 arithmetic; the gradients have no tolerance of their own
on the pages): every gradient element g of a tensor whose float64 value is r must
satisfy |g - r| <= TOL_REL * max|r over the tensor|, with TOL_REL = 2e-2.  The bf16
operands of the products (P and dS, relative rounding <= 2^-8 each), the bf16 O that
enters D = dO . O, and the final rounding of the gradient to bf16 (<= 2^-8 relative)
give errors of a few units of 2^-8 = 3.9e-3 of the tensor's scale.  The Frobenius-norm
relative error is also bounded, by TOL_FRO = 1e-2.
"""

import numpy as np
import pytest
import torch

import online_softmax_09_amd as osm
import oracle
import workloads
from parity import need_gpu, say

pytestmark = pytest.mark.gpu

TOL_REL = 2e-2
TOL_FRO = 1e-2


def _inputs(B, H, N, d, seed):
    q, k, v = workloads.attention_inputs(B, H, N, d, seed=seed, dtype="bf16")
    do = workloads.upstream_grad(B, H, N, d, seed=seed, dtype="bf16")
    return q, k, v, do


def _gpu_grads(q, k, v, do, scale, causal, dev):
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    o, lse = osm.fa_fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = osm.fa_bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy() for t in (dq, dk, dv))


def _compare(tag, got, ref):
    ok = True
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = np.asarray(g, dtype=np.float64)
        r = np.asarray(r, dtype=np.float64)
        scale = float(np.max(np.abs(r))) if r.size else 0.0
        err = float(np.max(np.abs(g - r))) if r.size else 0.0
        nr = float(np.linalg.norm(r))
        fro = float(np.linalg.norm(g - r)) / nr if nr > 0 else float(np.linalg.norm(g))
        say(f"  {tag} {name}: max abs {err:.3e}  max|ref| {scale:.3e}  ratio {err / max(scale, 1e-30):.3e}"
            f"  fro rel {fro:.3e}")
        if scale > 0:
            ok &= err <= TOL_REL * scale and fro <= TOL_FRO
        else:
            ok &= err <= 1e-6
    return ok


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 1, 1, 64, True), (1, 1, 7, 64, False), (1, 2, 64, 64, True), (2, 1, 127, 128, True),
    (1, 2, 128, 128, False), (1, 1, 129, 64, True), (1, 1, 200, 128, True), (2, 2, 383, 64, False),
    (1, 2, 1000, 128, True), (1, 1, 1000, 64, True), (1, 1, 513, 128, False),
    # d = 128 runs its query tiles in groups of six steps plus a remainder: blocks of one
    # step (N = 33; the last key block at N = 129 and 700), every remainder 0..5 (700
    # causal: 11, 9, 7, 5, 3, 1 steps; 1000 causal: 16, 14, ..., 2), a whole group and
    # nothing more (448: 7 steps)
    (1, 1, 33, 128, True), (1, 1, 129, 128, True), (1, 1, 700, 128, True), (1, 1, 448, 128, False),
    # causal grids with a multiple of eight heads per XCD take heads in groups of four,
    # with four heads per XCD in pairs: every head's gradients compared
    (1, 64, 256, 64, True), (2, 32, 300, 128, True), (1, 32, 256, 128, True)])
def test_bwd_small_shapes(B, H, N, d, causal):
    dev = need_gpu()
    say(f"case bwd B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v, do = _inputs(B, H, N, d, seed=workloads.SEED_BASE + 7000 + N + d)
    scale = workloads.default_scale(d)
    got = _gpu_grads(q, k, v, do, scale, causal, dev)
    ref = oracle.attention_backward(q, k, v, do, scale, causal)
    assert _compare("small", got, ref)


def test_bwd_full_size_sampled_heads():
    """The bench's launch configuration (causal 2 x 32 x 8192 x 128); the oracle checks
    two whole heads (every dQ, dK and dV row of them)."""
    dev = need_gpu()
    name = "attn_bf16_causal_b2h32n8192d128"
    c = workloads.CONFIGS[name]
    say(f"case bwd full {name}")
    q, k, v = workloads.attention_inputs_for(name)
    do = workloads.upstream_grad(c["B"], c["H"], c["N"], c["d"], seed=c["seed"])
    scale = workloads.default_scale(c["d"])
    got = _gpu_grads(q, k, v, do, scale, True, dev)
    heads = [(0, 0), (1, 31)]
    ref = oracle.attention_backward(q, k, v, do, scale, True, heads=heads)
    sel = tuple(np.stack([g[b, h] for b, h in heads]) for g in got)
    assert _compare("full", sel, ref)
    # every head: the key-gradients sum to zero over keys, and the value-gradients sum
    # to the sum of dO (both follow from the rows of P summing to one)
    dk_sum = got[1].astype(np.float64).sum(axis=2)
    dv_sum = got[2].astype(np.float64).sum(axis=2)
    do_sum = do.float().numpy().astype(np.float64).sum(axis=2)
    say(f"  invariants: max |sum dK| {np.abs(dk_sum).max():.3e}  max |sum dV - sum dO| "
        f"{np.abs(dv_sum - do_sum).max():.3e}")
    assert np.abs(dk_sum).max() <= 0.5 and np.abs(dv_sum - do_sum).max() <= 0.5


def test_bwd_ragged_full_size_heads():
    """N = 8191 (ragged last tile), one head checked in full."""
    dev = need_gpu()
    B, H, N, d = 1, 2, 8191, 128
    say(f"case bwd ragged N={N}")
    q, k, v, do = _inputs(B, H, N, d, seed=workloads.SEED_BASE + 7100)
    scale = workloads.default_scale(d)
    got = _gpu_grads(q, k, v, do, scale, True, dev)
    ref = oracle.attention_backward(q, k, v, do, scale, True, heads=[(0, 1)])
    assert _compare("ragged", tuple(g[:, 1] for g in got), ref)


@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 0.5])
def test_bwd_scale_edge_cases(scale):
    dev = need_gpu()
    B, H, N, d = 1, 2, 300, 128
    say(f"case bwd scale={scale}")
    q, k, v, do = _inputs(B, H, N, d, seed=workloads.SEED_BASE + 7200)
    got = _gpu_grads(q, k, v, do, scale, True, dev)
    ref = oracle.attention_backward(q, k, v, do, scale, True)
    assert _compare(f"scale {scale}", got, ref)


def test_bwd_constant_values_give_zero_qk_gradients():
    """V with identical rows: O does not depend on Q or K, so dQ = dK = 0 (closed form)."""
    dev = need_gpu()
    B, H, N, d = 1, 1, 700, 64
    q, k, v, do = _inputs(B, H, N, d, seed=workloads.SEED_BASE + 7300)
    v = v[:, :, :1, :].expand(B, H, N, d).contiguous()
    dq, dk, dv = _gpu_grads(q, k, v, do, workloads.default_scale(d), True, dev)
    say(f"  const V: max |dQ| {np.abs(dq).max():.3e}  max |dK| {np.abs(dk).max():.3e}")
    # D = dO . O is formed from the bf16-rounded O, so dS is zero only up to that rounding
    assert np.abs(dq).max() <= 2e-2 and np.abs(dk).max() <= 2e-2


@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (64, True), (64, False)])
def test_bwd_deterministic(d, causal):
    """Two calls on the same inputs give bitwise equal gradients, for both dK/dV kernels
    (pipelined at d = 128, two phases at d = 64)."""
    dev = need_gpu()
    say(f"case bwd determinism d={d} causal={causal}")
    q, k, v, do = _inputs(1, 4, 1500, d, seed=workloads.SEED_BASE + 7400 + d)
    a = _gpu_grads(q, k, v, do, 0.09, causal, dev)
    b = _gpu_grads(q, k, v, do, 0.09, causal, dev)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
