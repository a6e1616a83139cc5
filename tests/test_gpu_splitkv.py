"""GPU parity of fa_fwd_splitkv and attn_merge_states (through the C ABI) against the
float64 oracle (attention_rect, merge_attention_states).

Gates: the attention outputs take the forward's bf16 gates (O max abs <= 2e-2, LSE max
abs <= 1e-2).  The merge of given float32 partials is exact up to float32 rounding before
the single bf16 rounding of O: O within 2e-2 absolute (one bf16 rounding of |O| < 4 plus
float32 noise), LSE within 1e-5 + 2^-22 |LSE| (a few float32 ulps, which at LSE ~ 1000
exceeds 1e-5).
"""

import numpy as np
import pytest
import torch

import online_softmax_09_amd as osm
import oracle
import workloads
from parity import TOL_BF16_LSE, TOL_BF16_O, max_abs, need_gpu, say, split_bounds

pytestmark = pytest.mark.gpu


def _gpu_splitkv(q, k, v, scale, causal, n_splits, dev):
    o, lse = osm.fa_fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal, n_splits=n_splits)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,n_splits", [
    (1, 2, 1, 1000, 128, True, 4), (1, 2, 1, 1000, 128, False, 1), (2, 3, 5, 777, 64, True, 7),
    (1, 1, 32, 4096, 128, True, 16), (1, 2, 40, 300, 64, False, 3), (1, 1, 1, 1, 64, True, 1),
    (1, 1, 3, 3, 128, True, 2), (1, 1, 1, 64, 128, True, 8), (1, 1, 7, 100, 64, True, 4096),
    (2, 2, 16, 2049, 128, True, 32), (1, 1, 33, 33, 128, True, 3), (1, 2, 70, 50, 128, False, 2),
    (1, 3, 1, 4999, 64, False, 5), (2, 2, 1, 3000, 128, True, 40), (1, 1, 1, 300, 64, True, 64),
    # at least two blocks per CU on 256 CUs (512 blocks): the multi-query kernel waits for
    # the next K copy as well as the current sub-tile's (the cases above keep both in flight)
    (2, 64, 20, 2000, 64, True, 4), (1, 128, 33, 2049, 128, True, 2), (1, 128, 40, 1500, 64, False, 2)])
def test_splitkv_shapes(B, H, Nq, Nk, d, causal, n_splits):
    dev = need_gpu()
    say(f"case splitkv B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} n_splits={n_splits}")
    q, k, v = workloads.decode_inputs(B, H, Nq, Nk, d, seed=workloads.SEED_BASE + 8000 + Nq + Nk + d)
    scale = workloads.default_scale(d)
    o, lse = _gpu_splitkv(q, k, v, scale, causal, n_splits, dev)
    o_ref, lse_ref = oracle.attention_rect(q, k, v, scale, causal)
    eo, el = max_abs(o, o_ref), max_abs(lse, lse_ref)
    say(f"  O max abs {eo:.3e}  LSE max abs {el:.3e}")
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


@pytest.mark.parametrize("name", ["decode_bf16_b1h8q1k131072d128", "decode_bf16_b4h32q16k32768d128"])
def test_splitkv_decode_workloads(name):
    """The bench's decode configurations, every output row against the oracle."""
    dev = need_gpu()
    c = workloads.CONFIGS[name]
    say(f"case splitkv {name}")
    q, k, v = workloads.decode_inputs_for(name)
    scale = workloads.default_scale(c["d"])
    o, lse = _gpu_splitkv(q, k, v, scale, c["causal"], c["n_splits"], dev)
    o_ref = np.empty(o.shape)
    lse_ref = np.empty(lse.shape)
    for b in range(c["B"]):  # one batch at a time bounds host memory
        o_ref[b:b + 1], lse_ref[b:b + 1] = oracle.attention_rect(q[b:b + 1], k[b:b + 1], v[b:b + 1], scale,
                                                                 c["causal"])
    eo, el = max_abs(o, o_ref), max_abs(lse, lse_ref)
    say(f"  O max abs {eo:.3e}  LSE max abs {el:.3e}")
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


def test_splitkv_matches_square_forward():
    """With Nq = Nk, bottom-right and top-left alignment coincide: fa_fwd_splitkv agrees
    with fa_fwd within the bf16 gates, for several part counts."""
    dev = need_gpu()
    q, k, v = workloads.attention_inputs(1, 2, 500, 128, seed=workloads.SEED_BASE + 8100)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o0, l0 = osm.fa_fwd(qd, kd, vd, causal=True)
    for n in (1, 3, 8):
        o1, l1 = osm.fa_fwd_splitkv(qd, kd, vd, causal=True, n_splits=n)
        torch.cuda.synchronize()
        eo = max_abs(o1.float().cpu().numpy(), o0.float().cpu().numpy())
        el = max_abs(l1.cpu().numpy(), l0.cpu().numpy())
        say(f"  n_splits={n}: vs fa_fwd O {eo:.3e} LSE {el:.3e}")
        assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


@pytest.mark.parametrize("n_parts,rows,d", [(1, 5, 64), (2, 9, 128), (7, 33, 64), (256, 8, 128), (1000, 3, 128)])
def test_merge_states(n_parts, rows, d):
    dev = need_gpu()
    say(f"case merge n_parts={n_parts} rows={rows} d={d}")
    op, lp = workloads.merge_parts(n_parts, rows, d, seed=workloads.SEED_BASE + 8200 + n_parts + rows)
    o, lse = osm.attn_merge_states(op.to(dev), lp.to(dev))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.merge_attention_states(op.numpy(), lp.numpy())
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    eo = max_abs(o, o_ref)
    el = float(np.max(np.abs(lse - lse_ref) - 2.0 ** -22 * np.abs(lse_ref)))
    say(f"  O max abs {eo:.3e}  LSE excess over 2^-22 |LSE| {el:.3e}")
    assert eo <= TOL_BF16_O and el <= 1e-5


def test_splitkv_deterministic():
    dev = need_gpu()
    q, k, v = workloads.decode_inputs(2, 4, 3, 5000, 128, seed=workloads.SEED_BASE + 8300)
    a = _gpu_splitkv(q, k, v, 0.09, True, 17, dev)
    b = _gpu_splitkv(q, k, v, 0.09, True, 17, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,H,Nq,Nk,d,n_splits", [(1, 2, 3, 1000, 128, 4), (1, 1, 5, 300, 64, 16),
                                                  (1, 2, 1, 1000, 64, 4), (1, 1, 1, 2000, 128, 3)])
def test_splitkv_scales(scale, causal, B, H, Nq, Nk, d, n_splits):
    """The partial kernels' own scale handling (negated Q for a negative scale, c = |scale|
    log2 e) at scale 0 (uniform weights over the visible keys), a negative scale and a
    large one, for the multi-query kernel and the one-query kernel.  n_splits = 16 over
    300 keys leaves trailing parts empty."""
    dev = need_gpu()
    say(f"case splitkv scale={scale} causal={causal} B={B} H={H} Nq={Nq} Nk={Nk} d={d} n_splits={n_splits}")
    q, k, v = workloads.decode_inputs(B, H, Nq, Nk, d, seed=workloads.SEED_BASE + 8400 + Nk + d)
    o, lse = _gpu_splitkv(q, k, v, scale, causal, n_splits, dev)
    o_ref, lse_ref = oracle.attention_rect(q, k, v, scale, causal)
    eo, el = max_abs(o, o_ref), max_abs(lse, lse_ref)
    say(f"  O max abs {eo:.3e}  LSE max abs {el:.3e}")
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_merge_states_of_partials_at_scales(scale):
    """attn_merge_states on partial results the oracle computes over disjoint key ranges
    (a causal split with empty parts) at the same scales: the merge recovers the oracle's
    attention over all keys."""
    dev = need_gpu()
    say(f"case merge of oracle partials scale={scale}")
    B, H, Nq, Nk, d, n = 1, 2, 4, 700, 128, 8  # parts of 128 keys: the last two are empty
    q, k, v = workloads.decode_inputs(B, H, Nq, Nk, d, seed=workloads.SEED_BASE + 8500)
    qn, kn, vn = (t.float().numpy().astype(np.float64) for t in (q, k, v))
    rows = B * H * Nq
    o_parts = np.zeros((n, rows, d))
    lse_parts = np.full((n, rows), -np.inf)
    for p, (lo, hi) in enumerate(split_bounds(Nk, n)):
        for i in range(Nq):
            e = min(hi, Nk - Nq + i + 1)
            if e <= lo:
                continue
            op, lp = oracle.attention_rect(qn[:, :, i:i + 1], kn[:, :, lo:e], vn[:, :, lo:e], scale, False)
            o_parts[p, i::Nq] = op.reshape(B * H, d)
            lse_parts[p, i::Nq] = lp.reshape(B * H)
    o_ref, lse_ref = oracle.attention_rect(q, k, v, scale, True)
    o, lse = osm.attn_merge_states(torch.from_numpy(o_parts).float().to(dev),
                                   torch.from_numpy(lse_parts).float().to(dev))
    torch.cuda.synchronize()
    eo = max_abs(o.float().cpu().numpy().reshape(B, H, Nq, d), o_ref)
    el = max_abs(lse.cpu().numpy().reshape(B, H, Nq), lse_ref)
    say(f"  O max abs {eo:.3e}  LSE max abs {el:.3e}")
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


@pytest.mark.parametrize("Nq", [5, 1])
@pytest.mark.parametrize("causal", [True, False])
def test_splitkv_partials_follow_the_part_contract(causal, Nq):
    """The workspace after a call holds each part's normalised output and LSE over exactly
    the keys [lo, hi) the header states (64-key multiples), with (0, -inf) for a row that
    sees no key of its part (multi-query and one-query kernels)."""
    dev = need_gpu()
    B, H, Nk, d = 1, 2, 1000, 128
    n = 6 if Nq > 1 else 24  # one query: 64-key parts, the last eight empty
    say(f"case splitkv partials causal={causal} B={B} H={H} Nq={Nq} Nk={Nk} d={d} n_splits={n}")
    q, k, v = workloads.decode_inputs(B, H, Nq, Nk, d, seed=workloads.SEED_BASE + 8600)
    scale = workloads.default_scale(d)
    rows = B * H * Nq
    ws = torch.empty(osm._lib.load().fa_fwd_splitkv_workspace_bytes(B, H, Nq, d, n) // 4, dtype=torch.float32,
                     device=dev)
    osm.fa_fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal, n_splits=n, workspace=ws)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    o_parts = w[:n * rows * d].reshape(n, B, H, Nq, d)
    lse_parts = w[n * rows * d:n * rows * (d + 1)].reshape(n, B, H, Nq)
    qn, kn, vn = (t.float().numpy().astype(np.float64) for t in (q, k, v))
    worst_o = worst_l = 0.0
    for p, (lo, hi) in enumerate(split_bounds(Nk, n)):
        for i in range(Nq):
            e = min(hi, Nk - Nq + i + 1) if causal else hi
            if e <= lo:
                assert np.all(lse_parts[p, :, :, i] == -np.inf), (p, i)
                assert np.all(o_parts[p, :, :, i] == 0.0), (p, i)
                continue
            op, lp = oracle.attention_rect(qn[:, :, i:i + 1], kn[:, :, lo:e], vn[:, :, lo:e], scale, False)
            worst_o = max(worst_o, max_abs(o_parts[p, :, :, i], op[:, :, 0]))
            worst_l = max(worst_l, max_abs(lse_parts[p, :, :, i], lp[:, :, 0]))
    say(f"  partial O max abs {worst_o:.3e}  partial LSE max abs {worst_l:.3e}")
    assert worst_o <= TOL_BF16_O and worst_l <= TOL_BF16_LSE
