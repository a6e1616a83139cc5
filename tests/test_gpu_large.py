"""GPU parity at sizes whose element offsets pass 2^31: every entry point whose tensors hold
more than 2^31 elements, checked against the float64 oracle on the heads or rows that lie
past that boundary (and on the first ones).  An offset computed in 32 bits anywhere in a
kernel or launcher would read or write the wrong memory there.

Inputs are iid N(0, 1) drawn on the GPU from a seeded generator (workloads.device_normal):
at 4-9 GB per tensor, drawing on the host would take longer than the tests.  The oracle
evaluates the same values, copied back for the heads or rows it checks.  Gates as in the
other parity tests: bf16 O <= 2e-2 and LSE <= 1e-2 absolute; gradients <= 2e-2 of the
tensor's largest value; norms within one bf16 rounding plus 2e-3; softmax <= 1e-5.
"""

import numpy as np
import pytest
import torch

import online_softmax_09_amd as osm
import oracle
import workloads
from parity import TOL_BF16_LSE, TOL_BF16_O, TOL_F32, max_abs, need_gpu, say

pytestmark = pytest.mark.gpu

BIG = 1 << 31


def _heads_past(BH, per_head):
    """Flat head indices to check: the first, the two around element 2^31, and the last."""
    first_past = -(-BIG // per_head)
    return sorted({0, first_past - 1, first_past, BH - 1})


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,H,N,d,causal", [(33, 1024, 1024, 64, False), (17, 1024, 1024, 128, True)])
def test_forward_past_2_31(B, H, N, d, causal):
    dev = need_gpu()
    assert B * H * N * d > BIG
    say(f"case fa_fwd past 2^31 B={B} H={H} N={N} d={d} causal={causal}")
    seed = workloads.SEED_BASE + 9900 + d
    q = workloads.device_normal((B, H, N, d), seed, torch.bfloat16, dev)
    k = workloads.device_normal((B, H, N, d), seed + 1, torch.bfloat16, dev)
    v = workloads.device_normal((B, H, N, d), seed + 2, torch.bfloat16, dev)
    scale = workloads.default_scale(d)
    o, lse = osm.fa_fwd(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    worst_o = worst_l = 0.0
    for bh in _heads_past(B * H, N * d):
        b, h = divmod(bh, H)
        qs, ks, vs = (t[b:b + 1, h:h + 1].cpu() for t in (q, k, v))
        o_ref, l_ref = oracle.attention(qs, ks, vs, scale, causal)
        worst_o = max(worst_o, max_abs(o[b:b + 1, h:h + 1].float().cpu().numpy(), o_ref))
        worst_l = max(worst_l, max_abs(lse[b:b + 1, h:h + 1].cpu().numpy(), l_ref))
    say(f"  O max abs {worst_o:.3e}  LSE max abs {worst_l:.3e}")
    del q, k, v, o, lse
    _free()
    assert worst_o <= TOL_BF16_O and worst_l <= TOL_BF16_LSE


def test_backward_past_2_31():
    dev = need_gpu()
    B, H, N, d = 17, 1024, 1024, 128
    say(f"case fa_bwd past 2^31 B={B} H={H} N={N} d={d} causal")
    seed = workloads.SEED_BASE + 9910
    q = workloads.device_normal((B, H, N, d), seed, torch.bfloat16, dev)
    k = workloads.device_normal((B, H, N, d), seed + 1, torch.bfloat16, dev)
    v = workloads.device_normal((B, H, N, d), seed + 2, torch.bfloat16, dev)
    do = workloads.device_normal((B, H, N, d), seed + 3, torch.bfloat16, dev)
    scale = workloads.default_scale(d)
    o, lse = osm.fa_fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv = osm.fa_bwd(q, k, v, o, lse, do, scale=scale, causal=True)
    torch.cuda.synchronize()
    ok = True
    for bh in _heads_past(B * H, N * d):
        b, h = divmod(bh, H)
        qs, ks, vs, dos = (t[b:b + 1, h:h + 1].cpu() for t in (q, k, v, do))
        refs = oracle.attention_backward(qs, ks, vs, dos, scale, True)
        for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
            g = got[b:b + 1, h:h + 1].float().cpu().numpy()
            err, top = max_abs(g, ref), float(np.max(np.abs(ref)))
            say(f"  head {bh} {name}: max abs {err:.3e} (max |ref| {top:.3e})")
            ok &= err <= 2e-2 * top
    del q, k, v, do, o, lse, dq, dk, dv
    _free()
    assert ok


@pytest.mark.parametrize("Nq,n_splits", [(1, 24), (16, 16)])
def test_splitkv_past_2_31(Nq, n_splits):
    dev = need_gpu()
    B, H, Nk, d = 1, 66, 262144, 128
    assert B * H * Nk * d > BIG
    say(f"case fa_fwd_splitkv past 2^31 B={B} H={H} Nq={Nq} Nk={Nk} n_splits={n_splits}")
    seed = workloads.SEED_BASE + 9920 + Nq
    q = workloads.device_normal((B, H, Nq, d), seed, torch.bfloat16, dev)
    k = workloads.device_normal((B, H, Nk, d), seed + 1, torch.bfloat16, dev)
    v = workloads.device_normal((B, H, Nk, d), seed + 2, torch.bfloat16, dev)
    scale = workloads.default_scale(d)
    o, lse = osm.fa_fwd_splitkv(q, k, v, scale=scale, causal=True, n_splits=n_splits)
    torch.cuda.synchronize()
    worst_o = worst_l = 0.0
    for h in _heads_past(H, Nk * d):
        qs, ks, vs = (t[:, h:h + 1].cpu() for t in (q, k, v))
        o_ref, l_ref = oracle.attention_rect(qs, ks, vs, scale, True)
        worst_o = max(worst_o, max_abs(o[:, h:h + 1].float().cpu().numpy(), o_ref))
        worst_l = max(worst_l, max_abs(lse[:, h:h + 1].cpu().numpy(), l_ref))
    say(f"  O max abs {worst_o:.3e}  LSE max abs {worst_l:.3e}")
    del q, k, v, o, lse
    _free()
    assert worst_o <= TOL_BF16_O and worst_l <= TOL_BF16_LSE


def test_softmax_rows_past_2_31():
    dev = need_gpu()
    rows, cols = 540672, 4096
    assert rows * cols > BIG
    say(f"case online_softmax_rows past 2^31 rows={rows} cols={cols}")
    x = workloads.device_normal((rows, cols), workloads.SEED_BASE + 9930, torch.float32, dev)
    y = osm.online_softmax_rows(x)
    torch.cuda.synchronize()
    first_past = -(-BIG // cols)
    sel = torch.tensor([0, first_past - 1, first_past, rows // 2 + 7, rows - 1], device=dev)
    xs, ys = x[sel].double().cpu().numpy(), y[sel].double().cpu().numpy()
    err = max_abs(ys, oracle.softmax_rows(xs)[0])
    say(f"  y max abs {err:.3e}")
    del x, y
    _free()
    assert err <= TOL_F32


def test_rmsnorm_past_2_31():
    dev = need_gpu()
    rows, cols = 270336, 8192
    assert rows * cols > BIG
    say(f"case fused_add_rmsnorm past 2^31 rows={rows} cols={cols}")
    seed = workloads.SEED_BASE + 9940
    x = workloads.device_normal((rows, cols), seed, torch.bfloat16, dev)
    r = workloads.device_normal((rows, cols), seed + 1, torch.bfloat16, dev)
    g = workloads.device_normal((cols,), seed + 2, torch.bfloat16, dev)
    y, hsum = osm.fused_add_rmsnorm(x, r, g, eps=1e-5)
    torch.cuda.synchronize()
    first_past = -(-BIG // cols)
    sel = torch.tensor([0, first_past - 1, first_past, rows - 1], device=dev)
    y_ref, h_ref = oracle.rms_norm(x[sel].cpu(), g.cpu(), 1e-5, residual=r[sel].cpu())
    yy = y[sel].double().cpu().numpy()
    excess = float(np.max(np.abs(yy - y_ref) - (2.0 ** -8 * np.abs(y_ref) + 2e-3)))
    h_err = max_abs(hsum[sel].double().cpu().numpy(), h_ref)
    say(f"  y max excess over the gate {excess:.3e}  h max abs {h_err:.3e}")
    del x, r, g, y, hsum
    _free()
    assert excess <= 0.0 and h_err <= 2.0 ** -7 * float(np.max(np.abs(h_ref)))
