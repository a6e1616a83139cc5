"""GPU parity of fa_fwd_f16 (fp16 twin of the bf16 forward, through the C ABI) against the
float64 oracle on the same fp16 inputs.

Gates (derived from fp16 arithmetic, in the way the bf16 gates follow from bf16): fp16 has
a unit roundoff of 2^-11 = 4.9e-4, eight times finer than bf16.  P is rounded to fp16 for
P V and O once at the end, so |O| < 4 gives errors of a few 1e-3 at most: O max abs
<= 5e-3.  LSE depends only on float32 arithmetic on fp16 products: LSE max abs <= 1e-3.
"""

import numpy as np
import pytest
import torch

import online_softmax_09_amd as osm
import oracle
import workloads
from parity import max_abs, need_gpu, oracle_rows_per_head, say

pytestmark = pytest.mark.gpu

TOL_F16_O = 5e-3
TOL_F16_LSE = 1e-3


def _gpu(q, k, v, scale, causal, dev):
    o, lse = osm.fa_fwd_f16(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 1, 1, 64, True), (1, 2, 7, 128, False), (2, 1, 64, 64, True), (1, 2, 129, 128, True),
    (1, 1, 383, 64, False), (1, 2, 1000, 128, True), (2, 2, 513, 128, False), (1, 1, 2048, 64, True)])
def test_f16_shapes(B, H, N, d, causal):
    dev = need_gpu()
    say(f"case f16 B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = workloads.attention_inputs(B, H, N, d, seed=workloads.SEED_BASE + 9000 + N + d, dtype="f16")
    scale = workloads.default_scale(d)
    o, lse = _gpu(q, k, v, scale, causal, dev)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    eo, el = max_abs(o, o_ref), max_abs(lse, lse_ref)
    say(f"  O max abs {eo:.3e}  LSE max abs {el:.3e}")
    assert eo <= TOL_F16_O and el <= TOL_F16_LSE


def test_f16_full_size_sampled_rows():
    """The causal 2 x 32 x 8192 x 128 shape in fp16; 64 seeded rows per head plus 0 and N-1."""
    dev = need_gpu()
    c = workloads.CONFIGS["attn_bf16_causal_b2h32n8192d128"]
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    say("case f16 full causal 2x32x8192x128")
    q, k, v = workloads.attention_inputs(B, H, N, d, seed=c["seed"], dtype="f16")
    scale = workloads.default_scale(d)
    o, lse = _gpu(q, k, v, scale, True, dev)
    rows = workloads.sampled_query_rows(B, H, N, 64, seed=c["seed"])
    o_ref, lse_ref = oracle_rows_per_head(q, k, v, scale, True, rows)
    o_s = np.take_along_axis(o, rows[..., None], axis=2)
    l_s = np.take_along_axis(lse, rows, axis=2)
    eo, el = max_abs(o_s, o_ref), max_abs(l_s, lse_ref)
    say(f"  O max abs {eo:.3e}  LSE max abs {el:.3e}")
    assert eo <= TOL_F16_O and el <= TOL_F16_LSE


def test_f16_worked_example():
    """The pages' worked row (scores 0, 1, 2; values 10, 20, 30) embedded in attention."""
    dev = need_gpu()
    from test_oracle_attention import worked_example_inputs

    for shift in (False, True):
        q, k, v = (torch.from_numpy(x).to(torch.float16) for x in worked_example_inputs(d=64, shift=shift))
        o, lse = _gpu(q, k, v, 1.0, False, dev)
        o_ref, lse_ref = oracle.attention(q, k, v, 1.0, False)
        say(f"  shift={shift}: O[0,0] {o[0, 0, 0, 0]:.6f} (exact {o_ref[0, 0, 0, 0]:.6f})  LSE {lse[0, 0, 0]:.5f}")
        assert max_abs(o, o_ref) <= TOL_F16_O
        assert max_abs(lse, lse_ref) <= TOL_F16_LSE
