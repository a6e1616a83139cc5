"""GPU check of fa_fwd_splitkv_noalloc (the split-KV forward with the partial results in
the library's per-device scratch) through the C ABI, against fa_fwd_splitkv with a
caller-supplied workspace on the same inputs.

Both run the same kernels in the same order, so the outputs must agree bit for bit; they
are also held to the bf16 gates against the float64 oracle (O max abs <= 2e-2, LSE max
abs <= 1e-2).  Three calls run in a row, each smaller than the one before, so each reads a
scratch that still holds the earlier call's partials; the last has one query per head and
takes the one-query partial kernel.
"""

import ctypes

import numpy as np
import pytest
import torch

import online_softmax_09_amd as osm
import oracle
import workloads
from online_softmax_09_amd import _lib
from parity import TOL_BF16_LSE, TOL_BF16_O, max_abs, need_gpu, say

pytestmark = pytest.mark.gpu


def _noalloc_raw(q, k, v, scale, causal, n_splits):
    """One call of the C entry point on torch's current stream, outputs from torch."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    rc = _lib.load().fa_fwd_splitkv_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
        ctypes.c_float(scale), 1 if causal else 0, n_splits, torch.cuda.current_stream().cuda_stream)
    assert rc == _lib.OK, _lib.strerror(rc)
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
def test_noalloc_matches_workspace_entry(causal):
    dev = need_gpu()
    # each call smaller than the one before; the last takes the one-query kernel
    cases = [(2, 8, 16, 4096, 128, 24), (1, 3, 5, 1000, 64, 7), (1, 2, 1, 900, 128, 3)]
    for i, (B, H, Nq, Nk, d, n) in enumerate(cases):
        say(f"case noalloc call {i} causal={causal} B={B} H={H} Nq={Nq} Nk={Nk} d={d} n_splits={n}")
        q, k, v = workloads.decode_inputs(B, H, Nq, Nk, d, seed=workloads.SEED_BASE + 8700 + i)
        scale = workloads.default_scale(d)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o_na, l_na = _noalloc_raw(qd, kd, vd, scale, causal, n)
        torch.cuda.synchronize()
        o_na, l_na = o_na.float().cpu().numpy(), l_na.cpu().numpy()
        o_ws, l_ws = osm.fa_fwd_splitkv(qd, kd, vd, scale=scale, causal=causal, n_splits=n)
        torch.cuda.synchronize()
        o_ws, l_ws = o_ws.float().cpu().numpy(), l_ws.cpu().numpy()
        assert np.array_equal(o_na, o_ws) and np.array_equal(l_na, l_ws)
        o_ref, l_ref = oracle.attention_rect(q, k, v, scale, causal)
        eo, el = max_abs(o_na, o_ref), max_abs(l_na, l_ref)
        say(f"  bitwise equal to fa_fwd_splitkv; vs oracle O {eo:.3e} LSE {el:.3e}")
        assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


def test_noalloc_binding_and_limit():
    dev = need_gpu()
    say("case noalloc binding, then a call beyond the scratch")
    q, k, v = workloads.decode_inputs(1, 2, 3, 2000, 128, seed=workloads.SEED_BASE + 8710)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o1, l1 = osm.fa_fwd_splitkv_noalloc(qd, kd, vd, causal=True, n_splits=5)
    o2, l2 = osm.fa_fwd_splitkv(qd, kd, vd, causal=True, n_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # 32 heads x 16 queries x 129 floats x 128 parts (33.8 MB) is past the 32 MiB scratch
    qb = torch.zeros((1, 32, 16, 128), dtype=torch.bfloat16, device=dev)
    kb = torch.zeros((1, 32, 64, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(RuntimeError, match="unsupported"):
        osm.fa_fwd_splitkv_noalloc(qb, kb, kb, n_splits=128)
