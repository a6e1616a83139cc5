"""Capture of the library's entry points in a HIP graph (torch.cuda.CUDAGraph).

Every entry point enqueues its kernels on the caller's stream and allocates, copies and
synchronises nothing, so a sequence of calls can be captured once and replayed; the launch
cost of short calls (a decoding step is two kernels of well under 100 us) is then paid per
graph rather than per kernel.  The test captures one call of each entry point into one
graph, then three times writes new inputs into the captured buffers, replays the graph and
runs the same calls eagerly on those inputs, with the program's own eager work and
synchronisations in between.  Every replay must equal the eager calls bit for bit (same
kernels, same launch shapes), and the first replay must also meet the float64 oracle's
gates on the attention output.
"""

import numpy as np
import pytest
import torch

import online_softmax_09_amd as osm
import oracle
import workloads
from parity import TOL_BF16_LSE, TOL_BF16_O, TOL_F32, max_abs, need_gpu, say

pytestmark = pytest.mark.gpu


def _inputs(seed):
    """CPU tensors for every captured call, drawn from one seed."""
    d = {}
    d["q"], d["k"], d["v"] = workloads.attention_inputs(1, 2, 300, 128, seed=seed)
    d["do"] = workloads.attention_inputs(1, 2, 300, 128, seed=seed + 1)[0]
    d["q32"], d["k32"], d["v32"] = workloads.attention_inputs(1, 1, 256, 64, seed=seed + 2, dtype="f32")
    d["dq"], d["dk"], d["dv"] = workloads.decode_inputs(1, 8, 1, 4096, 128, seed=seed + 3)
    d["x"], _ = workloads.softmax_inputs(64, 4095, seed=seed + 4)
    g = torch.Generator().manual_seed(seed + 5)
    d["nx"] = torch.randn(16, 2048, generator=g).to(torch.bfloat16)
    d["nr"] = torch.randn(16, 2048, generator=g).to(torch.bfloat16)
    d["ng"] = (1.0 + 0.1 * torch.randn(2048, generator=g)).to(torch.bfloat16)
    return d


def _calls(t):
    """One call of each entry point on the device tensors t; returns every output."""
    scale = workloads.default_scale(128)
    o, lse = osm.fa_fwd(t["q"], t["k"], t["v"], scale=scale, causal=True)
    dq, dk, dv = osm.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], scale=scale, causal=True)
    o32, lse32 = osm.fa_fwd_f32(t["q32"], t["k32"], t["v32"], scale=workloads.default_scale(64))
    od, lsed = osm.fa_fwd_splitkv(t["dq"], t["dk"], t["dv"], scale=scale, causal=True, n_splits=8)
    on, lsen = osm.fa_fwd_splitkv_noalloc(t["dq"], t["dk"], t["dv"], scale=scale, causal=True, n_splits=8)
    y = osm.online_softmax_rows(t["x"])
    h_out, r_out = osm.fused_add_rmsnorm(t["nx"], t["nr"], t["ng"])
    return [o, lse, dq, dk, dv, o32, lse32, od, lsed, on, lsen, y, h_out, r_out]


def test_graph_replays_match_eager_calls():
    dev = need_gpu()
    host = _inputs(workloads.SEED_BASE + 9700)
    t = {k: v.to(dev) for k, v in host.items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        _calls(t)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = _calls(t)
    torch.cuda.synchronize()
    for rep in range(3):
        new = _inputs(workloads.SEED_BASE + 9710 + 10 * rep)
        for k, v in new.items():
            t[k].copy_(v.to(dev))
        torch.cuda.synchronize()
        say(f"case graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        eager = _calls(t)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(captured, eager)):
            assert torch.equal(a, b), (rep, i)
        if rep == 0:
            q, k, v = new["q"], new["k"], new["v"]
            ref_o, ref_lse = oracle.attention(q, k, v, workloads.default_scale(128), True)
            eo = max_abs(captured[0].float().cpu().numpy(), ref_o)
            el = max_abs(captured[1].cpu().numpy(), ref_lse)
            ref32, _ = oracle.attention(new["q32"], new["k32"], new["v32"], workloads.default_scale(64), False)
            e32 = max_abs(captured[5].cpu().numpy(), ref32)
            say(f"  replay 0 vs oracle: bf16 O {eo:.2e} LSE {el:.2e}; f32 O {e32:.2e}")
            assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE and e32 <= TOL_F32
            assert np.isfinite(captured[11].cpu().numpy()).all()
