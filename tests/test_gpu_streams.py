"""Calls from several host threads on their own streams at once.

The library keeps no mutable state between calls (the allocation-free split-KV entry
point aside, whose shared scratch makes overlapping calls race by contract, so it is left
out here) and caches only the device's CU count, so calls from different host threads on
different streams may run concurrently.  Two threads each run a loop of attention,
backward, split-KV, row-softmax and norm calls on their own inputs and streams (default
priority); every output must equal the same calls made one at a time on the default
stream, bit for bit.
"""

import threading

import pytest
import torch

import online_softmax_09_amd as osm
import workloads
from parity import need_gpu, say

pytestmark = pytest.mark.gpu


def _inputs(seed, dev):
    t = {}
    t["q"], t["k"], t["v"] = (x.to(dev) for x in workloads.attention_inputs(2, 4, 1000, 128, seed=seed))
    t["do"] = workloads.attention_inputs(2, 4, 1000, 128, seed=seed + 1)[0].to(dev)
    t["dq"], t["dk"], t["dv"] = (x.to(dev) for x in workloads.decode_inputs(2, 8, 4, 20000, 128, seed=seed + 2))
    t["x"] = workloads.softmax_inputs(512, 4096, seed=seed + 3)[0].to(dev)
    g = torch.Generator().manual_seed(seed + 4)
    t["nx"] = torch.randn(64, 4096, generator=g).to(torch.bfloat16).to(dev)
    t["nr"] = torch.randn(64, 4096, generator=g).to(torch.bfloat16).to(dev)
    t["ng"] = torch.ones(4096, dtype=torch.bfloat16).to(dev)
    return t


def _calls(t, stream):
    scale = workloads.default_scale(128)
    o, lse = osm.fa_fwd(t["q"], t["k"], t["v"], scale=scale, causal=True, stream=stream)
    grads = osm.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], scale=scale, causal=True, stream=stream)
    od, lsed = osm.fa_fwd_splitkv(t["dq"], t["dk"], t["dv"], scale=scale, causal=True, n_splits=6, stream=stream)
    y = osm.online_softmax_rows(t["x"], stream=stream)
    yn, hn = osm.fused_add_rmsnorm(t["nx"], t["nr"], t["ng"], stream=stream)
    return [o, lse, *grads, od, lsed, y, yn, hn]


def test_two_threads_on_their_own_streams():
    dev = need_gpu()
    seeds = [workloads.SEED_BASE + 9800, workloads.SEED_BASE + 9900]
    ins = [_inputs(s, dev) for s in seeds]
    torch.cuda.synchronize()
    ref = [[r.clone() for r in _calls(t, None)] for t in ins]
    torch.cuda.synchronize()
    rounds = 8
    got = [None, None]
    errors = []

    def worker(i):
        try:
            torch.cuda.set_device(dev)
            s = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(s):
                last = None
                for _ in range(rounds):
                    last = _calls(ins[i], s)
            s.synchronize()
            got[i] = last
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))

    say("case two host threads, own streams, 8 rounds each")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(2):
        for j, (a, b) in enumerate(zip(got[i], ref[i])):
            assert torch.equal(a, b), (i, j)
