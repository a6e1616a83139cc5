"""Host-side checks of the seeded input recipe (no method arithmetic here)."""

import math

import numpy as np
import torch

import workloads


def test_attention_inputs_deterministic_and_bf16():
    a = workloads.attention_inputs(1, 2, 33, 64, seed=1, dtype="bf16")
    b = workloads.attention_inputs(1, 2, 33, 64, seed=1, dtype="bf16")
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (1, 2, 33, 64)
        assert torch.equal(x, y)
    f = workloads.attention_inputs(1, 2, 33, 64, seed=1, dtype="f32")
    # bf16 is the round-to-nearest-even cast of the same fp32 draw
    assert torch.equal(f[0].to(torch.bfloat16), a[0])


def test_key_outliers_are_exact_powers_of_two():
    q0, k0, v0 = workloads.attention_inputs(1, 2, 4000, 8, seed=3, dtype="f32")
    q1, k1, v1 = workloads.attention_inputs(1, 2, 4000, 8, seed=3, dtype="f32", k_outlier_frac=0.001)
    assert torch.equal(q0, q1)
    ratio = (k1 / k0).flatten(0, 2)
    rows = (ratio != 1).any(dim=-1)
    assert int(rows.sum()) == 2 * 4
    assert torch.all(ratio[rows] == 8.0)


def test_softmax_specials():
    x, sp = workloads.softmax_inputs(1000, 37, seed=4)
    sets = [set(v.tolist()) for v in sp.values()]
    assert all(len(s) == 10 for s in sets)
    assert not (sets[0] & sets[1]) and not (sets[0] & sets[2]) and not (sets[1] & sets[2])
    ae = torch.from_numpy(sp["all_equal"])
    assert torch.all(x[ae] == x[ae, :1])
    assert torch.all(x[torch.from_numpy(sp["plus1000"])] > 900)
    assert torch.all(x[torch.from_numpy(sp["minus1000"])] < -900)


def test_scalar_rows_recipe():
    rows = workloads.scalar_rows()
    assert rows[0] == ("worked", [0.0, 1.0, 2.0], [10.0, 20.0, 30.0])
    rnd = [r for r in rows if r[0].startswith("len")]
    assert len(rnd) == 390
    for n in range(1, 40):
        assert sum(1 for r in rnd if len(r[1]) == n) == 10
    assert all(-10 <= v <= 10 for r in rnd for v in r[2])


def test_sampled_rows():
    r = workloads.sampled_query_rows(1, 3, 131072, 1024, seed=5)
    assert r.shape == (1, 3, 1026)
    for h in range(3):
        assert r[0, h, 0] == 0 and r[0, h, -1] == 131071
        assert len(np.unique(r[0, h])) == 1026


def test_default_scale():
    assert workloads.default_scale(64) == 0.125
    assert math.isclose(workloads.default_scale(128), 1 / math.sqrt(128), rel_tol=1e-7)


def test_device_normal_is_seeded_and_chunked():
    """The device-side generator of the very large inputs: the same seed and chunk size
    give the same values (the chunk size is part of the recipe: drawing in pieces gives
    other values than one draw), and the values are the generator's N(0, 1) draws rounded
    once to the requested type.  Checked on the host device."""
    import torch

    a = workloads.device_normal((7, 13), 1234, torch.float32, "cpu")
    b = workloads.device_normal((7, 13), 1234, torch.float32, "cpu", chunk=10)
    g = torch.Generator(device="cpu")
    g.manual_seed(1234)
    ref = torch.randn(91, generator=g, dtype=torch.float32).view(7, 13)
    assert torch.equal(a, ref)
    assert not torch.equal(b, ref)  # chunked draws continue the same stream in pieces
    c = workloads.device_normal((7, 13), 1234, torch.bfloat16, "cpu")
    assert torch.equal(c, ref.to(torch.bfloat16))
    assert not torch.equal(a, workloads.device_normal((7, 13), 1235, torch.float32, "cpu"))
