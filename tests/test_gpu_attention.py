"""GPU parity of fa_fwd (bf16) and fa_fwd_f32 (through the C ABI) against the float64 oracle.

Gates: float32 path max abs error <= 1e-5 on O and LSE; bf16 path max abs error
<= 2e-2 on O and <= 1e-2 on LSE.  Small shapes are compared on every output; the
full-size workloads (the bench's launch configuration) on seeded sampled query rows
that the oracle evaluates one by one.
"""

import math

import numpy as np
import pytest
import torch

import online_softmax_09_amd as osm
import oracle
import workloads
from parity import (TOL_BF16_LSE, TOL_BF16_O, TOL_F32, max_abs, max_rel, need_gpu,
                    oracle_rows_per_head, say)

pytestmark = pytest.mark.gpu


def _gpu(fn, q, k, v, scale, causal, dev):
    o, lse = fn(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _report(tag, o, lse, o_ref, lse_ref, floor):
    eo, el = max_abs(o, o_ref), max_abs(lse, lse_ref)
    say(f"  {tag}: O max abs {eo:.3e} rel {max_rel(o, o_ref, floor):.3e} | LSE max abs {el:.3e}")
    return eo, el


# ---------------------------------------------------------------------------
# float32 path
# ---------------------------------------------------------------------------

def test_f32_single_head_workload():
    dev = need_gpu()
    c = workloads.CONFIGS["attn_f32_b1h1n256d64"]
    q, k, v = workloads.attention_inputs_for("attn_f32_b1h1n256d64")
    scale = workloads.default_scale(c["d"])
    say("case attn_f32_b1h1n256d64")
    o, lse = _gpu(osm.fa_fwd_f32, q, k, v, scale, False, dev)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, False)
    eo, el = _report("f32", o, lse, o_ref, lse_ref, 1e-6)
    assert eo <= TOL_F32 and el <= TOL_F32


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 1, 1, 64, False), (1, 1, 1, 64, True), (2, 3, 65, 64, True), (2, 2, 100, 128, False),
    (1, 2, 300, 128, True), (1, 1, 257, 64, True), (3, 1, 500, 64, False), (1, 1, 129, 128, True)])
def test_f32_shapes(B, H, N, d, causal):
    dev = need_gpu()
    q, k, v = workloads.attention_inputs(B, H, N, d, seed=workloads.SEED_BASE + 5000 + N + d,
                                         dtype="f32")
    scale = workloads.default_scale(d)
    say(f"case f32 B={B} H={H} N={N} d={d} causal={causal}")
    o, lse = _gpu(osm.fa_fwd_f32, q, k, v, scale, causal, dev)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    eo, el = _report("f32", o, lse, o_ref, lse_ref, 1e-6)
    assert eo <= TOL_F32 and el <= TOL_F32


def _worked(d, shift, dtype):
    """The pages' worked row as attention: q_i = e1 (+e2), k_j = j e1 (+1000 e2),
    v_j = 10 (j + 1) e1, N = 3, scale = 1: every row has scores [0, 1, 2] (+1000)
    and values [10, 20, 30].  All entries are exact in bf16."""
    q = torch.zeros(1, 1, 3, d)
    k = torch.zeros(1, 1, 3, d)
    v = torch.zeros(1, 1, 3, d)
    q[..., 0] = 1.0
    for j in range(3):
        k[0, 0, j, 0] = float(j)
        v[0, 0, j, 0] = 10.0 * (j + 1)
    if shift:
        q[..., 1] = 1.0
        k[..., 1] = 1000.0
    if dtype == "bf16":
        q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    return q, k, v


@pytest.mark.parametrize("shift", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_f32_worked_example(d, shift):
    dev = need_gpu()
    q, k, v = _worked(d, shift, "f32")
    say(f"case f32 worked row d={d} shift={shift}")
    o, lse = _gpu(osm.fa_fwd_f32, q, k, v, 1.0, False, dev)
    o_ref, lse_ref = oracle.attention(q, k, v, 1.0, False)
    assert round(float(o[0, 0, 0, 0]), 6) == 25.752104
    assert max_abs(o, o_ref) <= TOL_F32
    # LSE near 1002.4 is compared to two float32 ulps (an ulp there is about 6.1e-5).
    ulp = float(np.spacing(np.float32(abs(lse_ref).max())))
    assert max_abs(lse, lse_ref) <= max(TOL_F32, 2 * ulp)


def test_f32_random_scalar_rows():
    """The 390 random rows (ten of each length 1..39) as one-column attention: row r
    of length n becomes head r with keys k_j = s_j e1, values v_j e1, q_i = e1."""
    dev = need_gpu()
    rows = [r for r in workloads.scalar_rows() if r[0].startswith("len")]
    say("case f32 390 scalar rows")
    worst = 0.0
    for n in range(1, 40):
        group = [r for r in rows if len(r[1]) == n]
        H = len(group)
        q = torch.zeros(1, H, n, 64)
        k = torch.zeros(1, H, n, 64)
        v = torch.zeros(1, H, n, 64)
        q[..., 0] = 1.0
        for h, (_, s, vals) in enumerate(group):
            k[0, h, :, 0] = torch.tensor(s, dtype=torch.float32)
            v[0, h, :, 0] = torch.tensor(vals, dtype=torch.float32)
        o, _ = _gpu(osm.fa_fwd_f32, q, k, v, 1.0, False, dev)
        o_ref, _ = oracle.attention(q, k, v, 1.0, False)
        worst = max(worst, max_abs(o, o_ref))
        # the float32-rounded row against the scalar online instrument
        for h, (_, s, vals) in enumerate(group):
            s32 = [float(np.float32(t)) for t in s]
            v32 = [float(np.float32(t)) for t in vals]
            ref = oracle.online_weighted(s32, v32)[0]
            assert abs(float(o[0, h, 0, 0]) - ref) <= TOL_F32
    say(f"  max abs err {worst:.3e}")
    assert worst <= TOL_F32


# ---------------------------------------------------------------------------
# bf16 path: small shapes, every output compared
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 7, 64, 127, 128, 129, 200, 383, 1000])
def test_bf16_small_shapes(N, d, causal):
    dev = need_gpu()
    B, H = 2, 3
    q, k, v = workloads.attention_inputs(B, H, N, d, seed=workloads.SEED_BASE + 6000 + N + d)
    scale = workloads.default_scale(d)
    say(f"case bf16 B={B} H={H} N={N} d={d} causal={causal}")
    o, lse = _gpu(osm.fa_fwd, q, k, v, scale, causal, dev)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    eo, el = _report("bf16", o, lse, o_ref, lse_ref, 1e-3)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


def test_bf16_non_causal_workload_full():
    dev = need_gpu()
    name = "attn_bf16_b4h16n2048d64"
    c = workloads.CONFIGS[name]
    q, k, v = workloads.attention_inputs_for(name)
    scale = workloads.default_scale(c["d"])
    say(f"case {name} (every output)")
    o, lse = _gpu(osm.fa_fwd, q, k, v, scale, c["causal"], dev)
    rows = np.broadcast_to(np.arange(c["N"]), (c["B"], c["H"], c["N"]))
    o_ref, lse_ref = oracle_rows_per_head(q, k, v, scale, c["causal"], rows)
    eo, el = _report("bf16", o, lse, o_ref, lse_ref, 1e-3)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


def _sampled(name, per_head, extra_rows=()):
    dev = need_gpu()
    c = workloads.CONFIGS[name]
    q, k, v = workloads.attention_inputs_for(name)
    scale = workloads.default_scale(c["d"])
    B, H, N = c["B"], c["H"], c["N"]
    rows = workloads.sampled_query_rows(B, H, N, per_head, seed=c["seed"])
    if extra_rows:
        ex = np.array([r for r in extra_rows if r < N], dtype=np.int64)
        rows = np.concatenate([rows, np.broadcast_to(ex, (B, H, len(ex)))], axis=2)
    say(f"case {name}: {rows.shape[2]} sampled rows per head")
    o, lse = _gpu(osm.fa_fwd, q, k, v, scale, c["causal"], dev)
    o_ref, lse_ref = oracle_rows_per_head(q, k, v, scale, c["causal"], rows)
    bi = np.arange(B)[:, None, None]
    hi = np.arange(H)[None, :, None]
    eo, el = _report("bf16", o[bi, hi, rows], lse[bi, hi, rows], o_ref, lse_ref, 1e-3)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE
    # causal row 0 sees key 0 only: O_0 = V_0 exactly
    if c["causal"]:
        assert np.array_equal(o[:, :, 0], v[:, :, 0].float().numpy())
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


TILE_EDGES = (1, 31, 32, 63, 64, 127, 128, 129, 255, 256, 4095, 4096, 8190, 8191)


def test_bf16_causal_workload_sampled():
    _sampled("attn_bf16_causal_b2h32n8192d128", 126, TILE_EDGES)


def test_bf16_causal_ragged_workload_sampled():
    _sampled("attn_bf16_causal_b2h32n8191d128", 126, TILE_EDGES)


def test_bf16_long_causal_workload_sampled():
    _sampled("attn_bf16_causal_b1h8n131072d128", 1024)


# ---------------------------------------------------------------------------
# bf16 path: closed forms, worked row, determinism
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
def test_bf16_constant_values(d):
    dev = need_gpu()
    q, k, v = workloads.attention_inputs(1, 2, 700, d, seed=workloads.SEED_BASE + 7000 + d)
    v = v[:, :, :1].expand_as(v).contiguous()
    say(f"case bf16 constant V d={d}")
    for causal in (False, True):
        o, _ = _gpu(osm.fa_fwd, q, k, v, workloads.default_scale(d), causal, dev)
        # every row is a convex combination of identical rows
        assert max_abs(o, np.broadcast_to(v.float().numpy(), o.shape)) <= TOL_BF16_O


@pytest.mark.parametrize("shift", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_worked_example(d, shift):
    dev = need_gpu()
    q, k, v = _worked(d, shift, "bf16")
    say(f"case bf16 worked row d={d} shift={shift}")
    o, lse = _gpu(osm.fa_fwd, q, k, v, 1.0, False, dev)
    o_ref, lse_ref = oracle.attention(q, k, v, 1.0, False)
    assert abs(float(o[0, 0, 0, 0]) - 25.752104) <= TOL_BF16_O
    assert max_abs(o, o_ref) <= TOL_BF16_O
    assert max_abs(lse, lse_ref) <= TOL_BF16_LSE


def test_bf16_repeat_runs_bitwise_identical():
    dev = need_gpu()
    q, k, v = workloads.attention_inputs(2, 4, 1500, 128, seed=workloads.SEED_BASE + 7100)
    say("case bf16 determinism")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    a = osm.fa_fwd(qd, kd, vd, causal=True)
    b = osm.fa_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_unsupported_head_dim_is_an_error():
    dev = need_gpu()
    q = torch.zeros(1, 1, 16, 96, dtype=torch.bfloat16, device=dev)
    with pytest.raises(RuntimeError, match="unsupported"):
        osm.fa_fwd(q, q.clone(), q.clone())


@pytest.mark.parametrize("scale", [0.0, -0.0883883461356163, 0.5])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("fn,dtype,tol_o,tol_l", [("fa_fwd", "bf16", TOL_BF16_O, TOL_BF16_LSE),
                                                   ("fa_fwd_f32", "f32", TOL_F32, TOL_F32)])
def test_scale_edge_cases(fn, dtype, tol_o, tol_l, causal, scale):
    """scale = 0 (uniform weights over the visible keys), negative and large scales.

    The float32 score error grows with |scale| * sqrt(d) (a d-term dot product of
    N(0, 1) entries, times scale), so the float32 gate is widened by that factor when
    it exceeds 1; at scale = 1/sqrt(d) it is the plain 1e-5."""
    dev = need_gpu()
    q, k, v = workloads.attention_inputs(1, 2, 333, 128, seed=workloads.SEED_BASE + 7200, dtype=dtype)
    say(f"case {fn} scale={scale} causal={causal}")
    o, lse = _gpu(getattr(osm, fn), q, k, v, scale, causal, dev)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    eo, el = _report(fn, o, lse, o_ref, lse_ref, 1e-3)
    if dtype == "f32":
        widen = max(1.0, abs(scale) * math.sqrt(q.shape[-1]))
        tol_o, tol_l = tol_o * widen, tol_l * widen
    assert eo <= tol_o and el <= tol_l


@pytest.mark.parametrize("fn,dtype,tol_o,tol_l", [("fa_fwd", "bf16", TOL_BF16_O, TOL_BF16_LSE),
                                                   ("fa_fwd_f16", "f16", 5e-3, 1e-3)])
@pytest.mark.parametrize("f", [2, 8, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_score_jumps(d, causal, f, fn, dtype, tol_o, tol_l):
    """Keys far above the running maximum arrive late in the key loop: key rows 130,
    300 and 611 are multiplied by f, 2 f and 4 f (powers of two, exact in both
    formats), so a row's maximum jumps, in later key tiles, by a few to several hundred
    powers of two.  Small jumps stay under the kernel's lazy threshold (the reference
    maximum does not move and the probabilities exceed 1); large ones move it and
    rescale O by alpha, where exp2 of the jump against the old maximum would overflow
    float32 by far."""
    dev = need_gpu()
    q, k, v = workloads.attention_inputs(1, 2, 700, d, seed=workloads.SEED_BASE + 7300 + d, dtype=dtype)
    k = k.clone()
    for row, mult in ((130, f), (300, 2 * f), (611, 4 * f)):
        k[:, :, row] *= mult
    say(f"case {fn} score jumps d={d} causal={causal} f={f}")
    o, lse = _gpu(getattr(osm, fn), q, k, v, workloads.default_scale(d), causal, dev)
    o_ref, lse_ref = oracle.attention(q, k, v, workloads.default_scale(d), causal)
    eo, el = _report(fn, o, lse, o_ref, lse_ref, 1e-3)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert eo <= tol_o and el <= tol_l


@pytest.mark.parametrize("fn,dtype,tol_o,tol_l", [("fa_fwd", "bf16", TOL_BF16_O, TOL_BF16_LSE),
                                                   ("fa_fwd_f16", "f16", 5e-3, 1e-3)])
@pytest.mark.parametrize("N,causal", [(2048, False), (2049, False), (4096, False), (10240, True), (10241, True)])
def test_both_block_forms(N, causal, fn, dtype, tol_o, tol_l):
    """The host runs d = 128 with 4-wavefront blocks (two per CU) up to causal N = 10240
    and non-causal N = 2048, and with the 8-wavefront ping-pong above; these lengths sit
    on both sides of each switch (and N = 4096, ping-pong without key masks), in both
    16-bit formats.  Sampled rows include both ends and tile edges."""
    dev = need_gpu()
    B, H, d = 1, 2, 128
    q, k, v = workloads.attention_inputs(B, H, N, d, seed=workloads.SEED_BASE + 7400 + N, dtype=dtype)
    scale = workloads.default_scale(d)
    rows = workloads.sampled_query_rows(B, H, N, 96, seed=workloads.SEED_BASE + 7400 + N)
    edges = np.array([r for r in TILE_EDGES + (N - 2, N - 1) if r < N], dtype=np.int64)
    rows = np.concatenate([rows, np.broadcast_to(edges, (B, H, len(edges)))], axis=2)
    say(f"case {fn} block forms N={N} causal={causal}")
    o, lse = _gpu(getattr(osm, fn), q, k, v, scale, causal, dev)
    o_ref, lse_ref = oracle_rows_per_head(q, k, v, scale, causal, rows)
    bi = np.arange(B)[:, None, None]
    hi = np.arange(H)[None, :, None]
    eo, el = _report(fn, o[bi, hi, rows], lse[bi, hi, rows], o_ref, lse_ref, 1e-3)
    assert eo <= tol_o and el <= tol_l
    if causal:
        assert np.array_equal(o[:, :, 0], v[:, :, 0].float().numpy())


@pytest.mark.parametrize("B,H,N,d", [(4, 16, 4096, 64), (4, 16, 4100, 64), (1, 2, 8192, 128), (1, 2, 8200, 128),
                                     (1, 2, 2048, 128)])
def test_non_causal_key_tail_forms(B, H, N, d):
    """Non-causal kernels are built twice: with key masks for a last key tile that runs
    past N (N not a multiple of 64) and without them.  At d = 64 the build without masks
    fits three blocks per CU, and the host holds it to two for grids of four blocks per
    CU (the full B=4 H=16 N=2048 workload covers that case); 2048 blocks here run three
    per CU.  At d = 128 both builds are taken in both block forms (N = 2048 plain,
    N = 8192 ping-pong).  Sampled rows include both ends and tile edges."""
    dev = need_gpu()
    q, k, v = workloads.attention_inputs(B, H, N, d, seed=workloads.SEED_BASE + 7500 + N + d)
    scale = workloads.default_scale(d)
    rows = workloads.sampled_query_rows(B, H, N, 48, seed=workloads.SEED_BASE + 7500 + N)
    edges = np.array([r for r in TILE_EDGES + (N - 2, N - 1) if r < N], dtype=np.int64)
    rows = np.concatenate([rows, np.broadcast_to(edges, (B, H, len(edges)))], axis=2)
    say(f"case bf16 non-causal key tail B={B} H={H} N={N} d={d}")
    o, lse = _gpu(osm.fa_fwd, q, k, v, scale, False, dev)
    o_ref, lse_ref = oracle_rows_per_head(q, k, v, scale, False, rows)
    bi = np.arange(B)[:, None, None]
    hi = np.arange(H)[None, :, None]
    eo, el = _report("bf16", o[bi, hi, rows], lse[bi, hi, rows], o_ref, lse_ref, 1e-3)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


@pytest.mark.parametrize("B,H,N", [(2, 8, 2048), (1, 8, 1024), (1, 16, 4096)])
def test_causal_d64_dispatch_order(B, H, N):
    """Causal d = 64 launches whose blocks divide evenly over the 8 XCDs take a dispatch
    order that holds back the shortest quarter of every head's query tiles (one head per
    XCD, pairs of heads, two pairs).  Every output row is compared, so a tile computed
    twice or never shows up."""
    dev = need_gpu()
    d = 64
    q, k, v = workloads.attention_inputs(B, H, N, d, seed=workloads.SEED_BASE + 7600 + N + H)
    scale = workloads.default_scale(d)
    say(f"case bf16 causal d=64 dispatch order B={B} H={H} N={N}")
    o, lse = _gpu(osm.fa_fwd, q, k, v, scale, True, dev)
    rows = np.broadcast_to(np.arange(N), (B, H, N))
    o_ref, lse_ref = oracle_rows_per_head(q, k, v, scale, True, rows)
    eo, el = _report("bf16", o, lse, o_ref, lse_ref, 1e-3)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE
    assert np.array_equal(o[:, :, 0], v[:, :, 0].float().numpy())


@pytest.mark.parametrize("B,H,N,d", [(8, 8, 512, 64), (4, 16, 1024, 128), (2, 32, 2048, 64), (1, 64, 1000, 128)])
def test_causal_head_groups_of_four(B, H, N, d):
    """Causal launches of rows up to 4096 whose XCDs hold a multiple of eight heads take the
    heads in groups of four (with the held-back shortest quarter at d = 64), a ragged N
    included.  Every output row is compared, so a tile computed twice or never shows up."""
    dev = need_gpu()
    q, k, v = workloads.attention_inputs(B, H, N, d, seed=workloads.SEED_BASE + 7700 + N + H + d)
    scale = workloads.default_scale(d)
    say(f"case bf16 causal head groups B={B} H={H} N={N} d={d}")
    o, lse = _gpu(osm.fa_fwd, q, k, v, scale, True, dev)
    rows = np.broadcast_to(np.arange(N), (B, H, N))
    o_ref, lse_ref = oracle_rows_per_head(q, k, v, scale, True, rows)
    eo, el = _report("bf16", o, lse, o_ref, lse_ref, 1e-3)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE
    assert np.array_equal(o[:, :, 0], v[:, :, 0].float().numpy())
