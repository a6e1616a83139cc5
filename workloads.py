"""Seeded synthetic inputs shaped like the pages' workloads.

Shared by ``tests/``, ``bench.py`` and ``__graft_entry__.smoke()``.  This module holds
none of the method's arithmetic: it only draws random numbers, applies the input
recipe (shifts, constant rows, outlier keys) and casts to the storage dtype, so both
the GPU path and the CPU oracle receive the very same bits.

Recipe (all draws from NumPy's PCG64, in float32, in the order listed):

* attention: Q, K, V iid N(0, 1) of shape [B, H, N, d]; optionally a fraction of the
  key rows of every head (chosen without replacement) multiplied by 8, which is
  exact in both fp32 and bf16; then cast to bf16 by round-to-nearest-even where the
  workload is bf16.
* row softmax: x iid N(0, sigma) of shape [rows, cols]; three disjoint row sets of
  floor(1% of rows) each get +1000 added, -1000 added, or every entry replaced by
  the row's first entry (an all-equal row).
* scalar rows: the pages' worked row (scores 0, 1, 2 with values 10, 20, 30), the
  same with every score +1000, and 390 random rows, ten of each length 1..39, with
  scores N(0, 2) and values U(-10, 10).
* sampled query rows for the long-sequence check: per head 1024 distinct rows drawn
  uniformly from 1..N-2, plus rows 0 and N-1.

The second parameter of N(0, 2) / N(0, 3) is read as the standard deviation.
"""

import math

import numpy as np

SEED_BASE = 20261202

# The workloads, keyed by what they are.  ``seed`` is SEED_BASE + the workload's
# position in the list; variants of one workload add a fixed offset.
CONFIGS = {
    "attn_f32_b1h1n256d64": dict(kind="attn", dtype="f32", B=1, H=1, N=256, d=64,
                                 causal=False, seed=SEED_BASE + 0),
    "softmax_f32_65536x4096": dict(kind="softmax", rows=65536, cols=4096, sigma=3.0,
                                   seed=SEED_BASE + 1),
    "softmax_f32_65536x4095": dict(kind="softmax", rows=65536, cols=4095, sigma=3.0,
                                   seed=SEED_BASE + 1 + 1000),
    "softmax_f32_65536x1": dict(kind="softmax", rows=65536, cols=1, sigma=3.0,
                                seed=SEED_BASE + 1 + 2000),
    "attn_bf16_b4h16n2048d64": dict(kind="attn", dtype="bf16", B=4, H=16, N=2048, d=64,
                                    causal=False, seed=SEED_BASE + 2),
    "attn_bf16_causal_b2h32n8192d128": dict(kind="attn", dtype="bf16", B=2, H=32, N=8192,
                                            d=128, causal=True, seed=SEED_BASE + 3),
    "attn_bf16_causal_b2h32n8191d128": dict(kind="attn", dtype="bf16", B=2, H=32, N=8191,
                                            d=128, causal=True, seed=SEED_BASE + 3 + 1000),
    "attn_bf16_causal_b1h8n131072d128": dict(kind="attn", dtype="bf16", B=1, H=8, N=131072,
                                             d=128, causal=True, seed=SEED_BASE + 4,
                                             k_outlier_frac=0.001, k_outlier_scale=8.0,
                                             sample_rows=1024),
    # Decoding against a key/value cache: the long causal workload's heads with one new
    # query each (bottom-right aligned), keys cut into parts merged in the log domain.
    "decode_bf16_b1h8q1k131072d128": dict(kind="decode", dtype="bf16", B=1, H=8, Nq=1, Nk=131072,
                                          d=128, causal=True, n_splits=32, seed=SEED_BASE + 5),
    # A batch of decoding streams with 16 queries each (speculative or chunked decoding).
    "decode_bf16_b4h32q16k32768d128": dict(kind="decode", dtype="bf16", B=4, H=32, Nq=16, Nk=32768,
                                           d=128, causal=True, n_splits=4, seed=SEED_BASE + 6),
    # Residual add + normalisation of 16384 tokens with a hidden size of 8192.
    "norm_bf16_16384x8192": dict(kind="norm", rows=16384, cols=8192, eps=1e-5, seed=SEED_BASE + 7),
}


def generator(seed):
    """The one random source: NumPy PCG64 seeded with ``seed``."""
    return np.random.Generator(np.random.PCG64(int(seed)))


def default_scale(d):
    """1/sqrt(d) rounded to float32, the value every caller passes as ``scale``."""
    return float(np.float32(1.0 / math.sqrt(d)))


def _to_torch(a, dtype):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)  # round-to-nearest-even
    elif dtype == "f16":
        t = t.to(torch.float16)   # round-to-nearest-even
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return t


def attention_inputs(B, H, N, d, seed, dtype="bf16", k_outlier_frac=0.0,
                     k_outlier_scale=8.0):
    """Q, K, V as CPU torch tensors [B, H, N, d] of ``dtype`` ('bf16' or 'f32')."""
    g = generator(seed)
    shape = (B, H, N, d)
    q = g.standard_normal(shape, dtype=np.float32)
    k = g.standard_normal(shape, dtype=np.float32)
    v = g.standard_normal(shape, dtype=np.float32)
    n_out = int(math.floor(k_outlier_frac * N))
    if n_out:
        for b in range(B):
            for h in range(H):
                idx = g.choice(N, size=n_out, replace=False)
                k[b, h, idx, :] *= np.float32(k_outlier_scale)
    return _to_torch(q, dtype), _to_torch(k, dtype), _to_torch(v, dtype)


def upstream_grad(B, H, N, d, seed, dtype="bf16"):
    """An upstream gradient dL/dO as a CPU torch tensor [B, H, N, d]: iid N(0, 1) drawn
    from its own stream (seed + 31), so it never repeats Q, K or V of the same seed."""
    g = generator(seed + 31)
    return _to_torch(g.standard_normal((B, H, N, d), dtype=np.float32), dtype)


def decode_inputs(B, H, Nq, Nk, d, seed, dtype="bf16"):
    """q [B, H, Nq, d] and k, v [B, H, Nk, d] as CPU torch tensors, iid N(0, 1)."""
    g = generator(seed)
    q = g.standard_normal((B, H, Nq, d), dtype=np.float32)
    k = g.standard_normal((B, H, Nk, d), dtype=np.float32)
    v = g.standard_normal((B, H, Nk, d), dtype=np.float32)
    return _to_torch(q, dtype), _to_torch(k, dtype), _to_torch(v, dtype)


def decode_inputs_for(name):
    c = CONFIGS[name]
    return decode_inputs(c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["seed"], c["dtype"])


def merge_parts(n_parts, rows, d, seed, empty_frac=0.1):
    """Partial results for the merge: o_parts [n_parts, rows, d] float32 N(0, 1) and
    lse_parts [n_parts, rows] float32 N(0, sd 3), with a seeded share of parts marked
    empty (-inf; never all parts of a row) and the last row's LSE shifted by +1000."""
    import torch

    g = generator(seed)
    o = g.standard_normal((n_parts, rows, d), dtype=np.float32)
    lse = (g.standard_normal((n_parts, rows)) * 3.0).astype(np.float32)
    empty = g.random((n_parts, rows)) < empty_frac
    empty[0] = False
    lse[empty] = -np.inf
    lse[:, -1] += np.float32(1000.0)
    return torch.from_numpy(o), torch.from_numpy(lse)


def norm_inputs(rows, cols, seed, special_frac=0.01):
    """x, residual [rows, cols] and gamma, beta [cols] as bf16 CPU torch tensors.

    x ~ N(0, 1), residual ~ N(0, sd 2); gamma ~ 1 + 0.1 N(0, 1), beta ~ 0.1 N(0, 1).  Seeded
    disjoint row sets (each special_frac of the rows): rows whose sum h = x + residual is
    constant (residual = c - x is not representable, so x and residual are both set to the
    row's first draws), and rows shifted by +1000 in x (a large mean, where a one-pass
    variance in float32 would cancel).
    """
    g = generator(seed)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    r = g.standard_normal((rows, cols), dtype=np.float32) * np.float32(2.0)
    gamma = (1.0 + 0.1 * g.standard_normal(cols)).astype(np.float32)
    beta = (0.1 * g.standard_normal(cols)).astype(np.float32)
    n_sp = int(math.floor(special_frac * rows))
    pick = g.choice(rows, size=2 * n_sp, replace=False)
    const_rows, shift_rows = np.sort(pick[:n_sp]), np.sort(pick[n_sp:])
    x[const_rows] = x[const_rows, :1]
    r[const_rows] = r[const_rows, :1]
    x[shift_rows] += np.float32(1000.0)
    t = [_to_torch(a, "bf16") for a in (x, r, gamma, beta)]
    return t[0], t[1], t[2], t[3], {"constant": const_rows, "plus1000": shift_rows}


def attention_inputs_for(name):
    c = CONFIGS[name]
    return attention_inputs(c["B"], c["H"], c["N"], c["d"], c["seed"], c["dtype"],
                            c.get("k_outlier_frac", 0.0), c.get("k_outlier_scale", 8.0))


def softmax_inputs(rows, cols, seed, sigma=3.0, special_frac=0.01):
    """x as a CPU float32 torch tensor [rows, cols], plus the special row sets.

    Returns (x, specials) where specials maps 'plus1000', 'minus1000' and
    'all_equal' to sorted int64 arrays of row indices (disjoint).
    """
    import torch

    g = generator(seed)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    x *= np.float32(sigma)
    n_sp = int(math.floor(special_frac * rows))
    pick = g.choice(rows, size=3 * n_sp, replace=False)
    specials = {
        "plus1000": np.sort(pick[:n_sp]),
        "minus1000": np.sort(pick[n_sp:2 * n_sp]),
        "all_equal": np.sort(pick[2 * n_sp:]),
    }
    x[specials["plus1000"]] += np.float32(1000.0)
    x[specials["minus1000"]] -= np.float32(1000.0)
    ae = specials["all_equal"]
    x[ae] = x[ae, :1]
    return torch.from_numpy(x), specials


def softmax_inputs_for(name):
    c = CONFIGS[name]
    return softmax_inputs(c["rows"], c["cols"], c["seed"], c["sigma"])


def scalar_rows(seed=SEED_BASE + 0, per_length=10, max_length=39):
    """The scalar rows: list of (label, scores, values) with Python float lists."""
    rows = [
        ("worked", [0.0, 1.0, 2.0], [10.0, 20.0, 30.0]),
        ("worked_plus1000", [1000.0, 1001.0, 1002.0], [10.0, 20.0, 30.0]),
    ]
    g = generator(seed + 500)
    for n in range(1, max_length + 1):
        for r in range(per_length):
            s = g.normal(0.0, 2.0, size=n)
            v = g.uniform(-10.0, 10.0, size=n)
            rows.append((f"len{n}_{r}", s.tolist(), v.tolist()))
    return rows


def device_normal(shape, seed, dtype, device, chunk=1 << 27):
    """A tensor of ``shape`` on ``device`` filled with iid N(0, 1) values from torch's
    seeded generator on that device, rounded to ``dtype`` (a torch dtype), drawn in
    chunks so that no float32 copy of the whole tensor is made.  For inputs too large to
    draw on the host (more than 2^31 elements); the same seed, device and chunk size give
    the same values."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for s0 in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - s0)
        flat[s0:s0 + n] = torch.randn(n, generator=g, device=device, dtype=torch.float32).to(dtype)
    return out


def sampled_query_rows(B, H, N, per_head, seed):
    """int64 [B, H, per_head + 2]: distinct rows from 1..N-2 per head, plus 0 and N-1."""
    g = generator(seed + 7)
    out = np.empty((B, H, per_head + 2), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            mid = g.choice(np.arange(1, N - 1), size=per_head, replace=False)
            out[b, h] = np.sort(np.concatenate([[0, N - 1], mid]))
    return out
