"""Benchmark of the hot path on one MI355X: bf16 causal attention forward and fp32 row softmax.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one fa_fwd over the causal bf16 workload B=2, H=32, N=8192, d=128 followed by
one online_softmax_rows over the fp32 workload 65536 x 4096, inputs resident in HBM.
W untimed steps, then exactly K timed steps between two device synchronisations.
Kernel durations come from HIP events recorded on the stream the kernels run on
(torch's current stream, which the binding passes to the C ABI).

Prints ONE JSON line:
  value      attention TFLOP/s = (4 B H N^2 d / 2) per launch / mean attention launch time
  softmax    row-softmax GB/s = (8 bytes x rows x cols) per launch / mean launch time
  roofline   attention against the dense bf16 matrix-core peak (2500 TFLOP/s)
  roofline_softmax   row softmax against the HBM3E peak (8000 GB/s)
  clock      the sustained shader clock of the attention kernel (GRBM_GUI_ACTIVE per XCD over
             the dispatch time, from a committed rocprofv3 counter run of the same source)
             and the attention throughput against the matrix-core peak at that clock
  configs    every workload and batch, one record each: latency (mean, median, min, max of
             the per-launch times of batches of back-to-back launches, timed in interleaved
             rounds after their own warm-up), throughput, the
             fraction of its roofline, the device bytes the call touches (the library
             allocates nothing) and, from the cpu_baseline leg, the max abs and max rel
             error against the float64 oracle on sampled outputs
  cpu_baseline       the float64 oracle on whole heads of the same attention workload, timed on
                     the host (about 10-30 s), in the same TFLOP/s convention
  parity     max abs error of the headline attention output on the heads the oracle evaluated
  flushed    attention and softmax launch times with L2 and MALL flushed (a 512 MiB device
             write between calls), next to the unflushed means above

Only the cpu_baseline leg imports the oracle: it times the oracle and computes the errors
that the configs records carry.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

ATTN = "attn_bf16_causal_b2h32n8192d128"
SOFTMAX = "softmax_f32_65536x4096"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 (and fp16) matrix-core peak
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E peak
CUS = 256                   # compute units
FLOP_PER_CLK_CU = 4096      # dense bf16 matrix-core flop per clock per compute unit

CSRC = os.path.join(ROOT, "online_softmax_09_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
CLOCK_FILE = os.path.join(ROOT, "profiles", "clock_attn_fwd_bf16_causal_b2h32n8192d128.txt")
# kernel-name prefix in rocprofv3 output -> sources whose hash stamps its counters
KERNEL_SOURCES = {
    "attn_fwd_bf16": ["attn_fwd_bf16.hip", "device_common.hpp", "mfma_bf16.hpp"],
    "softmax_rows": ["softmax_rows.hip", "device_common.hpp"],
}


def sources_sha(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _stamped_records(path):
    """{kernel: {field: value}} for the 'kernel <name> k v k v ...' lines of a profile
    summary whose sources still hash to the recorded value."""
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        f = line.split()
        if len(f) >= 4 and f[0] == "kernel" and f[1] in KERNEL_SOURCES:
            rec = dict(zip(f[2::2], f[3::2]))
            if rec.get("sources_sha256_16") == sources_sha(f[1]):
                out[f[1]] = rec
    return out


def read_traffic():
    """{kernel: bytes per launch} from profiles/hbm_traffic.txt, only for kernels whose
    sources are unchanged since the counters were taken."""
    return {k: float(r["fetch_bytes"]) + float(r["write_bytes"]) for k, r in _stamped_records(TRAFFIC_FILE).items()}


def read_clock():
    """The attention kernel's sustained clock record, if its sources are unchanged."""
    return _stamped_records(CLOCK_FILE).get("attn_fwd_bf16")


def _per_kernel(path, counter):
    import csv

    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def write_traffic(fetch_csv, write_csv, copy_mib):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) of
    `bench.py --calib-copy-mib copy_mib` into profiles/hbm_traffic.txt.  The plain
    device copy of known size in the same runs calibrates each counter."""
    f = _per_kernel(fetch_csv, "FETCH_SIZE")
    w = _per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib * (1 << 20)
    # the calibration copy is the largest copy dispatch (host transfers run as many small
    # copies of the same kernel)
    def calib(vals):
        cv = [v for k, vs in vals.items() if "copyBuffer" in k for v in vs]
        return [v for v in cv if v >= 0.9 * max(cv)]

    cf, cw = calib(f), calib(w)
    fetch_scale = copy_bytes / (np.median(cf) * 1024.0)
    write_scale = copy_bytes / (np.median(cw) * 1024.0)
    lines = [
        "# HBM bytes per launch, from two rocprofv3 --pmc runs of bench.py (FETCH_SIZE, then",
        "# WRITE_SIZE, KiB per dispatch, median over dispatches), each scaled by what the same",
        f"# counter read for a plain {copy_mib} MiB device copy in the same run:",
        f"#   fetch scale {fetch_scale:.4f}  write scale {write_scale:.4f}",
        "# commands (from the repository root, one GPU):",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- python3 bench.py --steps 2 --warmup 1 --cpu-budget 0 --no-configs --calib-copy-mib {copy_mib}",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- python3 bench.py --steps 2 --warmup 1 --cpu-budget 0 --no-configs --calib-copy-mib {copy_mib}",
        "#   python bench.py --write-traffic <fetch csv> <write csv>",
        "# bench.py reports a kernel's traffic only while its sources hash to sources_sha256_16.",
    ]
    for kern in KERNEL_SOURCES:
        fk = [v for k, vs in f.items() if kern in k for v in vs]
        wk = [v for k, vs in w.items() if kern in k for v in vs]
        if not fk or not wk:
            continue
        lines.append(f"kernel {kern} sources_sha256_16 {sources_sha(kern)} "
                     f"fetch_bytes {np.median(fk) * 1024.0 * fetch_scale:.0f} "
                     f"write_bytes {np.median(wk) * 1024.0 * write_scale:.0f} "
                     f"fetch_kib_raw {np.median(fk):.1f} write_kib_raw {np.median(wk):.1f}")
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_clock(counter_csv, trace_csv):
    """Turn a rocprofv3 run with --pmc GRBM_GUI_ACTIVE and --kernel-trace of
    `bench.py --only attn` into the clock summary: GRBM_GUI_ACTIVE counts GPU-busy
    cycles summed over the 8 XCDs, so busy cycles per XCD / dispatch time = clock."""
    import csv

    grbm = {}
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and "attn_fwd_bf16" in r["Kernel_Name"]:
            grbm[r["Dispatch_Id"]] = grbm.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    ghz = []
    for r in csv.DictReader(open(trace_csv)):
        if r["Dispatch_Id"] in grbm:
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            ghz.append(grbm[r["Dispatch_Id"]] / 8.0 / dur / 1e9)
    ghz = ghz[len(ghz) // 4:]  # the warm dispatches
    lines = [
        "# Sustained shader clock of the attention forward at B=2 H=32 N=8192 d=128 causal (bf16):",
        "# GRBM_GUI_ACTIVE (GPU-busy cycles, summed over the 8 XCDs) / 8 / dispatch duration.",
        "# The same ratio read 2.39, 2.00 and 2.08 GHz on three probe kernels whose shader",
        "# clock was also read in-kernel (s_memtime against s_memrealtime), agreeing to 1%.",
        "# commands (from the repository root, one GPU):",
        "#   rocprofv3 --pmc GRBM_GUI_ACTIVE --kernel-trace --output-format csv -d <dir> -o run -- \\",
        "#       python3 bench.py --only attn --steps 30 --warmup 30 --cpu-budget 0",
        "#   python bench.py --write-clock <dir>/run_counter_collection.csv <dir>/run_kernel_trace.csv",
        "# bench.py reports the clock only while the kernel's sources hash to sources_sha256_16.",
        f"kernel attn_fwd_bf16 sources_sha256_16 {sources_sha('attn_fwd_bf16')} "
        f"ghz_median {np.median(ghz):.4f} ghz_min {min(ghz):.4f} ghz_max {max(ghz):.4f} dispatches {len(ghz)}",
    ]
    with open(CLOCK_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def attn_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def sha256(t):
    return hashlib.sha256(t.contiguous().view(-1).view(dtype=__import__("torch").uint8).numpy()).hexdigest()[:16]


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def nbytes(*ts):
    return int(sum(t.numel() * t.element_size() for t in ts))


# ------------------------------------------------------------------------------------
# The workloads as timed cases.  Each case holds its device buffers, a closure that
# launches one call, its work per call and roofline, and what the oracle leg needs.
# ------------------------------------------------------------------------------------


class Case:
    def __init__(self, name, run, work, unit, bound, peak, dtype, device_bytes, oracle=None, note=None):
        self.name, self.run, self.work, self.unit = name, run, work, unit
        self.bound, self.peak, self.dtype, self.device_bytes = bound, peak, dtype, device_bytes
        self.oracle = oracle  # callable(oracle module) -> error record, run in the cpu_baseline leg
        self.note = note
        self.ms = []  # per-launch time of each timed batch
        self.launches = 0

    def record(self):
        ms = np.array(self.ms)
        mean = float(ms.mean())
        thr = self.work / (mean * 1e-3) / (1e12 if self.unit == "TFLOP/s" else 1e9)
        rec = {"dtype": self.dtype, "ms_mean": round(mean, 4), "ms_median": round(float(np.median(ms)), 4),
               "ms_min": round(float(ms.min()), 4), "ms_max": round(float(ms.max()), 4), "batches": len(ms),
               "launches": self.launches,
               "work_per_launch": self.work, "throughput": round(thr, 2), "unit": self.unit,
               "roofline": {"bound": self.bound, "peak": self.peak,
                            "frac": round(thr / self.peak, 4) if self.peak else None},
               "device_bytes": self.device_bytes}
        if self.note:
            rec["note"] = self.note
        return rec


def sample_rows(n_rows, specials, count, seed):
    """Row indices: `count` seeded distinct rows plus up to 16 of each special set."""
    g = np.random.Generator(np.random.PCG64(seed))
    rows = set(g.choice(n_rows, size=min(count, n_rows), replace=False).tolist())
    for v in (specials or {}).values():
        rows.update(np.asarray(v)[:16].tolist())
    return np.array(sorted(rows), dtype=np.int64)


def gather_rows(t, rows):
    """t [B, H, N, ...] on the GPU, rows [B, H, R] -> CPU float64 array [B, H, R, ...]."""
    import torch

    idx = torch.from_numpy(rows).to(t.device)
    shape = idx.shape + t.shape[3:]
    flat = idx.reshape(idx.shape[0], idx.shape[1], -1, *([1] * (t.dim() - 3))).expand(*shape)
    return torch.gather(t, 2, flat).double().cpu().numpy()


def errors(got, ref, floor):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    return {"max_abs": float(d.max()), "max_rel": float((d / np.maximum(np.abs(ref), floor)).max()),
            "rel_floor": floor}


def attn_case(osm, workloads, torch, dev, name, rows_per_head, fn_name="fa_fwd", dtype_key=None, inputs=None):
    c = workloads.CONFIGS[name]
    B, H, N, d, causal = c["B"], c["H"], c["N"], c["d"], c["causal"]
    dt = dtype_key or c["dtype"]
    if inputs is None:
        q, k, v = workloads.attention_inputs(B, H, N, d, c["seed"], dt, c.get("k_outlier_frac", 0.0),
                                             c.get("k_outlier_scale", 8.0))
    else:
        q, k, v = inputs
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    od = torch.empty_like(qd)
    lsed = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    scale = workloads.default_scale(d)
    fn = getattr(osm, "fa_fwd_f32" if dt == "f32" else fn_name)

    def run():
        fn(qd, kd, vd, scale=scale, causal=causal, out=od, lse=lsed)

    if rows_per_head is None:
        rows = np.broadcast_to(np.arange(N), (B, H, N)).copy()
    else:
        rows = workloads.sampled_query_rows(B, H, N, rows_per_head, seed=c["seed"] + 31)
    gates = {"f32": (1e-5, 1e-5), "f16": (5e-3, 1e-3)}.get(dt, (2e-2, 1e-2))

    def oracle(orc):
        run()
        torch.cuda.synchronize()
        o_ref, l_ref = orc.attention_rows(q, k, v, scale, causal, rows)
        eo = errors(gather_rows(od, rows), o_ref, 1e-6 if dt == "f32" else 1e-3)
        el = errors(gather_rows(lsed, rows), l_ref, 1e-6)
        return {"rows_checked": int(rows.size), "o": eo, "lse": el, "o_gate": gates[0], "lse_gate": gates[1],
                "within_gate": eo["max_abs"] <= gates[0] and el["max_abs"] <= gates[1]}

    tf_dt = {"f32": "f32", "bf16": "bf16", "f16": "f16"}[dt]
    if dt == "f32":
        return Case(name, run, attn_flops(B, H, N, d, causal), "TFLOP/s", "latency", None, tf_dt,
                    nbytes(qd, kd, vd, od, lsed), oracle, note="fp32 FMA path, latency bound; no matrix-core roofline"), \
            (qd, kd, vd, od, lsed)
    return Case(name if dt != "f16" else name.replace("bf16", "f16"), run, attn_flops(B, H, N, d, causal),
                "TFLOP/s", "mfma", PEAK_BF16_TFLOPS, tf_dt, nbytes(qd, kd, vd, od, lsed), oracle), \
        (qd, kd, vd, od, lsed)


def softmax_case(osm, workloads, torch, dev, name, inputs=None):
    c = workloads.CONFIGS[name]
    x, sp = inputs if inputs is not None else workloads.softmax_inputs_for(name)
    xd = x.to(dev)
    yd = torch.empty_like(xd)

    def run():
        osm.online_softmax_rows(xd, out=yd)

    rows = sample_rows(c["rows"], sp, 256, c["seed"] + 17)

    def oracle(orc):
        run()
        torch.cuda.synchronize()
        ref = orc.softmax_rows(x.numpy()[rows])[0]
        e = errors(yd[torch.from_numpy(rows).to(dev)].double().cpu().numpy(), ref, 1e-6)
        return {"rows_checked": int(len(rows)), "y": e, "gate": 1e-5, "within_gate": e["max_abs"] <= 1e-5}

    bytes_ = 8.0 * c["rows"] * c["cols"]
    return Case(name, run, bytes_, "GB/s", "hbm", PEAK_HBM_GBPS, "f32", nbytes(xd, yd), oracle), (xd, yd)


def build_cases(osm, workloads, torch, dev, head, soft, want=None):
    """Every workload and batch as a Case; head / soft are the step's own buffers.
    want(name) -> bool, if given, limits the list (inputs are only made for those)."""
    def attn(name, rows, **kw):
        return lambda: attn_case(osm, workloads, torch, dev, name, rows, **kw)[0]

    makers = [
        # cfg 1: fp32 attention, every output
        ("attn_f32_b1h1n256d64", attn("attn_f32_b1h1n256d64", None)),
        # cfg 2: the step's softmax buffers, and the ragged 4095- and 1-column batches
        (soft.name, lambda: soft),
    ]
    for n in ("softmax_f32_65536x4095", "softmax_f32_65536x1"):
        makers.append((n, lambda n=n: softmax_case(osm, workloads, torch, dev, n)[0]))
    # cfg 3, cfg 4 (the step's buffers), cfg 4' and cfg 5
    makers += [
        ("attn_bf16_b4h16n2048d64", attn("attn_bf16_b4h16n2048d64", 32)),
        (head.name, lambda: head),
        ("attn_bf16_causal_b2h32n8191d128", attn("attn_bf16_causal_b2h32n8191d128", 16)),
        ("attn_bf16_causal_b1h8n131072d128", attn("attn_bf16_causal_b1h8n131072d128", 64)),
        # beyond the hot path: fp16 forward, gradients, split-KV decoding, fused norms
        (ATTN.replace("bf16", "f16"), attn(ATTN, 16, fn_name="fa_fwd_f16", dtype_key="f16")),
        ("attn_bwd_bf16_causal_b2h32n8192d128", lambda: bwd_case(osm, workloads, torch, dev)),
    ]
    for n in ("decode_bf16_b1h8q1k131072d128", "decode_bf16_b4h32q16k32768d128"):
        makers.append((n, lambda n=n: decode_case(osm, workloads, torch, dev, n)))
    cases = [make() for name, make in makers if want is None or want(name)]
    if want is None or any(want(p + "norm_bf16_16384x8192") for p in ("rmsnorm_", "layernorm_")):
        cases.extend(c for c in norm_cases(osm, workloads, torch, dev) if want is None or want(c.name))
    return cases


def bwd_case(osm, workloads, torch, dev):
    """fa_bwd on the headline shape; TFLOP/s counted as 2.5x the forward's flops (the five
    matrix products of the gradients).  The oracle checks one whole head."""
    c = workloads.CONFIGS[ATTN]
    B, H, N, d, causal = c["B"], c["H"], c["N"], c["d"], c["causal"]
    q, k, v = workloads.attention_inputs_for(ATTN)
    do = workloads.upstream_grad(B, H, N, d, seed=c["seed"])
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    scale = workloads.default_scale(d)
    od, lsed = osm.fa_fwd(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    ws = torch.empty(B * H * N * 2, dtype=torch.float32, device=dev)

    def run():
        osm.fa_bwd(qd, kd, vd, od, lsed, dod, scale=scale, causal=causal, dq=dq, dk=dk, dv=dv, workspace=ws)

    def oracle(orc):
        run()
        torch.cuda.synchronize()
        refs = orc.attention_backward(q, k, v, do, scale, causal, heads=[(0, 0)])
        out = {"heads_checked": 1}
        ok = True
        for nm, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
            gg = g[0, 0].double().cpu().numpy()
            rr = r[0]
            scale_r = float(np.max(np.abs(rr)))
            e = float(np.max(np.abs(gg - rr)))
            fro = float(np.linalg.norm(gg - rr) / np.linalg.norm(rr))
            out[nm] = {"max_abs": e, "max_abs_over_max_ref": e / scale_r, "frobenius_rel": fro}
            ok = ok and e <= 2e-2 * scale_r and fro <= 1e-2
        out["gate"] = "max_abs <= 2e-2 max|ref| and Frobenius rel <= 1e-2 per tensor"
        out["within_gate"] = ok
        return out

    return Case("attn_bwd_bf16_causal_b2h32n8192d128", run, 2.5 * attn_flops(B, H, N, d, causal), "TFLOP/s", "mfma",
                PEAK_BF16_TFLOPS, "bf16", nbytes(qd, kd, vd, od, lsed, dod, dq, dk, dv, ws), oracle,
                note="flops counted as 2.5x the forward's (five products); the kernels execute seven")


def decode_case(osm, workloads, torch, dev, name):
    c = workloads.CONFIGS[name]
    B, H, Nq, Nk, d = c["B"], c["H"], c["Nq"], c["Nk"], c["d"]
    q, k, v = workloads.decode_inputs_for(name)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    scale = workloads.default_scale(d)
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    need = osm._lib.load().fa_fwd_splitkv_workspace_bytes(B, H, Nq, d, c["n_splits"])
    ws = torch.empty(need // 4, dtype=torch.float32, device=dev)

    def run():
        osm.fa_fwd_splitkv(qd, kd, vd, scale=scale, causal=c["causal"], n_splits=c["n_splits"], out=o, lse=lse,
                           workspace=ws)

    def oracle(orc):
        run()
        torch.cuda.synchronize()
        eo = {"max_abs": 0.0, "max_rel": 0.0, "rel_floor": 1e-3}
        el = {"max_abs": 0.0, "max_rel": 0.0, "rel_floor": 1e-6}
        for b in range(B):  # one batch at a time bounds host memory
            o_ref, l_ref = orc.attention_rect(q[b:b + 1], k[b:b + 1], v[b:b + 1], scale, c["causal"])
            e1 = errors(o[b:b + 1].double().cpu().numpy(), o_ref, 1e-3)
            e2 = errors(lse[b:b + 1].double().cpu().numpy(), l_ref, 1e-6)
            for acc, e in ((eo, e1), (el, e2)):
                acc["max_abs"] = max(acc["max_abs"], e["max_abs"])
                acc["max_rel"] = max(acc["max_rel"], e["max_rel"])
        return {"rows_checked": B * H * Nq, "o": eo, "lse": el, "o_gate": 2e-2, "lse_gate": 1e-2,
                "within_gate": eo["max_abs"] <= 2e-2 and el["max_abs"] <= 1e-2}

    algo = 2.0 * B * H * Nk * d * 2 + 2.0 * B * H * Nq * d * 2 + 4.0 * B * H * Nq
    return Case(name, run, algo, "GB/s", "hbm", PEAK_HBM_GBPS, "bf16", nbytes(qd, kd, vd, o, lse, ws), oracle,
                note=f"{c['n_splits']} key parts merged in the log domain; bytes = K and V once plus Q, O and LSE")


def norm_cases(osm, workloads, torch, dev):
    name = "norm_bf16_16384x8192"
    c = workloads.CONFIGS[name]
    x, r, g, b, sp = workloads.norm_inputs(c["rows"], c["cols"], c["seed"])
    xd, rd, gd, bd = (t.to(dev) for t in (x, r, g, b))
    y, h = torch.empty_like(xd), torch.empty_like(xd)
    rows = sample_rows(c["rows"], sp, 256, c["seed"] + 19)
    algo = 8.0 * c["rows"] * c["cols"]
    out = []
    for layer in (False, True):
        if layer:
            def run():
                osm.fused_add_layernorm(xd, rd, gd, bd, eps=c["eps"], out=y, residual_out=h)
        else:
            def run():
                osm.fused_add_rmsnorm(xd, rd, gd, eps=c["eps"], out=y, residual_out=h)

        def oracle(orc, run=run, layer=layer):
            run()
            torch.cuda.synchronize()
            xs, rs = x[rows], r[rows]
            if layer:
                y_ref, h_ref = orc.layer_norm(xs, g, b, c["eps"], residual=rs)
            else:
                y_ref, h_ref = orc.rms_norm(xs, g, c["eps"], residual=rs)
            idx = torch.from_numpy(rows).to(dev)
            yy = y[idx].double().cpu().numpy()
            ey = errors(yy, y_ref, 1e-3)
            excess = float(np.max(np.abs(yy - y_ref) - (2.0 ** -8 * np.abs(y_ref) + 2e-3)))
            return {"rows_checked": int(len(rows)), "y": ey, "gate": "|y - ref| <= 2^-8 |ref| + 2e-3",
                    "max_excess_over_gate": excess, "within_gate": excess <= 0.0}

        out.append(Case(("layernorm_" if layer else "rmsnorm_") + name, run, algo, "GB/s", "hbm", PEAK_HBM_GBPS,
                        "bf16", nbytes(xd, rd, gd, bd, y, h), oracle,
                        note="bytes = read x and residual, write y and h (8 per element)"))
    return out


def time_rounds(torch, cases, rounds=3, target_s=0.04, batches=4):
    """Time every case in interleaved rounds: in each round each case gets a short
    warm-up and then `batches` batches of back-to-back launches, each batch between
    two HIP events, so that all cases see the same mix of clock and thermal states.
    A sample is one batch's time per launch (short kernels are not charged for an
    event between every two launches)."""
    est = {}
    for cs in cases:  # first call: compile-free, but caches and clocks settle
        cs.run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cs.run()
        e1.record()
        torch.cuda.synchronize()
        est[cs.name] = max(e0.elapsed_time(e1) * 1e-3, 1e-6)
    for _ in range(rounds):
        for cs in cases:
            n = int(min(48, max(batches, target_s / est[cs.name])))
            per = max(1, n // batches)
            for _ in range(max(2, n // 4)):
                cs.run()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(batches)]
            for a, b in evs:
                a.record()
                for _ in range(per):
                    cs.run()
                b.record()
            torch.cuda.synchronize()
            cs.ms.extend(a.elapsed_time(b) / per for a, b in evs)
            cs.launches += per * batches


def cpu_baseline_leg(q, k, v, scale, causal, o_gpu, lse_gpu, budget_s, cases):
    """The oracle leg.  (1) Times the float64 oracle on whole heads of the headline
    workload for about budget_s seconds (with BLAS pinned to the host's cores) and
    records the GPU's error on those heads; (2) computes every case's error against
    the oracle on sampled outputs."""
    import oracle

    cores = host_cores()
    try:
        from threadpoolctl import threadpool_limits

        pinned = threadpool_limits(limits=cores)
    except Exception:
        import contextlib

        pinned = contextlib.nullcontext()
    with pinned:
        B, H, N, d = q.shape
        done, t_total = [], 0.0
        err_o = err_l = rel_o = 0.0
        for bh in range(B * H):
            b, h = divmod(bh, H)
            t0 = time.perf_counter()
            o_ref, lse_ref = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], scale,
                                              causal)
            t_total += time.perf_counter() - t0
            og = o_gpu[b, h].float().numpy()
            err_o = max(err_o, float(np.max(np.abs(og - o_ref[0, 0]))))
            rel_o = max(rel_o, float(np.max(np.abs(og - o_ref[0, 0]) / np.maximum(np.abs(o_ref[0, 0]), 1e-3))))
            err_l = max(err_l, float(np.max(np.abs(lse_gpu[b, h].numpy() - lse_ref[0, 0]))))
            done.append(bh)
            if t_total >= budget_s:
                break
        flops = attn_flops(1, len(done), N, d, causal)
        cpu = {
            "value": flops / t_total / 1e12,
            "unit": "TFLOP/s",
            "cores": cores,
            "kind": "oracle",
            "sample": (f"{len(done)} of {B * H} heads of the same workload (every query row), "
                       f"{t_total:.1f} s on {cores} host cores (BLAS threads pinned to that count); "
                       f"float64 NumPy, S materialised per 256-row block, three-pass softmax; "
                       f"flops counted as 4 N^2 d / 2 per head"),
        }
        parity = {"heads_checked": len(done), "o_max_abs": err_o, "o_max_rel_floor1e-3": rel_o,
                  "lse_max_abs": err_l, "o_tol": 2e-2, "lse_tol": 1e-2}
        errs = {}
        t0 = time.perf_counter()
        for cs in cases:
            if cs.oracle is not None:
                errs[cs.name] = cs.oracle(oracle)
        cpu["errors_s"] = round(time.perf_counter() - t0, 1)
        return cpu, parity, errs


def time_flushed(torch, run, calls, flush):
    """Mean launch time of run() with flush() (a large device write) before every call."""
    ms = []
    for _ in range(calls):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return round(float(np.mean(ms)), 4)


def calib_copy(torch, dev, mib):
    """Two plain device copies of `mib` MiB: the known byte count that calibrates the HBM
    byte counters of a profiler run."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the cpu_baseline leg (0 disables the leg)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload records")
    ap.add_argument("--only", choices=["attn", "softmax"], default=None,
                    help="time one kernel of the step only (for profiler runs; not the bench line)")
    ap.add_argument("--records", metavar="SUBSTR[,SUBSTR...]", default=None,
                    help="time only the per-workload records whose name contains one of the given "
                         "substrings and print them (for profiler runs; not the bench line)")
    ap.add_argument("--loop-seconds", type=float, default=0.0,
                    help="with --only: run that kernel back to back for this many seconds (for power "
                         "and clock sampling from outside the process), then exit")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB "
                         "(calibrates HBM byte counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.txt from two rocprofv3 counter CSVs and exit")
    ap.add_argument("--write-clock", nargs=2, metavar=("COUNTER_CSV", "TRACE_CSV"),
                    help="write the attention clock summary from a GRBM_GUI_ACTIVE run and exit")
    args = ap.parse_args()

    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], args.calib_copy_mib or 1024)
        return
    if args.write_clock:
        write_clock(*args.write_clock)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the attention heads and softmax rows would shard across "
              f"GPUs with no exchange, but no multi-GPU figure is produced here.", file=sys.stderr)
        sys.exit(2)

    import torch

    import online_softmax_09_amd as osm
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ca = workloads.CONFIGS[ATTN]
    cs = workloads.CONFIGS[SOFTMAX]
    B, H, N, d, causal = ca["B"], ca["H"], ca["N"], ca["d"], ca["causal"]
    scale = workloads.default_scale(d)

    t0 = time.perf_counter()
    q, k, v = workloads.attention_inputs_for(ATTN)
    x, x_sp = workloads.softmax_inputs_for(SOFTMAX)
    t_gen = time.perf_counter() - t0
    hashes = {"q": sha256(q), "k": sha256(k), "v": sha256(v), "x": sha256(x)}

    head, (qd, kd, vd, od, lsed) = attn_case(osm, workloads, torch, dev, ATTN, 16, inputs=(q, k, v))
    soft, (xd, yd) = softmax_case(osm, workloads, torch, dev, SOFTMAX, inputs=(x, x_sp))
    torch.cuda.synchronize()

    if args.records is not None:
        subs = [x for x in args.records.split(",") if x]
        cases = build_cases(osm, workloads, torch, dev, head, soft, want=lambda n: any(x in n for x in subs))
        if not cases:
            sys.exit(f"bench.py: no per-workload record matches {args.records!r}")
        time_rounds(torch, cases, rounds=max(1, args.steps // 10) if args.steps else 3)
        if args.calib_copy_mib:
            calib_copy(torch, dev, args.calib_copy_mib)
        print(json.dumps({"records": {c.name: c.record() for c in cases}}))
        return

    run_attn = args.only in (None, "attn")
    run_sm = args.only in (None, "softmax")

    def step(ev=None):
        if run_attn:
            if ev is not None:
                ev[0].record()
            osm.fa_fwd(qd, kd, vd, scale=scale, causal=causal, out=od, lse=lsed)
            if ev is not None:
                ev[1].record()
        if run_sm:
            if ev is not None:
                ev[2].record()
            osm.online_softmax_rows(xd, out=yd)
            if ev is not None:
                ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    if args.loop_seconds > 0:
        if args.only is None:
            sys.exit("bench.py: --loop-seconds needs --only")
        t0, n, mark = time.perf_counter(), 0, 0.0
        while time.perf_counter() - t0 < args.loop_seconds:
            for _ in range(20):
                step()
            torch.cuda.synchronize()
            n += 20
            if time.perf_counter() - t0 >= mark:
                print(f"loop {args.only}: {n} calls in {time.perf_counter() - t0:.1f} s", flush=True)
                mark += 5.0
        print(json.dumps({"only": args.only, "loop_calls": n, "loop_s": round(time.perf_counter() - t0, 2)}))
        return

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for s in range(args.steps):
        step(evs[s])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    total_ms = t_start.elapsed_time(t_end)
    attn_ms = [e[0].elapsed_time(e[1]) for e in evs] if run_attn else []
    sm_ms = [e[2].elapsed_time(e[3]) for e in evs] if run_sm else []

    if args.calib_copy_mib:
        calib_copy(torch, dev, args.calib_copy_mib)

    fl = attn_flops(B, H, N, d, causal)
    attn_min_bytes = 2.0 * B * H * N * d * 4 + 4.0 * B * H * N  # read Q, K, V; write O; write LSE
    sm_bytes = 8.0 * cs["rows"] * cs["cols"]
    attn_avg = float(np.mean(attn_ms)) if attn_ms else float("nan")
    sm_avg = float(np.mean(sm_ms)) if sm_ms else float("nan")
    tflops = fl / (attn_avg * 1e-3) / 1e12 if attn_ms else None
    gbps = sm_bytes / (sm_avg * 1e-3) / 1e9 if sm_ms else None

    if args.only is not None:
        print(json.dumps({"only": args.only, "attn_ms_mean": attn_avg, "softmax_ms_mean": sm_avg,
                          "attn_tflops": tflops, "softmax_gbps": gbps, "steps": args.steps}))
        return

    flush_buf = torch.empty(512 * (1 << 20) // 4, dtype=torch.float32, device=dev)
    flushed = {
        "attn_ms_mean": time_flushed(torch, lambda: osm.fa_fwd(qd, kd, vd, scale=scale, causal=causal, out=od,
                                                              lse=lsed), 10, lambda: flush_buf.fill_(1.0)),
        "softmax_ms_mean": time_flushed(torch, lambda: osm.online_softmax_rows(xd, out=yd), 10,
                                        lambda: flush_buf.fill_(1.0)),
        "flush": "512 MiB device write (fill_) before every call",
    }
    del flush_buf

    # the step's outputs for the oracle leg, before the per-workload runs reuse the buffers
    o_cpu, lse_cpu = (od.cpu(), lsed.cpu()) if args.cpu_budget > 0 else (None, None)

    cases = []
    configs = None
    if not args.no_configs:
        cases = build_cases(osm, workloads, torch, dev, head, soft)
        time_rounds(torch, cases)
        configs = {c.name: c.record() for c in cases}

    cpu = parity = None
    if args.cpu_budget > 0:
        cpu, parity, errs = cpu_baseline_leg(q, k, v, scale, causal, o_cpu, lse_cpu, args.cpu_budget, cases)
        for name, e in errs.items():
            configs[name]["error"] = e

    traffic = read_traffic()
    clk = read_clock()
    clock = None
    if clk is not None:
        ghz = float(clk["ghz_median"])
        adj = CUS * FLOP_PER_CLK_CU * ghz * 1e9 / 1e12
        clock = {"sustained_ghz": ghz, "ghz_range": [float(clk["ghz_min"]), float(clk["ghz_max"])],
                 "source": os.path.relpath(CLOCK_FILE, ROOT),
                 "clock_adjusted_peak_tflops": round(adj, 1),
                 "frac_of_clock_adjusted_peak": round(tflops / adj, 4),
                 "note": "peak at 2.4 GHz is 256 CU x 4096 flop/clk = 2516.6 TFLOP/s; the roofline uses 2500"}
    line = {
        "metric": "attn fwd TFLOP/s & % bf16 MFMA peak (causal N=8192 d=128); softmax GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{ATTN} + {SOFTMAX}", "B": B, "H": H, "N": N, "d": d,
                   "causal": causal, "scale": scale, "softmax_rows": cs["rows"],
                   "softmax_cols": cs["cols"], "softmax_dtype": "f32"},
        "attn": {"ms_mean": round(attn_avg, 4), "ms_min": round(min(attn_ms), 4),
                 "ms_max": round(max(attn_ms), 4), "tflops": round(tflops, 2),
                 "flops_per_launch": fl},
        "softmax": {"ms_mean": round(sm_avg, 4), "ms_min": round(min(sm_ms), 4),
                    "ms_max": round(max(sm_ms), 4), "gbps": round(gbps, 1),
                    "bytes_per_launch": sm_bytes, "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic.get("attn_fwd_bf16"),
                     "traffic_algorithmic_min": attn_min_bytes},
        "roofline_softmax": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                             "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                             "traffic": traffic.get("softmax_rows"),
                             "traffic_algorithmic": sm_bytes},
        "clock": clock,
        "cpu_baseline": cpu,
        "parity": parity,
        "configs": configs,
        "flushed": flushed,
        "timing": {"method": "HIP events on the launch stream", "l2_flush": False,
                   "configs": "3 interleaved rounds; per case and round a warm-up, then 4 batches of "
                              "back-to-back launches, each batch between two HIP events "
                              "(ms_* are per-launch times of the batches)",
                   "wall_s_timed_region": round(wall, 3), "input_gen_s": round(t_gen, 1),
                   "device_peak_allocated_bytes": int(torch.cuda.max_memory_allocated(dev))},
        "inputs_sha256_16": hashes,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
