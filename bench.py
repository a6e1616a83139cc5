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
  cpu_baseline       the float64 oracle on whole heads of the same attention workload, timed on
                     the host (about 10-30 s), in the same TFLOP/s convention
  parity     max abs error of the GPU output on the heads the oracle evaluated
  next       kernels beyond the hot path, timed after it on the same inputs (not part of the
             step): attn_bwd = fa_bwd on the attention workload, in TFLOP/s counted as 2.5x
             the forward's flops (the five matrix products of the gradients); decode_* =
             fa_fwd_splitkv on the decoding workloads, in GB/s of algorithmic HBM traffic
             (K and V once, plus Q, O and LSE) against the HBM3E peak; attn_fwd_f16 = fa_fwd_f16
             on the attention workload's shape in fp16, in TFLOP/s; rmsnorm / layernorm =
             fused_add_rmsnorm / fused_add_layernorm on the 16384 x 8192 bf16 rows, in GB/s of
             algorithmic traffic (read x and residual, write y and h: 8 bytes per element)
  flushed    attention and softmax launch times with L2 and MALL flushed (a 512 MiB device
             write between calls), next to the unflushed means above
  other_configs      the forward on the other attention workloads (bf16 4x16x2048x64
             non-causal, causal N = 8191, causal 1x8x131072x128 with 0.1% outlier keys;
             fp32 1x1x256x64 latency), timed the same way

Only the cpu_baseline leg imports the oracle.
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


CSRC = os.path.join(ROOT, "online_softmax_09_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
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


def read_traffic():
    """{kernel: bytes per launch} from profiles/hbm_traffic.txt, only for kernels whose
    sources are unchanged since the counters were taken."""
    out = {}
    if not os.path.exists(TRAFFIC_FILE):
        return out
    for line in open(TRAFFIC_FILE):
        f = line.split()
        if len(f) >= 9 and f[0] == "kernel" and f[1] in KERNEL_SOURCES:
            rec = dict(zip(f[2::2], f[3::2]))
            if rec.get("sources_sha256_16") == sources_sha(f[1]):
                out[f[1]] = float(rec["fetch_bytes"]) + float(rec["write_bytes"])
    return out


def write_traffic(fetch_csv, write_csv, copy_mib):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) of
    `bench.py --calib-copy-mib copy_mib` into profiles/hbm_traffic.txt.  The plain
    device copy of known size in the same runs calibrates each counter."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib * (1 << 20)
    cf = [v for k, vs in f.items() if "copyBuffer" in k for v in vs]
    cw = [v for k, vs in w.items() if "copyBuffer" in k for v in vs]
    fetch_scale = copy_bytes / (np.median(cf) * 1024.0)
    write_scale = copy_bytes / (np.median(cw) * 1024.0)
    lines = [
        "# HBM bytes per launch, from two rocprofv3 --pmc runs of bench.py (FETCH_SIZE, then",
        "# WRITE_SIZE, KiB per dispatch, median over dispatches), each scaled by what the same",
        f"# counter read for a plain {copy_mib} MiB device copy in the same run:",
        f"#   fetch scale {fetch_scale:.4f}  write scale {write_scale:.4f}",
        "# commands (from the repository root, one GPU):",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- python3 bench.py --steps 2 --warmup 1 --cpu-budget 0 --calib-copy-mib {copy_mib}",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- python3 bench.py --steps 2 --warmup 1 --cpu-budget 0 --calib-copy-mib {copy_mib}",
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


def attn_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def sha256(t):
    return hashlib.sha256(t.contiguous().view(-1).view(dtype=__import__("torch").uint8).numpy()).hexdigest()[:16]


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def cpu_baseline(q, k, v, scale, causal, o_gpu, lse_gpu, budget_s):
    """Time the oracle on whole heads until about budget_s seconds; also return the
    GPU's error on those heads."""
    import oracle

    B, H, N, d = q.shape
    done, t_total = [], 0.0
    err_o = err_l = 0.0
    rel_o = 0.0
    for bh in range(B * H):
        b, h = divmod(bh, H)
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                          v[b:b + 1, h:h + 1], scale, causal)
        t_total += time.perf_counter() - t0
        og = o_gpu[b, h].float().numpy()
        err_o = max(err_o, float(np.max(np.abs(og - o_ref[0, 0]))))
        rel_o = max(rel_o, float(np.max(np.abs(og - o_ref[0, 0]) / np.maximum(np.abs(o_ref[0, 0]), 1e-3))))
        err_l = max(err_l, float(np.max(np.abs(lse_gpu[b, h].numpy() - lse_ref[0, 0]))))
        done.append(bh)
        if t_total >= budget_s:
            break
    flops = attn_flops(1, len(done), N, d, causal)
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"{len(done)} of {B * H} heads of the same workload (every query row), "
                   f"{t_total:.1f} s; float64 NumPy, S materialised per 256-row block, "
                   f"three-pass softmax; flops counted as 4 N^2 d / 2 per head"),
    }, {"heads_checked": len(done), "o_max_abs": err_o, "o_max_rel_floor1e-3": rel_o,
        "lse_max_abs": err_l, "o_tol": 2e-2, "lse_tol": 1e-2}


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


def time_bwd(osm, workloads, torch, dev, ca, qd, kd, vd, od, lsed, scale, steps, warmup):
    """fa_bwd on the attention workload (O and LSE from fa_fwd, a seeded upstream gradient),
    timed with HIP events per launch."""
    B, H, N, d, causal = ca["B"], ca["H"], ca["N"], ca["d"], ca["causal"]
    do = workloads.upstream_grad(B, H, N, d, seed=ca["seed"]).to(dev)
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    ws = torch.empty(B * H * N * 2, dtype=torch.float32, device=dev)

    def run():
        osm.fa_bwd(qd, kd, vd, od, lsed, do, scale=scale, causal=causal, dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    fl = 2.5 * attn_flops(B, H, N, d, causal)
    avg = float(np.mean(ms))
    tf = fl / (avg * 1e-3) / 1e12
    return {"workload": ATTN, "ms_mean": round(avg, 4), "ms_min": round(min(ms), 4), "ms_max": round(max(ms), 4),
            "launches": steps, "flops_per_launch": fl, "tflops": round(tf, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def time_decode(osm, workloads, torch, dev, name, steps, warmup):
    """fa_fwd_splitkv on a decoding workload, timed with HIP events per call."""
    c = workloads.CONFIGS[name]
    B, H, Nq, Nk, d = c["B"], c["H"], c["Nq"], c["Nk"], c["d"]
    q, k, v = (t.to(dev) for t in workloads.decode_inputs_for(name))
    scale = workloads.default_scale(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    need = osm._lib.load().fa_fwd_splitkv_workspace_bytes(B, H, Nq, d, c["n_splits"])
    ws = torch.empty(need // 4, dtype=torch.float32, device=dev)

    def run():
        osm.fa_fwd_splitkv(q, k, v, scale=scale, causal=c["causal"], n_splits=c["n_splits"], out=o, lse=lse,
                           workspace=ws)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    avg = float(np.mean(ms))
    algo = 2.0 * B * H * Nk * d * 2 + 2.0 * B * H * Nq * d * 2 + 4.0 * B * H * Nq
    gbps = algo / (avg * 1e-3) / 1e9
    return {"workload": name, "n_splits": c["n_splits"], "ms_mean": round(avg, 4), "ms_min": round(min(ms), 4),
            "ms_max": round(max(ms), 4), "launches": steps, "bytes_algorithmic": algo, "gbps": round(gbps, 1),
            "workspace_bytes": need,
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(gbps / PEAK_HBM_GBPS, 4)}}


DECODE = ["decode_bf16_b1h8q1k131072d128", "decode_bf16_b4h32q16k32768d128"]


def time_fwd_f16(osm, workloads, torch, dev, ca, scale, steps, warmup):
    """fa_fwd_f16 on the attention workload's shape with the same seeded values in fp16."""
    B, H, N, d, causal = ca["B"], ca["H"], ca["N"], ca["d"], ca["causal"]
    q, k, v = (t.to(dev) for t in workloads.attention_inputs(B, H, N, d, seed=ca["seed"], dtype="f16"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        osm.fa_fwd_f16(q, k, v, scale=scale, causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        osm.fa_fwd_f16(q, k, v, scale=scale, causal=causal, out=o, lse=lse)
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    avg = float(np.mean(ms))
    fl = attn_flops(B, H, N, d, causal)
    tf = fl / (avg * 1e-3) / 1e12
    return {"workload": ATTN.replace("bf16", "f16"), "ms_mean": round(avg, 4), "ms_min": round(min(ms), 4),
            "launches": steps, "flops_per_launch": fl, "tflops": round(tf, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


NORM = "norm_bf16_16384x8192"
OTHER_ATTN = ["attn_bf16_b4h16n2048d64", "attn_bf16_causal_b2h32n8191d128", "attn_bf16_causal_b1h8n131072d128",
              "attn_f32_b1h1n256d64"]


def time_other_configs(osm, workloads, torch, dev, steps, warmup):
    """fa_fwd (fa_fwd_f32 for the fp32 workload) on the other attention workloads."""
    out = {}
    for name in OTHER_ATTN:
        c = workloads.CONFIGS[name]
        q, k, v = (t.to(dev) for t in workloads.attention_inputs_for(name))
        fn = osm.fa_fwd_f32 if c["dtype"] == "f32" else osm.fa_fwd
        scale = workloads.default_scale(c["d"])
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        n = max(3, steps // 4) if c["N"] > 65536 else steps
        for _ in range(warmup):
            fn(q, k, v, scale=scale, causal=c["causal"], out=o, lse=lse)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in evs:
            e0.record()
            fn(q, k, v, scale=scale, causal=c["causal"], out=o, lse=lse)
            e1.record()
        torch.cuda.synchronize()
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        avg = float(np.mean(ms))
        fl = attn_flops(c["B"], c["H"], c["N"], c["d"], c["causal"])
        tf = fl / (avg * 1e-3) / 1e12
        rec = {"ms_mean": round(avg, 4), "ms_min": round(min(ms), 4), "launches": n, "flops_per_launch": fl,
               "tflops": round(tf, 2)}
        if c["dtype"] != "f32":
            rec["frac_of_bf16_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
        else:
            rec["note"] = "fp32 FMA path, latency bound; no matrix-core roofline"
        out[name] = rec
        del q, k, v, o, lse
    return out


def time_norms(osm, workloads, torch, dev, steps, warmup):
    """fused_add_rmsnorm and fused_add_layernorm on the norm workload, HIP events per call."""
    c = workloads.CONFIGS[NORM]
    x, r, g, b, _ = workloads.norm_inputs(c["rows"], c["cols"], c["seed"])
    x, r, g, b = (t.to(dev) for t in (x, r, g, b))
    y, h = torch.empty_like(x), torch.empty_like(x)
    algo = 8.0 * c["rows"] * c["cols"]
    out = {}
    for name, run in (("rmsnorm", lambda: osm.fused_add_rmsnorm(x, r, g, eps=c["eps"], out=y, residual_out=h)),
                      ("layernorm", lambda: osm.fused_add_layernorm(x, r, g, b, eps=c["eps"], out=y,
                                                                    residual_out=h))):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in evs:
            e0.record()
            run()
            e1.record()
        torch.cuda.synchronize()
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        avg = float(np.mean(ms))
        gbps = algo / (avg * 1e-3) / 1e9
        out[name] = {"workload": NORM, "ms_mean": round(avg, 4), "ms_min": round(min(ms), 4), "launches": steps,
                     "bytes_algorithmic": algo, "gbps": round(gbps, 1),
                     "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                  "frac": round(gbps / PEAK_HBM_GBPS, 4)}}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the cpu_baseline leg (0 disables it)")
    ap.add_argument("--no-next", action="store_true", help="skip the kernels beyond the hot path")
    ap.add_argument("--only", choices=["attn", "softmax", "bwd", "decode", "norm", "other", "f16"], default=None,
                    help="time one kernel only (for profiler runs; not the bench line)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB "
                         "(calibrates HBM byte counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.txt from two rocprofv3 counter CSVs and exit")
    args = ap.parse_args()

    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], args.calib_copy_mib or 1024)
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
    x, _ = workloads.softmax_inputs_for(SOFTMAX)
    t_gen = time.perf_counter() - t0
    hashes = {"q": sha256(q), "k": sha256(k), "v": sha256(v), "x": sha256(x)}

    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    od = torch.empty_like(qd)
    lsed = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    xd = x.to(dev)
    yd = torch.empty_like(xd)
    torch.cuda.synchronize()

    run_attn = args.only in (None, "attn")
    run_sm = args.only in (None, "softmax")
    if args.only == "f16":
        print(json.dumps({"only": "f16", **time_fwd_f16(osm, workloads, torch, dev, ca, scale, args.steps,
                                                        args.warmup)}))
        return
    if args.only == "other":
        print(json.dumps({"only": "other", **time_other_configs(osm, workloads, torch, dev, args.steps, args.warmup)}))
        return
    if args.only == "norm":
        print(json.dumps({"only": "norm", **time_norms(osm, workloads, torch, dev, args.steps, args.warmup)}))
        return
    if args.only == "decode":
        print(json.dumps({"only": "decode", "runs": [time_decode(osm, workloads, torch, dev, n, args.steps,
                                                                   args.warmup) for n in DECODE]}))
        return
    if args.only == "bwd":
        osm.fa_fwd(qd, kd, vd, scale=scale, causal=causal, out=od, lse=lsed)
        r = time_bwd(osm, workloads, torch, dev, ca, qd, kd, vd, od, lsed, scale, args.steps, args.warmup)
        print(json.dumps({"only": "bwd", **r}))
        return

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
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()

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

    cpu = None
    parity = None
    if args.cpu_budget > 0:
        o_cpu, lse_cpu = od.cpu(), lsed.cpu()
        cpu, parity = cpu_baseline(q, k, v, scale, causal, o_cpu, lse_cpu, args.cpu_budget)

    nxt = None
    other = None
    if not args.no_next:
        nxt = {"attn_bwd": time_bwd(osm, workloads, torch, dev, ca, qd, kd, vd, od, lsed, scale,
                                    min(args.steps, 10), 2)}
        for n in DECODE:
            nxt[n] = time_decode(osm, workloads, torch, dev, n, min(args.steps, 20), 3)
        nxt["attn_fwd_f16"] = time_fwd_f16(osm, workloads, torch, dev, ca, scale, min(args.steps, 20), 3)
        nxt.update(time_norms(osm, workloads, torch, dev, min(args.steps, 20), 3))
        other = time_other_configs(osm, workloads, torch, dev, min(args.steps, 20), 2)

    traffic = read_traffic()
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
        "cpu_baseline": cpu,
        "parity": parity,
        "next": nxt,
        "other_configs": other,
        "flushed": flushed,
        "timing": {"method": "HIP events on the launch stream", "l2_flush": False,
                   "wall_s_timed_region": round(wall, 3), "input_gen_s": round(t_gen, 1)},
        "inputs_sha256_16": hashes,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
