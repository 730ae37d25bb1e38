"""Benchmark of the fused-attention hot path on one MI355X.

One step = the whole path once over resident synthetic inputs:
  * causal GQA prefill, B=1 H=32 Hkv=8 N=8192 d=128, bf16 (sharpened Q/K);
  * split-K decode, B=64 H=32 Hkv=8 Nk=32768 d=128, bf16, 16 splits + merge;
  * fp32 single-head forward, N=256 d=64 (the fp32 variant).
The headline value is the prefill's algorithmic TFLOP/s (4 d per visible
query-key pair); the decode's algorithmic GB/s (K/V cache read once + q + O +
LSE) is reported beside it. Kernel durations come from HIP events recorded on
the stream the kernels are launched on, around each call inside the timed
steps.

Beside the step, and timed in a loop of their own over the same number of
steps, these variants are measured: the causal d = 64 prefill (B4 H16 N2048),
the causal sliding-window prefill (window 4096 over 32768 tokens), the
prefill with Q and K in fp8, packed-document prefill (four 8k contexts filled
with documents of log-uniform length, the mask restarting at every
document) and its backward, the decode over the same cache buffers with a
random length per sequence, that decode with its keys in 16-key pages
scattered over one pool, and the backward of the prefill.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extensions]
    python bench.py --trace-summary run_kernel_trace.csv --trace-skip W
    python bench.py --counter-summary run_counter_collection.csv --trace-skip W
    python bench.py --write-traffic FETCH.csv WRITE.csv --trace-skip W --calib-copy MIB
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (% bf16 MFMA peak) at N=8k d=128; decode GB/s (% HBM)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "fwd_bf16": ["exact_io_aware_06_amd/csrc/fwd_bf16.hip", "exact_io_aware_06_amd/csrc/common.hpp"],
    "decode": ["exact_io_aware_06_amd/csrc/decode.hip", "exact_io_aware_06_amd/csrc/common.hpp"],
}


def source_digest(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kind: str):
    """Counter-derived HBM bytes per launch, if measured on this exact source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(kind)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_digest") != source_digest(kind):
        return None
    return t.get("bytes_per_launch")


def trace_summary(path: str, skip: int) -> str:
    """Markdown table of the library's kernels in a rocprofv3 kernel_trace.csv,
    over each kernel's launches after its first `skip` (the warm-up calls):
    launches, mean, median, min and max duration in ns."""
    import csv
    import re
    import statistics

    pat = re.compile(r"miattn::\(anonymous namespace\)::(\w+(<[^()]*>)?)\(")
    runs = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            m = pat.search(r["Kernel_Name"])
            if m is None:
                continue
            # one kernel serves several workloads: the grid tells them apart
            wgs = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            runs.setdefault((m.group(1), wgs), []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    lines = [f"| kernel | work-groups | launches (after the first {skip}) | mean ns | median ns | "
             f"min ns | max ns |", "|---|---|---|---|---|---|---|"]
    order = sorted(runs, key=lambda k: -sum(d for _, d in runs[k]))
    for name, wgs in order:
        ds = [d for _, d in sorted(runs[(name, wgs)])][skip:]
        if not ds:
            continue
        lines.append(f"| `{name}` | {wgs} | {len(ds)} | {statistics.fmean(ds):.0f} | "
                     f"{statistics.median(ds):.0f} | {min(ds)} | {max(ds)} |")
    return "\n".join(lines)


def _short_kernel(name: str):
    import re
    m = re.search(r"miattn::\(anonymous namespace\)::(\w+(<[^()]*>)?)\(", name)
    return m.group(1) if m else None


def counter_table(path: str, skip: int):
    """{(kernel, work-groups): {counter: [values per dispatch, in order]}} for
    this library's kernels in a rocprofv3 counter_collection.csv, plus the
    values of the largest runtime copy kernel (the calibration copy)."""
    import csv
    per, copy = {}, {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            name, ctr, val = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
            if "copyBuffer" in name:
                copy[ctr] = max(copy.get(ctr, 0.0), val)
                continue
            k = _short_kernel(name)
            if k is None:
                continue
            wgs = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
            per.setdefault((k, wgs), {}).setdefault(ctr, []).append(
                (int(r["Dispatch_Id"]), val))
    out = {key: {c: [v for _, v in sorted(vs)][skip:] for c, vs in d.items()}
           for key, d in per.items()}
    return out, copy


def counter_summary(path: str, skip: int) -> str:
    """Markdown: mean value per dispatch of every counter, per kernel and grid."""
    import statistics
    tab, copy = counter_table(path, skip)
    lines = []
    for (k, wgs), d in sorted(tab.items()):
        lines.append(f"`{k}`, {wgs} work-groups (launches after the first {skip}):\n")
        lines.append("| counter | launches | mean per launch |")
        lines.append("|---|---|---|")
        for c, vs in sorted(d.items()):
            if vs:
                lines.append(f"| `{c}` | {len(vs)} | {statistics.fmean(vs):,.1f} |")
        lines.append("")
    if copy:
        lines.append("Largest runtime copy kernel (the calibration copy): "
                     + ", ".join(f"`{c}` = {v:,.1f}" for c, v in sorted(copy.items())))
    return "\n".join(lines)


def write_traffic(fetch_csv: str, write_csv: str, skip: int, copy_mib: int) -> dict:
    """HBM bytes per launch of the headline prefill and decode kernels from a
    FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch), each scaled so
    that the calibration copy of `copy_mib` MiB reads and writes exactly its
    size; stored in profiles/traffic.json with the digest of the sources."""
    import statistics

    from exact_io_aware_06_amd import accounting
    import synth
    fe, cf = counter_table(fetch_csv, skip)
    wr, cw = counter_table(write_csv, skip)
    kib = copy_mib * 1024.0
    sf, sw = kib / cf["FETCH_SIZE"], kib / cw["WRITE_SIZE"]
    cp = synth.CONFIGS["causal_gqa_n8192_d128"]
    cd = synth.CONFIGS["decode_b64_nk32768_d128"]
    want = {
        "fwd_bf16": (("fwd_bf16_kernel<128, false, false, true>", cp.B * cp.H * (cp.Nq // 128)),
                     accounting.prefill_bytes(cp.B, cp.H, cp.Hkv, cp.Nq, cp.Nk, cp.d)),
        "decode": (("decode_split_kernel<128, false, false, false>", cd.B * cd.Hkv * cd.splits),
                   accounting.decode_bytes(cd.B, cd.H, cd.Hkv, cd.Nk, cd.d)),
    }
    out = {}
    for kind, (key, alg) in want.items():
        f = statistics.fmean(fe[key]["FETCH_SIZE"]) * 1024 * sf
        w = statistics.fmean(wr[key]["WRITE_SIZE"]) * 1024 * sw
        out[kind] = {"source_digest": source_digest(kind), "bytes_per_launch": int(round(f + w)),
                     "fetch_bytes": int(round(f)), "write_bytes": int(round(w)),
                     "algorithmic_bytes": alg, "launches_averaged": len(fe[key]["FETCH_SIZE"]),
                     "fetch_scale": round(sf, 4), "write_scale": round(sw, 4)}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores(threadpool_info):
    """The host threads the oracle ran on: its BLAS thread pool (the
    matrix products; NumPy's elementwise work is single-threaded), bounded by
    the CPUs this process may run on, plus that CPU set and the CPU model."""
    affinity = len(os.sched_getaffinity(0))
    blas = max([i.get("num_threads", 1) for i in threadpool_info()
                if i.get("user_api") == "blas"] or [1])
    return {"cores": min(blas, affinity), "affinity_cpus": affinity, "blas_threads": blas,
            "cpu_model": cpu_model()}


def cpu_baseline_prefill(cfg, heads: int, q, k, v):
    """The oracle, untuned, on the first `heads` heads of the prefill workload.

    q, k, v are host copies of the benchmarked tensors (first `heads` query
    heads and their K/V heads).
    """
    from threadpoolctl import threadpool_info

    import oracle
    from exact_io_aware_06_amd import accounting

    sub = cfg.with_(H=heads, Hkv=max(1, heads * cfg.Hkv // cfg.H))
    t0 = time.perf_counter()
    oracle.attention_ref(q, k, v, sub.scale, sub.causal, sub.window)
    dt = time.perf_counter() - t0
    flops = accounting.prefill_flops(1, heads, sub.Nq, sub.Nk, sub.d, sub.causal, sub.window)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", **host_cores(threadpool_info),
            "kind": "oracle",
            "sample": f"{heads} of {cfg.H} heads of the prefill workload (fp64, full score "
                      f"matrix per head), {dt:.2f} s wall",
            "seconds": dt}


def cpu_baseline_decode(cfg, seqs: int, q, kc, vc):
    """The oracle, untuned, on host copies of the first `seqs` decode sequences."""
    from threadpoolctl import threadpool_info

    import oracle
    from exact_io_aware_06_amd import accounting

    sub = cfg.with_(B=seqs)
    t0 = time.perf_counter()
    oracle.decode_ref(q, kc, vc, sub.scale, sub.window)
    dt = time.perf_counter() - t0
    nbytes = accounting.decode_bytes(seqs, sub.H, sub.Hkv, sub.Nk, sub.d, window=sub.window)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", **host_cores(threadpool_info),
            "kind": "oracle",
            "sample": f"{seqs} of {cfg.B} sequences of the decode workload, {dt:.2f} s wall",
            "seconds": dt}


def measure_ceilings(torch, mi, dev):
    """Sustained bf16 matrix-core rate and streaming-read bandwidth on this GPU."""
    sink = torch.zeros(4096, dtype=torch.float32, device=dev)
    best_tf = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = mi.api.calib_mfma(1024, 8000, sink)
        e1.record()
        torch.cuda.synchronize()
        best_tf = max(best_tf, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    usink = torch.zeros(4, dtype=torch.int32, device=dev)
    best_gb = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        nbytes = mi.api.calib_read(buf, usink, 2048)
        e1.record()
        torch.cuda.synchronize()
        best_gb = max(best_gb, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(best_tf, 1), "hbm_read_gbs": round(best_gb, 1),
            "method": "attn_calib_mfma (1024 WGs x 4 waves x 8000 x 8 independent 32x32x16 "
                      "bf16 MFMAs) and attn_calib_read (2 GiB, 16-byte non-temporal loads), "
                      "best of 3"}


SWEEP_N = [1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072]


def context_sweep(torch, synth, mi, accounting, dev, steps, warmup):
    """Causal GQA prefill (B1 H32 Hkv8 d128, scale 1/sqrt(d)) over context lengths."""
    base = synth.CONFIGS["window4096_gqa_n32768_d128"].with_(window=0)
    rows = []
    for n in SWEEP_N:
        c = base.with_(name=f"causal{n}", Nq=n, Nk=n)
        q, k, v = synth.prefill_inputs(c, 0, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty(c.B, c.H, c.Nq, dtype=torch.float32, device=dev)
        call = lambda: mi.attn_fwd(q, k, v, scale=c.scale, causal=1, out=o, lse=lse)
        for _ in range(warmup):
            call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)
        flops = accounting.prefill_flops(c.B, c.H, n, n, c.d, 1, 0)
        med = ms[len(ms) // 2]
        tf = flops / (med * 1e-3) / 1e12
        rows.append({"N": n, "ms_median": round(med, 4), "ms_min": round(ms[0], 4),
                     "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "algorithmic_flops": flops})
        print(f"sweep N={n}: {med:.4f} ms, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--cpu-seqs", type=int, default=64)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "fp32", "packed", "kvlens", "window",
                                       "paged", "backward", "fp8", "packed_backward",
                                       "prefill_d64", "kvlens_skewed"],
                    default="all", help="launch only one part (for profiling runs)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step: causal prefill over N = 1k..128k, one JSON line")
    ap.add_argument("--no-extensions", action="store_true",
                    help="skip the packed-document prefill and mixed-length decode legs")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured matrix-core / read-bandwidth ceilings")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print the steady-state launch durations of this library's kernels "
                         "from a rocprofv3 kernel_trace.csv (no GPU needed) and exit")
    ap.add_argument("--trace-skip", type=int, default=None,
                    help="with --trace-summary: leading launches per kernel to drop "
                         "(default: --warmup)")
    ap.add_argument("--counter-summary", metavar="CSV",
                    help="print the mean counter values per launch of this library's kernels "
                         "from a rocprofv3 counter_collection.csv (no GPU needed) and exit")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="compute the headline kernels' HBM bytes per launch from a FETCH_SIZE "
                         "and a WRITE_SIZE counter run (with --calib-copy) into "
                         "profiles/traffic.json and exit")
    args = ap.parse_args()
    skip = args.warmup if args.trace_skip is None else args.trace_skip
    if args.trace_summary:
        print(trace_summary(args.trace_summary, skip))
        return
    if args.counter_summary:
        print(counter_summary(args.counter_summary, skip))
        return
    if args.write_traffic:
        print(json.dumps(write_traffic(*args.write_traffic, skip, args.calib_copy or 1024),
                         indent=1))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(each GPU's share of prefill or decode is the single-GPU workload).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import exact_io_aware_06_amd as mi
    from exact_io_aware_06_amd import accounting

    if not os.path.exists(mi.library_path()):
        from exact_io_aware_06_amd import build
        build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep:
        rows = context_sweep(torch, synth, mi, accounting, dev, max(3, min(args.steps, 20)),
                             max(1, min(args.warmup, 3)))
        print(json.dumps({"sweep": "causal GQA prefill B1 H32 Hkv8 d128 bf16, scale 1/sqrt(d), "
                                   "N(0,1) inputs", "unit": "TFLOP/s", "points": rows}))
        return

    cp = synth.CONFIGS["causal_gqa_n8192_d128"]
    cd = synth.CONFIGS["decode_b64_nk32768_d128"]
    cf = synth.CONFIGS["f32_n256_d64"]
    c2 = synth.CONFIGS["causal_b4_h16_n2048_d64"]
    q, k, v = synth.prefill_inputs(cp, seed=0, device=dev)
    qd, kc, vc = synth.decode_inputs(cd, seed=0, device=dev)
    qf, kf, vf = synth.prefill_inputs(cf, seed=0, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(cp.B, cp.H, cp.Nq, dtype=torch.float32, device=dev)
    od = torch.empty_like(qd)
    lsed = torch.empty(cd.B, cd.H, dtype=torch.float32, device=dev)
    ws = torch.empty(mi.decode_workspace_bytes(cd.B, cd.H, cd.Hkv, cd.Nk, cd.d, cd.splits),
                     dtype=torch.uint8, device=dev)
    of = torch.empty_like(qf)
    lsef = torch.empty(cf.B, cf.H, cf.Nq, dtype=torch.float32, device=dev)

    # Packed documents (four 8k contexts of log-uniform documents) and decode
    # over the same cache buffers with per-sequence lengths.
    cpk = synth.inputs.PACKED["packed_24docs_4x8192_d128"]
    pk_lens = cpk.lengths(0)
    pk_cu = synth.inputs.cu_seqlens(pk_lens)
    pk_total = int(pk_cu[-1])
    qp, kp, vp = synth.inputs.packed_inputs(cpk, pk_total, pk_total, seed=0, device=dev)
    cu_dev = torch.from_numpy(pk_cu).to(dev)
    op = torch.empty_like(qp)
    lsep = torch.empty(cpk.H, pk_total, dtype=torch.float32, device=dev)
    # the packed backward: the packed forward's O and LSE, a seeded dO
    dout_p = synth.gen_normal((cpk.H, pk_total, cpk.d), 0, 4, 0, "bf16", 1.0, dev)
    dqp, dkp, dvp = torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(vp)
    bws_p = torch.empty(mi.bwd_workspace_bytes(1, cpk.H, cpk.Hkv, pk_total, pk_total, cpk.d),
                        dtype=torch.uint8, device=dev)
    ck = synth.inputs.DECODE_KVLENS
    kv_lens = synth.inputs.kv_lengths(0, ck.B, ck.Nk)
    kv_lens_dev = torch.from_numpy(kv_lens).to(dev)
    # A skewed batch over the same cache: every eighth sequence full, the rest 512 keys.
    sk_lens = synth.inputs.skewed_kv_lengths(ck.B, ck.Nk)
    sk_lens_dev = torch.from_numpy(sk_lens).to(dev)
    # The same lengths stored in 16-key pages scattered over one pool.
    cg = synth.inputs.PAGED["decode"]
    page_size = synth.inputs.PAGED["page_size"]
    pg_table, num_pages = synth.inputs.paged_block_table(0, kv_lens, page_size)
    qg, kpg, vpg = synth.inputs.paged_inputs(cg, num_pages, page_size, seed=0, device=dev)
    pg_table_dev = torch.from_numpy(pg_table).to(dev)
    # The headline prefill with Q and K in fp8 e4m3 (per-tensor descales).
    q8, k8, v8b, q8_ds, k8_ds = synth.inputs.fp8_prefill_inputs(cp, seed=0, device=dev)
    o8 = torch.empty_like(o)
    lse8 = torch.empty_like(lse)
    # The causal d = 64 prefill (B4 H16 N2048).
    q2, k2, v2 = synth.prefill_inputs(c2, seed=0, device=dev)
    o2 = torch.empty_like(q2)
    lse2 = torch.empty(c2.B, c2.H, c2.Nq, dtype=torch.float32, device=dev)
    # The causal sliding-window prefill (window 4096 over 32768 tokens).
    cw = synth.CONFIGS["window4096_gqa_n32768_d128"]
    qw, kw, vw = synth.prefill_inputs(cw, seed=0, device=dev)
    ow = torch.empty_like(qw)
    lsew = torch.empty(cw.B, cw.H, cw.Nq, dtype=torch.float32, device=dev)
    # Backward of the headline prefill: the forward's O and LSE, a seeded dO.
    dout = synth.gen_normal((cp.B, cp.H, cp.Nq, cp.d), 0, 4, 0, "bf16", 1.0, dev)
    dq_b, dk_b, dv_b = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(mi.bwd_workspace_bytes(cp.B, cp.H, cp.Hkv, cp.Nq, cp.Nk, cp.d),
                      dtype=torch.uint8, device=dev)

    parts = {
        "prefill": lambda: mi.attn_fwd(q, k, v, scale=cp.scale, causal=cp.causal,
                                       window=cp.window, out=o, lse=lse),
        "decode": lambda: mi.attn_decode(qd, kc, vc, scale=cd.scale, window=cd.window,
                                         num_splits=cd.splits, out=od, lse=lsed, workspace=ws),
        "fp32": lambda: mi.attn_fwd(qf, kf, vf, scale=cf.scale, causal=cf.causal,
                                    window=cf.window, out=of, lse=lsef),
        "packed": lambda: mi.attn_fwd_varlen(qp, kp, vp, cu_dev, cu_dev, max(pk_lens),
                                             scale=cpk.scale, causal=cpk.causal,
                                             window=cpk.window, out=op, lse=lsep),
        "kvlens": lambda: mi.attn_decode_varlen(qd, kc, vc, kv_lens_dev, scale=ck.scale,
                                                window=ck.window, num_splits=ck.splits,
                                                out=od, lse=lsed, workspace=ws),
        "kvlens_skewed": lambda: mi.attn_decode_varlen(qd, kc, vc, sk_lens_dev, scale=ck.scale,
                                                       window=ck.window, num_splits=ck.splits,
                                                       out=od, lse=lsed, workspace=ws),
        "packed_backward": lambda: mi.attn_bwd_varlen(
            qp, kp, vp, op, lsep, dout_p, cu_dev, cu_dev, max(pk_lens), max(pk_lens),
            scale=cpk.scale, causal=cpk.causal, window=cpk.window, dq=dqp, dk=dkp, dv=dvp,
            workspace=bws_p),
        "window": lambda: mi.attn_fwd(qw, kw, vw, scale=cw.scale, causal=cw.causal,
                                      window=cw.window, out=ow, lse=lsew),
        "prefill_d64": lambda: mi.attn_fwd(q2, k2, v2, scale=c2.scale, causal=c2.causal,
                                           window=c2.window, out=o2, lse=lse2),
        "fp8": lambda: mi.attn_fwd_fp8(q8, k8, v8b, q8_ds, k8_ds, scale=cp.scale,
                                       causal=cp.causal, window=cp.window, out=o8, lse=lse8),
        "backward": lambda: mi.attn_bwd(q, k, v, o, lse, dout, scale=cp.scale,
                                        causal=cp.causal, window=cp.window, dq=dq_b, dk=dk_b,
                                        dv=dv_b, workspace=bws),
        "paged": lambda: mi.attn_decode_paged(qg, kpg, vpg, pg_table_dev, kv_lens_dev,
                                              scale=cg.scale, window=cg.window,
                                              num_splits=cg.splits, out=od, lse=lsed,
                                              workspace=ws),
    }
    core = ["prefill", "decode", "fp32"]
    ext = [] if args.no_extensions else ["prefill_d64", "window", "fp8", "packed",
                                         "packed_backward", "kvlens", "kvlens_skewed", "paged",
                                         "backward"]
    if args.only != "all":
        core, ext = [args.only], []

    if args.calib_copy > 0:
        nbytes = args.calib_copy << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"calibration copy: {nbytes} bytes read, {nbytes} bytes written", file=sys.stderr)
        del src, dst

    def timed(names):
        """Warm up, then time `args.steps` passes over `names`; per-part event times."""
        for _ in range(args.warmup):
            for n in names:
                parts[n]()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            evs[i][0].record()
            for j, n in enumerate(names):
                parts[n]()
                evs[i][j + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = {n: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, n in enumerate(names)}
        return wall, ms

    if "backward" in core:
        parts["prefill"]()  # O and LSE, inputs of the backward
    if "packed_backward" in core:
        parts["packed"]()
        torch.cuda.synchronize()
    wall, ms = timed(core)
    ext_ms = timed(ext)[1] if ext else {}
    ms.update(ext_ms)
    pre_ms = ms.get("prefill", [0.0])
    dec_ms = ms.get("decode", [0.0])
    f32_ms = ms.get("fp32", [0.0])
    mean = lambda xs: sum(xs) / len(xs)

    pre_flops = accounting.prefill_flops(cp.B, cp.H, cp.Nq, cp.Nk, cp.d, cp.causal, cp.window)
    dec_bytes = accounting.decode_bytes(cd.B, cd.H, cd.Hkv, cd.Nk, cd.d, window=cd.window)
    f32_flops = accounting.prefill_flops(cf.B, cf.H, cf.Nq, cf.Nk, cf.d, cf.causal, cf.window)
    rate = lambda work, ms: work / (ms * 1e-3) if ms > 0 else 0.0
    ceilings = None if args.no_ceilings else measure_ceilings(torch, mi, dev)
    pre_tflops = rate(pre_flops, mean(pre_ms)) / 1e12
    dec_gbs = rate(dec_bytes, mean(dec_ms)) / 1e9
    pk_flops = accounting.packed_flops(cpk.H, pk_cu, pk_cu, cpk.d, cpk.causal, cpk.window)
    kvl_bytes = accounting.decode_kvlens_bytes(ck.H, ck.Hkv, kv_lens, ck.d, window=ck.window)
    sk_bytes = accounting.decode_kvlens_bytes(ck.H, ck.Hkv, sk_lens, ck.d, window=ck.window)
    pg_bytes = accounting.decode_paged_bytes(cg.H, cg.Hkv, kv_lens, cg.d, page_size,
                                             window=cg.window)
    bwd_flops = accounting.backward_flops(cp.B, cp.H, cp.Nq, cp.Nk, cp.d, cp.causal, cp.window)
    win_flops = accounting.prefill_flops(cw.B, cw.H, cw.Nq, cw.Nk, cw.d, cw.causal, cw.window)
    d64_flops = accounting.prefill_flops(c2.B, c2.H, c2.Nq, c2.Nk, c2.d, c2.causal, c2.window)
    if args.only != "all":
        xs = ms[args.only]
        val, unit = {"prefill": (pre_tflops, "TFLOP/s"), "decode": (dec_gbs, "GB/s"),
                     "fp32": (rate(f32_flops, mean(f32_ms)) / 1e12, "TFLOP/s"),
                     "packed": (rate(pk_flops, mean(xs)) / 1e12, "TFLOP/s"),
                     "kvlens": (rate(kvl_bytes, mean(xs)) / 1e9, "GB/s"),
                     "kvlens_skewed": (rate(sk_bytes, mean(xs)) / 1e9, "GB/s"),
                     "paged": (rate(pg_bytes, mean(xs)) / 1e9, "GB/s"),
                     "backward": (rate(bwd_flops, mean(xs)) / 1e12, "TFLOP/s"),
                     "fp8": (rate(pre_flops, mean(xs)) / 1e12, "TFLOP/s"),
                     "window": (rate(win_flops, mean(xs)) / 1e12, "TFLOP/s"),
                     "prefill_d64": (rate(d64_flops, mean(xs)) / 1e12, "TFLOP/s"),
                     "packed_backward": (rate(2.5 * pk_flops, mean(xs)) / 1e12,
                                         "TFLOP/s")}[args.only]
        print(json.dumps({"only": args.only, "ms": round(mean(xs), 4),
                          "ms_min": round(min(xs), 4), "value": round(val, 2),
                          "unit": unit, "steps": args.steps}))
        return

    out = {
        "metric": METRIC,
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) (prefill Q and K times 3*d^-1/4 before the bf16 cast)",
        "config": {
            "workload": "causal GQA prefill B1 H32 Hkv8 N8192 d128 bf16 (sharpened, scale 1.0) "
                        "+ split-K decode B64 H32 Hkv8 Nk32768 d128 bf16 16 splits "
                        "+ fp32 forward B1 H1 N256 d64",
            "prefill": {"B": cp.B, "H": cp.H, "Hkv": cp.Hkv, "N": cp.Nq, "d": cp.d,
                        "causal": cp.causal, "window": cp.window, "scale": cp.scale,
                        "algorithmic_flops": pre_flops},
            "decode": {"B": cd.B, "H": cd.H, "Hkv": cd.Hkv, "Nk": cd.Nk, "d": cd.d,
                       "splits": cd.splits, "algorithmic_bytes": dec_bytes},
        },
        "prefill_ms": round(mean(pre_ms), 4),
        "prefill_ms_min": round(min(pre_ms), 4),
        "decode": {"value": round(dec_gbs, 1), "unit": "GB/s", "ms": round(mean(dec_ms), 4),
                   "ms_min": round(min(dec_ms), 4), "frac_hbm": round(dec_gbs / PEAK_HBM_GBS, 4)},
        "fp32_forward": {"ms": round(mean(f32_ms), 4),
                         "tflops": round(rate(f32_flops, mean(f32_ms)) / 1e12, 3)},
        "roofline": {"kernel": "fwd_bf16_kernel<128>", "bound": "mfma",
                     "achieved": round(pre_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for("fwd_bf16")},
        "ceilings": ceilings,
        "roofline_decode": {"kernel": "decode_split_kernel<128, false, false, false> + decode_merge_kernel<128>",
                            "bound": "hbm", "achieved": round(dec_gbs, 1),
                            "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                            "traffic": traffic_for("decode")},
    }
    if "prefill_d64" in ms:
        d64_tf = rate(d64_flops, mean(ms["prefill_d64"])) / 1e12
        out["prefill_d64"] = {
            "workload": f"causal prefill B{c2.B} H{c2.H} Hkv{c2.Hkv} N{c2.Nq} d{c2.d} bf16, "
                        f"scale 1/sqrt(d)",
            "algorithmic_flops": d64_flops,
            "algorithmic_bytes": accounting.prefill_bytes(c2.B, c2.H, c2.Hkv, c2.Nq, c2.Nk, c2.d),
            "ms": round(mean(ms["prefill_d64"]), 4), "ms_min": round(min(ms["prefill_d64"]), 4),
            "value": round(d64_tf, 2), "unit": "TFLOP/s",
            "frac_peak": round(d64_tf / PEAK_BF16_TFLOPS, 4)}
    if "window" in ms:
        w_tf = rate(win_flops, mean(ms["window"])) / 1e12
        out["window_prefill"] = {
            "workload": f"causal sliding-window GQA prefill B{cw.B} H{cw.H} Hkv{cw.Hkv} "
                        f"N{cw.Nq} d{cw.d} bf16, window {cw.window}, scale 1/sqrt(d)",
            "algorithmic_flops": win_flops,
            "algorithmic_bytes": accounting.prefill_bytes(cw.B, cw.H, cw.Hkv, cw.Nq, cw.Nk, cw.d),
            "ms": round(mean(ms["window"]), 4), "ms_min": round(min(ms["window"]), 4),
            "value": round(w_tf, 2), "unit": "TFLOP/s",
            "frac_peak": round(w_tf / PEAK_BF16_TFLOPS, 4)}
    if "packed" in ms:
        pk_tf = rate(pk_flops, mean(ms["packed"])) / 1e12
        out["packed_prefill"] = {
            "workload": f"packed causal GQA prefill: {len(pk_lens)} documents (log-uniform "
                        f"{cpk.min_len}..{cpk.max_len}) in {cpk.contexts} x {cpk.context_len} "
                        f"tokens, H{cpk.H} Hkv{cpk.Hkv} d{cpk.d} bf16",
            "documents": len(pk_lens), "tokens": pk_total, "algorithmic_flops": pk_flops,
            "ms": round(mean(ms["packed"]), 4), "ms_min": round(min(ms["packed"]), 4),
            "value": round(pk_tf, 2), "unit": "TFLOP/s",
            "frac_peak": round(pk_tf / PEAK_BF16_TFLOPS, 4)}
    if "kvlens" in ms:
        kv_gbs = rate(kvl_bytes, mean(ms["kvlens"])) / 1e9
        out["decode_kvlens"] = {
            "workload": f"split-K decode B{ck.B} H{ck.H} Hkv{ck.Hkv} d{ck.d}, cache slots of "
                        f"{ck.Nk} keys holding uniform random lengths in [1, {ck.Nk}] "
                        f"(total {int(kv_lens.sum())} keys), {ck.splits} splits",
            "algorithmic_bytes": kvl_bytes,
            "ms": round(mean(ms["kvlens"]), 4), "ms_min": round(min(ms["kvlens"]), 4),
            "value": round(kv_gbs, 1), "unit": "GB/s", "frac_hbm": round(kv_gbs / PEAK_HBM_GBS, 4)}
    if "kvlens_skewed" in ms:
        sk_gbs = rate(sk_bytes, mean(ms["kvlens_skewed"])) / 1e9
        out["decode_kvlens_skewed"] = {
            "workload": f"split-K decode B{ck.B} H{ck.H} Hkv{ck.Hkv} d{ck.d} over the same cache "
                        f"slots, every eighth sequence at {ck.Nk} keys and the rest at 512 "
                        f"(total {int(sk_lens.sum())} keys), {ck.splits} splits",
            "algorithmic_bytes": sk_bytes,
            "ms": round(mean(ms["kvlens_skewed"]), 4),
            "ms_min": round(min(ms["kvlens_skewed"]), 4),
            "value": round(sk_gbs, 1), "unit": "GB/s", "frac_hbm": round(sk_gbs / PEAK_HBM_GBS, 4)}
    if "paged" in ms:
        pg_gbs = rate(pg_bytes, mean(ms["paged"])) / 1e9
        out["decode_paged"] = {
            "workload": f"the mixed-length decode with its keys in {page_size}-key pages "
                        f"scattered over one pool of {num_pages} pages",
            "algorithmic_bytes": pg_bytes,
            "ms": round(mean(ms["paged"]), 4), "ms_min": round(min(ms["paged"]), 4),
            "value": round(pg_gbs, 1), "unit": "GB/s", "frac_hbm": round(pg_gbs / PEAK_HBM_GBS, 4)}
    if "fp8" in ms:
        f8_tf = rate(pre_flops, mean(ms["fp8"])) / 1e12
        out["fp8_prefill"] = {
            "workload": "the headline prefill (B1 H32 Hkv8 N8192 d128 causal, sharpened) with Q "
                        "and K in fp8 e4m3 (one descale per tensor), V bf16",
            "algorithmic_flops": pre_flops,
            "ms": round(mean(ms["fp8"]), 4), "ms_min": round(min(ms["fp8"]), 4),
            "value": round(f8_tf, 2), "unit": "TFLOP/s",
            "frac_peak_bf16": round(f8_tf / PEAK_BF16_TFLOPS, 4),
            "note": "Q K^T runs on the fp8 matrix cores (5.0 PFLOP/s dense), P V on bf16 "
                    "(2.5 PFLOP/s); half the FLOPs at each rate gives a 3.33 PFLOP/s ceiling"}
    if "packed_backward" in ms:
        pb_tf = rate(2.5 * pk_flops, mean(ms["packed_backward"])) / 1e12
        out["packed_backward"] = {
            "workload": "backward of the packed prefill (24 documents in 4 x 8192 tokens, "
                        "H32 Hkv8 d128 causal), seeded N(0,1) dO",
            "algorithmic_flops": int(2.5 * pk_flops),
            "ms": round(mean(ms["packed_backward"]), 4),
            "ms_min": round(min(ms["packed_backward"]), 4),
            "value": round(pb_tf, 2), "unit": "TFLOP/s",
            "frac_peak": round(pb_tf / PEAK_BF16_TFLOPS, 4)}
    if "backward" in ms:
        bw_tf = rate(bwd_flops, mean(ms["backward"])) / 1e12
        out["backward"] = {
            "workload": "backward of the causal GQA prefill (B1 H32 Hkv8 N8192 d128, sharpened), "
                        "seeded N(0,1) dO, O and LSE from the forward",
            "algorithmic_flops": bwd_flops,
            "executed_flops": accounting.backward_executed_flops(cp.B, cp.H, cp.Nq, cp.Nk, cp.d,
                                                                 cp.causal, cp.window),
            "ms": round(mean(ms["backward"]), 4), "ms_min": round(min(ms["backward"]), 4),
            "value": round(bw_tf, 2), "unit": "TFLOP/s",
            "frac_peak": round(bw_tf / PEAK_BF16_TFLOPS, 4)}
    if ceilings:
        out["roofline"]["frac_of_measured_ceiling"] = round(
            pre_tflops / ceilings["mfma_bf16_tflops"], 4)
        out["roofline_decode"]["frac_of_measured_ceiling"] = round(
            dec_gbs / ceilings["hbm_read_gbs"], 4)
    if not args.no_cpu_baseline:
        nh = max(1, min(args.cpu_heads, cp.H))
        nkv = max(1, nh * cp.Hkv // cp.H)
        host = [t.cpu() for t in (q[:, :nh], k[:, :nkv], v[:, :nkv])]
        ns = max(1, min(args.cpu_seqs, cd.B))
        host_d = [t.cpu() for t in (qd[:ns], kc[:ns], vc[:ns])]
    del kc, vc
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        cb = cpu_baseline_prefill(cp, nh, *host)
        out["cpu_baseline"] = {kk: (round(vv, 6) if isinstance(vv, float) else vv)
                               for kk, vv in cb.items() if kk != "seconds"}
        cbd = cpu_baseline_decode(cd, ns, *host_d)
        out["cpu_baseline_decode"] = {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                                      for kk, vv in cbd.items() if kk != "seconds"}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
