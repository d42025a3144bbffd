"""Throughput benchmark of the fused attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--sweep] [--decode] [--masked] [--rows] [--fp8]

A step is one pass of the whole path over one batch of resident synthetic input:
the forward kernel (O and LSE) followed by the backward (D preprocess, dK/dV
kernel, dQ kernel).  Default workload: bf16, B=4, H=16 (B*H = 64), N = 8192,
d = 128, non-causal.  Prints ONE JSON line.

FLOP accounting: forward 4*B*H*N^2*d (two N^2*d matmuls), backward 2.5x that
(five: the S recompute, dV, dP, dK, dQ), both halved for a causal mask.  The dQ
kernel's extra recompute of S and dP is real work that is not counted.

Timing: HIP events recorded on the stream the kernels run on (torch's current
stream, which the binding passes to the library), around each pass of each of the
K timed steps, after W untimed warm-up steps.  Between steps, outside the events, a
512 MiB buffer is overwritten (a fill kernel) so that no step starts with the
previous one's data in L2 or the 256 MB MALL (--no-flush turns this off).  The
backward is enqueued as its three kernels (attn_bwd_preprocess, attn_bwd_dkdv,
attn_bwd_dq: exactly what attn_bwd launches) so that an event sits between every
two launches.  ``value`` and ``ms_per_step`` use the median step time (mean, min and
p90 are reported beside it).  ``kernels`` gives each launch's mean/median/min/p90
time and its roofline: achieved = the algorithmic FLOP (or bytes, for the HBM-bound
preprocess) per launch / mean launch time (the figure a rocprofv3 kernel trace's
average duration reproduces), against the dense bf16/fp16 MFMA peak of 2516.6
TFLOP/s (256 CUs x 4096 flop/clk x 2.4 GHz) or HBM's 8 TB/s, and, for the MFMA
kernels, against the same peak at the core clock measured during the timed steps
(``sclk``: the current level of amdgpu's pp_dpm_sclk, read every 5 ms from the start
of the warm-up; that level lags the load, so only samples from the timed steps taken
at least 0.3 s after the warm-up began give the clock, and a shorter run gives no
clock-referenced fraction).  ``roofline`` repeats the entry of the kernel
with the largest share of the step.  ``traffic`` is the HBM bytes per launch from
committed rocprofv3 counter runs, or null once the kernel source has changed since
they were taken.  ``cpu_baseline`` times the fp64 oracle on the host for a bounded
sample (16 heads of the headline workload; fewer at longer N).
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp32": 157.3, "fp8": 5033.2}
METRIC = "attention fwd/bwd TFLOP/s + % of bf16 MFMA peak, B*H=64 N=8192 d=128"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "online_softmax_attn_amd", "csrc")
FWD_SOURCES = [os.path.join(CSRC, f) for f in ("fwd_mfma.hip", "common.h")]
BWD_SOURCES = [os.path.join(CSRC, f) for f in ("bwd_mfma.hip", "common.h")]
F32_SOURCES = [os.path.join(CSRC, "f32_kernels.hip")]
ROW_SOURCES = [os.path.join(CSRC, f) for f in ("rowsoftmax.hip", "common.h")]


def kernel_source_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def traffic_of(traffic, kt, workload_name: str):
    """HBM bytes per launch of one kernel from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs, scaled by the copy-kernel calibration; None unless the counters
    were taken on the kernel's current source."""
    ent = traffic.get("kernels", {}).get(kt["name"], {})
    if ent.get("source_sha") != kernel_source_sha(kt["sources"]):
        return None
    return ent.get("workloads", {}).get(workload_name, {}).get("hbm_bytes_per_launch")


COPY_BYTES = 512 * 1024 * 1024
COPY_KERNEL = "copyBuffer"  # the runtime's device-to-device copy kernel


def _counter_means(folder: str, counter: str):
    """Mean per-dispatch value of one counter, per kernel name, from a rocprofv3
    --pmc output folder (run_counter_collection.csv)."""
    import csv
    import glob
    sums, counts = {}, {}
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                sums[name] = sums.get(name, 0.0) + float(r["Counter_Value"])
                counts[name] = counts.get(name, 0) + 1
    return {n: sums[n] / counts[n] for n in sums}


def _pick(means, short):
    keys = short if isinstance(short, (list, tuple)) else [short]
    hits = [v for n, v in means.items() if any(k in n for k in keys)]
    if not hits:
        raise SystemExit(f"no dispatch of {short} in the counter output")
    return sum(hits) / len(hits)


# How a kernel's element type shows in a rocprofv3 name (mangled or demangled).
_TYPE_TOKENS = {"bf16": ("IDF16b", "<__bf16"), "fp16": ("IDF16_", "<_Float16"),
                "fp32": ("If", "<float")}


def row_kernel_table(w):
    """The forward and backward launch of a row workload, with the substrings that
    pick their dispatches out of a counter run (kernel template and element type)."""
    fb, bb = row_bytes(w)
    if w.op == "xent":
        bases = (("xent_fwd_kernel",), ("xent_bwd_flat", "xent_bwd_kernel"))
    else:
        bases = (("rs_fwd_reg", "rs_fwd_stream"), ("rs_bwd_reg", "rs_bwd_stream"))
    out = []
    for base, nbytes in zip(bases, (fb, bb)):
        out.append({"name": f"{'/'.join(base)}<{w.dtype}>", "bytes": nbytes, "sources": ROW_SOURCES,
                    "match": [b + t for b in base for t in _TYPE_TOKENS[w.dtype]]})
    return out


def write_traffic(folders, workload_name, rows: bool = False):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each kernel of the step by
    what the same counters read for a plain copy of COPY_BYTES, and record the
    result with the sha of each kernel's source.  rows: the counter runs are of
    `bench.py --rows` and every row workload is recorded."""
    import synthetic as S
    if rows:
        tables = [(w, row_kernel_table(w)) for w in S.ROWS.values()]
    else:
        w = S.WORKLOADS[workload_name] if workload_name else S.HEADLINE
        tables = [(w, kernel_table(w))]
    fetch, write, cfetch, cwrite = folders
    fm, wm = _counter_means(fetch, "FETCH_SIZE"), _counter_means(write, "WRITE_SIZE")
    cf = _pick(_counter_means(cfetch, "FETCH_SIZE"), COPY_KERNEL)
    cw = _pick(_counter_means(cwrite, "WRITE_SIZE"), COPY_KERNEL)
    fetch_scale, write_scale = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    old = load_traffic()
    out = {"note": "HBM bytes per launch = FETCH_SIZE*1024*fetch_scale + WRITE_SIZE*1024*write_scale; "
                   "the scales make a plain device copy of known size read and write its own size",
           "copy_calibration": {"bytes_read_and_written": COPY_BYTES, "FETCH_SIZE_KiB": cf,
                                "WRITE_SIZE_KiB": cw, "fetch_scale": round(fetch_scale, 5),
                                "write_scale": round(write_scale, 5)},
           "kernels": old.get("kernels", {})}
    for w, kt in ((w, kt) for w, table in tables for kt in table):
        key = kt.get("match", kt["name"])
        f_kib, w_kib = _pick(fm, key), _pick(wm, key)
        hbm = f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale
        ent = out["kernels"].get(kt["name"], {})
        sha = kernel_source_sha(kt["sources"])
        if ent.get("source_sha") != sha:
            ent = {"source_sha": sha, "source_files": [os.path.relpath(p, ROOT) for p in kt["sources"]],
                   "workloads": {}}
        ent["workloads"][w.name] = {"FETCH_SIZE_KiB_per_dispatch": round(f_kib, 1),
                                    "WRITE_SIZE_KiB_per_dispatch": round(w_kib, 1),
                                    "hbm_bytes_per_launch": int(hbm),
                                    "algorithmic_bytes_per_launch": kt["bytes"],
                                    "ratio_to_algorithmic": round(hbm / kt["bytes"], 4)}
        out["kernels"][kt["name"]] = ent
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def blas_threads() -> int:
    """Threads the oracle's matrix products run on (BLAS pool), else the affinity size."""
    try:
        from threadpoolctl import threadpool_info
        return int(max((i.get("num_threads", 1) for i in threadpool_info()
                        if i.get("user_api") == "blas"), default=1))
    except Exception:
        return len(os.sched_getaffinity(0))


def baseline_groups(w, heads: int = 0):
    """The (batch, kv head) groups of the oracle sample: `heads` query heads, by default
    16 at N = 8192 scaled by (8192 / N)^2 so that the sample stays near 10-15 s of oracle
    time; whole KV groups of batch 0, at least one, at most all of them."""
    n_rep = w.H // w.Hkv
    if heads <= 0:
        heads = max(1, min(16, int(16 * (8192 / w.N) ** 2)))
    return [(0, g) for g in range(min(w.Hkv, max(1, heads // n_rep)))]


def cpu_baseline(w, inp, gpu_out, heads: int = 0):
    """Time the fp64 oracle (fwd + bwd) on the query heads of baseline_groups."""
    import numpy as np

    import oracle.attention as A
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:  # threadpoolctl missing: report the affinity size
        threads = len(os.sched_getaffinity(0))
    n_rep = w.H // w.Hkv
    groups = baseline_groups(w, heads)
    n_heads = len(groups) * n_rep
    t0 = time.perf_counter()
    ref = A.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.causal,
                               heads=groups)
    dt = time.perf_counter() - t0
    flop = (w.fwd_flop() + w.bwd_flop()) / (w.B * w.H) * n_heads
    # Same sample from the GPU run, as a sanity figure for the record.
    o, dq = gpu_out
    hs = slice(0, n_heads)
    err_o = float(np.max(np.abs(o[0, hs].float().cpu().double().numpy() - ref["o"][0, hs])))
    dq_ref = ref["dq"][0, hs]
    err_dq = float(np.max(np.abs(dq[0, hs].float().cpu().double().numpy() - dq_ref))
                   / np.max(np.abs(dq_ref)))
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle fwd+bwd on {n_heads} of {w.B * w.H} heads (b=0, kv groups "
                      f"{[g for _, g in groups]}), {dt:.2f} s; dense S/P, FLOP counted as for the GPU",
            "seconds": dt, "gpu_vs_oracle_on_sample": {"o_max_abs": err_o, "dq_rel": err_dq}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not overwrite a 512 MiB buffer between timed steps")
    ap.add_argument("--sweep", action="store_true",
                    help="time every point of the bf16 sweep (one JSON line each)")
    ap.add_argument("--decode", action="store_true",
                    help="time the split-KV forward on the decoding workloads (one line each)")
    ap.add_argument("--masked", action="store_true",
                    help="time the interval-masked fwd+bwd on the masked workloads (one line each)")
    ap.add_argument("--fp8", action="store_true",
                    help="time the fp8 (e4m3) forward on the B4 H16 N8192 shape, d = 128 and 64, "
                         "non-causal and causal (one line each)")
    ap.add_argument("--rows", action="store_true",
                    help="time row softmax / log-softmax / cross-entropy fwd+bwd on the row "
                         "workloads (one line each)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run three plain 512 MiB device copies (for scaling HBM counters)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="no GPU: turn four rocprofv3 --pmc output folders into "
                         "profiles/hbm_traffic.json")
    args = ap.parse_args()

    if args.traffic_from:
        write_traffic(args.traffic_from, args.workload, rows=args.rows)
        return

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (--gpus {args.gpus} requested); the path would "
              "shard over (batch, kv-head group) pairs with no communication", file=sys.stderr)
        sys.exit(2)

    import torch

    import online_softmax_attn_amd as osa
    import synthetic as S

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    osa.library()

    if args.copy_calibration:
        a = torch.randn(COPY_BYTES // 4, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES}))
        return

    if args.sweep:
        for w in S.sweep_points():
            print(json.dumps(run_one(w, args, osa, torch, with_cpu=False)), flush=True)
        return
    if args.decode:
        for w in S.DECODE.values():
            print(json.dumps(run_decode(w, args, osa, torch, with_cpu=not args.no_cpu_baseline)),
                  flush=True)
        return
    if args.masked:
        for name, (w, kind, mk) in S.MASKED.items():
            print(json.dumps(run_masked(name, w, kind, mk, args, osa, torch,
                                        with_cpu=not args.no_cpu_baseline)), flush=True)
        return
    if args.fp8:
        for d in (128, 64):
            for causal in (False, True):
                w = S.custom("bf16", 4, 16, 16, 8192, d, causal, seed_base=34000)
                print(json.dumps(run_fp8(w, args, osa, torch, with_cpu=not args.no_cpu_baseline)),
                      flush=True)
        return
    if args.rows:
        for w in S.ROWS.values():
            print(json.dumps(run_rows(w, args, osa, torch, with_cpu=not args.no_cpu_baseline)),
                  flush=True)
        return
    w = S.WORKLOADS[args.workload] if args.workload else S.HEADLINE
    print(json.dumps(run_one(w, args, osa, torch, with_cpu=not args.no_cpu_baseline)), flush=True)


def kernel_table(w):
    """The four launches of one step, in order, with the algorithmic work each one
    is charged: FLOP for the MFMA kernels (the counted matmuls of the method), bytes
    for the HBM-bound preprocess."""
    e = {"bf16": 2, "fp16": 2, "fp32": 4}[w.dtype]
    qb = w.B * w.H * w.N * w.d * e      # one of Q, O, dO, dQ
    kb = w.B * w.Hkv * w.N * w.d * e    # one of K, V, dK, dV
    rb = w.B * w.H * w.N * 4            # one float32 per query row
    f32 = w.dtype == "fp32"
    fsrc = F32_SOURCES if f32 else FWD_SOURCES
    bsrc = F32_SOURCES if f32 else BWD_SOURCES
    rows = w.B * w.H * w.N
    fwd_f, bwd_f = w.fwd_flop(), w.bwd_flop()
    return [
        # S = Q K^T and O = P V.
        {"name": "fwd_mfma_kernel" if w.dtype != "fp32" else "fwd_f32_kernel", "bound": "mfma",
         "work": fwd_f, "unit": "flop", "sources": fsrc, "bytes": 2 * qb + 2 * kb + rb},
        # Reads O and dO (d elements each) and LSE; writes D and LSE*log2(e).
        {"name": "bwd_preprocess_kernel", "bound": "hbm", "work": rows * (2 * w.d * e + 3 * 4),
         "unit": "byte", "sources": BWD_SOURCES, "bytes": 2 * qb + 3 * rb},
        # S recompute, dV = P^T dO, dP = dO V^T, dK = dS^T Q: four of the five matmuls.
        {"name": "bwd_dkdv_kernel" if w.dtype != "fp32" else "bwd_dkdv_f32_kernel",
         "bound": "mfma", "work": 0.8 * bwd_f, "unit": "flop", "sources": bsrc,
         "bytes": 2 * qb + 4 * kb + 2 * rb},
        # dQ = dS K (counted); the kernel also recomputes S and dP (executed, not counted).
        {"name": "bwd_dq_kernel" if w.dtype != "fp32" else "bwd_dq_f32_kernel", "bound": "mfma",
         "work": 0.2 * bwd_f, "unit": "flop", "sources": bsrc, "executed_work": 0.6 * bwd_f,
         "bytes": 3 * qb + 2 * kb + 2 * rb},
    ]


def run_decode(w, args, osa, torch, with_cpu: bool = False):
    """One split-KV forward (chunk kernel + merge kernel) per step on a decoding
    workload; HBM-bound, so the roofline is bytes: K and V read once, plus Q read and
    O and LSE written (the fp32 chunk results in the workspace are overhead)."""
    import synthetic as S

    inp = S.make_inputs(w, with_grad=False)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), device="cuda", dtype=torch.float32)
    need = osa.attn_fwd_splitkv_workspace_bytes(w.B, w.H, w.Hkv, w.N, w.nk, w.d, w.causal, q.dtype)
    ws = torch.empty(need, device="cuda", dtype=torch.uint8)

    def step():
        osa.attn_fwd_splitkv(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    st = stats([e[0].elapsed_time(e[1]) for e in ev])
    e = q.element_size()
    algo = w.kv_bytes() + 2 * q.numel() * e + lse.numel() * 4
    gbs = algo / (st["mean"] * 1e-3) / 1e9
    line = {"metric": "split-KV decode forward: compulsory HBM bytes per second",
            "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(st["mean"], 4), "higher_is_better": True,
            "dtype": w.dtype, "data": "synthetic", "config": w.describe(),
            "tflops": round(w.fwd_flop() / (st["mean"] * 1e-3) / 1e12, 2),
            "workspace_bytes": need,
            "roofline": {"bound": "hbm", "kernel": "splitkv_partial_kernel + splitkv_merge_kernel",
                         "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": algo,
                         "ms": {k2: round(x, 4) for k2, x in st.items()}}}
    if with_cpu:
        line["cpu_baseline"] = decode_cpu_baseline(w, inp, o, algo)
    return line


def decode_cpu_baseline(w, inp, o_gpu, algo_bytes: int, budget_s: float = 10.0):
    """Time the fp64 oracle forward over the batch entries in order (all heads of each)
    until every entry is done or budget_s seconds have been spent; the rate is the
    compulsory bytes of the entries done over that time, as for the GPU."""
    import numpy as np

    import oracle.attention as A
    done, dt, err = 0, 0.0, 0.0
    while done < w.B and dt < budget_s:
        b = slice(done, done + 1)
        t0 = time.perf_counter()
        ref_o, _ = A.attention_forward(inp["q"][b], inp["k"][b], inp["v"][b], w.scale, w.causal)
        dt += time.perf_counter() - t0
        err = max(err, float(np.max(np.abs(o_gpu[b].float().cpu().double().numpy() - ref_o))))
        done += 1
    return {"value": round(algo_bytes * done / w.B / dt / 1e9, 3), "unit": "GB/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"fp64 oracle forward on batch entries 0-{done - 1} of {w.B} (all {w.H} "
                      f"query heads each), {dt:.2f} s; bytes counted as for the GPU",
            "seconds": round(dt, 3), "gpu_vs_oracle_o_max_abs": err}


def run_masked(name, w, kind, mk, args, osa, torch, with_cpu: bool = False):
    """Interval-masked forward + backward; FLOP counted on the visible (query, key)
    pairs only: 4*d per pair and head forward, 2.5x that backward."""
    import synthetic as S

    inp = S.make_inputs(w, with_grad=True)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    lo, hi = S.mask_intervals(kind, w.B, w.N, w.nk, **mk)
    pairs = S.visible_pairs(lo, hi, w.nk)
    lo, hi = lo.cuda(), hi.cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), device="cuda", dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(osa.attn_bwd_masked_workspace_bytes(w.B, w.H, w.Hkv, w.N, w.nk, w.d, q.dtype),
                     device="cuda", dtype=torch.uint8)
    fwd = lambda: osa.attn_fwd_masked(q, k, v, lo, hi, scale=w.scale, out=o, lse=lse)
    bwd = lambda: osa.attn_bwd_masked(q, k, v, o, lse, do, lo, hi, scale=w.scale, dq=dq, dk=dk,
                                      dv=dv, workspace=ws)
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    f_ms = stats([e[0].elapsed_time(e[1]) for e in ev])["mean"]
    b_ms = stats([e[1].elapsed_time(e[2]) for e in ev])["mean"]
    ff = 4.0 * w.H * w.d * pairs
    bf = 2.5 * ff
    peak = PEAK_TFLOPS[w.dtype]
    val = (ff + bf) / ((f_ms + b_ms) * 1e-3) / 1e12
    dense = 4.0 * w.B * w.H * w.N * w.nk * w.d
    line = {"metric": "interval-masked attention fwd+bwd TFLOP/s on visible pairs",
            "value": round(val, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(f_ms + b_ms, 4), "higher_is_better": True,
            "dtype": w.dtype, "data": "synthetic",
            "config": dict(w.describe(), workload=name, mask=kind,
                           mask_params={k2: (v2 if k2 != "doc_lens" else "per batch")
                                        for k2, v2 in mk.items()}),
            "visible_fraction": round(pairs * w.H / (dense / (4.0 * w.d)), 4),
            "fwd": {"ms": round(f_ms, 4), "tflops": round(ff / (f_ms * 1e-3) / 1e12, 2),
                    "frac_peak": round(ff / (f_ms * 1e-3) / 1e12 / peak, 4)},
            "bwd": {"ms": round(b_ms, 4), "tflops": round(bf / (b_ms * 1e-3) / 1e12, 2),
                    "frac_peak": round(bf / (b_ms * 1e-3) / 1e12 / peak, 4)}}
    if with_cpu:
        line["cpu_baseline"] = masked_cpu_baseline(w, inp, lo.cpu(), hi.cpu(), o, dq)
    return line


def masked_cpu_baseline(w, inp, lo, hi, o_gpu, dq_gpu, budget_s: float = 10.0):
    """Time the fp64 oracle forward + backward under the same intervals, one KV group of
    batch 0 at a time, until every group is done or budget_s seconds have been spent;
    FLOP counted on the visible pairs of batch 0, as for the GPU."""
    import numpy as np

    import oracle.attention as A
    import synthetic as S
    n_rep = w.H // w.Hkv
    lo_n, hi_n = lo.numpy(), hi.numpy()
    done, dt, err_o, err_dq = 0, 0.0, 0.0, 0.0
    while done < w.Hkv and dt < budget_s:
        t0 = time.perf_counter()
        ref = A.attention_backward_intervals(inp["q"], inp["k"], inp["v"], inp["do"], w.scale,
                                             lo_n, hi_n, heads=[(0, done)])
        dt += time.perf_counter() - t0
        hs = slice(done * n_rep, (done + 1) * n_rep)
        err_o = max(err_o, float(np.max(np.abs(o_gpu[0, hs].float().cpu().double().numpy()
                                               - ref["o"][0, hs]))))
        dq_ref = ref["dq"][0, hs]
        err_dq = max(err_dq, float(np.max(np.abs(dq_gpu[0, hs].float().cpu().double().numpy() - dq_ref))
                                   / max(float(np.max(np.abs(dq_ref))), 1e-300)))
        done += 1
    n_heads = done * n_rep
    flop = 14.0 * w.d * S.visible_pairs(lo[:1], hi[:1], w.nk) * n_heads
    return {"value": round(flop / dt / 1e12, 5), "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"fp64 oracle fwd+bwd on {n_heads} of {w.B * w.H} heads (b=0, kv groups "
                      f"0-{done - 1}), {dt:.2f} s; dense S/P under the mask, FLOP counted on "
                      f"visible pairs as for the GPU",
            "seconds": round(dt, 3), "gpu_vs_oracle_on_sample": {"o_max_abs": err_o, "dq_rel": err_dq}}


def run_fp8(w, args, osa, torch, with_cpu: bool):
    """One attn_fwd_fp8 call per step (the V transpose pass and the forward kernel);
    FLOP 4 * N^2 * d per head (halved when causal), against the dense fp8 peak."""
    import synthetic as S

    inp = S.make_fp8_inputs(w)
    q8, k8, v8 = (inp[n].cuda() for n in ("q8", "k8", "v8"))
    ws = torch.empty(osa.attn_fwd_fp8_workspace_bytes(w.B, w.Hkv, w.N, w.d), device="cuda",
                     dtype=torch.uint8)
    o = torch.empty(q8.shape, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((w.B, w.H, w.N), device="cuda", dtype=torch.float32)
    fwd = lambda: osa.attn_fwd_fp8(q8, k8, v8, inp["dq"], inp["dk"], inp["dv"], causal=w.causal,
                                   scale=w.scale, out=o, lse=lse, workspace=ws)
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    st = stats([e[0].elapsed_time(e[1]) for e in ev])
    flop = w.fwd_flop()
    tf = flop / (st["mean"] * 1e-3) / 1e12
    line = {"metric": "fp8 (e4m3) attention forward TFLOP/s", "value": round(tf, 2),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(st["mean"], 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8-e4m3 (fp32 accumulate, bf16 out)",
            "data": "synthetic", "config": dict(w.describe(), dtype="fp8_e4m3",
                                                workload=f"fp8_e4m3_B4_H16_N8192_d{w.d}"
                                                + ("_causal" if w.causal else "")),
            "roofline": {"bound": "mfma", "kernel": "vt_kernel + fwd_fp8_kernel (one call)",
                         "achieved": round(tf, 2), "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_TFLOPS["fp8"], 4), "flop_per_launch": flop,
                         "traffic": None, "ms": {k: round(x, 4) for k, x in st.items()}}}
    if with_cpu:
        import numpy as np

        import oracle.fp8 as F8
        t0 = time.perf_counter()
        sub = {n: inp[n][:1, :1].numpy() for n in ("q8", "k8", "v8")}
        ref_o, _ = F8.attention_forward_fp8(sub["q8"], sub["k8"], sub["v8"], inp["dq"], inp["dk"],
                                            inp["dv"], w.scale, w.causal)
        dt = time.perf_counter() - t0
        err = float(np.max(np.abs(o[0, 0].float().cpu().double().numpy() - ref_o[0, 0])))
        line["cpu_baseline"] = {"value": round(flop / (w.B * w.H) / dt / 1e12, 5), "unit": "TFLOP/s",
                                "cores": blas_threads(), "kind": "oracle",
                                "sample": f"fp64 oracle forward (decoded fp8 inputs) on head (0,0) of "
                                          f"{w.B * w.H}, {dt:.2f} s",
                                "seconds": round(dt, 3), "gpu_vs_oracle_o_max_abs": err}
    return line


def row_bytes(w):
    """Compulsory HBM bytes of the forward and the backward launch of a row workload:
    every element read or written once (fp32 loss / lse / dloss, int32 targets)."""
    el = w.rows * w.cols * w.elem_bytes()
    if w.op == "xent":
        return el + w.rows * (4 + 8), 2 * el + w.rows * 12
    return 2 * el, 3 * el


def row_cpu_baseline(w, inp, budget_s: float = 10.0):
    """Time the fp64 oracle's forward + backward over the rows in order, in chunks of
    about 4e7 elements, until every row is done or budget_s seconds of oracle time
    have been spent (the conversion of each chunk to fp64 is not timed)."""
    import numpy as np

    import oracle.rowsoftmax as R
    chunk = max(1, int(4e7 // w.cols))
    done, dt = 0, 0.0
    while done < w.rows and dt < budget_s:
        n = min(chunk, w.rows - done)
        x = inp["x"][done:done + n].double().numpy()
        if w.op == "xent":
            t = inp["targets"][done:done + n].numpy().astype(np.int64)
            dl = inp["dloss"][done:done + n].numpy()
            t0 = time.perf_counter()
            R.cross_entropy(x, t)
            R.cross_entropy_backward(x, t, dl)
        else:
            log = w.op == "log_softmax"
            dy = inp["dy"][done:done + n].double().numpy()
            t0 = time.perf_counter()
            y = R.log_softmax(x) if log else R.softmax(x)
            (R.log_softmax_backward if log else R.softmax_backward)(y, dy)
        dt += time.perf_counter() - t0
        done += n
    fb, bb = row_bytes(w)
    frac = done / w.rows
    return {"value": round((fb + bb) * frac / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"fp64 oracle fwd+bwd on rows 0-{done - 1} of {w.rows} (chunks of {chunk} "
                      f"rows), {dt:.2f} s; bytes counted as for the GPU (dtype-sized elements)",
            "seconds": round(dt, 3)}


def run_rows(w, args, osa, torch, with_cpu: bool):
    """One forward and one backward launch per step on a row workload; both are
    HBM-bound, so the roofline is compulsory bytes over time."""
    import synthetic as S

    inp = S.row_inputs(w)
    x = inp["x"].cuda()
    if w.op == "xent":
        t, dloss = inp["targets"].cuda(), inp["dloss"].cuda()
        loss = torch.empty(w.rows, device="cuda", dtype=torch.float32)
        lse = torch.empty_like(loss)
        dx = torch.empty_like(x)
        fwd = lambda: osa.rowxent_fwd(x, t, loss=loss, lse=lse)
        bwd = lambda: osa.rowxent_bwd(x, t, lse, dloss, out=dx)
        names = ("xent_fwd_kernel", "xent_bwd_flat / xent_bwd_kernel")
    else:
        log = w.op == "log_softmax"
        dy = inp["dy"].cuda()
        y, dx = torch.empty_like(x), torch.empty_like(x)
        fwd = lambda: osa.rowsoftmax_fwd(x, log_softmax=log, out=y)
        bwd = lambda: osa.rowsoftmax_bwd(y, dy, log_softmax=log, out=dx)
        names = ("rs_fwd_reg / rs_fwd_stream", "rs_bwd_reg / rs_bwd_stream")
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps * 1e3
    f_ms = stats([e[0].elapsed_time(e[1]) for e in ev])["mean"]
    b_ms = stats([e[1].elapsed_time(e[2]) for e in ev])["mean"]
    fb, bb = row_bytes(w)
    gbs = (fb + bb) / ((f_ms + b_ms) * 1e-3) / 1e9
    f_gbs, b_gbs = fb / (f_ms * 1e-3) / 1e9, bb / (b_ms * 1e-3) / 1e9
    kt_f, kt_b = row_kernel_table(w)
    dom = ((names[0], f_gbs, fb, f_ms, kt_f) if f_ms >= b_ms else
           (names[1], b_gbs, bb, b_ms, kt_b))
    line = {"metric": f"row {w.op} fwd+bwd: compulsory HBM bytes per second",
            "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(f_ms + b_ms, 4),
            "wall_ms_per_step": round(wall, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": w.dtype, "data": "synthetic", "config": w.describe(),
            "fwd": {"kernel": names[0], "ms": round(f_ms, 4), "bytes": fb, "gbs": round(f_gbs, 1),
                    "frac": round(f_gbs / HBM_PEAK_GBS, 4)},
            "bwd": {"kernel": names[1], "ms": round(b_ms, 4), "bytes": bb, "gbs": round(b_gbs, 1),
                    "frac": round(b_gbs / HBM_PEAK_GBS, 4)},
            "roofline": {"bound": "hbm", "kernel": dom[0], "achieved": round(dom[1], 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dom[1] / HBM_PEAK_GBS, 4), "bytes_per_launch": dom[2],
                         "ms": round(dom[3], 4), "traffic": traffic_of(load_traffic(), dom[4],
                                                                       w.name)}}
    if with_cpu:
        line["cpu_baseline"] = row_cpu_baseline(w, inp)
    return line


def stats(xs):
    ys = sorted(xs)
    n = len(ys)
    med = ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])
    return {"mean": sum(ys) / n, "median": med, "min": ys[0],
            "p90": ys[min(n - 1, int(math.ceil(0.9 * n)) - 1)]}


def sclk_path():
    """The sysfs file that reports the GPU core clock levels with the current one
    starred (amdgpu's pp_dpm_sclk), if exactly one GPU exposes it."""
    import glob
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    return paths[0] if len(paths) == 1 else None


def read_sclk_mhz(path):
    """Current core clock in MHz from pp_dpm_sclk (the starred level), or None."""
    try:
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().rstrip("*").strip().lower()
                                 .replace("mhz", ""))
    except (OSError, ValueError, IndexError, TypeError):
        return None
    return None


SCLK_SETTLE_S = 0.3  # seconds of load before the sysfs clock level is taken as settled


class ClockSampler:
    """Reads the current core clock (every `period` seconds, from a thread) from the
    start of the warm-up to the end of the timed region.  The clock under load is what
    the matrix cores run at; the spec peak assumes 2.4 GHz.  The sysfs level lags the
    load: it climbs for a couple of hundred milliseconds after work starts while the
    kernels already run at full speed (the same kernel timed the same at readings of
    1200 and 2228 MHz), so only samples taken SCLK_SETTLE_S or more after the load
    began, and inside the timed region, count as the measured clock."""

    def __init__(self, period: float = 0.005, settle_s: float = SCLK_SETTLE_S):
        self.path = sclk_path()
        self.period = period
        self.settle_s = settle_s
        self.samples = []  # (seconds since start, MHz)
        self.before = self.after = None
        self.t_start = self.t_timed = None
        self._stop = None
        self._thread = None

    def start(self):
        """Call when the load begins (before the warm-up)."""
        import threading
        self.t_start = time.perf_counter()
        if not self.path:
            return
        self.before = read_sclk_mhz(self.path)
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                v = read_sclk_mhz(self.path)
                if v is not None:
                    self.samples.append((time.perf_counter() - self.t_start, v))
                self._stop.wait(self.period)
        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()

    def mark_timed(self):
        """Call where the timed region begins."""
        self.t_timed = time.perf_counter() - (self.t_start or time.perf_counter())

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        if self.path:
            self.after = read_sclk_mhz(self.path)

    def timed_samples(self):
        t0 = self.t_timed or 0.0
        return [v for t, v in self.samples if t >= t0]

    def settled_samples(self):
        t0 = max(self.t_timed or 0.0, self.settle_s)
        return [v for t, v in self.samples if t >= t0]

    def record(self):
        """{'source', 'before_mhz', 'after_mhz', 'during_mhz': all samples of the timed
        region, 'settled_mhz': those at least settle_s into the load (the clock used)}."""
        out = {"source": self.path or "unavailable", "before_mhz": self.before,
               "after_mhz": self.after, "during_mhz": None, "settled_mhz": None,
               "settle_s": self.settle_s}
        for key, vals in (("during_mhz", self.timed_samples()), ("settled_mhz", self.settled_samples())):
            if vals:
                st = stats(vals)
                out[key] = {"median": st["median"], "min": st["min"], "max": max(vals), "n": len(vals)}
        if out["settled_mhz"] is None and self.path:
            out["note"] = (f"timed region ended before {self.settle_s} s of load: the sysfs level "
                           "had not settled, so no clock-referenced fraction is given")
        return out

    def median_ghz(self):
        """Median settled clock in GHz, or None."""
        vals = self.settled_samples()
        return stats(vals)["median"] / 1000.0 if vals else None


def peak_at_clock(peak_spec: float, ghz):
    """The dense peak scaled from the spec clock (2.4 GHz) to a measured clock."""
    return peak_spec * ghz / 2.4 if ghz else None


FLUSH_BYTES = 512 << 20  # more than the 256 MB last-level cache (MALL) and every L2


class CacheFlush:
    """Overwrites a 512 MiB device buffer between timed steps, outside the timed
    region (a fill kernel on the current stream before the step's first event), so
    that no step starts with the previous step's data in L2 or the MALL."""

    def __init__(self, torch, enabled: bool = True):
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda") if enabled else None
        self.count = 0

    def __call__(self):
        if self.buf is not None:
            self.count += 1
            self.buf.fill_(self.count & 0xFF)


def run_one(w, args, osa, torch, with_cpu: bool):
    import synthetic as S

    inp = S.make_inputs(w, with_grad=True)
    dev = {k: v.cuda() for k, v in inp.items()}
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), device="cuda", dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = osa.new_bwd_workspace(q, k)
    kw = dict(causal=w.causal, scale=w.scale)

    # One step = the forward, then the backward's three kernels.  attn_bwd enqueues
    # exactly these three; calling them one by one lets an event sit between them.
    launches = [
        lambda: osa.attn_fwd(q, k, v, out=o, lse=lse, **kw),
        lambda: osa.attn_bwd_preprocess(q, k, o, lse, do, ws),
        lambda: osa.attn_bwd_dkdv(q, k, v, o, lse, do, ws, dk=dk, dv=dv, **kw),
        lambda: osa.attn_bwd_dq(q, k, v, o, lse, do, ws, dq=dq, **kw),
    ]

    # Between steps (outside the timed region) a 512 MiB buffer is overwritten so that
    # no step finds the previous step's data in L2 or the MALL.
    flush = CacheFlush(torch, enabled=not getattr(args, "no_flush", False))
    # Events on the stream the library launches on (the binding passes torch's
    # current stream to every call).
    stream = torch.cuda.current_stream()
    nl = len(launches)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    clock = ClockSampler()
    clock.start()
    for _ in range(args.warmup):
        flush()
        for f in launches:
            f()
    torch.cuda.synchronize()
    clock.mark_timed()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        ev[i][0].record(stream)
        for j, f in enumerate(launches):
            f()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock.stop()
    ghz = clock.median_ghz()

    step_ms = [ev[i][0].elapsed_time(ev[i][nl]) for i in range(args.steps)]
    per_ms = [[ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)] for j in range(nl)]
    peak = PEAK_TFLOPS[w.dtype]
    peak_clk = peak_at_clock(peak, ghz)
    step_st = stats(step_ms)
    ms_step = step_st["median"]
    fwd_f, bwd_f = w.fwd_flop(), w.bwd_flop()
    value = (fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12
    fwd_ms = stats(per_ms[0])
    bwd_ms = stats([sum(per_ms[j][i] for j in range(1, nl)) for i in range(args.steps)])
    fwd_tf = fwd_f / (fwd_ms["median"] * 1e-3) / 1e12
    bwd_tf = bwd_f / (bwd_ms["median"] * 1e-3) / 1e12
    traffic = load_traffic()

    kernels = []
    for kt, ms in zip(kernel_table(w), per_ms):
        st = stats(ms)
        secs = st["mean"] * 1e-3
        if kt["bound"] == "mfma":
            ach, pk, unit = kt["work"] / secs / 1e12, peak, "TFLOP/s"
        else:
            ach, pk, unit = kt["work"] / secs / 1e9, HBM_PEAK_GBS, "GB/s"
        ent = {"kernel": kt["name"], "bound": kt["bound"], "achieved": round(ach, 2), "peak": pk,
               "unit": unit, "frac": round(ach / pk, 4),
               "traffic": traffic_of(traffic, kt, w.name),
               ("flop_per_launch" if kt["unit"] == "flop" else "bytes_per_launch"): kt["work"],
               "ms": {k2: round(x, 4) for k2, x in st.items()}}
        if kt["bound"] == "mfma" and peak_clk:
            ent["frac_at_measured_sclk"] = round(ach / peak_clk, 4)
        if "executed_work" in kt:
            ent["executed_flop_per_launch"] = kt["executed_work"]
            ent["executed_tflops"] = round(kt["executed_work"] / secs / 1e12, 2)
        kernels.append(ent)
    dominant = max(kernels, key=lambda e: e["ms"]["mean"])

    props = torch.cuda.get_device_properties(0)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_stats": {k2: round(x, 4) for k2, x in step_st.items()},
        "value_basis": "median step time over the timed steps",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": dict(w.describe(), step="fwd+bwd", parallelism="single GPU"),
        "fwd": {"ms_mean": round(fwd_ms["mean"], 4), "ms_median": round(fwd_ms["median"], 4),
                "tflops": round(fwd_tf, 2), "frac_peak": round(fwd_tf / peak, 4),
                "frac_at_measured_sclk": round(fwd_tf / peak_clk, 4) if peak_clk else None},
        "bwd": {"ms_mean": round(bwd_ms["mean"], 4), "ms_median": round(bwd_ms["median"], 4),
                "tflops": round(bwd_tf, 2), "frac_peak": round(bwd_tf / peak, 4),
                "frac_at_measured_sclk": round(bwd_tf / peak_clk, 4) if peak_clk else None,
                "launches": nl - 1},
        "frac_peak_step": round(value / peak, 4),
        "frac_peak_step_at_measured_sclk": round(value / peak_clk, 4) if peak_clk else None,
        "sclk": dict(clock.record(), peak_at_median_tflops=round(peak_clk, 1) if peak_clk else None),
        "cache_flush_bytes_between_steps": FLUSH_BYTES if flush.buf is not None else 0,
        "roofline": {k2: dominant[k2] for k2 in dominant if k2 != "ms"},
        "kernels": kernels,
        "wall_s_timed": round(wall, 3),
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count},
        "torch": torch.__version__,
    }
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(w, inp, (o, dq))
    return out


if __name__ == "__main__":
    main()
