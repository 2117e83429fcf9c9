#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--configs 1,2,3,4] [--headline 4] [--gpus 1]

Workloads: the decode configurations of paged_kv_gqa_decode_amd.workloads.CONFIGS
that the 70 %-of-HBM target covers (1: Llama-3-8B shaped batch, 2: long-context
split, 3: multi-row causal, 4: ragged serving), seeded synthetic data generated
on the GPU; the headline is the ragged-serving batch (B=256, H=64, KV=8, D=128,
BLOCK=32, bf16, lognormal context lengths), the largest of them.

One step = one paged_attn_decode call (pass 1 and, for split plans, the
combine). Per workload: W untimed steps, then `--repeats` regions of K steps
back to back, each bracketed by torch.cuda.synchronize() and two HIP events on
the launch stream; the reported time per step is the median over the regions
(p10 / p90 beside it). Pools are rotated over `--replicas` copies so the
working set exceeds the 256 MB Infinity Cache. The dominant kernel (pass 1) is
then timed alone: K pass-1 launches back to back between two HIP events on the
same stream (an event between two kernels would add its own drain), and the
combine the same way.

Prints ONE JSON line (stdout):
  value  = KV GB/s of the headline workload, KV bytes = sum_b (L_b + NQ)*KV*D*2*s
  roofline.achieved = KV bytes per pass-1 launch / mean pass-1 launch duration
  configs = the same figures for every workload measured
  cpu_baseline = the oracle (plain C, fp64) on this host's cores, a bounded
                 sample of the headline workload
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/step + achieved KV GB/s (% of MI355X HBM peak)"
HBM_PEAK_GBPS = 8000.0
KERNEL_NAMES = {1: "valu", 2: "mfma"}
CSRC = os.path.join(ROOT, "paged_kv_gqa_decode_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kv_bytes: int):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("kernel_source_sha") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def _counter_rows(d):
    """Rows of a rocprofv3 --pmc run's counter CSV under directory d."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, match):
    """Mean Counter_Value per dispatch of the kernels whose name contains `match`."""
    vals = {}
    for r in rows:
        if match in r["Kernel_Name"]:
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return (sum(vals.values()) / len(vals), len(vals)) if vals else (None, 0)


def summarize_traffic(d: str):
    """profiles/traffic_counters.json and a markdown table from the counter runs
    under d: fetch_<workload>/ and write_<workload>/ (FETCH_SIZE, WRITE_SIZE of a
    `--configs N --lean` bench run, its stdout JSON in <dir>.out), cal_fetch/ and
    cal_write/ (a --calibrate-copy run: 256 MiB device copies). Counter KiB are
    scaled by what the same counter reads for the copy."""
    import statistics
    cal = {}
    for ctr, sub in (("FETCH_SIZE", "cal_fetch"), ("WRITE_SIZE", "cal_write")):
        vals = {}
        for r in _counter_rows(os.path.join(d, sub)):
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        big = [v for v in vals.values() if v > 1024]  # the copies (setup kernels are tiny)
        cal[ctr] = (256 << 20) / (statistics.median(big) * 1024)
    out = {"kernel_source_sha": kernel_source_hash(), "copy_scale": cal,
           "command_fetch": "rocprofv3 --pmc FETCH_SIZE -d <dir>/fetch_<workload> -o pmc "
                            "--output-format csv -- python3 bench.py --configs N --headline N "
                            "--lean --steps 10 --warmup 2 --repeats 1 --no-cpu-baseline",
           "command_write": "(the same with --pmc WRITE_SIZE -d <dir>/write_<workload>)",
           "command_calibration": "rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE -d <dir>/cal_fetch|"
                                  "cal_write -o pmc --output-format csv -- python3 bench.py "
                                  "--calibrate-copy",
           "command_summary": "python3 bench.py --summarize-traffic <dir>"}
    lines = ["| workload | kernel | dispatches | FETCH_SIZE KiB/dispatch (raw) | read bytes (scaled) "
             "| WRITE_SIZE KiB/dispatch (raw) | written bytes (scaled) | algorithmic KV bytes "
             "| read / algorithmic |", "|---|---|---|---|---|---|---|---|---|"]
    for sub in sorted(os.listdir(d)):
        if not sub.startswith("fetch_") or not os.path.isdir(os.path.join(d, sub)):
            continue
        name = sub[len("fetch_"):]
        with open(os.path.join(d, sub + ".out")) as fh:
            line = [l for l in fh.read().splitlines() if l.startswith("{")][-1]
        kvb = json.loads(line)["configs"][name]["kv_bytes_per_step"]
        frows = _counter_rows(os.path.join(d, sub))
        wrows = _counter_rows(os.path.join(d, "write_" + name))
        entry = {"kernel_source_sha": kernel_source_hash(), "kv_bytes": kvb}
        total = 0.0
        for kname, match in (("pass 1", "decode_"), ("combine", "combine_")):
            fk, n = _per_dispatch(frows, match)
            wk, _ = _per_dispatch(wrows, match)
            if fk is None:
                continue
            rd, wr = fk * 1024 * cal["FETCH_SIZE"], (wk or 0.0) * 1024 * cal["WRITE_SIZE"]
            entry[kname] = {"fetch_kib_raw": fk, "write_kib_raw": wk, "read_bytes": rd,
                            "write_bytes": wr, "dispatches": n}
            if kname == "pass 1":
                total = rd + wr
            lines.append(f"| {name} | {kname} | {n} | {fk:.1f} | {rd / 1e6:.2f} MB | {wk or 0:.1f} "
                         f"| {wr / 1e6:.2f} MB | {kvb / 1e6:.2f} MB | "
                         + (f"{rd / kvb:.3f} |" if kname == "pass 1" else "- |"))
        entry["hbm_bytes_per_launch"] = total
        out[name] = entry
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(f"kernel sources sha256[:16]: {kernel_source_hash()}")
    print(f"copy calibration (256 MiB device copy, median dispatch): FETCH_SIZE x "
          f"{cal['FETCH_SIZE']:.4f}, WRITE_SIZE x {cal['WRITE_SIZE']:.4f}\n")
    print("\n".join(lines))


def _kernel_name(name: str) -> str:
    """The library's kernels as pa::name<args> when the trace gives them mangled
    (template arguments: _Float16, bf16_t, float, integers, booleans)."""
    import re
    m = re.match(r"_ZN2pa(\d+)", name)
    if not m:
        return name
    pos = m.end()
    n = int(m.group(1))
    base, pos = name[pos:pos + n], pos + n
    if not name.startswith("I", pos):
        return "pa::" + base
    pos += 1
    args = []
    while pos < len(name) and name[pos] != "E":
        for pat, fmt in ((r"DF16_", lambda g: "_Float16"), (r"NS_6bf16_tE", lambda g: "pa::bf16_t"),
                         (r"f", lambda g: "float"), (r"Li(\d+)E", lambda g: g.group(1)),
                         (r"Lb([01])E", lambda g: "true" if g.group(1) == "1" else "false")):
            t = re.match(pat, name[pos:])
            if t:
                args.append(fmt(t))
                pos += t.end()
                break
        else:
            return name
    return f"pa::{base}<{', '.join(args)}>"


def summarize_trace(d: str):
    """A markdown table of the kernel statistics of a rocprofv3 --kernel-trace
    --stats run under d."""
    import csv
    import glob
    f = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))[0]
    with open(f, newline="") as fh:
        rows = list(csv.DictReader(fh))
    names = [_kernel_name(r["Name"]) for r in rows]
    print("| kernel | calls | avg us | min us | max us | share of GPU time |")
    print("|---|---|---|---|---|---|")
    for r, name in zip(rows, names):
        short = name.split("(")[0]
        if short.startswith("void "):
            short = short[5:]
        print(f"| {short[:110]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.1f}% |")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, seconds: float):
    """Time the oracle on the host: one warm-up, then repeats until `seconds`."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_gqa_decode_amd import workloads as W

    host = W.Workload(w.spec, w.context_lens, w.block_table, w.num_blocks, w.q.cpu(),
                      w.k_pool.cpu(), w.v_pool.cpu(), w.new_k.cpu(), w.new_v.cpu(), w.scale)
    # Probe on one sequence to bound the sample.
    def run(nseq):
        lens = host.context_lens[:nseq]
        t0 = time.perf_counter()
        oracle.paged_decode(host.q[:nseq], host.k_pool, host.v_pool, host.block_table[:nseq],
                            lens, host.new_k[:nseq], host.new_v[:nseq], host.scale,
                            causal=w.spec.causal)
        return time.perf_counter() - t0

    B = w.spec.B
    probe = run(1)
    per_seq = max(probe, 1e-4)
    nseq = B if per_seq * B <= seconds / 3 else max(1, int(seconds / 3 / per_seq))
    run(nseq)  # warm-up
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_start < seconds and len(times) < 1000):
        times.append(run(nseq))
    t = statistics.median(times)
    s = w.spec
    sample_bytes = int(sum(int(L) + s.NQ for L in host.context_lens[:nseq])) * s.KV * s.D * 2 * w.elem_bytes
    return {
        "value": sample_bytes / t / 1e9,
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"{'all' if nseq == B else 'first'} {nseq} of {B} sequences of the same "
                   f"workload, median of {len(times)} runs after 1 warm-up "
                   f"({sum(times):.1f} s of CPU time)"),
        "us_per_step_equiv": t / nseq * B * 1e6,
        "cpu_model": cpu_model(),
    }


MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix-core peak
SPIN_CYCLES = 200_000  # about 0.1 ms of GPU time ahead of each timed region


def dense_prefill(torch, pa, timed, warmup: int) -> dict:
    """pa_dense_attention on a Llama-3-8B-shaped causal prefill (one sequence of
    2048 tokens, 32 query heads over 8 KV heads, D = 128, fp16, synthetic):
    algorithmic flops 4*D per visible (query, key) pair, against the fp16
    matrix-core peak."""
    B, HQ, HK, S, D = 1, 32, 8, 2048, 128
    g = torch.Generator(device="cuda:0").manual_seed(1100)
    q = torch.randn(B, HQ, S, D, generator=g, device="cuda:0").half()
    k = torch.randn(B, HK, S, D, generator=g, device="cuda:0").half()
    v = torch.randn(B, HK, S, D, generator=g, device="cuda:0").half()
    out = torch.empty_like(q)
    scale = 1.0 / D ** 0.5

    def call(i):
        pa.dense_attention(q, k, v, scale, causal=True, out=out)

    for i in range(min(warmup, 50)):
        call(i)
    ms = timed(call, 50)
    flop = 4 * D * HQ * B * S * (S + 1) // 2
    tflops = flop / (ms / 1e3) / 1e12
    log(f"[bench] dense causal prefill {ms * 1e3:.1f} us, {tflops:.1f} TFLOP/s")
    return {
        "entry_point": "pa_dense_attention",
        "config": {"workload": "causal prefill", "batch": B, "num_heads": HQ,
                   "num_kv_heads": HK, "q_len": S, "kv_len": S, "head_dim": D,
                   "dtype": "f16", "causal": True, "mask": None},
        "us_per_call": round(ms * 1e3, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "algorithmic_flop_per_call": flop},
    }


def dense_backward(torch, pa, timed, warmup: int) -> dict:
    """pa_dense_attention_backward on the same causal prefill (dq, dk, dv for a
    synthetic output gradient): algorithmic flops 10*D per visible pair (five
    products of 2*D: the score recompute, dP, dV, dQ and dK), against the fp16
    matrix-core peak."""
    B, HQ, HK, S, D = 1, 32, 8, 2048, 128
    g = torch.Generator(device="cuda:0").manual_seed(1200)
    q = torch.randn(B, HQ, S, D, generator=g, device="cuda:0").half()
    k = torch.randn(B, HK, S, D, generator=g, device="cuda:0").half()
    v = torch.randn(B, HK, S, D, generator=g, device="cuda:0").half()
    dout = torch.randn(B, HQ, S, D, generator=g, device="cuda:0").half()
    scale = 1.0 / D ** 0.5
    prob = pa.make_dense_problem(q, k, causal=True)
    _, need = pa.pa_dense_backward_workspace_size(prob)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream()

    def call(i):
        pa.pa_dense_attention_backward(prob, q, k, v, None, dout, scale, dq, dk, dv, ws, need,
                                       stream)

    for i in range(min(warmup, 50)):
        call(i)
    ms = timed(call, 50)
    flop = 10 * D * HQ * B * S * (S + 1) // 2
    tflops = flop / (ms / 1e3) / 1e12
    log(f"[bench] dense causal backward {ms * 1e3:.1f} us, {tflops:.1f} TFLOP/s")
    return {
        "entry_point": "pa_dense_attention_backward",
        "config": {"workload": "causal prefill backward", "batch": B, "num_heads": HQ,
                   "num_kv_heads": HK, "q_len": S, "kv_len": S, "head_dim": D,
                   "dtype": "f16", "causal": True, "mask": None},
        "us_per_call": round(ms * 1e3, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "algorithmic_flop_per_call": flop},
    }


def percentile(sorted_values, q) -> float:
    """Linear-interpolation percentile of an ascending list."""
    x = (len(sorted_values) - 1) * q / 100.0
    lo = int(x)
    hi = min(lo + 1, len(sorted_values) - 1)
    return sorted_values[lo] + (sorted_values[hi] - sorted_values[lo]) * (x - lo)


def copy_bandwidth(torch, nbytes=1 << 30, reps=10) -> float:
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del a, b
    return 2 * nbytes / sec / 1e9


def prepare_workload(torch, W, spec, args):
    """The workload's inputs on the GPU, pools in `replicas` copies."""
    dev = "cuda:0"
    log(f"[bench] generating {spec.name} on {dev}")
    w = W.make_workload(spec, device=dev)
    table = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    kpools = [w.k_pool] + [w.k_pool.clone() for _ in range(args.replicas - 1)]
    vpools = [w.v_pool] + [w.v_pool.clone() for _ in range(args.replicas - 1)]
    return w, table, lens, kpools, vpools


def measure_workload(torch, pa, W, spec, args, stream, timed, prepared):
    """Every figure of one workload: the step (median of regions), pass 1 and
    the combine alone, and the slot-patched step against the plain one."""
    w, table, lens, kpools, vpools = prepared
    # the step users make: one paged_attn_decode call (merge included)
    dec = pa.Decoder(w.q, w.k_pool, table, max_context_len=w.max_context_len, causal=spec.causal,
                     num_partitions=args.partitions, kernel=args.kernel)
    # the same plan with the merge left to the caller, to time the two kernels apart
    dec_d = pa.Decoder(w.q, w.k_pool, table, max_context_len=w.max_context_len,
                       causal=spec.causal, num_partitions=args.partitions, kernel=args.kernel,
                       flags=pa.PA_FLAG_DEFER_COMBINE)
    kvb = W.kv_bytes(w)
    two = dec.partitions > 1
    kname = KERNEL_NAMES.get(dec.kernel, dec.kernel)
    log(f"[bench] {spec.name}: kv bytes/step {kvb}, partitions {dec.partitions}, chunk "
        f"{dec.chunk_tokens}, kernel {kname}, workspace {dec.workspace_bytes} B")

    def step(i):
        r = i % len(kpools)
        dec(w.q, kpools[r], vpools[r], table, lens, w.new_k, w.new_v, w.scale, stream=stream,
            check=False)

    def pass1(i):
        r = i % len(kpools)
        dec_d(w.q, kpools[r], vpools[r], table, lens, w.new_k, w.new_v, w.scale, stream=stream,
              check=False)

    def combine(i):
        pa.paged_attn_combine(dec_d.problem, lens, dec_d.workspace, dec_d.workspace_bytes,
                              dec_d.out, stream=stream)

    # the tensors are checked once here; the timed loops call with check=False
    for r in range(len(kpools)):
        pa.check_decode_args(w.q, kpools[r], vpools[r], table, lens, w.new_k, w.new_v, dec.out)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    regions = [timed(step, K) * 1e3 for _ in range(max(1, args.repeats))]
    wall = time.perf_counter() - t0
    srt = sorted(regions)
    us = statistics.median(regions)
    mean_pass1 = timed(pass1, K) * 1e3
    mean_comb = timed(combine, K) * 1e3 if two else 0.0
    gbps = kvb / (us / 1e6) / 1e9
    achieved = kvb / (mean_pass1 / 1e6) / 1e9
    log(f"[bench] {spec.name}: {us:.2f} us/step (median of {len(regions)} regions of {K}), "
        f"{gbps:.1f} GB/s ({gbps / HBM_PEAK_GBPS:.1%}); pass 1 {mean_pass1:.2f} us "
        f"({achieved / HBM_PEAK_GBPS:.1%}), combine {mean_comb:.2f} us; wall "
        f"{wall / K / len(regions) * 1e6:.2f} us/step")
    res = {
        "us_per_step": round(us, 2),
        "p10_us_per_step": round(percentile(srt, 10), 2),
        "p90_us_per_step": round(percentile(srt, 90), 2),
        "region_us_per_step": [round(x, 2) for x in regions],
        "kv_bytes_per_step": kvb,
        "kv_gbps": round(gbps, 2),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "config": {
            "workload": spec.name,
            "batch": spec.B, "num_heads": spec.H, "num_kv_heads": spec.KV, "head_dim": spec.D,
            "block_size": spec.BS, "nq": spec.NQ, "causal": spec.causal, "io_dtype": spec.dtype,
            "context_lens": list(spec.lengths), "kv_bytes_per_step": kvb, "accumulate": "f32",
            "partitions": dec.partitions, "chunk_tokens": dec.chunk_tokens, "kernel": kname,
            "pool_replicas": len(kpools), "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(spec.name, kvb),
            "kernel": f"pass 1 ({kname} decode kernel), timed alone: {K} launches back to back "
                      f"between two HIP events",
            "mean_launch_us": round(mean_pass1, 3),
            "algorithmic_bytes_per_launch": kvb,
            "combine_mean_us": round(mean_comb, 3),
        },
    }
    if not args.lean:
        res["append_step"] = append_step(torch, pa, spec, w, table, lens, kpools, vpools, args,
                                         stream, timed, step, kvb)
    del kpools, vpools, dec, dec_d, w
    torch.cuda.empty_cache()
    return res


def append_step(torch, pa, spec, w, table, lens, kpools, vpools, args, stream, timed, step, kvb):
    """The slot-patched step (paged_attn_decode_append): the same step also
    storing every new row into a spare slot past the cached blocks (the pools
    get ceil(B*NQ/BS) extra blocks; nothing cached is overwritten, so no read
    is patched): what the store and the per-sub-page slot checks cost, against
    the plain step on the same extended pools."""
    dev = "cuda:0"
    spare = -(-(spec.B * spec.NQ) // spec.BS)
    nb = kpools[0].shape[0]
    kx = [torch.cat([p, p.new_zeros((spare,) + tuple(p.shape[1:]))]) for p in kpools]
    vx = [torch.cat([p, p.new_zeros((spare,) + tuple(p.shape[1:]))]) for p in vpools]
    flat = torch.arange(spec.B * spec.NQ, device=dev, dtype=torch.int64)
    slots = ((nb + flat // spec.BS) * spec.BS + flat % spec.BS).to(torch.int32).view(spec.B, spec.NQ)
    dec_a = pa.Decoder(w.q, kx[0], table, max_context_len=w.max_context_len, causal=spec.causal,
                       num_partitions=args.partitions, kernel=args.kernel)

    def step_append(i):
        r = i % len(kx)
        dec_a(w.q, kx[r], vx[r], table, lens, w.new_k, w.new_v, w.scale, stream=stream,
              slot_mapping=slots, check=False)

    def step_plain(i):
        r = i % len(kx)
        dec_a(w.q, kx[r], vx[r], table, lens, w.new_k, w.new_v, w.scale, stream=stream,
              check=False)

    for r in range(len(kx)):
        pa.check_decode_args(w.q, kx[r], vx[r], table, lens, w.new_k, w.new_v, dec_a.out, slots)
    for i in range(args.warmup):
        step_append(i)
    K = args.steps
    app, plain = [], []
    for _ in range(3):  # interleaved, so that clock drift hits both alike
        app.append(timed(step_append, K) * 1e3)
        plain.append(timed(step_plain, K) * 1e3)
    ua, up = statistics.median(app), statistics.median(plain)
    elem = 4 if spec.dtype == "f32" else 2
    stored = spec.B * spec.NQ * spec.KV * spec.D * 2 * elem
    log(f"[bench] {spec.name}: slot-patched step {ua:.2f} us/step, plain step on the same pools "
        f"{up:.2f} us/step ({(ua / up - 1):+.1%})")
    del kx, vx, dec_a
    return {
        "entry_point": "paged_attn_decode_append",
        "us_per_step": round(ua, 2),
        "plain_step_same_pools_us": round(up, 2),
        "overhead_frac": round(ua / up - 1, 4),
        "kv_gbps": round(kvb / (ua / 1e6) / 1e9, 2),
        "stored_bytes_per_step": stored,
        "slots": "every new row into a spare slot past the cached blocks (no read patched)",
        "timing": "median of 3 regions of K steps each, interleaved with the plain step",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed regions of K steps per workload; the reported time per step is "
                         "their median")
    ap.add_argument("--configs", default="1,2,3,4",
                    help="comma-separated workload indices of CONFIGS, measured in this order")
    ap.add_argument("--headline", type=int, default=4,
                    help="workload whose figures are the line's value / roofline")
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--kernel", type=int, default=0, help="0 auto, 1 valu, 2 mfma")
    ap.add_argument("--partitions", type=int, default=0, help="0 = launch heuristic")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lean", action="store_true",
                    help="decode steps, pass 1 and the combine only (for profiler runs): no "
                         "slot-patched step, dense legs, copy bandwidth or CPU baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run device-to-device copies of a known size (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters of a profiler run)")
    ap.add_argument("--summarize-traffic", metavar="DIR",
                    help="write profiles/traffic_counters.json from the FETCH_SIZE / WRITE_SIZE "
                         "counter runs under DIR and print their table (no GPU)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print the kernel statistics of a rocprofv3 kernel-trace run under DIR "
                         "as a table (no GPU)")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library runs every kernel on a single "
              "MI355X and has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        nbytes, reps = 256 << 20, 10
        a = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(reps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": nbytes,
                          "bytes_written_per_copy": nbytes, "copies": reps}), flush=True)
        return

    import paged_kv_gqa_decode_amd as pa
    from paged_kv_gqa_decode_amd import workloads as W

    order = [int(x) for x in args.configs.split(",") if x.strip()]
    if args.headline not in order:
        order.append(args.headline)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    def timed(fn, count):
        """Mean ms per call of `count` calls of fn issued back to back between two
        HIP events on the launch stream. A short spin kernel ahead of the first
        event keeps the GPU busy while the host enqueues the first calls, so
        the region holds the calls back to back and not the host's latency to
        launch the first one."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(SPIN_CYCLES)
        e0.record(stream)
        for i in range(count):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / count

    # every workload is generated first (on the GPU), then each is measured
    prepared = {c: prepare_workload(torch, W, W.CONFIGS[c], args) for c in order}
    torch.cuda.synchronize()
    results = {}
    for c in order:
        results[W.CONFIGS[c].name] = measure_workload(torch, pa, W, W.CONFIGS[c], args, stream,
                                                      timed, prepared.pop(c))
    spec = W.CONFIGS[args.headline]
    head = results[spec.name]

    extra = {}
    if not args.lean:
        extra["dense_prefill"] = dense_prefill(torch, pa, timed, args.warmup)
        extra["dense_backward"] = dense_backward(torch, pa, timed, args.warmup)
        copy_gbps = copy_bandwidth(torch)
        log(f"[bench] device copy bandwidth {copy_gbps:.0f} GB/s (read+write)")
        extra["device_copy_gbps"] = round(copy_gbps, 1)

    cpu = None
    if not args.no_cpu_baseline and not args.lean:
        log(f"[bench] timing the oracle on the host ({spec.name})")
        w = W.make_workload(spec, device="cuda:0")
        cpu = cpu_baseline(w, args.cpu_seconds)
        del w
        log(f"[bench] oracle {cpu['value']:.3f} GB/s on {cpu['cores']} threads")

    result = {
        "metric": METRIC,
        "value": head["kv_gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 5),
        "us_per_step": head["us_per_step"],
        "hbm_frac": head["hbm_frac"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": head["config"],
        "timing": {
            "statistic": f"median over {len(head['region_us_per_step'])} timed regions of "
                         f"{args.steps} steps each (one paged_attn_decode call per step)",
            "p10_us_per_step": head["p10_us_per_step"],
            "p90_us_per_step": head["p90_us_per_step"],
            "region_us_per_step": head["region_us_per_step"],
        },
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "configs": {
            name: {k: v for k, v in r.items() if k not in ("region_us_per_step",)}
            for name, r in results.items()
        },
        **extra,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
