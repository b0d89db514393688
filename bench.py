#!/usr/bin/env python3
"""Benchmark of the MI355X MLA decode path (one GPU).

A step is one full decode call (the split kernel, which plans its own work
item, and the combine) over one batch of synthetic inputs already resident in
HBM.  Default workload:
B=64, H=128, L=4096 for every sequence, fp16, contiguous cache, i.i.d. N(0,1)
inputs, softmax_scale = 1/sqrt(576), planner-chosen splits.

Prints ONE JSON line.  Throughput is TFLOPS of the algorithmic work
2·H·(576 + 512) per valid cache row; the line also carries KV GB/s, µs per
call, the fraction of the per-workload roofline min(8 TB/s × intensity, 2.5
PFLOP/s dense fp16/bf16), the split kernel against the HBM peak with its
measured traffic (`roofline`), and the fp64 CPU oracle timed on a sample of
the workload (`cpu_baseline`).

Kernel times.  The timed region (events on the launch stream around K calls)
gives the time of a call.  A second pass times each launch from its own
dispatch events; those events slow the launches down by a few percent, so that
pass only gives each kernel's share of the call, and a kernel's time is its
share of the timed-region time (the per-kernel times add up to the call).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0     # dense fp16 / bf16
D_QK, D_V = 576, 512

METRIC = "MLA decode TFLOPS + KV GB/s (% roofline), B=64/128 h=128 d=576/512"


def workload_figures(lens, heads: int, seqlen_q: int = 1, kv_elt: int = 2):
    """Algorithmic flops and bytes of one call (cache rows, Q, out, lse).

    `heads` counts query rows (seqlen_q tokens x heads per token); with several
    query tokens, token t of s is charged only the L - (s - 1 - t) rows it
    sees.  kv_elt: bytes per cache value (2, or 1 for an FP8 cache)."""
    import numpy as np
    L = np.maximum(np.asarray(lens, dtype=np.int64), 0)
    rows = float(np.sum(L))
    B, s = len(lens), seqlen_q
    seen = float(sum(np.sum(np.maximum(L - (s - 1 - t), 0)) for t in range(s)))
    flops = 2.0 * (heads // s) * (D_QK + D_V) * seen
    kv_bytes = rows * D_QK * kv_elt
    total_bytes = kv_bytes + B * heads * (D_QK * 2 + D_V * 2 + 4)
    return flops, kv_bytes, total_bytes


def code_sha256(text: str) -> str:
    """sha256 of C/HIP source text with comments, trailing blanks and blank
    lines removed (string literals holding "//" or "/*" are not expected)."""
    import hashlib
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
    return hashlib.sha256("\n".join(line for line in lines if line.strip()).encode()).hexdigest()


def kernel_code_sha256() -> str:
    """code_sha256 of the kernel source: the fingerprint a counter summary is
    taken on (a comment edit keeps it, a code edit does not)."""
    src = os.path.join(ROOT, "deepseek_mla_decode_amd", "csrc", "mla_kernels.hip")
    with open(src) as f:
        return code_sha256(f.read())


def measured_counters(workload: str, profiles_dir: str = os.path.join(ROOT, "profiles"), sha: str = None):
    """From the committed rocprofv3 summary of this workload (profiles/*.md):
    HBM bytes per split-kernel launch (FETCH_SIZE + WRITE_SIZE, scaled by a
    plain-copy calibration), the split kernel's MFMA-busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES)) and the file.
    None for each when there is no summary for this workload or the kernel
    code changed since the counters were taken (kernel_code_sha256)."""
    import glob
    sha = sha or kernel_code_sha256()
    traffic = busy = source = None
    for f in sorted(glob.glob(os.path.join(profiles_dir, "*.md"))):
        with open(f) as fh:
            lines = fh.readlines()
        for line in lines:
            for tag in ("traffic-json:", "counters-json:"):
                if line.startswith(tag):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("workload") != workload or rec.get("code_sha256") != sha:
                        continue
                    source = os.path.relpath(f, ROOT)
                    if tag == "traffic-json:":
                        traffic = int(rec["fetch_bytes"]) + int(rec["write_bytes"])
                    else:
                        busy = float(rec["mfma_busy"])
    return traffic, busy, source


def split_bounds(flops: float, total_bytes: float, split_ms: float, traffic):
    """The split kernel's launch against its two peaks, binding bound first.

    Algorithmic bytes per launch time against 8 TB/s and algorithmic flops per
    launch time against 2.5 PFLOP/s; the binding one is the one whose peak times
    the launch's intensity (flops / bytes) is smaller."""
    ok = split_ms > 0
    gbs = total_bytes / (split_ms * 1e-3) / 1e9 if ok else None
    tfs = flops / (split_ms * 1e-3) / 1e12 if ok else None
    hbm = {"bound": "hbm", "achieved": None if gbs is None else round(gbs, 1),
           "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": None if gbs is None else round(gbs / HBM_PEAK_GBS, 4),
           "traffic": traffic, "kernel": "split_kernel"}
    mfma = {"bound": "mfma", "achieved": None if tfs is None else round(tfs, 1),
            "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": None if tfs is None else round(tfs / MFMA_PEAK_TFLOPS, 4),
            "traffic": traffic, "kernel": "split_kernel"}
    hbm_bound = HBM_PEAK_GBS * 1e9 * flops < MFMA_PEAK_TFLOPS * 1e12 * total_bytes
    return (hbm, mfma) if hbm_bound else (mfma, hbm)


def host_cpu():
    """(logical CPUs this process may run on, CPU model name)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return n, model


def cpu_baseline(inp, budget_s: float):
    """Time the fp64 oracle on the workload's sequences, in order and again from
    the first, until ~budget_s of work (at least one sequence).  `cores` is the
    thread count of the BLAS pool the oracle's matrix products run on (the
    rest of the oracle is single-threaded NumPy)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    nproc, model = host_cpu()
    done, t0 = 0, time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        oracle.mla_decode_ref(inp, batches=[done % inp.batch])
        done += 1
    el = time.perf_counter() - t0
    passes, rest = divmod(done, inp.batch)
    full, _, _ = workload_figures(inp.cache_seqlens, inp.heads, inp.seqlen_q)   # flops only
    part, _, _ = workload_figures(inp.cache_seqlens[:rest], inp.heads, inp.seqlen_q)
    flops = passes * full + part
    return {"value": flops / el / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} sequence decode{'s' if done != 1 else ''} ({passes} passes over all "
                      f"{inp.batch} sequences + {rest}; "
                      f"all {inp.heads} query rows each), fp64 NumPy, {el:.1f} s wall",
            "host": {"nproc": nproc, "cpu_model": model}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults long enough for the clocks to settle under sustained load (the
    # first hundreds of calls run at a lower clock): about 0.25 s each at B=64.
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=2000)
    # The GPU leaves its idle clocks only after some hundreds of milliseconds
    # of load, so a short --warmup alone times the ramp (measured 3-9 % low
    # with 5 warm-up and 20 timed calls).  The same calls run untimed for this
    # long before the warm-up steps; the line reports how many.
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="seconds of untimed calls before the warm-up steps (0 = none)")
    ap.add_argument("--config", type=int, default=1, help="workload 0..4 (default 1: B=64 L=4096 fp16)")
    ap.add_argument("--num-split", type=int, default=0, help="0 = planner")
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated per step (0 = auto)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time (0 = skip)")
    ap.add_argument("--check", action="store_true", help="check sampled outputs against the oracle")
    ap.add_argument("--heads", type=int, default=0,
                    help="query heads per token instead of the workload's (e.g. one tensor-parallel shard)")
    ap.add_argument("--seqlen-q", type=int, default=1,
                    help="query tokens per sequence (speculative / multi-token decode), each of H heads")
    ap.add_argument("--plan-once", action="store_true",
                    help="make the split plan once (mla_plan_device) and decode with it every step "
                         "(mla_decode_planned), as a model's layers share one plan per decode step; "
                         "by default every call plans for itself")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="store the workload's cache as FP8 E4M3 bytes with one scale (workloads 0..3)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "the decode path has no multi-GPU mode", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import deepseek_mla_decode_amd as mla
    import mla_inputs as mi
    from mla_inputs.torch_io import to_device

    t_gen = time.perf_counter()
    inp = mi.make_config(args.config, seqlen_q=args.seqlen_q, heads=args.heads or None,
                         kv_dtype="fp8" if args.kv_fp8 else None)
    gen_s = time.perf_counter() - t_gen
    dev = to_device(inp, "cuda")
    kv_elt = 1 if inp.cache_dtype == "fp8" else 2
    flops, kv_bytes, total_bytes = workload_figures(inp.cache_seqlens, inp.heads, inp.seqlen_q, kv_elt)
    # Rotate copies of the cache when one copy would fit in the 256 MiB last-level cache.
    copies = args.copies or (1 if kv_bytes > 1.5 * 2**30 else 3)
    devs = [dev]
    for _ in range(copies - 1):
        d2 = dict(dev)
        if inp.paged:
            pool = dev["pool"].clone()
            d2.update(pool=pool, kv_latent=pool[..., :512], k_pe=pool[..., 512:])
        else:
            d2.update(kv_latent=dev["kv_latent"].clone(), k_pe=dev["k_pe"].clone())
        d2["q_nope"], d2["q_pe"] = dev["q_nope"].clone(), dev["q_pe"].clone()
        devs.append(d2)
    B, H, S = inp.batch, inp.heads, inp.seqlen_q   # H: query rows (S tokens x H / S heads)
    outs = [torch.empty((B, H, 512), dtype=dev["q_nope"].dtype, device="cuda") for _ in devs]
    lses = [torch.empty((B, H), dtype=torch.float32, device="cuda") for _ in devs]
    desc = mla.make_desc(dev["q_nope"], dev["q_pe"], dev["kv_latent"], dev["k_pe"], dev["block_table"], outs[0],
                         seqlen_q=S, kv_scale=dev["kv_scale"])
    ws = torch.empty(mla.mla_workspace_size(desc, args.num_split, mla.mla_num_cus()), dtype=torch.uint8,
                     device="cuda")

    def tokens(t):   # query rows [B, H, ...] -> [B, S, H / S, ...] when S > 1
        return t if S == 1 else t.view(B, S, H // S, *t.shape[2:])

    # One plan for every copy (their lengths are the same), made before the
    # timed region when --plan-once asks for it.
    plan = (mla.mla_plan_device(dev["cache_seqlens"], H, args.num_split, mla.mla_num_cus(), seqlen_q=S)
            if args.plan_once else None)

    def step(i):
        d = devs[i % len(devs)]
        a = (tokens(d["q_nope"]), tokens(d["q_pe"]), d["kv_latent"], d["k_pe"], d["block_table"],
             d["cache_seqlens"], inp.softmax_scale)
        kw = dict(num_split=args.num_split, out=tokens(outs[i % len(devs)]), lse=tokens(lses[i % len(devs)]),
                  workspace=ws, kv_scale=d["kv_scale"])
        if plan is not None:
            mla.mla_decode_planned(*a, plan, **kw)
        else:
            mla.mla_decode(*a, **kw)

    prewarm_calls = 0
    if args.prewarm_s > 0:
        t_end = time.perf_counter() + args.prewarm_s
        while time.perf_counter() < t_end:
            for _ in range(64):
                step(prewarm_calls)
                prewarm_calls += 1
            torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps), timing {args.steps} steps", file=sys.stderr, flush=True)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # Each kernel's share of a call, from the launches' own dispatch events
    # (a second pass; those events slow the launches, so only the shares are
    # used), applied to the timed-region time of a call.
    mla.mla_timing_enable(True)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    split_ev, comb_ev, calls = mla.mla_timing_read()
    mla.mla_timing_enable(False)
    share = split_ev / (split_ev + comb_ev) if split_ev + comb_ev > 0 else 1.0
    split_avg = ms * share
    comb_avg = ms - split_avg
    assert split_avg + comb_avg <= ms * (1 + 1e-9)

    check = None
    if args.check:
        import oracle
        from mla_inputs.torch_io import from_device
        b = [0, B - 1]
        ro, rl = oracle.mla_decode_ref(inp, batches=b)
        o = from_device(outs[0][b])
        l = from_device(lses[0][b])
        ex = float((np.abs(o - ro) - (2e-3 + 1e-2 * np.abs(ro))).max())
        check = {"sequences": b, "max_excess_out": ex, "max_lse_err": float(np.abs(l - rl).max()), "ok": ex <= 0}

    cpu = cpu_baseline(inp, args.cpu_budget) if args.cpu_budget > 0 else None

    workload = (inp.meta["config"] + (f"_q{S}" if S > 1 else "")
                + (f"_heads{H // S}" if args.heads else ""))
    tflops = flops / (ms * 1e-3) / 1e12
    ai = flops / total_bytes
    roof_tflops = min(HBM_PEAK_GBS * 1e9 * ai / 1e12, MFMA_PEAK_TFLOPS)
    mean_L = float(np.mean(inp.cache_seqlens))
    traffic, mfma_busy, counter_file = measured_counters(workload)
    bounds = split_bounds(flops, total_bytes, split_avg, traffic)
    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm": {"seconds": args.prewarm_s, "calls": prewarm_calls},
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic (seeded N(0,1), no dataset)",
        "config": {"workload": workload, "batch": B, "heads": H // S, "seqlen_q": S,
                   "seqlen_kv_mean": mean_L, "layout": "paged" if inp.paged else "contiguous",
                   "kv_cache": "fp8_e4m3 (one scale)" if kv_elt == 1 else inp.dtype,
                   "num_split": args.num_split or "planner", "input_copies": len(devs),
                   "plan": "made once, reused by every step" if args.plan_once else "in every call"},
        "us_per_call": round(ms * 1e3, 2),
        "kv_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
        "arith_intensity": round(ai, 1),
        "roofline_tflops": round(roof_tflops, 1),
        "frac_of_roofline": round(tflops / roof_tflops, 4),
        "kernel_ms": {"split": round(split_avg, 5), "combine": round(comb_avg, 5),
                      "split_share": round(share, 4),
                      "event_pass_ms": {"split": round(split_ev / max(calls, 1), 5),
                                        "combine": round(comb_ev / max(calls, 1), 5)}},
        # The binding bound of the split kernel: HBM below the ridge intensity
        # (8 TB/s x intensity < 2.5 PFLOP/s, one query token per sequence), MFMA above it
        # (several query tokens share each cache row); the other bound beside it.
        "roofline": bounds[0],
        "other_bound": bounds[1],
        # Counter-measured share of the split kernel's cycles with the MFMA
        # unit busy (the committed rocprofv3 summary of this workload).
        "counters": {"mfma_busy": mfma_busy, "source": counter_file},
        "cpu_baseline": cpu,
        "input_gen_s": round(gen_s, 1),
    }
    if check is not None:
        line["check"] = check
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
