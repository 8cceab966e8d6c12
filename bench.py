#!/usr/bin/env python3
"""Throughput of the GPT-OSS decode sampling tail on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-sweep]

A step is one tail_forward call (RMSNorm -> lm_head -> top-k -> sampler) over
one batch of synthetic, seeded inputs already resident in HBM.  The headline
workload is the GPT-OSS-shaped decode step: gbs 1, H 2880, V 201088, k 256,
bf16 hidden, sampling at top_k 256, top_p 1, T 1, u 0.5, logits not emitted.
`value` is tokens/s = gbs * K / (time of K steps), timed with HIP events on
the stream the library launches on, bracketed by device synchronizations.

Also reported: per-step p10/p50/p90, the step with logits emitted, the
gbs-256 step with the top-k and sampler fused into the lm_head kernel
(`ms_per_step_fused_select`, an opt-in variant), per-stage times, the page-precision mode's step and lm_head (`page_precision`), the
step on one vocabulary shard's shape (V / 8 columns, `vocab_shard_points`), the lm_head kernel's algorithmic HBM rate against the 8 TB/s peak
(`roofline`), the same numbers at gbs 8 / 64 / 256 (`by_gbs`, with the
matrix-core kernels' executed TFLOP/s against the 2.5 PFLOP/s dense bf16
peak; `rooflines` adds the gbs-256 matrix-core kernel against that peak),
and the fp64 CPU oracle timed on a bounded sample of every workload on the
host's cores (`cpu_baseline`, whole steps at gbs 1, 8 and 64, 64 rows of
the gbs-256 step).  Every timed loop follows `--settle` seconds of untimed
steps (`settle_s_per_loop`).  Progress goes to stderr; stdout carries
exactly one JSON line.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# the CPU oracle's BLAS threads: every core this process may run on (set
# before numpy loads its BLAS; an explicit setting by the caller wins)
HOST_CORES = len(os.sched_getaffinity(0))
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(HOST_CORES))

METRIC = "tail tokens/s at gbs 1/8/64/256, V=201088; lm_head HBM GB/s & MFMA % of peak"
HBM_PEAK = 8000.0  # GB/s, MI355X HBM3E
MFMA_PEAK = 2500.0  # TFLOP/s, MI355X dense bf16 matrix cores
GEMV_MAX_BATCH = 3  # larger batches run the lm_head on the matrix cores
COUNTERS = os.path.join(ROOT, "profiles", "rmsnorm_lm_head_gbs1_counters.md")
ROWS_COUNTERS = os.path.join(ROOT, "profiles", "lm_head_rows_gbs256_counters.md")
# GPU time every timed loop is preceded by: after an idle period the first
# 20-40 ms of steps run slower while the memory and fabric clocks come up
# from their idle states (measured: gbs 1 302 -> 178 us, gbs 64 377 -> 226
# us, gbs 256 864 -> 650 us, flat for seconds afterwards)
SETTLE_S = 0.3


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the step time settles only after tens of milliseconds of work following
    # the input upload (measured: about 12 ms at gbs 1, 40 ms at gbs 64), so
    # the default warm-up runs 200 untimed steps
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed steps before every timed loop (on top of --warmup)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="headline workload only")
    ap.add_argument("--workload", default=None,
                    help="time only this workload label (for per-workload profiling runs)")
    ap.add_argument("--no-shard", action="store_true", help="skip the vocabulary-shard points")
    ap.add_argument("--fused-select", choices=("auto", "off", "only"), default="auto",
                    help="auto: also time the gbs-256 step with the top-k fused into the lm_head "
                         "kernel; off: do not; only: fuse it in every step of the run (profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of exactly 1 GiB, three times: the HBM
    byte counters of this known-size copy scale the lm_head's counter reads."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(copy_calibration_bytes=n, copies=3)), flush=True)


# the sources the gbs-1 RMSNorm + lm_head kernel and the large-batch
# matrix-core kernel (with its activation producer) are built from
GEMV_SOURCES = ("lm_head_gemv.hip", "tail_internal.h")
ROWS_SOURCES = ("lm_head_rows.hip", "lds_copy.h", "rmsnorm.hip", "tail_internal.h", "select_row.h",
                "sampler_row.h")


def kernel_source_hash(sources=GEMV_SOURCES):
    """Hash of a kernel's sources; a committed counter summary carries the
    hash it was measured on."""
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "decode_sampling_tail_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def counter_traffic(path=COUNTERS, sources=GEMV_SOURCES):
    """Per-launch HBM bytes (fetch + write, each scaled by the copy
    calibration) of a kernel, from its committed rocprofv3 counter summary;
    None if absent or taken on other sources."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_hash:\s*(\w+)", text)
    b = re.search(r"hbm_bytes_per_dispatch:\s*([\d.eE+]+)", text)
    if not m or not b or m.group(1) != kernel_source_hash(sources):
        return None
    return float(b.group(1))


def workloads():
    import synth
    # (label, config id): the shapes and distributions of the five workloads;
    # the padded gbs-64 one is timed without its planted ties (timing only)
    return [("gptoss_tail_gbs1", 1), ("gbs8_sampling", 2), ("gbs64_padded", 3), ("gbs256_dense", 4)]


def gpu_inputs(cid, torch, np):
    import synth
    inp = synth.make_config(cid)
    dev = torch.device("cuda")
    if inp.dtype == synth.DT_BF16:
        hidden = torch.from_numpy(inp.hidden.view(np.int16)).view(torch.bfloat16)
    else:
        hidden = torch.from_numpy(inp.hidden)
    run = len(inp.params) - 1  # the sampling run of the gbs-1 workload
    return inp, dict(hidden=hidden.to(dev), gamma=torch.from_numpy(inp.gamma).to(dev),
                     w_t=torch.from_numpy(inp.w_t.view(np.int16)).view(torch.bfloat16).to(dev),
                     params=torch.from_numpy(np.ascontiguousarray(inp.params[run])).to(dev)), run


def settle(torch, fn, seconds):
    """Untimed calls until `seconds` of wall time have passed (the GPU kept
    busy: a synchronization every 10 calls); returns the seconds spent."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    return time.perf_counter() - t0


EVENT_STRIDE = 5  # calls between the events of the percentile loop


def time_loop(torch, fn, steps, warmup, per_step=False, settle_s=0.0):
    """Seconds per call over `steps` calls after `warmup` untimed ones and
    `settle_s` seconds of untimed calls, from HIP events on the stream the
    library launches on, bracketed by device synchronizations.  With
    per_step, an event also follows every EVENT_STRIDE calls and (mean,
    [p10, p50, p90] of the per-call time of each stride) is returned (an
    event between every two calls would add its own microseconds to each)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    settle(torch, fn, settle_s)
    st = torch.cuda.current_stream()
    stride = EVENT_STRIDE if per_step else steps
    n_int = max(1, steps // stride)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_int + 1)]
    ev[0].record(st)
    for i in range(n_int * stride):
        fn()
        if (i + 1) % stride == 0:
            ev[(i + 1) // stride].record(st)
    torch.cuda.synchronize()
    mean = ev[0].elapsed_time(ev[-1]) / 1000.0 / (n_int * stride)
    if not per_step:
        return mean
    import numpy as np
    d = np.array([ev[i].elapsed_time(ev[i + 1]) / 1000.0 / stride for i in range(n_int)])
    return mean, [float(np.percentile(d, q)) for q in (10, 50, 90)]


def time_graph(torch, fn, reps=20, replays=10):
    """Seconds per call of `fn` from replays of a HIP graph holding `reps`
    calls: the device time of short stages without the host's cost of a
    Python call (which exceeds a few-microsecond kernel).  The entry points
    launch only kernels on the caller's stream, so the capture is exact."""
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(replays):
        graph.replay()
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1000.0 / (replays * reps)


def bench_workload(cid, args, torch, np):
    import decode_sampling_tail_amd as dst
    inp, g, run = gpu_inputs(cid, torch, np)
    f = dst.Forward(inp.gbs, inp.H, inp.V, inp.k, inp.H_u, inp.eps, inp.zero_pad, deferred=True,
                    emit_logits=False)
    step = lambda: f(g["hidden"], g["gamma"], g["w_t"], g["params"])
    ss = args.settle
    t_step = time_loop(torch, step, args.steps, args.warmup, settle_s=ss)
    # percentiles from a second loop with an event every few steps (the mean
    # above comes from the plain loop)
    _, pct = time_loop(torch, step, args.steps, 0, per_step=True)
    # the same step with the fp32 logits emitted (an extra gbs*V*4-byte write)
    fe = dst.Forward(inp.gbs, inp.H, inp.V, inp.k, inp.H_u, inp.eps, inp.zero_pad, deferred=True,
                     emit_logits=True)
    t_emit = time_loop(torch, lambda: fe(g["hidden"], g["gamma"], g["w_t"], g["params"]),
                       max(10, args.steps // 4), args.warmup, settle_s=ss)
    del fe
    fused_timed = inp.gbs >= 129 and args.fused_select == "auto"
    if fused_timed:
        # the same step with the top-k and sampler run by the large-batch
        # lm_head kernel after its grid barrier (not the default: slower)
        os.environ["TAIL_FUSED_SELECT"] = "1"
        try:
            t_fused = time_loop(torch, step, max(10, args.steps // 4), args.warmup, settle_s=ss)
        finally:
            os.environ.pop("TAIL_FUSED_SELECT", None)
    # stage by stage.  rmsnorm_lm_head runs the same kernels and launch shapes
    # as tail_forward's first stage (there they also emit the group maxima);
    # topk and sample are the standalone calls (inside tail_forward the group
    # maxima come from the lm_head epilogue and the sampler is fused into the
    # top-k kernel).
    logits = torch.empty((inp.gbs, inp.V), dtype=torch.float32, device="cuda")
    r = torch.empty((inp.gbs,), dtype=torch.float32, device="cuda")
    ws = torch.empty(dst.workspace_size(inp.gbs, inp.H, inp.H_u, inp.V, inp.k, dst.EMIT_LOGITS),
                     dtype=torch.uint8, device="cuda")
    norm_lm = lambda: dst.rmsnorm_lm_head(g["hidden"], g["gamma"], g["w_t"], inp.H_u, inp.eps,
                                          inp.zero_pad, True, out=logits, out_r=r, ws=ws)
    norm_lm()
    vals, idx = dst.topk(logits, inp.k, ws=ws)
    t_lm = time_loop(torch, norm_lm, args.steps, args.warmup, settle_s=ss)
    # the short standalone stages as graph replays (device time per call)
    t_topk = time_graph(torch, lambda: dst.topk(logits, inp.k, vals, idx, ws))
    tok = torch.empty((inp.gbs,), dtype=torch.int32, device="cuda")
    t_samp = time_graph(torch, lambda: dst.sample(vals, idx, g["params"], tok))
    hid_bytes = inp.hidden.dtype.itemsize
    # algorithmic bytes: the real lanes of weight, hidden and gamma once, the
    # logits and the row scale written once
    lm_bytes = (inp.H_u * inp.V * 2 + inp.gbs * inp.H_u * hid_bytes + inp.H_u * 4 +
                inp.gbs * inp.V * 4 + inp.gbs * 4)
    flops = 2.0 * inp.gbs * inp.H_u * inp.V
    res = dict(gbs=inp.gbs, tokens_per_s=inp.gbs / t_step, steps_per_s=1.0 / t_step,
               ms_per_step=t_step * 1e3, ms_p10_p50_p90_evented=[x * 1e3 for x in pct],
               settle_s_per_loop=ss,
               ms_per_step_emit_logits=t_emit * 1e3,
               **(dict(ms_per_step_fused_select=t_fused * 1e3) if fused_timed else {}),
               stage_us=dict(rmsnorm_lm_head=t_lm * 1e6, topk=t_topk * 1e6, sample=t_samp * 1e6),
               lm_head_gbs=lm_bytes / t_lm / 1e9, lm_head_tflops=flops / t_lm / 1e12,
               lm_head_bytes=lm_bytes)
    if inp.gbs > GEMV_MAX_BATCH:
        # matrix-core path: 2 bf16 activation terms over the padded rows
        exec_flops = 2.0 * rows_padded(inp.gbs) * 2 * inp.H_u * inp.V
        res["lm_head_mfma_exec_tflops"] = exec_flops / t_lm / 1e12
        res["lm_head_mfma_frac"] = exec_flops / t_lm / 1e12 / MFMA_PEAK
        res["lm_head_mfma_alg_tflops"] = flops / t_lm / 1e12
        res["lm_head_mfma_alg_frac"] = flops / t_lm / 1e12 / MFMA_PEAK
    # the page-precision mode (bf16 GEMM input, top-k over the bf16 mirror):
    # the same step and stage, one activation term on the matrix cores
    fp = dst.Forward(inp.gbs, inp.H, inp.V, inp.k, inp.H_u, inp.eps, inp.zero_pad, deferred=True,
                     emit_logits=False, page=True)
    t_page = time_loop(torch, lambda: fp(g["hidden"], g["gamma"], g["w_t"], g["params"]),
                       args.steps, args.warmup, settle_s=ss)
    del fp
    wsp = torch.empty(dst.workspace_size(inp.gbs, inp.H, inp.H_u, inp.V, inp.k,
                                         dst.EMIT_LOGITS | dst.PAGE_PRECISION),
                      dtype=torch.uint8, device="cuda")
    t_lm_page = time_loop(torch, lambda: dst.rmsnorm_lm_head(
        g["hidden"], g["gamma"], g["w_t"], inp.H_u, inp.eps, inp.zero_pad, True, out=logits, out_r=r,
        ws=wsp, page=True), args.steps, args.warmup, settle_s=ss)
    page = dict(tokens_per_s=inp.gbs / t_page, ms_per_step=t_page * 1e3,
                rmsnorm_lm_head_us=t_lm_page * 1e6, lm_head_gbs=lm_bytes / t_lm_page / 1e9)
    if inp.gbs > GEMV_MAX_BATCH:
        exec_flops = 2.0 * rows_padded(inp.gbs) * inp.H_u * inp.V
        page["lm_head_mfma_exec_tflops"] = exec_flops / t_lm_page / 1e12
        page["lm_head_mfma_frac"] = exec_flops / t_lm_page / 1e12 / MFMA_PEAK
    res["page_precision"] = page
    del g, f, logits, ws, wsp, r
    torch.cuda.empty_cache()
    return inp, run, res


def rows_padded(gbs):
    """Rows the matrix-core kernels multiply at the full vocabulary: 16-row
    tiles up to 64 rows, then 32-row tiles (the large-batch kernel skips the
    MFMAs of its all-padding tiles)."""
    if gbs <= 64:
        return (gbs + 15) // 16 * 16
    return (gbs + 31) // 32 * 32


SHARDS = 8  # vocabulary shards of the multi-GPU design; one shard's shape is timed here


def bench_shard(cid, args, torch, np):
    """tail_forward on one vocabulary shard's real shape: the workload's hidden
    rows and params against shard 0 of its weight, W[:, :V / SHARDS] (what one
    of 8 GPUs computes before the candidate exchange)."""
    import decode_sampling_tail_amd as dst
    inp, g, run = gpu_inputs(cid, torch, np)
    Vs = inp.V // SHARDS
    w = g["w_t"][:, :Vs].contiguous()
    del g["w_t"]
    f = dst.Forward(inp.gbs, inp.H, Vs, inp.k, inp.H_u, inp.eps, inp.zero_pad, deferred=True,
                    emit_logits=False)
    t_step = time_loop(torch, lambda: f(g["hidden"], g["gamma"], w, g["params"]), args.steps,
                       args.warmup, settle_s=args.settle)
    logits = torch.empty((inp.gbs, Vs), dtype=torch.float32, device="cuda")
    ws = torch.empty(dst.workspace_size(inp.gbs, inp.H, inp.H_u, Vs, inp.k, dst.EMIT_LOGITS),
                     dtype=torch.uint8, device="cuda")
    t_lm = time_loop(torch, lambda: dst.rmsnorm_lm_head(g["hidden"], g["gamma"], w, inp.H_u, inp.eps,
                                                        inp.zero_pad, True, out=logits, ws=ws),
                     args.steps, args.warmup, settle_s=args.settle)
    lm_bytes = (inp.H_u * Vs * 2 + inp.gbs * inp.H_u * inp.hidden.dtype.itemsize + inp.H_u * 4 +
                inp.gbs * Vs * 4 + inp.gbs * 4)
    res = dict(gbs=inp.gbs, V_shard=Vs, ms_per_step=t_step * 1e3, tokens_per_s=inp.gbs / t_step,
               rmsnorm_lm_head_us=t_lm * 1e6, lm_head_gbs=lm_bytes / t_lm / 1e9)
    del g, w, f, logits, ws
    torch.cuda.empty_cache()
    return res


def blas_threads():
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])


# rows of the oracle's bounded sample per workload: whole steps where a step
# costs seconds, a row subset of the gbs-256 workload (rows are independent)
CPU_SAMPLE_ROWS = {1: None, 8: None, 64: None, 256: 64}


def cpu_oracle_leg(inp, run, budget_s):
    """The fp64 oracle, as it stands, on this workload's inputs: whole tail
    steps (repeated while the budget lasts) or a fixed subset of the rows."""
    import numpy as np
    import oracle
    n_rows = CPU_SAMPLE_ROWS.get(inp.gbs)
    rows = None if n_rows is None or n_rows >= inp.gbs else np.arange(n_rows)
    per_call = inp.gbs if rows is None else len(rows)
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.tail(inp.hidden, inp.dtype, inp.gamma, inp.w_t, inp.H_u, inp.k, inp.eps, inp.zero_pad,
                    params=inp.params[run], rows=rows)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 20 or rows is not None:
            break
    what = (f"{n} whole tail step{'s' if n > 1 else ''}" if rows is None else
            f"rows 0..{per_call - 1} of one step")
    log(f"cpu oracle gbs {inp.gbs}: {what}, {el:.1f} s")
    return dict(gbs=inp.gbs, rows=n * per_call, seconds=el, tokens_per_s=n * per_call / el,
                seconds_per_row=el / (n * per_call),
                sample=f"{what} of the gbs-{inp.gbs} workload (fp64 RMSNorm, fp64 lm_head, "
                       f"full stable sort, fp64 sampler)")


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the tail runs with the whole vocabulary on one device)", file=sys.stderr)
        sys.exit(2)
    if args.fused_select == "only":
        os.environ["TAIL_FUSED_SELECT"] = "1"  # the library reads it at every call
    import numpy as np
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.init()

    results, cpu = {}, {}
    for label, cid in workloads():
        if args.no_sweep and cid != 1:
            continue
        if args.workload and label != args.workload:
            continue
        log(f"workload {label}: generating inputs and timing {args.steps} steps")
        inp, run, res = bench_workload(cid, args, torch, np)
        log(f"{label}: {res['tokens_per_s']:.1f} tok/s, {res['ms_per_step']:.3f} ms/step, "
            f"lm_head {res['lm_head_gbs']:.0f} GB/s, stages {res['stage_us']}; page precision "
            f"{res['page_precision']['tokens_per_s']:.1f} tok/s, lm_head "
            f"{res['page_precision']['rmsnorm_lm_head_us']:.1f} us")
        results[label] = res
        if not args.no_cpu_baseline:
            # the oracle on the same inputs, in the same run, on this host's cores
            cpu[label] = cpu_oracle_leg(inp, run, 6.0 if inp.gbs == 1 else 0.0)
        del inp

    shard = {}
    if not args.no_sweep and not args.no_shard and not args.workload:
        for label, cid in workloads():
            log(f"shard point {label}: V / {SHARDS} columns")
            shard[label] = bench_shard(cid, args, torch, np)
            log(f"shard {label}: {shard[label]['ms_per_step'] * 1e3:.1f} us/step, "
                f"lm_head {shard[label]['lm_head_gbs']:.0f} GB/s")

    if "gptoss_tail_gbs1" not in results:  # a profiling run of another workload
        print(json.dumps(dict(metric=METRIC, by_gbs=results)), flush=True)
        return
    head = results["gptoss_tail_gbs1"]
    traffic = counter_traffic()
    roof = dict(bound="hbm", achieved=head["lm_head_gbs"], peak=HBM_PEAK, unit="GB/s",
                frac=head["lm_head_gbs"] / HBM_PEAK, traffic=traffic,
                kernel="gemv_kernel<1,2,4,6>: RMSNorm-fused weight-streaming lm_head, gbs 1",
                bytes_per_launch=head["lm_head_bytes"],
                launch_us=head["stage_us"]["rmsnorm_lm_head"])
    # the matrix-core kernel of the dense workload, against the bf16 peak:
    # algorithmic flops 2*gbs*H_u*V, executed ones with both activation terms
    rooflines = [roof]
    if "gbs256_dense" in results:
        r = results["gbs256_dense"]
        rooflines.append(dict(
            bound="mfma", achieved=r["lm_head_mfma_alg_tflops"], peak=MFMA_PEAK, unit="TFLOP/s",
            frac=r["lm_head_mfma_alg_frac"], executed=r["lm_head_mfma_exec_tflops"],
            frac_executed=r["lm_head_mfma_frac"],
            traffic=counter_traffic(ROWS_COUNTERS, ROWS_SOURCES),
            kernel="rows_kernel<2,13,8,3,1>: 32x32x16 matrix-core lm_head, gbs 256 (the time "
                   "includes its RMSNorm/bf16-split producer kernel)",
            flops_per_launch=2.0 * 256 * 2880 * 201088,
            launch_us=r["stage_us"]["rmsnorm_lm_head"]))
    out = dict(metric=METRIC, value=head["tokens_per_s"], unit="tokens/s", n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=head["ms_per_step"],
               higher_is_better=True, scaling="weak", vs_baseline=None, dtype="fp32",
               data="synthetic",
               config=dict(workload="gptoss_tail_gbs1", gbs=1, H=2880, H_u=2880, V=201088, k=256,
                           hidden_dtype="bf16", weight_dtype="bf16",
                           sampling="top_k=256 top_p=1 T=1 u=0.5", emit_logits=False,
                           parallelism="none (one GPU, whole vocabulary)"),
               stage_us=head["stage_us"], roofline=roof, rooflines=rooflines,
               settle_s_per_loop=args.settle,
               ms_p10_p50_p90_evented=head["ms_p10_p50_p90_evented"],
               by_gbs={lbl: dict(r, lm_head_hbm_frac=r["lm_head_gbs"] / HBM_PEAK)
                       for lbl, r in results.items()},
               source_hash=kernel_source_hash(),
               vocab_shard_points=shard or None)
    if cpu:
        h = cpu["gptoss_tail_gbs1"]
        out["cpu_baseline"] = dict(value=h["tokens_per_s"], unit="tokens/s", cores=HOST_CORES,
                                   blas_threads=blas_threads(), kind="oracle", sample=h["sample"],
                                   by_gbs=cpu)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
