#!/usr/bin/env python3
"""Throughput of the verify-and-resample step on one MI355X.

One step = one spec_verify_run call over a batch of B=64 sequences, K=4
draft tokens, V=128256 bf16 logits, nucleus top-p 0.8 at temperature 0.8 on
both models (target N(0, 4^2) plus +8 on 20 tokens per position, draft =
target + N(0, 0.7^2)): the whole hot path (filter thresholds, softmax
statistics, accept walk, resample / bonus draw) in the library's kernels.

Inputs are synthetic and resident in HBM before timing; R input sets rotate
so the 256 MB Infinity Cache cannot serve repeated reads.  Draft tokens are
drawn by the library itself (the step with K = 0 on the draft rows).

Prints one JSON line: value = rows/s; roofline = algorithmic logit bytes per
call / average time of the row kernel (the streaming pass over the logit
rows with each row's finish; HIP events the library attaches to that
kernel's own dispatches on the launch stream) against the 8 TB/s HBM peak;
streaming_ceiling = the read rate of the library's read-only probe over the
same rotating logits; per_call_us = p10 / median / p90 of single calls;
cpu_baseline = the fp64 oracle on a bounded sample, on one thread and on
disjoint sequences in up to 16 threads.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "verify rows/s and logits GB/s (% of HBM peak), B=64 K=4 V=128256 bf16"


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("sv_kernels.hip", "sv_host.hip", "sv_internal.h"):
        with open(os.path.join(ROOT, "speculative_sampling_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"row_kernel_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4, help="rotating input sets (>= 4 defeats the MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run --steps plain device copies of BYTES bytes (HBM counter calibration)")
    ap.add_argument("--workload", default=None,
                    help="another named workload (speculative_sampling_amd.workloads.config); "
                         "default: the headline, B=64 K=4 V=128256 bf16 nucleus")
    ap.add_argument("--batch", type=int, default=None, help="B of the named workload")
    ap.add_argument("--no-draft", action="store_true",
                    help="greedy workloads: call without the draft's logits (only target rows are read)")
    ap.add_argument("--probe-sweep", action="store_true",
                    help="only sweep the read-only probe's loads per lane and waves per CU over rotating "
                         "buffers of the headline's logit bytes and of 2 GiB; one JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(rows are independent; a multi-GPU run would shard B with row_offset).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        calibrate_copy(torch, args.calibrate_copy, args.steps)
        return
    if args.probe_sweep:
        probe_sweep(torch, args.steps, args.warmup)
        return

    from speculative_sampling_amd import binding, loop_model, workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    name = args.workload or workloads.HEADLINE
    kw = {} if args.batch is None else {"B": args.batch}
    if args.batch is not None and name not in ("latency_b1", "worked_example"):
        kw = {}
        print("--batch applies to latency_b1 and worked_example only", file=sys.stderr)
    sets = []
    for r in range(args.sets):
        w = workloads.config(name, device=dev, gen_seed=1000 + r, seed=r, **kw)
        sets.append(w)
    w0 = sets[0]
    B, K, V = w0.B, w0.K_max, w0.V
    no_draft = args.no_draft
    if no_draft and (w0.mode is not None or w0.default_mode != workloads.GREEDY):
        print("--no-draft needs a greedy workload", file=sys.stderr)
        sys.exit(2)
    v = binding.Verifier(B, K, V, w0.target.dtype, 0)
    # draft tokens: one draw per draft row by the library itself (the step
    # with K = 0), from each row's own filtered distribution
    sampler = binding.Verifier(B * K, 0, V, w0.target.dtype, 0)
    for w in sets:
        md, tmp, tk, tp = w.row_params()
        toks, st = sampler.sample(w.draft, seed=w.draft_seed, mode=md, temperature=tmp, top_k=tk, top_p=tp,
                                  default_mode=w.default_mode, default_temperature=w.default_temperature,
                                  default_top_k=w.default_top_k, default_top_p=w.default_top_p)
        toks = toks.to(torch.int32)
        if w.k_per_row is not None:   # padding slots hold token 0
            pad = torch.arange(K, device=dev).unsqueeze(0) >= w.k_per_row.to(dev).unsqueeze(1)
            toks = torch.where(pad, torch.zeros_like(toks), toks)
        w.draft_tokens = toks.contiguous()
    torch.cuda.synchronize()
    sampler.close()
    alg_bytes = w0.algorithmic_bytes()
    if no_draft:   # only the target rows t <= K_b
        es = w0.target.element_size()
        kb = B * K if w0.k_per_row is None else int(w0.k_per_row.to(torch.int64).sum().item())
        alg_bytes = (kb + B) * V * es
    outs = [v.outputs(B, K) for _ in sets]
    stream = torch.cuda.current_stream(dev)
    argss = [binding.make_args(w.target, None if no_draft else w.draft, w.draft_tokens, accepted=o[0],
                               out_tokens=o[1], row_status=o[2], diag=o[3], k_per_row=w.k_per_row, mode=w.mode,
                               temperature=w.temperature, top_k=w.top_k, top_p=w.top_p,
                               default_mode=w.default_mode, default_temperature=w.default_temperature,
                               default_top_k=w.default_top_k, default_top_p=w.default_top_p, seed=w.seed)
             for w, o in zip(sets, outs)]

    def step(i):
        binding.spec_verify_run(v.handle, argss[i % len(argss)], stream.cuda_stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: torch events on the launch stream bracket the K calls
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    rows_per_s = B / (ms_per_step * 1e-3)
    gbs_step = alg_bytes / (ms_per_step * 1e-3) / 1e9

    # the same K calls again with the library's stage events (HIP events it
    # attaches to the start and end of each stage's kernel dispatches on the
    # launch stream); kept apart from the timed region above
    binding.spec_verify_profile_begin(v.handle, args.steps)
    for i in range(args.steps):
        step(i)
    runs, (stage0_ms, stage1_ms) = binding.spec_verify_profile_end(v.handle)
    stream_ms = stage0_ms / runs        # the row kernel: streaming pass and each row's finish
    seq_ms = stage1_ms / runs           # per-sequence accept walk and draw
    achieved = alg_bytes / (stream_ms * 1e-3) / 1e9

    # per-call spread: each call bracketed by its own pair of events
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(pairs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    per_call = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
    pct = lambda f: per_call[min(len(per_call) - 1, int(f * len(per_call)))]

    # streaming ceiling: the library's read-only probe over the same rotating
    # logits (same access pattern as the streaming pass, no arithmetic)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    probe_tensors = lambda w: (w.target,) if no_draft else (w.target, w.draft)
    probe_bytes = sum(x.numel() * x.element_size() for w in sets for x in probe_tensors(w)) / len(sets)

    def probe(i):
        w = sets[i % len(sets)]
        for x in probe_tensors(w):
            binding.spec_verify_stream_probe(x.data_ptr(), x.numel() * x.element_size(), sink.data_ptr(),
                                             stream.cuda_stream)

    for i in range(args.warmup):
        probe(i)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        probe(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ceiling = probe_bytes / (t0.elapsed_time(t1) / args.steps * 1e-3) / 1e9

    # acceptance actually achieved by the synthetic draft (context), and the
    # loop model: one round at the pages' model-call times (target 14.1 ms,
    # draft 1.8 ms per token) with this verify step's measured time added
    acc = torch.cat([o[0] for o in outs])
    alpha_tokens = float(acc.float().mean().item())
    mon = loop_model.AcceptanceMonitor(K)
    mon.update(acc.cpu().numpy())
    alphas = mon.alpha()
    t_verify_ms = ms_per_step
    loop = {"alpha_per_position": [round(float(a), 4) for a in alphas],
            "tokens_per_round": mon.tokens_per_round(),
            "predicted_tokens_per_round": mon.predicted_tokens_per_round(),
            "t_target_ms": 14.1, "t_draft_ms": 1.8, "t_verify_ms": t_verify_ms,
            "ms_per_token": loop_model.ms_per_token(alphas, K, 14.1, 1.8, t_verify_ms),
            "ms_per_token_without_verify": loop_model.ms_per_token(alphas, K, 14.1, 1.8),
            "verify_share_of_round": t_verify_ms / loop_model.round_ms(K, 14.1, 1.8, t_verify_ms)}

    cpu = cpu_all = None
    if not args.no_cpu:
        cpu = cpu_baseline(sets[0], args.cpu_seconds)
        cpu_all = cpu_baseline(sets[0], args.cpu_seconds, threads=min(16, os.cpu_count() or 1))

    traffic = stored_traffic(name)
    line = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # bf16 logits decoded exactly to fp32; fp32 terms, fp64 sums
        "data": "synthetic",
        "config": workload_config(w0, name, len(sets), no_draft),
        "logits_GBps": gbs_step,
        "pct_hbm_peak": 100.0 * gbs_step / HBM_PEAK_GBS,
        "stage_ms": {"stream": stream_ms, "sequence": seq_ms},
        "per_call_us": {"p10": pct(0.1), "median": pct(0.5), "p90": pct(0.9),
                        "note": "each call bracketed by its own events"},
        "streaming_ceiling": {"GBps": ceiling, "kernel": "stream_probe_kernel",
                              "pct_hbm_peak": 100.0 * ceiling / HBM_PEAK_GBS,
                              "row_kernel_frac_of_ceiling": achieved / ceiling,
                              "value_frac_of_ceiling": gbs_step / ceiling},
        "mean_accepted": alpha_tokens,
        "loop_model": loop,
        "roofline": {"bound": "hbm", "kernel": "row_kernel", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg_bytes},
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
    }
    v.close()
    print(json.dumps(line), flush=True)


def workload_config(w, name, nsets, no_draft):
    modes = {0: "plain", 1: "top-k", 2: "top-p", 3: "greedy"}
    c = {"workload": name, "B": w.B, "K": w.K_max, "V": w.V, "dtype": w.dtype,
         "mode": "per-sequence" if w.mode is not None else modes[w.default_mode]}
    if w.mode is None and w.default_mode == 2:
        c["top_p"] = w.default_top_p
    if w.mode is None and w.default_mode == 1:
        c["top_k"] = w.default_top_k
    if w.mode is not None or w.default_mode != 3:
        c["temperature"] = w.default_temperature
    if w.k_per_row is not None:
        c["k_per_row"] = "ragged"
    if no_draft:
        c["draft_logits"] = "none"
    c.update({"input_sets": nsets, "parallelism": "single-gpu"})
    return c


def calibrate_copy(torch, nbytes, steps):
    """A plain device-to-device copy of known size: its FETCH_SIZE and
    WRITE_SIZE counters give the scale factors from counter units to bytes."""
    dev = torch.device("cuda", 0)
    src = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1) for _ in range(4)]
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    for i in range(steps):
        torch.add(src[i % 4], 1, out=dst)  # one elementwise kernel: reads and writes nbytes
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
                      "launches": steps}), flush=True)


def probe_sweep(torch, steps, warmup):
    """Read rate of the persistent read-only probe for 4, 8 and 16 loads per
    lane and 1 to 32 waves per CU, over rotating buffers (4 of the
    headline's 147,750,912 logit bytes per call, 2 of 2 GiB), next to the
    fixed probe (one wave per 8 KB block).  Each point: warmup untimed
    launches, then steps launches between two events."""
    from speculative_sampling_amd import binding

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    sizes = [(147750912, 4), (2 << 30, 2)]
    out = {"probe_sweep": [], "steps": steps, "warmup": warmup}
    for nbytes, nbuf in sizes:
        bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev) for _ in range(nbuf)]

        def rate(launch):
            for i in range(warmup):
                launch(bufs[i % nbuf])
            torch.cuda.synchronize()
            t0.record(stream)
            for i in range(steps):
                launch(bufs[i % nbuf])
            t1.record(stream)
            torch.cuda.synchronize()
            return nbytes / (t0.elapsed_time(t1) / steps * 1e-3) / 1e9

        fixed = rate(lambda b: binding.spec_verify_stream_probe(b.data_ptr(), nbytes, sink.data_ptr(),
                                                                stream.cuda_stream))
        points = []
        for loads in (4, 8, 16):
            for waves in (1, 2, 4, 8, 12, 16, 24, 32):
                g = rate(lambda b: binding.spec_verify_stream_probe_sweep(b.data_ptr(), nbytes, loads, waves,
                                                                          sink.data_ptr(), stream.cuda_stream))
                points.append({"loads_per_lane": loads, "waves_per_cu": waves, "GBps": round(g, 1)})
                print(f"# bytes={nbytes} loads={loads} waves={waves}: {g:.1f} GB/s", file=sys.stderr, flush=True)
        best = max(points, key=lambda q: q["GBps"])
        out["probe_sweep"].append({"bytes_per_launch": nbytes, "buffers": nbuf,
                                   "fixed_probe_GBps": round(fixed, 1), "best": best,
                                   "best_pct_hbm_peak": 100.0 * best["GBps"] / HBM_PEAK_GBS, "points": points})
        del bufs
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def cpu_baseline(w, budget_s, threads=1):
    """The oracle, as it stands, on whole sequences of the same workload until
    the time budget is spent; reported in rows/s (sequences per second).
    With threads > 1 the same single-threaded oracle runs on disjoint
    sequences in that many threads (its calls release the GIL)."""
    import threading
    import oracle
    from speculative_sampling_amd import workloads

    tgt = workloads.host_array(w.target)
    drf = workloads.host_array(w.draft)
    toks = w.draft_tokens.cpu().numpy()
    lock = threading.Lock()
    state = {"next": 0, "done": 0}
    t0 = time.perf_counter()

    def worker():
        while True:
            with lock:
                b = state["next"]
                if b >= w.B or time.perf_counter() - t0 >= budget_s:
                    return
                state["next"] = b + 1
            oracle.verify(tgt[b:b + 1], drf[b:b + 1], toks[b:b + 1],
                          default_mode=w.default_mode, default_temperature=w.default_temperature,
                          default_top_p=w.default_top_p, seed=w.seed, row_offset=b)
            with lock:
                state["done"] += 1

    pool = [threading.Thread(target=worker) for _ in range(threads)]
    for t in pool:
        t.start()
    for t in pool:
        t.join()
    el = time.perf_counter() - t0
    done = state["done"]
    kind = "single-threaded fp64" if threads == 1 else f"fp64 oracle on disjoint sequences, {threads} threads"
    return {"value": done / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {w.B} sequences of input set 0 ({el:.1f} s, {kind})",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
