"""Benchmark: absorbed-MLA paged decode on the DeepSeek-V3-shaped workload.

Workload: B=128 requests, H=128 heads, latent 512 + rope 64 in bf16, page size
64 with kv_last_page_len, lengths lognormal (median 2048, sigma 0.8, clipped
to [16, 16384]), pages scattered over the pool (seeded, workloads.v3).

One step = one attention-layer call of the hot path: mla_decode (the decode
kernel plus the merge of split-KV partials). The host plan is built once per
batch and reused by every layer, so it is built before the timed region and
reported separately (plan_us). Two identical copies of the inputs (different
device addresses, about 1.2 GB together) alternate between steps so that the
256 MB Infinity Cache cannot serve one step's latent reads from the previous
step.

value = latent-cache GB/s = (sum of KV tokens x 1152 bytes) / step time;
also reported: decode tokens/s (query rows / step time) and the fraction of
MI355X's 8 TB/s HBM peak. The CPU oracle is timed on the host's cores on a
bounded prefix of the same batch (cpu_baseline).

With --workload projections it instead times the two per-head projections of
weight absorption at the same decode shape (128 query rows, 128 heads):
mla_absorb_query (W_UK into the query) then mla_project_output (W_UV on the
latent output), cycling over 8 distinct weight and activation sets (about 600
MB) so that no step is served from the Infinity Cache. value = their
algorithmic bytes (weights, inputs and outputs, each once) / step time.

With --workload tree_verify it times the tree-verify cascade of the PR 49477
analysis (16 requests, 2048-token prefix, 64 drafts at depth <= 8, H=128):
the suffix-table compaction, then every draft row's attention over its prefix
and its visible drafts in one pass (mla_decode_tree_verify). The two-pass
cascade (prefix decode, suffix decode, LSE merge) is timed beside it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from paged_mla_decode_amd import costs  # noqa: E402  (host arithmetic only)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha256():
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "paged_mla_decode_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def copy_bandwidth_gbs(torch, dev, mib=1024, reps=5):
    """Device-to-device copy rate of this machine (bytes read + written per second,
    median of `reps`): the second reference the measured rate is stated against."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    del src, dst
    return 2.0 * (mib << 20) / float(np.median(times)) / 1e9


def measured_traffic(summary, key="traffic_bytes_per_launch"):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    profiles/<summary>_counters.md, or None when there is none or the kernels
    changed since."""
    path = os.path.join(ROOT, "profiles", f"{summary}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in (key, "kernel_source_sha256"):
                k, v = line.split(":", 1)
                fields[k] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    if key not in fields:
        return None
    v = float(fields[key])
    return int(v) if v.is_integer() else v


def warm_until_steady(torch, stream, step, min_steps, min_s=1.5, max_s=5.0, batch=25):
    """Warm the GPU to steady clocks before a timed region, whatever --warmup
    asks: run `min_steps` steps, then batches of `batch` steps until at least
    `min_s` seconds have passed and two consecutive batches agree within 1%
    (at most `max_s` seconds). Returns (seconds, steps run)."""
    t0 = time.perf_counter()
    done = 0
    for _ in range(min_steps):
        step(done)
        done += 1
    torch.cuda.synchronize()
    if min_s <= 0:
        return time.perf_counter() - t0, done
    prev = None
    while True:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(batch):
            step(done)
            done += 1
        e1.record(stream)
        torch.cuda.synchronize()
        cur = e0.elapsed_time(e1)
        el = time.perf_counter() - t0
        steady = prev is not None and abs(cur - prev) <= 0.01 * prev
        if el >= max_s or (el >= min_s and steady):
            return el, done
        prev = cur


def median_plan_us(plan, reps=21):
    """Host plan time: the median of `reps` calls after a warm one (the plan is
    built once per batch and reused by every layer)."""
    plan()
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        plan()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)) * 1e6


def _timed_runs(fn, runs=3):
    """One untimed warm-up call, then `runs` timed calls; the median seconds."""
    fn()
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times))


def _sized_subset(batch, seconds):
    """The first requests of `batch` whose oracle run takes about `seconds`
    with the oracle's current thread count (calibrated on two requests)."""
    import oracle

    cal = batch.subset(range(min(2, batch.batch)))
    t0 = time.perf_counter()
    oracle.decode_batch(cal)
    dt = time.perf_counter() - t0
    rate = float(cal.seq_lens.sum()) / max(dt, 1e-9)  # tokens/s
    cum = np.cumsum(batch.seq_lens.astype(np.int64))
    n = int(min(batch.batch, max(1, np.searchsorted(cum, rate * seconds) + 1)))
    return batch.subset(range(n)), n


def cpu_baseline(batch, run_s=3.0, one_core_s=2.0):
    """The oracle's GB/s on a bounded prefix of the batch, on every host core:
    one warm-up and three timed runs of the same prefix, the median reported.
    The same protocol on one core for the tiny and the V2-Lite configurations."""
    import oracle
    import workloads

    oracle.set_num_threads(0)
    sub, n = _sized_subset(batch, run_s)
    dt = _timed_runs(lambda: oracle.decode_batch(sub))
    toks = int(sub.seq_lens.sum())
    res = {
        "value": toks * batch.cache_bytes_per_token / dt / 1e9,
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"first {n} of {batch.batch} requests ({toks} KV tokens, all {batch.num_heads} heads), "
                  f"fp64 C oracle, median of 3 runs after 1 warm-up, {dt:.2f} s per run",
        "tokens_per_s": sub.num_rows / dt,
    }
    one = {}
    oracle.set_num_threads(1)
    try:
        for name, make in (("tiny", workloads.tiny), ("v2_lite", workloads.v2_lite)):
            b = make()
            s1, n1 = _sized_subset(b, one_core_s)
            d1 = _timed_runs(lambda: oracle.decode_batch(s1))
            t1 = int(s1.seq_lens.sum())
            one[name] = {"value": t1 * b.cache_bytes_per_token / d1 / 1e9, "unit": "GB/s", "cores": 1,
                         "tokens_per_s": s1.num_rows / d1,
                         "sample": f"first {n1} of {b.batch} requests ({t1} KV tokens, all "
                                   f"{b.num_heads} heads), median of 3 runs after 1 warm-up, "
                                   f"{d1:.3f} s per run"}
    finally:
        oracle.set_num_threads(0)
    res["one_core"] = one
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warmup-seconds", type=float, default=1.5,
                    help="after --warmup steps, keep warming until this many seconds have passed and "
                         "two 25-step batches agree within 1%% (0: --warmup steps only, e.g. under a "
                         "profiler)")
    ap.add_argument("--workload", default="v3",
                    choices=["v3", "v2_lite", "skewed_fp8", "projections", "tree_verify"])
    ap.add_argument("--append", action="store_true",
                    help="decode workloads: time mla_decode_append (each request's new token "
                         "written into its cache row in the same launch) instead of mla_decode")
    ap.add_argument("--fp8-score", action="store_true",
                    help="skewed_fp8: the score on the fp8 matrix core with an e4m3fn-quantised "
                         "query (MLA_DECODE_FP8_SCORE)")
    ap.add_argument("--rows-per-request", type=int, default=1,
                    help="v2_lite: this many query rows per request over the same tokens (multi-token "
                         "prediction, speculative decoding), planned with MLA_DECODE_SHARED_ROWS")
    ap.add_argument("--compare-per-row", action="store_true",
                    help="with --rows-per-request: also time the batch with one work item per query row "
                         "(one_item_per_row in the JSON)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (a known-size "
                         "reference for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share: --gpus {args.gpus} is not supported "
              "(the library runs on a single MI355X; sharding is described, not built).",
              file=sys.stderr)
        sys.exit(2)

    if args.fp8_score and (args.workload != "skewed_fp8" or args.append):
        print("--fp8-score applies to the skewed_fp8 workload's mla_decode only", file=sys.stderr)
        sys.exit(2)
    if args.rows_per_request < 1 or (args.rows_per_request > 1 and
                                     (args.workload != "v2_lite" or args.append or args.fp8_score)):
        print("--rows-per-request applies to the v2_lite workload's mla_decode only", file=sys.stderr)
        sys.exit(2)
    if args.workload == "projections":
        return bench_projections(args)
    if args.workload == "tree_verify":
        return bench_tree_verify(args)

    import torch

    import workloads
    from paged_mla_decode_amd.decoder import PagedMlaDecoder

    dev = torch.device("cuda:0")
    make = {"v3": workloads.v3, "v2_lite": workloads.v2_lite, "skewed_fp8": workloads.skewed_fp8}
    t0 = time.perf_counter()
    R = args.rows_per_request
    batch = make[args.workload]() if R == 1 else workloads.v2_lite(rows_per_request=R)
    qo = None if R == 1 else batch.qo_indptr
    log(f"workload {batch.name}: B={batch.batch} H={batch.num_heads} ps={batch.page_size} "
        f"tokens={int(batch.seq_lens.sum())} gen {time.perf_counter() - t0:.1f}s")

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    qn = to_dev_bf16(batch.q_nope)
    qr = to_dev_bf16(batch.q_rope)
    if batch.cache_dtype == "bf16":
        cache = to_dev_bf16(batch.cache)
    else:
        cache = torch.from_numpy(np.ascontiguousarray(batch.cache)).to(dev)
    idx = torch.from_numpy(batch.kv_indices).to(dev)
    sets = [(qn, qr, cache, idx), (qn.clone(), qr.clone(), cache.clone(), idx.clone())]

    dec = PagedMlaDecoder(batch.num_heads, batch.page_size, max_batch=batch.batch,
                          max_rows=batch.num_rows, kv_dtype=batch.cache_dtype, out_dtype="bf16",
                          device=dev, fp8_score=args.fp8_score, shared_rows=R > 1)
    h = dec.plan(batch.kv_indptr, batch.kv_last_page_len, qo)
    plan_us = median_plan_us(lambda: dec.plan(batch.kv_indptr, batch.kv_last_page_len, qo))
    torch.cuda.synchronize()
    outs = [torch.empty((batch.num_rows, batch.num_heads, 512), dtype=torch.bfloat16, device=dev)
            for _ in sets]
    lses = [torch.empty((batch.num_rows, batch.num_heads), dtype=torch.float32, device=dev)
            for _ in sets]

    stream = torch.cuda.current_stream(dev)
    if args.append:
        # The new tokens (one per request), drawn like every other input.
        rng = np.random.Generator(np.random.PCG64(batch.seed + 1000))
        c_new = to_dev_bf16(workloads.f32_to_bf16_bits(
            rng.standard_normal((batch.num_rows, 512), dtype=np.float32) * np.float32(0.5)))
        k_pe_new = to_dev_bf16(workloads.f32_to_bf16_bits(
            rng.standard_normal((batch.num_rows, 64), dtype=np.float32) * np.float32(0.5)))

    def step(i, ev=None):
        s = sets[i % 2]
        if ev is not None:
            ev[0].record(stream)
        if args.append:
            dec.run_append(s[0], s[1], s[2], s[3], c_new, k_pe_new, batch.sm_scale, batch.kv_scale,
                           out=outs[i % 2], lse=lses[i % 2], stream=stream)
        else:
            dec.run(s[0], s[1], s[2], s[3], batch.sm_scale, batch.kv_scale, out=outs[i % 2],
                    lse=lses[i % 2], stream=stream)
        if ev is not None:
            ev[1].record(stream)

    if args.copy_mb:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    warm_s, warm_steps = warm_until_steady(torch, stream, step, args.warmup, min_s=args.warmup_seconds)
    # The timed region: K calls back to back, with no event between them (an
    # event record is a packet of its own in the stream), bracketed by
    # synchronisations; two events on the stream give its GPU time.
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record(stream)
    for i in range(args.steps):
        step(i)
    g1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gpu_step_us = g0.elapsed_time(g1) * 1e3 / args.steps
    # Then the same K calls again, each between two events of its own, for the
    # per-call times (average, p10/p50/p90) of the roofline.
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in events])

    profile_key = (f"mla_decode_{args.workload}" + ("_fp8_score" if args.fp8_score else "") +
                   (f"_rows{R}" if R > 1 else ""))
    tokens = int(batch.seq_lens.sum())
    latent_bytes = costs.mla_decode_latent_bytes(tokens, 1 if batch.cache_dtype != "bf16" else 2)
    assert latent_bytes == tokens * batch.cache_bytes_per_token
    # Every query row attends to all of its request's tokens.
    flops = float(costs.mla_decode_flops(tokens, batch.num_heads)) * R
    per_row = None
    if R > 1 and args.compare_per_row:
        # The same batch with one work item per query row, for comparison.
        dec1 = PagedMlaDecoder(batch.num_heads, batch.page_size, max_batch=batch.batch,
                               max_rows=batch.num_rows, device=dev)
        h1 = dec1.plan(batch.kv_indptr, batch.kv_last_page_len, qo)

        def step1(i, ev=None):
            s = sets[i % 2]
            dec1.run(s[0], s[1], s[2], s[3], batch.sm_scale, batch.kv_scale, out=outs[i % 2],
                     lse=lses[i % 2], stream=stream)

        warm_until_steady(torch, stream, step1, args.warmup, min_s=args.warmup_seconds)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            step1(i)
        e1.record(stream)
        torch.cuda.synchronize()
        per_row = {"us_per_call": round(e0.elapsed_time(e1) * 1e3 / args.steps, 2),
                   "items": h1.num_items, "merges": h1.num_merges}
        log(f"one item per row: {per_row['us_per_call']:.1f} us per call ({h1.num_items} items)")
    ms_per_step = elapsed * 1e3 / args.steps
    gbs = latent_bytes / (ms_per_step * 1e-3) / 1e9
    launch_avg_ms = float(launch_ms.mean())
    achieved = latent_bytes / (launch_avg_ms * 1e-3) / 1e9
    log(f"plan: workers={h.num_workers} items={h.num_items} merges={h.num_merges} "
        f"partials={h.num_partials} capacity={h.chunk_tokens} plan_us={plan_us:.0f}")
    log(f"step {ms_per_step * 1e3:.1f} us, launch avg {launch_avg_ms * 1e3:.1f} us "
        f"(p10 {np.percentile(launch_ms, 10) * 1e3:.1f}, p90 {np.percentile(launch_ms, 90) * 1e3:.1f}), "
        f"{gbs:.0f} GB/s, {achieved / HBM_PEAK_GBS * 100:.1f}% HBM, "
        f"{flops / (launch_avg_ms * 1e-3) / 1e12:.0f} TFLOP/s")

    res = {
        "metric": "MLA decode latent-cache GB/s (% of HBM peak) and tokens/s, DeepSeek-V3 shapes",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if batch.cache_dtype == "bf16" else
                 ("fp8_e4m3fn cache, fp8 score mfma, bf16 product mfma" if args.fp8_score
                  else "fp8_e4m3fn cache, bf16 mfma"),
        "data": "synthetic",
        "config": {
            "workload": f"{batch.name}: B={batch.batch} H={batch.num_heads} latent 512+64 "
                        f"page_size={batch.page_size} seed={batch.seed}",
            "batch": batch.batch, "num_heads": batch.num_heads, "kv_lora_rank": 512,
            "qk_rope_head_dim": 64, "page_size": batch.page_size, "kv_tokens": tokens,
            "query_rows": batch.num_rows, "parallelism": "single GPU",
            "fused_append": bool(args.append), "fp8_score": bool(args.fp8_score),
            "rows_per_request": R, "shared_rows": R > 1,
        },
        "tokens_per_s": round(batch.num_rows / (ms_per_step * 1e-3), 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "warmup_run": {"steps": warm_steps, "seconds": round(warm_s, 2),
                       "rule": "at least --warmup steps, then until two 25-step batches agree "
                               "within 1% after >= 1.5 s (at most 5 s)"},
        "plan_us": round(plan_us, 1),
        "plan_us_note": "host plan + its copy to the device, median of 21 calls after a warm call",
        "plan": {"workers": h.num_workers, "items": h.num_items, "merges": h.num_merges,
                 "partials": h.num_partials, "capacity_tokens": h.chunk_tokens},
        "roofline": {
            "kernel": ("mla_decode_append" if args.append else "mla_decode") +
                      (" launch (query quantisation + decode kernel + split-KV merge kernel)"
                       if args.fp8_score else " launch (decode kernel + split-KV merge kernel)"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if args.append else measured_traffic(profile_key),
            "algorithmic_bytes_per_launch": latent_bytes,
            "launch_avg_us": round(launch_avg_ms * 1e3, 2),
            "mfma_tflops": round(flops / (launch_avg_ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (launch_avg_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
        },
    }
    copy_gbs = copy_bandwidth_gbs(torch, dev)
    res["copy_gbs"] = round(copy_gbs, 1)
    res["frac_of_copy_bandwidth"] = round(achieved / copy_gbs, 4)
    res["launch_us_p10_p50_p90"] = [round(float(np.percentile(launch_ms, q)) * 1e3, 2) for q in (10, 50, 90)]
    res["gpu_us_per_step"] = round(gpu_step_us, 2)
    if per_row is not None:
        res["one_item_per_row"] = per_row
    mfma = None if args.append else measured_traffic(profile_key, "mfma_util_percent_decode")
    res["roofline"]["mfma_busy_counter"] = None if mfma is None else round(mfma / 100.0, 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline(batch)
    print(json.dumps(res), flush=True)


def cpu_baseline_projections(p, run_s=3.0):
    """Oracle absorb + project GB/s: one warm-up and three timed runs, each
    repeating the full shape for about run_s, the median reported."""
    import oracle
    import threadpoolctl
    import workloads

    f = workloads.bf16_bits_to_f32
    q, w_uk, w_uv, x = (f(a).astype(np.float64) for a in (p.q, p.w_uk, p.w_uv, p.x))
    N, H, D = q.shape
    nbytes = costs.absorb_bytes(N, H, D) + costs.project_bytes(N, H, D)

    def once():
        oracle.absorb_query(q, w_uk)
        oracle.project_output(x, w_uv)

    t0 = time.perf_counter()
    once()
    reps = max(1, int(run_s / max(time.perf_counter() - t0, 1e-6)))

    def run():
        for _ in range(reps):
            once()

    dt = _timed_runs(run)
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    return {"value": reps * nbytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} repetitions of the full shape (N={N}, H={H}) per run, fp64 numpy "
                      f"per-head products, median of 3 runs after 1 warm-up, {dt:.2f} s per run"}


def bench_projections(args):
    import torch

    import workloads
    from paged_mla_decode_amd import absorb_query, project_output

    dev = torch.device("cuda:0")
    N, H, D, A, SETS = 128, 128, 128, 512, 8
    p = workloads.projection_inputs(3, N, H, D)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    base = {"q": to_dev(p.q), "w_uk": to_dev(p.w_uk), "x": to_dev(p.x),
            # W_UV with the latent contiguous, as kv_b_proj stores it: [H, D, A], viewed (a, h, d)
            "w_uv_t": to_dev(np.ascontiguousarray(p.w_uv.transpose(1, 2, 0)))}
    sets = []
    for i in range(SETS):
        s = {k: (v if i == 0 else v.clone()) for k, v in base.items()}
        s["q_abs"] = torch.empty((N, H, A), dtype=torch.bfloat16, device=dev)
        s["o"] = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)
        sets.append(s)
    stream = torch.cuda.current_stream(dev)

    def absorb(i):
        s = sets[i % SETS]
        absorb_query(s["q"], s["w_uk"], out=s["q_abs"], stream=stream)

    def project(i):
        s = sets[i % SETS]
        project_output(s["x"], s["w_uv_t"].permute(2, 0, 1), out=s["o"], stream=stream)

    def step(i):
        absorb(i)
        project(i)

    if args.copy_mb:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    warm_s, warm_steps = warm_until_steady(torch, stream, step, args.warmup, min_s=args.warmup_seconds)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Per-kernel launch duration: the two kernels are a few microseconds each, so
    # events between them would cost as much as they measure. Each is timed
    # instead over `steps` back-to-back launches on the same rotating sets, with
    # one pair of HIP events on the launch stream around them.
    def launch_avg_us(fn):
        # A few untimed calls first: the first launch of a kernel the step does
        # not use loads its code.
        for i in range(10):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    absorb_us = launch_avg_us(absorb)
    project_us = launch_avg_us(project)

    # Algorithmic bytes, each tensor once: weight + input + output of each projection.
    absorb_bytes = costs.absorb_bytes(N, H, D, A)
    project_bytes = costs.project_bytes(N, H, D, A)
    step_bytes = absorb_bytes + project_bytes
    ms_per_step = elapsed * 1e3 / args.steps
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    kern = {"absorb": (absorb_us, absorb_bytes, "head_gemm_kernel<64, 1> (mla_absorb_query)"),
            "project": (project_us, project_bytes, "head_gemm_kernel<64, 4> (mla_project_output)")}
    dom = max(kern, key=lambda k: kern[k][0])
    us, nbytes, kname = kern[dom]
    achieved = nbytes / (us * 1e-6) / 1e9
    log(f"step {ms_per_step * 1e3:.2f} us; absorb {absorb_us:.2f} us "
        f"({absorb_bytes / absorb_us / 1e3:.0f} GB/s), project {project_us:.2f} us "
        f"({project_bytes / project_us / 1e3:.0f} GB/s)")
    res = {
        "metric": "W_UK absorption + W_UV projection GB/s (% of HBM peak), DeepSeek-V3 decode shape",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"projections: N={N} query rows, H={H} heads, head_dim {D}, latent {A}, "
                               f"bf16, {SETS} rotating weight sets, seed 3",
                   "query_rows": N, "num_heads": H, "head_dim": D, "kv_lora_rank": A,
                   "parallelism": "single GPU"},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "warmup_run": {"steps": warm_steps, "seconds": round(warm_s, 2)},
        "kernels_us": {"absorb": round(absorb_us, 2), "project": round(project_us, 2)},
        "roofline": {
            "kernel": kname,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("mla_projections_v3", f"traffic_bytes_per_launch_{dom}"),
            "algorithmic_bytes_per_launch": nbytes,
            "launch_avg_us": round(us, 2),
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline_projections(p)
    print(json.dumps(res), flush=True)


def cpu_baseline_tree(tv, run_s=4.0):
    """Oracle latent GB/s on the first rows of the cascade (each row's attention
    over its prefix and its visible drafts): one warm-up and three timed runs
    of a prefix of rows sized to about run_s each, the median reported."""
    import oracle

    pre, W = tv.prefix, tv.width

    def rows_args(rows):
        kv_indptr, kv_indices = [0], []
        for r in rows:
            req, plen = r // W, int(tv.prefix_lens[r // W])
            vis = np.nonzero(tv.tree_mask[r])[0]
            slots = np.concatenate([tv.req_to_token[req, :plen], tv.req_to_token[req, plen + vis]])
            kv_indices.append(slots)
            kv_indptr.append(kv_indptr[-1] + len(slots))
        return (np.asarray(kv_indptr, np.int32), np.concatenate(kv_indices).astype(np.int32))

    def run(rows, indptr, indices):
        oracle.mla_decode(pre.q_nope[rows], pre.q_rope[rows], pre.cache, indptr, indices, 1,
                          pre.sm_scale, kv_last_page_len=np.ones(len(rows), np.int32))

    oracle.set_num_threads(0)
    cal = list(range(2))
    a = rows_args(cal)
    t0 = time.perf_counter()
    run(cal, *a)
    dt = time.perf_counter() - t0
    n = int(min(pre.num_rows, max(2, 2 * run_s / max(dt, 1e-6))))
    rows = list(range(n))
    a = rows_args(rows)
    dt = _timed_runs(lambda: run(rows, *a))
    toks = int(a[0][-1])
    return {"value": toks * 1152 / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {n} of {pre.num_rows} draft rows (prefix + visible drafts, all 128 heads), "
                      f"fp64 C oracle, median of 3 runs after 1 warm-up, {dt:.2f} s per run"}


def bench_tree_verify(args):
    import torch

    import workloads
    from paged_mla_decode_amd.decoder import PagedMlaDecoder, merge_states, tree_suffix_compact

    dev = torch.device("cuda:0")
    tv = workloads.tree_verify()
    pre, W, D = tv.prefix, tv.width, tv.max_tree_depth
    B, N, H = pre.batch, pre.num_rows, pre.num_heads

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    base = {"qn": to_dev_bf16(pre.q_nope), "qr": to_dev_bf16(pre.q_rope), "cache": to_dev_bf16(pre.cache),
            "idx": torch.from_numpy(pre.kv_indices).to(dev), "mask": torch.from_numpy(tv.tree_mask).to(dev),
            "r2t": torch.from_numpy(tv.req_to_token).to(dev), "plen": torch.from_numpy(tv.prefix_lens).to(dev)}
    # Two input sets alternate so that one step's reads are not served from the
    # previous step's Infinity Cache lines.
    sets = [base, {k: v.clone() for k, v in base.items()}]
    dp = PagedMlaDecoder(H, 1, max_batch=B, max_rows=N, device=dev)
    t0 = time.perf_counter()
    hp = dp.plan(pre.kv_indptr, pre.kv_last_page_len, pre.qo_indptr)
    ds = PagedMlaDecoder(H, 1, max_batch=N, max_rows=N, device=dev)
    hs = ds.plan(np.arange(N + 1, dtype=np.int32) * D, np.ones(N, dtype=np.int32))
    plan_us = (time.perf_counter() - t0) * 1e6
    # Single pass: every row over its prefix and then its visible drafts.
    d1 = PagedMlaDecoder(H, 1, max_batch=B, max_rows=N, device=dev, suffix_tokens=D)
    h1 = d1.plan(pre.kv_indptr, pre.kv_last_page_len, pre.qo_indptr)
    plan1_us = median_plan_us(lambda: d1.plan(pre.kv_indptr, pre.kv_last_page_len, pre.qo_indptr))
    outs = [(torch.empty((N, H, 512), dtype=torch.bfloat16, device=dev),
             torch.empty((N, H), dtype=torch.float32, device=dev)) for _ in sets]
    tables = [tree_suffix_compact(s["mask"], s["r2t"], s["plen"], W) for s in sets]
    stream = torch.cuda.current_stream(dev)

    def compact(i):
        s = sets[i % 2]
        return tree_suffix_compact(s["mask"], s["r2t"], s["plen"], W, stream=stream)

    def prefix(i):
        s, (o, l) = sets[i % 2], outs[i % 2]
        dp.run(s["qn"], s["qr"], s["cache"], s["idx"], pre.sm_scale, out=o, lse=l, stream=stream)

    def suffix_separate(i, table_seqlens):
        s, (o, l) = sets[i % 2], outs[i % 2]
        table, seqlens = table_seqlens
        so, sl = ds.run(s["qn"], s["qr"], s["cache"], table[:, :D].contiguous().view(-1),
                        pre.sm_scale, kv_lens=seqlens, stream=stream)
        merge_states(o, l, so, sl, out=o, s_out=l, stream=stream)

    def single(i, table_seqlens):
        s, (o, l) = sets[i % 2], outs[i % 2]
        table, seqlens = table_seqlens
        d1.run_tree_verify(s["qn"], s["qr"], s["cache"], s["idx"], table, seqlens, pre.sm_scale,
                           out=o, lse=l, stream=stream)

    # The step: compaction, then one pass over prefix and visible drafts. The
    # two-pass cascade (prefix, then suffix and merge) is timed too.
    def step(i):
        single(i, compact(i))

    if args.copy_mb:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    warm_s, warm_steps = warm_until_steady(torch, stream, step, args.warmup, min_s=args.warmup_seconds)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    def launch_avg_us(fn):
        # A few untimed calls first: the first launch of a kernel the step does
        # not use loads its code.
        for i in range(10):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    compact_us = launch_avg_us(compact)
    prefix_us = launch_avg_us(prefix)
    separate_us = launch_avg_us(lambda i: suffix_separate(i, tables[i % 2]))
    single_us = launch_avg_us(lambda i: single(i, tables[i % 2]))

    seq = tables[0][1].cpu().numpy()
    prefix_tokens = int(pre.seq_lens.astype(np.int64).repeat(W).sum())
    attended = prefix_tokens + int(seq.sum())
    latent_bytes = costs.mla_decode_latent_bytes(attended, 2)
    unique_bytes = costs.mla_decode_latent_bytes(int(pre.seq_lens.sum()) + B * W, 2)
    ms_per_step = elapsed * 1e3 / args.steps
    gbs = latent_bytes / (ms_per_step * 1e-3) / 1e9
    prefix_flops = costs.mla_decode_flops(prefix_tokens, H)
    tflops = prefix_flops / (prefix_us * 1e-6) / 1e12
    single_flops = costs.mla_decode_flops(attended, H)
    single_tflops = single_flops / (single_us * 1e-6) / 1e12
    log(f"step {ms_per_step * 1e3:.1f} us: compaction {compact_us:.1f}, single pass {single_us:.1f} "
        f"({single_tflops:.0f} TFLOP/s); two-pass cascade: prefix {prefix_us:.1f} ({tflops:.0f} "
        f"TFLOP/s), suffix + merge_states {separate_us:.1f}; plans: single "
        f"{h1.num_items} items, prefix {hp.num_items}, suffix {hs.num_items}")
    res = {
        "metric": "MLA decode latent-cache GB/s (% of HBM peak) and tokens/s, DeepSeek-V3 shapes",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"tree_verify: B={B} prefix={int(pre.seq_lens[0])} W={W} depth<={D} "
                               f"H={H} page_size=1 seed={pre.seed}",
                   "batch": B, "draft_rows": N, "num_heads": H, "kv_tokens_attended": attended,
                   "unique_kv_tokens": int(pre.seq_lens.sum()) + B * W, "parallelism": "single GPU"},
        "tokens_per_s": round(N / (ms_per_step * 1e-3), 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "unique_latent_bytes": unique_bytes,
        "warmup_run": {"steps": warm_steps, "seconds": round(warm_s, 2)},
        "plan_us": round(plan1_us, 1),
        "phases_us": {"compaction": round(compact_us, 2), "single_pass": round(single_us, 2),
                      "two_pass_prefix": round(prefix_us, 2),
                      "two_pass_suffix_then_merge_states": round(separate_us, 2)},
        "roofline": {
            "kernel": "mla_decode_tree_verify launch (1024 draft rows x (2048 prefix + <= 8 draft) "
                      "tokens, H=128)",
            "bound": "mfma",
            "achieved": round(single_tflops, 2),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(single_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("mla_decode_tree_verify"),
            "algorithmic_flops_per_launch": single_flops,
            "launch_avg_us": round(single_us, 2),
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline_tree(tv)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
