"""Benchmark of the DSA-style decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sets R] [--no-cpu]
                    [--no-extra | --extra unplanted,ragged,two_stage,prefill,multilayer]

Workload: one request with 131072 cached tokens (64 indexer heads x 128,
fp8 E4M3FN keys with per-token scales, bf16 queries; k = 2048; sparse MLA with
128 heads over 576-wide bf16 latent rows).  A step is one lsi_decode_step call
(indexer scan -> top-k -> sparse MLA).  To keep every step's reads cold, R
independent requests live in one page pool (R*2048 pages, one global random
page permutation) and step i runs request i % R; with R = 32 the rotation
touches ~5.4 GB, far beyond the 256 MB last-level cache.  The steps are
captured into HIP graphs (one step per input set) and replayed, as a decode
loop would run them; the timed region covers exactly K steps.

Printed (one JSON line): tokens/s = 131072 * steps / time (whole step timed,
inputs resident in HBM), decode steps/s, per-phase averages from HIP events on
the launch stream, every kernel of the step timed with HIP events recorded on
its stream between launches (library profiling marks), the roofline of the
step's longest kernel (its algorithmic bytes per launch over its mean
duration, against 8 TB/s; the scan's algorithmic bytes are 132 per token:
128 key bytes and a 4-byte scale, the 4-byte score it writes being reported
as overhead), a sustained scan of 32 x 128K tokens in one launch, the CPU
oracle's throughput on a bounded sample of the same step, and (unless
--no-extra; --extra picks a subset) the un-planted twin of the step, the
ragged 64-request decode step, the two-stage compact-key search at 512K
(original keys on the device and in pinned host memory), the prefill
indexer chunk, and 61 layers of one 128K request under the serial, MLI and
IndexCache schedules.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

# the CPU oracle's BLAS pool: as many threads as this process may run on,
# unless the environment already fixes it (set before numpy is imported)
_AFFINITY = len(os.sched_getaffinity(0))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(_AFFINITY))

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer-scanned tokens/s and decode steps/s (index+top-k+sparse attn) @128K ctx"
HBM_PEAK_GBS = 8000.0
BYTES_PER_TOKEN = 132          # 128 fp8 key bytes + 4-byte scale (algorithmic scan bytes)
SCORE_BYTES_PER_TOKEN = 4      # the fp32 score the scan writes (implementation overhead)


EXTRAS = ("unplanted", "ragged", "two_stage", "prefill", "multilayer")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=320)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--sets", type=int, default=32)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-extra", action="store_true",
                   help="skip every workload but the one-request step and the sustained scan")
    p.add_argument("--extra", default=",".join(EXTRAS),
                   help="which other workloads to measure (comma-separated subset of "
                        + ", ".join(EXTRAS) + "; multilayer_r1: only retention 1 at "
                        "131072 tokens, plus each schedule's eager kernel timeline)")
    p.add_argument("--only-extra", action="store_true",
                   help="measure only the --extra workloads and print them (no step line; "
                        "for kernel traces of one workload group)")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a 512 MiB device copy (known traffic) for counter scaling")
    return p.parse_args()


def event_loop(fn, n, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(n):
        fn(i)
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n      # ms per call


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    from lightning_indexer_top_04_amd import lsi, synth

    torch.cuda.set_device(0)
    dev = "cuda:0"
    if args.only_extra:
        res = {"other_workloads": other_workloads(lsi, synth, torch, dev, tuple(args.extra.split(",")))}
        if args.calib_copy:
            res["calib_copy_bytes"] = calib_copy(torch, dev)
        print(json.dumps(res))
        return
    R = args.sets
    L = 131072
    wl = synth.scaled(synth.DSA_128K, seq_lens=tuple([L] * R), num_req=R)
    t0 = time.time()
    di = synth.make_decode_inputs(wl, device=dev)
    torch.cuda.synchronize()
    print(f"# inputs drawn in {time.time() - t0:.1f}s ({R} sets)", file=sys.stderr, flush=True)

    ik = lsi.Cache(di.ikeys, di.iscale, "fp8", 128)
    kv = lsi.Cache(di.kv, None, "bf16", 576)
    reqs = [lsi.Requests(di.seq_lens[r:r + 1], di.page_table[r:r + 1], L) for r in range(R)]
    k, H, dv = 2048, 128, 512
    idx = torch.empty(1, k, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    out = torch.empty(1, H, dv, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(1, H, dtype=torch.float32, device=dev)
    ws = lsi.decode_step_workspace(1, L, k, H, dv, dev)
    def step(r, stream=None):
        lsi.decode_step(ik, kv, None, reqs[r], q_idx[r], w[r], q_attn[r], k, wl.sm_scale, dv,
                        out=out, lse=lse, idx=idx, count=cnt, ws=ws, stream=stream)

    # per-set views, made once (slicing in the timed loop would cost host time)
    q_idx = [di.q_idx[r:r + 1] for r in range(R)]
    w = [di.w[r:r + 1] for r in range(R)]
    q_attn = [di.q_attn[r:r + 1] for r in range(R)]

    # eager warm-up (also initialises the library), then graphs: a decode loop
    # replays the same launch sequence every step, so the steps are captured
    # once (one step per input set) and replayed; the host then only launches
    # graphs and the timed region measures the device
    for i in range(max(args.warmup, 3)):
        step(i % R)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_eager = min(args.steps, 100)
    for i in range(n_eager):
        step(i % R)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / n_eager

    def capture(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        return g

    all_steps = [lambda r=r: step(r) for r in range(R)]
    g_all = capture(all_steps)
    nfull, rem = divmod(args.steps, R)
    g_rem = capture(all_steps[:rem]) if rem else None
    wfull, wrem = divmod(args.warmup, R)
    for _ in range(wfull):
        g_all.replay()
    for f in all_steps[:wrem]:
        f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(nfull):
        g_all.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    tokens_s = L * args.steps / dt
    print(f"# decode step {ms_step * 1e3:.1f} us (graph), {eager_ms * 1e3:.1f} us (eager)",
          file=sys.stderr, flush=True)

    # ---- per-phase timing: each phase captured over all sets in one graph,
    # timed with HIP events on the replay stream -----------------------------
    scores = torch.empty(R, L, dtype=torch.float32, device=dev)
    sc_rows = [scores[r:r + 1] for r in range(R)]
    for r in range(R):
        lsi.index_scores(ik, reqs[r], q_idx[r], w[r], scores=sc_rows[r])
    idx_sel = [lsi.topk(sc_rows[r], reqs[r], k)[0] for r in range(R)]
    torch.cuda.synchronize()
    g_scan = capture([lambda r=r: lsi.index_scores(ik, reqs[r], q_idx[r], w[r], scores=sc_rows[r])
                      for r in range(R)])
    g_topk = capture([lambda r=r: lsi.topk(sc_rows[r], reqs[r], k) for r in range(R)])
    g_mla = capture([lambda r=r: lsi.sparse_mla_decode(kv, None, reqs[r], q_attn[r], idx_sel[r],
                                                       wl.sm_scale, dv) for r in range(R)])

    def per_launch_ms(g, reps=5):
        g.replay()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            g.replay()
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1) / (reps * R)

    t_scan = per_launch_ms(g_scan)
    t_topk = per_launch_ms(g_topk)
    t_mla = per_launch_ms(g_mla)

    # ---- every kernel of the step, timed live: HIP events recorded on the
    # launch stream before the step's first kernel and after each kernel
    # (lsi_profile_events), over n_prof steps queued behind a sleep kernel so
    # that the device runs them back to back --------------------------------
    n_prof = 4 * R
    timer = lsi.KernelTimer(capacity=8 * n_prof)
    torch.cuda.synchronize()
    try:
        torch.cuda._sleep(2_000_000)
    except Exception:
        pass
    with timer:
        for i in range(n_prof):
            step(i % R)
    kern = {}
    for name, ms in timer.intervals():
        kern.setdefault(name, []).append(ms * 1e3)
    alg = {   # algorithmic HBM bytes per launch (one 131072-token request)
        "scan_dma_kernel<fp8>": L * BYTES_PER_TOKEN,
        "topk_hist_kernel": L * 4,
        "topk_select_kernel": L * 4 + k * 4,
        "topk_refine_kernel": k * 4,
        "mla_bf16_kernel": k * 576 * 2 + H * 576 * 2,
        "mla_combine_kernel": H * dv * 2,
    }
    kernels = {}
    for name, v in kern.items():
        mean_us = sum(v) / len(v)
        b = alg.get(name)
        kernels[name] = {"launches": len(v), "mean_us": mean_us,
                         "median_us": sorted(v)[len(v) // 2], "algorithmic_bytes": b,
                         "GB_s": None if b is None else b / (mean_us * 1e-6) / 1e9,
                         "frac_of_hbm_peak": None if b is None else b / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    dom = max(kernels, key=lambda n: kernels[n]["mean_us"])
    scan_us = kernels.get("scan_dma_kernel<fp8>", {}).get("mean_us", t_scan * 1e3)

    # ---- sustained scan: all R requests in one launch ---------------------
    req_all = lsi.Requests(di.seq_lens, di.page_table, L)
    scores_all = torch.empty(R, L, dtype=torch.float32, device=dev)
    n_sus = 20
    stream = torch.cuda.current_stream()
    # warm-up until the launch time has settled: the first windows after
    # the step benchmarks run fast, then slow for a few windows while the
    # device's clocks settle (seen as 95, 107, 107, 101, 99, 99, 98 us per
    # launch in consecutive 20-launch windows), so ~40 ms of launches go first
    for _ in range(400):
        lsi.index_scores(ik, req_all, di.q_idx, di.w, scores=scores_all, stream=stream)
    torch.cuda.synchronize()
    # back-to-back launches on the stream (the figure reported) and the same
    # launches replayed from one graph (for comparison: graph replays insert
    # their own inter-node synchronisation, which is slower here)
    # seven windows of 20 launches; the median window is reported
    sus_windows = sorted(event_loop(lambda i: lsi.index_scores(ik, req_all, di.q_idx, di.w,
                                                               scores=scores_all, stream=stream),
                                    n_sus, stream) for _ in range(7))
    t_sus = sus_windows[3]
    g_sus = capture([lambda: lsi.index_scores(ik, req_all, di.q_idx, di.w, scores=scores_all)
                     for _ in range(n_sus)])
    g_sus.replay()
    torch.cuda.synchronize()
    t_sus_graph = event_loop(lambda i: g_sus.replay(), 3, torch.cuda.current_stream()) / n_sus
    sus_gbs = R * L * BYTES_PER_TOKEN / (t_sus * 1e-3) / 1e9
    del g_sus

    # spread of the step time: the same graph of R steps replayed 10 more
    # times (after the timed region), each replay between HIP events
    per_replay = sorted(event_loop(lambda i: g_all.replay(), 1, stream) / R for _ in range(10))
    pct = lambda q: per_replay[min(len(per_replay) - 1, int(round(q * (len(per_replay) - 1))))]

    # achievable-bandwidth reference on the same device: plain streams over
    # 1 GiB (torch's full sum, a per-row sum that writes 1/4096 of what it
    # reads, and a copy counted as read + write); the best rate is reported
    big = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(big)
    rows = big.view(-1, 4096)
    refs = {"sum": (lambda i: big.sum(), 1 << 30),
            "row_sum": (lambda i: rows.sum(1), (1 << 30) + (1 << 18)),
            "copy": (lambda i: dst.copy_(big), 2 << 30)}
    ref_gbs = {}
    for name, (fn, nbytes) in refs.items():
        fn(0)
        torch.cuda.synchronize()
        ref_gbs[name] = nbytes / (event_loop(fn, 10, stream) * 1e-3) / 1e9
    read_gbs = max(ref_gbs.values())
    del big, dst, rows
    torch.cuda.empty_cache()
    traffic = measured_traffic(dom)

    step_bytes = L * BYTES_PER_TOKEN + k * 576 * 2 + H * 576 * 2 + H * dv * 2
    res = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; fp8 keys N(0,1) quantised per token, 2048 planted tokens)",
        "config": {"workload": "dsa-decode-L131072", "num_req": 1, "seq_len": L, "k": k,
                   "indexer_heads": 64, "indexer_dim": 128, "mla_heads": H, "dk": 576,
                   "dv": dv, "page_size": 64, "rotating_sets": R},
        "decode_steps_per_s": 1e3 / ms_step,
        "timing": "HIP graph replay (one step per input set); eager per-call figure below",
        "eager_ms_per_step": eager_ms,
        "step_us_p10_p50_p90": [pct(0.1) * 1e3, pct(0.5) * 1e3, pct(0.9) * 1e3],
        "phases_us": {"scan": t_scan * 1e3, "topk": t_topk * 1e3, "mla": t_mla * 1e3,
                      "how": "each phase's standalone entry point (index_scores, topk, "
                             "sparse_mla_decode) over the 32 sets, graph replays between HIP events"},
        "scan_tokens_per_s": L / (scan_us * 1e-6),
        "step_kernels": {"kernels": kernels,
                         "how": f"{n_prof} eager steps queued behind a sleep kernel; HIP events "
                                "recorded on the launch stream before the step's first kernel and "
                                "after each kernel (lsi_profile_events); mean of the intervals",
                         "sum_of_means_us": sum(x["mean_us"] for x in kernels.values())},
        "roofline": {"kernel": dom, "bound": "hbm",
                     "achieved": kernels[dom]["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": kernels[dom]["frac_of_hbm_peak"],
                     "traffic": traffic,
                     "traffic_GB_s": None if traffic is None else traffic / (kernels[dom]["mean_us"] * 1e-6) / 1e9,
                     "overfetch": None if traffic is None or not kernels[dom]["algorithmic_bytes"]
                     else traffic / kernels[dom]["algorithmic_bytes"],
                     "note": f"the step's longest kernel: {kernels[dom]['algorithmic_bytes']} "
                             f"algorithmic bytes per launch / its mean duration "
                             f"{kernels[dom]['mean_us']:.2f} us (step_kernels)"},
        "scan_roofline": {"kernel": "scan_dma_kernel<fp8>", "bound": "hbm",
                          "bytes_per_token": BYTES_PER_TOKEN,
                          "achieved_GB_s": L * BYTES_PER_TOKEN / (scan_us * 1e-6) / 1e9,
                          "frac": L * BYTES_PER_TOKEN / (scan_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "score_write_overhead_bytes_per_token": SCORE_BYTES_PER_TOKEN},
        "scan_sustained": {"tokens": R * L, "us": t_sus * 1e3,
                           "tokens_per_s": R * L / (t_sus * 1e-3), "GB_s": sus_gbs,
                           "frac": sus_gbs / HBM_PEAK_GBS,
                           "bytes_per_token": BYTES_PER_TOKEN,
                           "score_write_overhead_bytes_per_token": SCORE_BYTES_PER_TOKEN,
                           "timing": "HIP events around 20 back-to-back launches on one stream; "
                                     "median of 7 such windows after ~40 ms of warm-up launches",
                           "us_windows_min_max": [sus_windows[0] * 1e3, sus_windows[-1] * 1e3],
                           "us_windows_sorted": [w * 1e3 for w in sus_windows],
                           "us_graph_replay": t_sus_graph * 1e3,
                           "stream_reference_GB_s": read_gbs,
                           "frac_of_stream_reference": sus_gbs / read_gbs,
                           "stream_reference": {"GB_s": ref_gbs,
                                                "how": "HIP events around 10 launches each over "
                                                       "1 GiB of float32: torch sum, per-row sum, "
                                                       "copy (read + write)"}},
        # the whole step against its algorithmic HBM time: the scan's keys and
        # scales, the gathered latent rows, the query and the output
        "step_roofline": {"algorithmic_bytes": step_bytes,
                          "roofline_us": step_bytes / (HBM_PEAK_GBS * 1e3),
                          "frac": step_bytes / (HBM_PEAK_GBS * 1e3) / (ms_step * 1e3)},
    }

    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(di, wl, L, args.cpu_seconds)

    if not args.no_extra:
        # the other workloads of the pages' configurations, measured on the
        # same device after the 128K sets are released
        del g_all, g_rem, g_scan, g_topk, g_mla, di, scores, scores_all, sc_rows, idx_sel
        del q_idx, w, q_attn, reqs, ik, kv, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        res["other_workloads"] = other_workloads(lsi, synth, torch, dev, tuple(args.extra.split(",")))

    if args.calib_copy:
        res["calib_copy_bytes"] = calib_copy(torch, dev)

    print(json.dumps(res))


def calib_copy(torch, dev):
    """A plain elementwise copy of known size (512 MiB read, 512 MiB written
    per launch) and a plain sum (512 MiB read), for scaling the FETCH_SIZE /
    WRITE_SIZE counters of the same run."""
    src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)      # 512 MiB written (and read)
        src.sum()                         # 512 MiB read, nothing written
    torch.cuda.synchronize()
    return 512 << 20


def other_workloads(lsi, synth, torch, dev, extra=EXTRAS):
    """Throughput of the ragged 64-request decode step, the two-stage
    compact-key search at 512K and the prefill indexer chunk, each against
    its own roofline (HBM bytes, or bf16 MFMA flops for the prefill)."""
    out = {}

    def graph_ms(fn, n=8, reps=5):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            g.replay()
        e1.record(st)
        e1.synchronize()
        del g
        return e0.elapsed_time(e1) / (reps * n)

    if "unplanted" in extra:
        # the un-planted twin of the one-request step: no planted tokens, so the
        # scores are one continuous distribution and the k-th score falls in a
        # crowded histogram bin (thousands of candidates to refine); 8 rotating
        # input sets (1.3 GB, more than the last-level cache)
        nset, L1 = 8, 131072
        wl = synth.scaled(synth.DSA_128K, seq_lens=(L1,) * nset, num_req=nset)
        di = synth.make_decode_inputs(wl, device=dev, planted=False)
        ik = lsi.Cache(di.ikeys, di.iscale, "fp8", 128)
        kv = lsi.Cache(di.kv, None, "bf16", 576)
        reqs = [lsi.Requests(di.seq_lens[r:r + 1], di.page_table[r:r + 1], L1) for r in range(nset)]
        views = [(di.q_idx[r:r + 1], di.w[r:r + 1], di.q_attn[r:r + 1]) for r in range(nset)]
        k, H, dv = 2048, 128, 512
        idx = torch.empty(1, k, dtype=torch.int32, device=dev)
        cnt = torch.empty(1, dtype=torch.int32, device=dev)
        o = torch.empty(1, H, dv, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(1, H, dtype=torch.float32, device=dev)
        ws = lsi.decode_step_workspace(1, L1, k, H, dv, dev)

        def unplanted_steps():
            for r in range(nset):
                qi, wr, qa = views[r]
                lsi.decode_step(ik, kv, None, reqs[r], qi, wr, qa, k, wl.sm_scale, dv, out=o,
                                lse=lse, idx=idx, count=cnt, ws=ws)

        t = graph_ms(unplanted_steps, n=1, reps=10) / nset
        out["decode_step_unplanted_l131072"] = {
            "us_per_step": t * 1e3, "tokens_per_s": L1 / (t * 1e-3), "steps_per_s": 1e3 / t,
            "sets": nset}
        del di, ik, kv, reqs, views, idx, cnt, o, lse, ws
        torch.cuda.empty_cache()

    if "ragged" in extra:
        # ragged batch: 64 requests, L ~ U{10000..195000}
        wl = synth.BATCH_RAGGED
        di = synth.make_decode_inputs(wl, device=dev)
        seq = di.seq_lens
        maxL = int(seq.max().item())
        ik = lsi.Cache(di.ikeys, di.iscale, "fp8", 128)
        kv = lsi.Cache(di.kv, None, "bf16", 576)
        req = lsi.Requests(seq, di.page_table, maxL)
        B, k, H, dv = seq.numel(), 2048, 128, 512
        idx = torch.empty(B, k, dtype=torch.int32, device=dev)
        cnt = torch.empty(B, dtype=torch.int32, device=dev)
        o = torch.empty(B, H, dv, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(B, H, dtype=torch.float32, device=dev)
        ws = lsi.decode_step_workspace(B, maxL, k, H, dv, dev)
        t = graph_ms(lambda: lsi.decode_step(ik, kv, None, req, di.q_idx, di.w, di.q_attn, k,
                                             wl.sm_scale, dv, out=o, lse=lse, idx=idx, count=cnt,
                                             ws=ws), n=2, reps=5)
        tokens = int(seq.sum().item())
        byts = tokens * BYTES_PER_TOKEN + B * (k * 576 * 2 + H * 576 * 2 + H * dv * 2)
        out["ragged_decode_b64"] = {
            "requests": B, "tokens": tokens, "us_per_step": t * 1e3,
            "tokens_per_s": tokens / (t * 1e-3), "steps_per_s": 1e3 / t,
            "roofline": {"bound": "hbm", "algorithmic_bytes": byts,
                         "achieved_GB_s": byts / (t * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "frac": byts / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}}
        del di, ik, kv, req, idx, cnt, o, lse, ws
        torch.cuda.empty_cache()

    if "two_stage" in extra:
        # two-stage compact-key search at 524288 tokens: int4 scan, 8192
        # candidates, exact fp8 rescoring, 2048 kept; planted and un-planted
        # inputs, each with its recall against the exact top-2048 of the
        # fp8 scores (this library's one-stage scan + top-k, the same
        # arithmetic) and the recall of the int4 scores alone
        L = 524288
        res = {"tokens": L, "n_cand": 8192, "k": 2048}
        for planted in (True, False):
            wl = synth.TWO_STAGE_512K
            di = synth.make_decode_inputs(wl, device=dev, with_int4=True, with_attn=planted,
                                          planted=planted)
            ik8 = lsi.Cache(di.ikeys, di.iscale, "fp8", 128)
            ik4 = lsi.Cache(di.ikeys4, di.iscale4, "int4", 128)
            req = lsi.Requests(di.seq_lens, di.page_table, L)
            # one workspace for every call (its state words stay zero between calls)
            ws2 = lsi.two_stage_workspace(1, L, 8192, 2048, dev)
            t = graph_ms(lambda: lsi.two_stage_topk(ik4, ik8, req, di.q_idx, di.w, 8192, 2048, ws=ws2), n=4)
            idx, _ = lsi.two_stage_topk(ik4, ik8, req, di.q_idx, di.w, 8192, 2048, ws=ws2)
            exact, _ = lsi.topk(lsi.index_scores(ik8, req, di.q_idx, di.w), req, 2048)
            only4, _ = lsi.topk(lsi.index_scores(ik4, req, di.q_idx, di.w), req, 2048)
            torch.cuda.synchronize()
            ex = set(exact[0].tolist())
            byts = L * 68 + 8192 * BYTES_PER_TOKEN
            rec = {
                "us_per_call": t * 1e3, "tokens_per_s": L / (t * 1e-3),
                "recall": len(set(idx[0].tolist()) & ex) / 2048,
                "recall_int4_only": len(set(only4[0].tolist()) & ex) / 2048,
                "roofline": {"bound": "hbm", "algorithmic_bytes": byts,
                             "achieved_GB_s": byts / (t * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                             "frac": byts / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}}
            if planted:
                # the sparse MLA over the selection (128 heads), alone and
                # after the search in one graph: the decode step over 524288
                # tokens with the compact search as its indexer
                kv = lsi.Cache(di.kv, None, "bf16", 576)
                t_mla = graph_ms(lambda: lsi.sparse_mla_decode(kv, None, req, di.q_attn, idx,
                                                               wl.sm_scale, 512), n=8)

                def step():
                    sel, _ = lsi.two_stage_topk(ik4, ik8, req, di.q_idx, di.w, 8192, 2048, ws=ws2)
                    lsi.sparse_mla_decode(kv, None, req, di.q_attn, sel, wl.sm_scale, 512)

                t_step = graph_ms(step, n=4)
                rec["mla_over_selection_us"] = t_mla * 1e3
                rec["search_plus_mla_us"] = t_step * 1e3
                del kv
                # the original fp8 keys in pinned host memory: only the compact
                # keys (68 B/token) occupy GPU memory; the rescoring reads the
                # 8192 candidates' rows across the host bus
                ik8h = lsi.Cache(di.ikeys.cpu().pin_memory(), di.iscale.cpu().pin_memory(), "fp8", 128)
                th = graph_ms(lambda: lsi.two_stage_topk(ik4, ik8h, req, di.q_idx, di.w, 8192, 2048, ws=ws2),
                              n=4)
                rec["host_originals"] = {
                    "us_per_call": th * 1e3, "tokens_per_s": L / (th * 1e-3),
                    "gpu_bytes_per_token": 68, "gpu_bytes_per_token_device_originals": 68 + 132,
                    "bus_bytes_per_call": 8192 * 132}
                del ik8h
            res["planted" if planted else "unplanted"] = rec
            del di, ik8, ik4, req, idx, exact, only4, ws2
            torch.cuda.empty_cache()
        res["how"] = ("recall = |selection & exact| / 2048, exact = top-2048 of the fp8 scores of "
                      "all 524288 tokens; recall_int4_only = the same for the top-2048 of the int4 "
                      "scores; us_per_call from graph replays of 4 calls")
        out["two_stage_l524288"] = res

    if "prefill" in extra:
        # prefill chunk: 4096 queries over 65536 history + the chunk, causal
        wl = synth.PREFILL_CHUNK
        pi = synth.make_prefill_inputs(wl, device=dev)
        Hh = pi.hist_len
        hist_k_host = pi.keys[:Hh].cpu().pin_memory()
        hist_s_host = pi.scale[:Hh].cpu().pin_memory()
        hist_k_dev = pi.keys[:Hh].contiguous()
        hist_s_dev = pi.scale[:Hh].contiguous()
        chunk_k = pi.keys[Hh:].contiguous()
        chunk_s = pi.scale[Hh:].contiguous()
        copy_stream = torch.cuda.Stream()
        T = pi.T
        pairs = T * Hh + T * (T + 1) // 2
        flops = pairs * 64 * 128 * 2

        def prefill_ms(hk, hs, reps=5):
            lsi.prefill_index_topk(hk, hs, chunk_k, chunk_s, pi.q, pi.w, 2048, 8192,
                                   copy_stream=copy_stream)
            torch.cuda.synchronize()
            st = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(reps):
                lsi.prefill_index_topk(hk, hs, chunk_k, chunk_s, pi.q, pi.w, 2048, 8192,
                                       copy_stream=copy_stream)
            e1.record(st)
            e1.synchronize()
            return e0.elapsed_time(e1) / reps

        t_host = prefill_ms(hist_k_host, hist_s_host)
        t_dev = prefill_ms(hist_k_dev, hist_s_dev)
        out["prefill_t4096_h65536"] = {
            "queries": T, "pairs": pairs, "ms_history_from_pinned_host": t_host,
            "ms_history_on_device": t_dev,
            "workspace_bytes": int(lsi.workspace_bytes(lsi.OP_PREFILL, num_req=T, max_seq_len=Hh,
                                                       k=2048, dim=128, block_tokens=8192)),
            "roofline": {"bound": "mfma", "useful_flops": flops, "dtype": "bf16",
                         "achieved_TFLOP_s": flops / (t_dev * 1e-3) / 1e12, "peak": 2500.0,
                         "frac": flops / (t_dev * 1e-3) / 1e12 / 2500.0,
                         "note": "indexer scores of every (query, visible token) pair plus the "
                                 "per-query top-k, history on the device; the pinned-host "
                                 "figure includes the block copies over PCIe"}}
        del pi, hist_k_host, hist_s_host, hist_k_dev, hist_s_dev, chunk_k, chunk_s
        torch.cuda.empty_cache()
    if "multilayer" in extra:
        out["multilayer_l131072_x61"] = multilayer(lsi, synth, torch, dev, graph_ms)
    if "multilayer_r1" in extra:
        out["multilayer_l131072_x61_r1"] = multilayer(lsi, synth, torch, dev, graph_ms, quick=True)
    return out


def multilayer(lsi, synth, torch, dev, graph_ms, n_layers=61, quick=False):
    """Several layers of one decode step over one request, each layer with
    its own indexer keys and latent cache (one page table): an indexer in
    every layer, each finishing before its layer attends (serial), and the
    MLI schedule (each layer attends the previous indexer layer's selection
    while its own indexer runs on a second stream); IndexCache retention 1/r
    keeps an indexer in every r-th layer.  Swept over r = 1 .. 32 at 131072
    tokens, and over contexts of 10240 .. 199680 tokens at r = 1 and 4.  One
    graph replay per multi-layer step."""
    k, H, dv = 2048, 128, 512
    side = torch.cuda.Stream()
    attn_bytes = k * 576 * 2 + H * 576 * 2 + H * dv * 2

    def sweep(L, retentions):
        wl = synth.scaled(synth.DSA_128K, seq_lens=(L,))
        dis = [synth.make_decode_inputs(wl, device=dev, planted=False, layer=l)
               for l in range(n_layers)]
        req = lsi.Requests(dis[0].seq_lens, dis[0].page_table, L)
        kv = [lsi.Cache(d.kv, None, "bf16", 576) for d in dis]
        us, frac = {}, {}
        for r in retentions:
            has = [l % r == 0 for l in range(n_layers)]
            layers = lsi.Layers([lsi.Cache(d.ikeys, d.iscale, "fp8", 128) if h else None
                                 for d, h in zip(dis, has)], kv, req,
                                [d.q_idx if h else None for d, h in zip(dis, has)],
                                [d.w if h else None for d, h in zip(dis, has)],
                                [d.q_attn for d in dis], k, dv, r)
            byts = sum(has) * L * BYTES_PER_TOKEN + n_layers * attn_bytes
            for sched in ("serial", "mli"):
                t = graph_ms(lambda sched=sched: lsi.multilayer_decode(
                    layers, wl.sm_scale, sched, index_stream=side), n=1, reps=10)
                key = f"r{r}_{sched}"
                us[key] = t * 1e3
                frac[key] = byts / (t * 1e-3) / 1e9 / HBM_PEAK_GBS
            del layers
            print(f"# multilayer L={L} r={r}: serial {us[f'r{r}_serial']:.0f} us, "
                  f"mli {us[f'r{r}_mli']:.0f} us", file=sys.stderr, flush=True)
        del dis, kv, req
        torch.cuda.empty_cache()
        base = us["r1_serial"]
        return {"tokens_per_layer": L, "us_per_step": us,
                "us_per_layer": {kk: v / n_layers for kk, v in us.items()},
                "speedup_vs_unmodified": {kk: base / v for kk, v in us.items()},
                "hbm_roofline_frac": frac}

    res = sweep(131072, (1,) if quick else (1, 2, 4, 8, 16, 32))
    res["layers"] = n_layers
    if quick:
        res["eager_overlap"] = eager_overlap(lsi, synth, torch, dev, n_layers, side)
        return res
    res["by_context"] = {f"L{L}": sweep(L, (1, 4)) for L in (10240, 65536, 199680)}
    res["note"] = ("r = retention (one indexer every r layers); serial = each indexer finishes "
                   "before its layer attends; mli = the indexer of layer l runs beside layer l's "
                   "attention on a second stream, after layer l-1; speedups against r1_serial "
                   "of the same context")
    return res


def eager_overlap(lsi, synth, torch, dev, n_layers, side, L=131072):
    """Kernel timeline of one eager multi-layer step per schedule (r = 1),
    from the start/stop events each dispatch carries (lsi_profile_events):
    how long an indexer kernel (scan, top-k) and an attention kernel (MLA,
    combine) run at the same time, against the summed kernel time."""
    k, dv = 2048, 512
    wl = synth.scaled(synth.DSA_128K, seq_lens=(L,))
    dis = [synth.make_decode_inputs(wl, device=dev, planted=False, layer=l) for l in range(n_layers)]
    req = lsi.Requests(dis[0].seq_lens, dis[0].page_table, L)
    layers = lsi.Layers([lsi.Cache(d.ikeys, d.iscale, "fp8", 128) for d in dis],
                        [lsi.Cache(d.kv, None, "bf16", 576) for d in dis], req,
                        [d.q_idx for d in dis], [d.w for d in dis], [d.q_attn for d in dis], k, dv, 1)
    out = {}
    for sched in ("serial", "mli"):
        for _ in range(3):
            lsi.multilayer_decode(layers, wl.sm_scale, sched, index_stream=side)
        torch.cuda.synchronize()
        timer = lsi.KernelTimer(capacity=16 * n_layers)
        # queued behind a sleep kernel, so that the whole step is enqueued
        # before the device starts it and the host's launch time is not in
        # the timeline
        try:
            torch.cuda._sleep(30_000_000)
        except Exception:
            pass
        with timer:
            lsi.multilayer_decode(layers, wl.sm_scale, sched, index_stream=side)
        tl = timer.timeline()
        idx_side = [(a, b) for n, a, b in tl if n.startswith(("scan", "topk"))]
        att_side = [(a, b) for n, a, b in tl if n.startswith("mla")]

        def union(iv):
            tot, cs, ce = 0.0, None, None
            for a, b in sorted(iv):
                if ce is None or a > ce:
                    if ce is not None:
                        tot += ce - cs
                    cs, ce = a, b
                else:
                    ce = max(ce, b)
            return tot + (ce - cs if ce is not None else 0.0)

        u_all = union(idx_side + att_side)
        both = union(idx_side) + union(att_side) - u_all   # time with kernels of both kinds running
        out[sched] = {"kernels": len(tl), "span_us": (max(b for _, _, b in tl) - min(a for _, a, _ in tl)) * 1e3,
                      "kernel_sum_us": sum(b - a for _, a, b in tl) * 1e3,
                      "busy_union_us": u_all * 1e3, "indexer_and_attention_concurrent_us": both * 1e3}
    del layers, dis, req
    torch.cuda.empty_cache()
    out["note"] = ("one eager call per schedule, 61 layers at 131072 tokens, r = 1, enqueued behind "
                   "a sleep kernel; times from the "
                   "dispatch-carried HIP events of every kernel (lsi_profile_events): span of the "
                   "step, summed kernel durations, their union, and the time during which an "
                   "indexer kernel (scan, top-k) and an attention kernel (MLA, combine) run at once")
    return out


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` in the one-request step, from the
    committed counter summary (FETCH_SIZE + WRITE_SIZE, calibrated against a
    plain copy), or None when there is none for that kernel or its source
    file has changed since the counters were taken."""
    import hashlib
    summ = os.path.join(ROOT, "profiles", "kernel_counters_dsa128k.json")
    try:
        with open(summ) as f:
            rec = json.load(f)["kernels"][kernel]
        with open(os.path.join(ROOT, rec["source"]), "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != digest:
        return None
    return rec["bytes_per_launch"]


def cpu_baseline(di, wl, L, seconds):
    """The oracle's decode step for one 128K request, repeated for ~`seconds`."""
    import numpy as np

    import oracle as O
    from lightning_indexer_top_04_amd import synth
    try:   # the BLAS pool's size as numpy runs it (set from the environment at start-up)
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", _AFFINITY))
    pt = di.page_table[0].cpu().numpy()
    n_pages = L // 64
    pages = di.page_table[0, :n_pages].long()
    codes = synth.u8_bits(di.ikeys[pages])              # this request's pages, in order
    scale = di.iscale[pages].cpu().numpy()
    kvp = di.kv[pages].contiguous()
    kv_bits = synth.bf16_bits(kvp)
    q_idx = synth.bf16_bits(di.q_idx[0])
    w = di.w[0].cpu().double().numpy()
    q_attn = synth.bf16_bits(di.q_attn[0])
    local_pt = np.arange(n_pages)

    def run(budget):
        t0 = time.perf_counter()
        n = 0
        while True:
            K = O.decode_e4m3fn(O.request_rows(codes, local_pt, L, 64))
            s = O.request_rows(scale, local_pt, L, 64)
            I = O.index_scores(O.decode_bf16(q_idx), w, K, s)
            sel, _ = O.topk(I, 2048)
            rows = O.request_rows(kv_bits, local_pt, L, 64)[np.sort(sel)]
            O.mla_decode(O.decode_bf16(q_attn), O.decode_bf16(rows), 512, wl.sm_scale)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget or n >= 50:
                return n, el

    n, el = run(seconds)
    single = None
    try:   # the same step with the BLAS pool held to one thread
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            n1, el1 = run(seconds / 3)
        single = {"steps_per_s": n1 / el1, "tokens_per_s": L * n1 / el1,
                  "sample": f"{n1} steps ({el1:.1f}s)"}
    except Exception:
        pass
    del pt
    return {"value": L * n / el, "unit": "tokens/s", "cores": int(threads),
            "affinity_cpus": _AFFINITY, "kind": "oracle",
            "steps_per_s": n / el,
            "sample": f"{n} oracle decode steps of one 131072-token request "
                      f"(numpy float64, {el:.1f}s)",
            "single_thread": single}


if __name__ == "__main__":
    main()
