"""Benchmark of the DSA forward hot path on one MI355X.

One step = the whole path (lightning indexer -> top-k -> sparse MLA-MQA) over
all query rows of the 128K-context causal prefill (L = 131072, k = 2048,
H_I = 64 FP8 indexer heads, 128 MLA heads over 576-d bf16 latents), with
inputs already resident in HBM: one fused dsa_forward_prefill call.  Phase A
times K fused calls (the headline); phase B runs K more with the library's
launch timing on, which brackets every kernel stage with HIP events on the
stream it runs on (dsa_timing_begin / dsa_timing_end) and gives the per-kernel
durations.  Afterwards a stage-by-stage replay through the single-stage calls
must reproduce the fused outputs bit for bit (skipped with --fused-only).

Prints one JSON line: query-tokens/s, the dominant kernel's roofline, and the
CPU oracle's rate on a bounded sample of the same workload.

Other modes (not the headline line):
  --workload decode_b64_ctx32k | paged_decode_b32_ctx4k_128k
      one step = one fused decode call (indexer -> top-k -> split attention ->
      combine) for the whole batch, timed in the same two phases, then K
      replays of a HIP graph captured from one fused call (no host launch gaps;
      each replay's outputs must equal the eager call's; --no-graph skips it);
      the staged check replays it through the paged entry points (the
      contiguous cache is addressed through an identity page table for it).
  --workload paged_prefill_b4_ctx32k_q8k
      one step = one chunked prefill call into a paged cache (4 sequences of
      32K tokens, the last 8K of each new).
  --kl
      the sparse-stage indexer KL loss over all rows of a prefill workload.
  --copy-calibration
      copies a 1 GiB buffer three times with a plain device copy, so that HBM
      byte counters read under a profiler can be scaled against a known size.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA query-tokens/s at 128K ctx, k=2048 (indexer+topk+sparse MLA); %roofline"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0

# HBM bytes per stage launch read with rocprofv3 (FETCH_SIZE and WRITE_SIZE, one counter per run,
# on the timed calls alone: bench.py --fused-only, or --bwd --no-cpu for the backward), summed
# over the kernels of the stage, scaled by what the same counters read for a plain 1 GiB device
# copy (bytes read = FETCH_SIZE KiB x 1024 x 2.0, bytes written = WRITE_SIZE KiB x 1024 x 1.0).
# Each entry holds the hash of the device sources of the stage's kernels the counters were taken
# on (and of the host code that sizes the prefill's row tiles, where a launch covers one); once
# one changes, the figure no longer describes the launch and the roofline reports traffic as null.
COUNTER_TRAFFIC = {
    ("prefill_L128k", "indexer"): ("e80d6cb420658ad0", ('indexer.hip', 'indexer_exact.h', 'common.h', 'dsa_api.cpp'), 1009.2e6),
    ("prefill_L128k", "topk"): ("d879294fca012ffb", ('topk.hip', 'indexer_exact.h', 'common.h', 'dsa_api.cpp'), 991.0e6),
    ("prefill_L128k", "sparse_mla"): ("e286d380d79d225d", ('sparse_mla.hip', 'common.h'), 278029.8e6),
    ("decode_b64_ctx32k", "indexer"): ("aa70767aa971e6ed", ('indexer.hip', 'indexer_exact.h', 'common.h'), 281.4e6),
    ("decode_b64_ctx32k", "topk"): ("d1d997af9d4303a1", ('topk.hip', 'indexer_exact.h', 'common.h'), 9.3e6),
    ("decode_b64_ctx32k", "sparse_mla"): ("e286d380d79d225d", ('sparse_mla.hip', 'common.h'), 246.3e6),
    ("paged_decode_b32_ctx4k_128k", "indexer"): ("aa70767aa971e6ed", ('indexer.hip', 'indexer_exact.h', 'common.h'), 278.3e6),
    ("paged_decode_b32_ctx4k_128k", "topk"): ("d1d997af9d4303a1", ('topk.hip', 'indexer_exact.h', 'common.h'), 10.4e6),
    ("paged_decode_b32_ctx4k_128k", "sparse_mla"): ("e286d380d79d225d", ('sparse_mla.hip', 'common.h'), 157.6e6),
    ("paged_prefill_b4_ctx32k_q8k", "indexer"): ("e80d6cb420658ad0", ('indexer.hip', 'indexer_exact.h', 'common.h', 'dsa_api.cpp'), 924.6e6),
    ("paged_prefill_b4_ctx32k_q8k", "topk"): ("d879294fca012ffb", ('topk.hip', 'indexer_exact.h', 'common.h', 'dsa_api.cpp'), 989.3e6),
    ("paged_prefill_b4_ctx32k_q8k", "sparse_mla"): ("e286d380d79d225d", ('sparse_mla.hip', 'common.h'), 10447.6e6),
    ("prefill_L32k", "mla_bwd_dq"): ("d841631102c38279", ('sparse_mla_bwd.hip', 'common.h'), 5635.5e6),
    ("prefill_L32k", "mla_bwd_dkv"): ("d841631102c38279", ('sparse_mla_bwd.hip', 'common.h'), 7632.8e6),
    ("prefill_L32k", "mla_bwd_reduce"): ("d841631102c38279", ('sparse_mla_bwd.hip', 'common.h'), 5010.0e6),
}


def counter_traffic(workload: str, kernel: str):
    """Counter-measured HBM bytes per dispatch, or None if absent or taken on other sources."""
    import hashlib
    ent = COUNTER_TRAFFIC.get((workload, kernel))
    if ent is None:
        return None
    digest, files, nbytes = ent
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_attention_long_08_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return nbytes if h.hexdigest()[:16] == digest else None


def algorithmic_work(wl, T):
    """Per-stage algorithmic work of the whole step (causal prefill, q_pos0 = 0)."""
    import numpy as np
    pos = np.arange(T, dtype=np.float64)
    n = np.minimum(pos + 1, wl.N)
    pairs = n.sum()
    sel = np.minimum(n, wl.k).sum()
    idx_flops = pairs * 2 * wl.H_I * wl.d_I
    mla_flops = sel * 2 * wl.H * (wl.D_qk + wl.D_v)
    # bytes each stage must move at least once: inputs read, outputs written
    idx_bytes = T * (wl.H_I * wl.d_I + 4 * wl.H_I) + wl.N * wl.d_I
    topk_bytes = T * wl.k * 4
    mla_bytes = T * (wl.H * wl.D_qk * 2 + wl.H * wl.D_v * 4 + wl.H * 4) + sel * wl.D_qk * 2 + T * wl.k * 4
    return dict(pairs=pairs, selected=sel, idx_flops=idx_flops, mla_flops=mla_flops, idx_bytes=idx_bytes,
                topk_bytes=topk_bytes, mla_bytes=mla_bytes)


def cpu_baseline(wl, rows: int):
    """The oracle (plain C, fp64, one thread per process) on a bounded sample of
    the prefill workload's query rows, timed on this host's cores.

    Each row's indexer, top-k and attention are timed on their own (input
    generation excluded), first one row after another in this process, then
    with rows spread over one process per core (up to 16) running at once.
    From the single-threaded times, cost(t) = a + b n_t + c min(k, n_t) is
    fitted (n_t = candidates of row t) and summed over every row of the
    workload: an extrapolation of the whole-workload time on one core.  The
    concurrent run measures how much the cores slow each other down, which
    turns that sum into the host-aggregate time.  `value` is the concurrent
    run's rate in query rows per second."""
    import numpy as np
    from oracle import jobs
    from dsa_inputs import configs
    sample = configs.sample_rows(wl, rows)
    # a few rows with fewer than k candidates pin the fit's attention term
    short = [r for r in (17, 300, 900, 1500, 2040) if r < wl.T]
    single = np.unique(np.concatenate([sample, short])).astype(np.int64)
    jobs._prefill_keys(configs.WORKLOADS[wl.name], int(single.max()) + 1)  # key generation, untimed
    t0 = time.perf_counter()
    res = [jobs.timed_prefill_row_job((wl.name, int(t))) for t in single]
    wall1 = time.perf_counter() - t0
    n = np.array([r[0] for r in res], dtype=np.float64)
    sec = np.array([r[1] for r in res])
    A = np.stack([np.ones_like(n), n, np.minimum(n, wl.k)], axis=1)
    coef = np.linalg.lstsq(A, sec, rcond=None)[0]
    all_n = np.minimum(np.arange(wl.T, dtype=np.float64) + 1, wl.N)
    fit = lambda nn: coef[0] + coef[1] * nn + coef[2] * np.minimum(nn, wl.k)
    single_core_s = float(fit(all_n).sum())
    # concurrent run: two rows per process, one process per core
    procs = jobs.default_procs()
    conc = configs.sample_rows(wl, rows + 2 * procs)[-2 * procs:]
    t0 = time.perf_counter()
    res2 = jobs.run(jobs.timed_prefill_row_job, [(wl.name, int(t)) for t in conc], procs=procs)
    wall2 = time.perf_counter() - t0
    n2 = np.array([r[0] for r in res2], dtype=np.float64)
    sec2 = np.array([r[1] for r in res2])
    slowdown = float(sec2.sum() / fit(n2).sum())
    per_proc = sec2.sum() / procs  # oracle seconds each process spent, on average
    return {"value": len(conc) / per_proc, "unit": "query-tokens/s", "cores": procs, "kind": "oracle",
            "sample": f"{len(conc)} seeded-random query rows of {wl.name} ({procs} single-threaded processes at "
                      f"once, oracle time only) after {len(single)} rows one at a time in one process "
                      f"({wall1:.1f} s); indexer + top-k + attention per row, plain C oracle in fp64",
            "single_core_rows_per_s": len(single) / float(sec.sum()),
            "fit_seconds": {"a": float(coef[0]), "b_per_candidate": float(coef[1]),
                            "c_per_selected": float(coef[2])},
            "extrapolated_single_core_s": single_core_s,
            "extrapolated_host_aggregate_s": single_core_s * slowdown / procs,
            "concurrency_slowdown": slowdown, "host_nproc": os.cpu_count(),
            "note": "whole-workload times are extrapolations from the fit, not measurements"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 3 prefill, 200 decode)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 1 prefill, 20 decode)")
    ap.add_argument("--workload", default="prefill_L128k")
    ap.add_argument("--cpu-rows", type=int, default=60, help="query rows the CPU oracle baseline times")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--fused-only", action="store_true",
                    help="run only the fused calls (both timing phases): no staged-replay check and no CPU "
                         "baseline, so that a profiler sees the product path alone")
    ap.add_argument("--no-graph", action="store_true", help="decode: skip the HIP graph replay timing")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--dense-kl", action="store_true",
                    help="time the dense warm-up indexer KL loss (prefill_L32k unless --workload names another "
                         "prefill workload)")
    ap.add_argument("--bwd", action="store_true",
                    help="time the sparse attention backward (prefill_L32k unless --workload names another "
                         "prefill workload)")
    ap.add_argument("--kl", action="store_true",
                    help="time the sparse-stage indexer KL loss instead of the forward path (prefill_L32k unless "
                         "--workload names another prefill workload)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the DSA path here is a single-GPU kernel library).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        return copy_calibration()

    from dsa_inputs import configs

    if (args.kl or args.dense_kl or args.bwd) and args.workload == ap.get_default("workload"):
        args.workload = "prefill_L32k"
    wl = configs.WORKLOADS[args.workload]
    if wl.kind == "paged_prefill":
        args.steps = 3 if args.steps is None else args.steps
        args.warmup = 1 if args.warmup is None else args.warmup
        return bench_paged_prefill(args, wl)
    decode = wl.kind != "prefill"
    if args.dense_kl:
        if decode:
            print("--dense-kl needs a prefill workload", file=sys.stderr)
            sys.exit(2)
        args.steps = 3 if args.steps is None else args.steps
        args.warmup = 1 if args.warmup is None else args.warmup
        return bench_dense_kl(args, wl)
    if args.bwd:
        if decode:
            print("--bwd needs a prefill workload", file=sys.stderr)
            sys.exit(2)
        args.steps = 3 if args.steps is None else args.steps
        args.warmup = 1 if args.warmup is None else args.warmup
        return bench_bwd(args, wl)
    if args.kl:
        if decode:
            print("--kl needs a prefill workload", file=sys.stderr)
            sys.exit(2)
        args.steps = 3 if args.steps is None else args.steps
        args.warmup = 1 if args.warmup is None else args.warmup
        return bench_kl(args, wl)
    if args.steps is None:
        args.steps = 200 if decode else 3
    if args.warmup is None:
        args.warmup = 20 if decode else 1
    if decode:
        return bench_decode(args, wl)
    return bench_prefill(args, wl)


def copy_calibration():
    """Three plain device copies of 1 GiB (reads 1 GiB and writes 1 GiB each)."""
    import torch
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(3):
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy {i + 1}/3 of {nbytes} bytes done", file=sys.stderr, flush=True)
    print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 3}))


def launch_times(dsa, torch, stream, fused, steps: int):
    """Runs `steps` more fused calls with the library's launch timing on: each
    kernel stage is bracketed by two HIP events on the stream it is launched on.
    Returns ({kind: (summed ms, launches)}, ms per step of these calls)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    dsa.dsa_timing_begin()
    e0.record(stream)
    for _ in range(steps):
        fused()
    e1.record(stream)
    torch.cuda.synchronize()
    rec = dsa.dsa_timing_end()
    print(f"[bench] {steps} fused steps with launch events done", file=sys.stderr, flush=True)
    return rec, e0.elapsed_time(e1) / steps


def decode_graph_times(torch, stream, fused, outs, steps: int):
    """Captures one fused decode call into a HIP graph and times `steps`
    replays on `stream` (the decode path records no memset nodes).  Every
    replay's outputs must equal the eager call's: one replay is checked before
    the timed ones, the last timed one after them, with eager work in
    between."""
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fused()
    checks = []

    def scribble():  # so that the next call must rewrite every output
        for t in outs:
            t.fill_(-7)

    def check():
        torch.cuda.synchronize()
        checks.append(all(bool(torch.equal(a, b)) for a, b in zip(outs, ref)))

    scribble()
    g.replay()
    check()
    scribble()
    fused()  # eager work between replays
    check()
    scribble()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        g.replay()
    e1.record(stream)
    check()
    print(f"[bench] {steps} HIP graph replays done", file=sys.stderr, flush=True)
    return {"ms_per_step": e0.elapsed_time(e1) / steps, "replays_equal_eager": all(checks)}


def bench_prefill(args, wl):
    import numpy as np
    import torch

    import sparse_attention_long_08_amd as dsa
    from dsa_inputs import device

    dsa.load()
    T, N, k = wl.T, wl.N, wl.k
    print(f"[bench] generating {wl.name} inputs on the GPU", file=sys.stderr, flush=True)
    inp = device.make_prefill_inputs(wl)
    stream = torch.cuda.current_stream()
    tile_rows, ld = dsa.dsa_forward_prefill_plan(T, N)
    n_tiles = (T + tile_rows - 1) // tile_rows
    fws_bytes = dsa.dsa_forward_prefill_workspace_bytes(T, N, wl.H, wl.D_v, k)
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device="cuda")
    f_idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    f_out = torch.empty((T, wl.H, wl.D_v), dtype=torch.float32, device="cuda")
    f_lse = torch.empty((T, wl.H), dtype=torch.float32, device="cuda")

    def fused():
        dsa.dsa_forward_prefill(inp["q_idx"], inp["w"], inp["k_idx"], inp["q"], inp["kv"], T, N, wl.H_I, wl.d_I,
                                wl.H, wl.D_qk, wl.D_v, k, 0, wl.scale, f_idx, f_out, f_lse, fws, fws_bytes)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()
    # phase A, the timed region: K fused calls
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        fused()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gpu_ms_per_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} fused prefill steps done: {ms_per_step:.1f} ms per step", file=sys.stderr,
          flush=True)
    # phase B: K more fused calls with the library bracketing each kernel stage by
    # HIP events on the stream it runs on (the events would perturb phase A)
    rec_t, ev_ms_per_step = launch_times(dsa, torch, stream, fused, args.steps)
    stage_ms = {"indexer": rec_t["indexer"][0] / args.steps, "topk": rec_t["topk"][0] / args.steps,
                "sparse_mla": rec_t["attention"][0] / args.steps}
    stage_launches = {"indexer": rec_t["indexer"][1] // args.steps, "topk": rec_t["topk"][1] // args.steps,
                      "sparse_mla": rec_t["attention"][1] // args.steps}

    # the same path replayed stage by stage through the single-stage calls
    # (untimed): it must reproduce the fused call bit for bit
    del fws
    same = None
    if not args.fused_only:
        print("[bench] staged replay check", file=sys.stderr, flush=True)
        scores = torch.empty((tile_rows, ld), dtype=torch.float32, device="cuda")
        idx = torch.empty_like(f_idx)
        out = torch.empty_like(f_out)
        lse = torch.empty_like(f_lse)
        mla_ws_bytes = dsa.dsa_sparse_mla_fwd_workspace_bytes(T, wl.H, wl.D_v, k)
        mla_ws = torch.empty(max(mla_ws_bytes, 256), dtype=torch.uint8, device="cuda")
        for i in range(n_tiles):
            r0 = i * tile_rows
            tr = min(tile_rows, T - r0)
            dsa.dsa_indexer_scores(inp["q_idx"][r0:], inp["w"][r0:], inp["k_idx"], tr, N, wl.H_I, wl.d_I, r0,
                                   scores, ld)
            dsa.dsa_topk(scores, ld, tr, N, r0, None, k, idx[r0:])
        dsa.dsa_sparse_mla_fwd(inp["q"], inp["kv"], idx, T, N, wl.H, wl.D_qk, wl.D_v, k, wl.scale, out, lse, mla_ws,
                               mla_ws_bytes)
        torch.cuda.synchronize()
        del scores
        same = bool(torch.equal(f_idx, idx) and torch.equal(f_lse, lse) and torch.equal(f_out, out))
        del out
    del f_out
    w = algorithmic_work(wl, T)
    hbm_s = (w["idx_bytes"] + w["topk_bytes"] + w["mla_bytes"]) / (PEAK_HBM_GBS * 1e9)
    # the indexer's contraction is priced at the FP8 MFMA peak (the fused call scores
    # on the FP8 matrix cores), the attention at the bf16 peak
    t_roof = max(w["idx_flops"] / (PEAK_FP8_TFLOPS * 1e12) + w["mla_flops"] / (PEAK_BF16_TFLOPS * 1e12), hbm_s)
    kernels = {
        "sparse_mla": ("mfma", w["mla_flops"] / (stage_ms["sparse_mla"] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
        "indexer": ("mfma", w["idx_flops"] / (stage_ms["indexer"] * 1e-3) / 1e12, PEAK_FP8_TFLOPS, "TFLOP/s"),
        "topk": ("hbm", w["topk_bytes"] / (stage_ms["topk"] * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"),
    }
    dom = max(stage_ms, key=stage_ms.get)
    bound, ach, peak, unit = kernels[dom]
    launches = stage_launches[dom]
    rec = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "gpu_ms_per_step": gpu_ms_per_step,
        "ms_per_step_with_launch_events": ev_ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator, device-resident)",
        "config": {"workload": wl.name, "L": T, "k": k, "H_I": wl.H_I, "d_I": wl.d_I, "H": wl.H,
                   "D_qk": wl.D_qk, "D_v": wl.D_v, "causal": True, "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": bound, "achieved": ach, "peak": peak, "unit": unit,
                     "frac": ach / peak, "traffic": counter_traffic(wl.name, dom), "launches_per_step": launches,
                     "avg_launch_ms": stage_ms[dom] / launches},
        "stage_rooflines": {kk: {"bound": v[0], "achieved": v[1], "peak": v[2], "unit": v[3], "frac": v[1] / v[2],
                                 "traffic": counter_traffic(wl.name, kk), "launches_per_step": stage_launches[kk]}
                            for kk, v in kernels.items()},
        "stages_ms": stage_ms,
        "path_roofline": {"t_roof_ms": t_roof * 1e3, "frac": t_roof * 1e3 / ms_per_step},
        "staged_equals_fused": same,
    }
    if not (args.no_cpu or args.fused_only):
        print(f"[bench] CPU oracle baseline on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows)
        print("[bench] CPU oracle baseline done", file=sys.stderr, flush=True)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


def paged_prefill_work(wl):
    """Algorithmic work of one chunked paged-prefill call (every chunk row's
    causal candidates within its own sequence)."""
    import numpy as np
    from dsa_inputs import configs
    _, seq, pos = configs.chunk_rows(wl)
    n = (pos + 1).astype(np.float64)
    T = len(pos)
    pairs = n.sum()
    sel = np.minimum(n, wl.k).sum()
    keys = float(sum(wl.ctxs))
    return dict(pairs=pairs, selected=sel, idx_flops=pairs * 2 * wl.H_I * wl.d_I,
                mla_flops=sel * 2 * wl.H * (wl.D_qk + wl.D_v),
                idx_bytes=T * (wl.H_I * wl.d_I + 4 * wl.H_I) + keys * wl.d_I, topk_bytes=T * wl.k * 4,
                mla_bytes=T * (wl.H * wl.D_qk * 2 + wl.H * wl.D_v * 4 + wl.H * 4) + sel * wl.D_qk * 2 + T * wl.k * 4)


def bench_paged_prefill(args, wl):
    """Chunked prefill of several sequences into a paged cache: one
    dsa_forward_prefill_paged call per step, timed as the prefill (phase A: K
    calls; phase B: K calls with the library's launch events)."""
    import numpy as np
    import torch

    import oracle
    import sparse_attention_long_08_amd as dsa
    from dsa_inputs import configs, device

    dsa.load()
    T, k = wl.T, wl.k
    print(f"[bench] generating {wl.name} inputs on the GPU", file=sys.stderr, flush=True)
    inp = device.make_paged_prefill_inputs(wl)
    q_start, seq, pos = configs.chunk_rows(wl)
    ctx = inp["ctx_len"]
    pt = inp["page_table"]
    nb = dsa.dsa_forward_prefill_paged_workspace_bytes(T, int(ctx.max()), wl.H, wl.D_v, k)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, wl.H, wl.D_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, wl.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def fused():
        dsa.dsa_forward_prefill_paged(inp["q_idx"], inp["w"], inp["k_pool"], inp["q"], inp["kv_pool"], inp["n_pages"],
                                      pt, pt.shape[1], wl.page, q_start, ctx, wl.B, wl.H_I, wl.d_I, wl.H, wl.D_qk,
                                      wl.D_v, k, wl.scale, idx, out, lse, ws, nb)

    for _ in range(args.warmup):
        fused()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        fused()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    gpu_ms_per_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} paged prefill steps done: {ms_per_step:.1f} ms per step", file=sys.stderr,
          flush=True)
    rec_t, ev_ms_per_step = launch_times(dsa, torch, stream, fused, args.steps)
    stage_ms = {"indexer": rec_t["indexer"][0] / args.steps, "topk": rec_t["topk"][0] / args.steps,
                "sparse_mla": rec_t["attention"][0] / args.steps}
    stage_launches = {"indexer": rec_t["indexer"][1] // args.steps, "topk": rec_t["topk"][1] // args.steps,
                      "sparse_mla": rec_t["attention"][1] // args.steps}
    w = paged_prefill_work(wl)
    t_roof = w["idx_flops"] / (PEAK_FP8_TFLOPS * 1e12) + w["mla_flops"] / (PEAK_BF16_TFLOPS * 1e12)
    kernels = {
        "sparse_mla": ("mfma", w["mla_flops"] / (stage_ms["sparse_mla"] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
        # priced at the FP8 peak like the contiguous prefill; the chunked paged call scores on the
        # exact (bf16 MFMA) route, whose own peak is half that (frac_vs_bf16_peak)
        "indexer": ("mfma", w["idx_flops"] / (stage_ms["indexer"] * 1e-3) / 1e12, PEAK_FP8_TFLOPS, "TFLOP/s"),
        "topk": ("hbm", w["topk_bytes"] / (stage_ms["topk"] * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"),
    }
    dom = max(stage_ms, key=stage_ms.get)
    bound, ach, peak, unit = kernels[dom]
    rec = {
        "metric": "DSA chunked paged prefill query-tokens/s (indexer+topk+sparse MLA); %roofline",
        "value": T / (ms_per_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "gpu_ms_per_step": gpu_ms_per_step,
        "ms_per_step_with_launch_events": ev_ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator, device-resident)",
        "config": {"workload": wl.name, "B": wl.B, "ctx": list(wl.ctxs), "chunk": list(wl.chunks), "k": k,
                   "H_I": wl.H_I, "H": wl.H, "page": wl.page, "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": bound, "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
                     "traffic": counter_traffic(wl.name, dom), "launches_per_step": stage_launches[dom],
                     "avg_launch_ms": stage_ms[dom] / max(stage_launches[dom], 1),
                     "frac_vs_bf16_peak": (ach / PEAK_BF16_TFLOPS) if dom == "indexer" else None},
        "stages_ms": stage_ms,
        "path_roofline": {"t_roof_ms": t_roof * 1e3, "frac": t_roof * 1e3 / ms_per_step},
    }
    del inp, ws, idx, out, lse
    if args.no_cpu or args.fused_only:
        rec["cpu_baseline"] = None
    else:
        rows = configs.sample_rows(wl, max(1, args.cpu_rows // 4))
        print(f"[bench] CPU oracle baseline on {len(rows)} rows", file=sys.stderr, flush=True)
        keys = {b: configs.k_idx_bytes(wl, b, np.arange(int(wl.ctxs[b]))) for b in set(int(seq[r]) for r in rows)}
        t1 = time.perf_counter()
        for r in rows:
            oracle.paged_prefill_row(wl, int(seq[r]), int(pos[r]), keys[int(seq[r])])
        dt = time.perf_counter() - t1
        rec["cpu_baseline"] = {"value": len(rows) / dt, "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{len(rows)} seeded-random query rows of {wl.name}, indexer+top-k+"
                                         f"attention per row over its own sequence, single-threaded C oracle in "
                                         f"fp64, {dt:.1f} s"}
    print(json.dumps(rec))


def kl_cpu_baseline(wl, rows: int):
    """The oracle's KL loss (single thread) on `rows` seeded-random query rows; the
    oracle's own scores and selection feed it and are computed outside the timed part."""
    import numpy as np
    import oracle
    from dsa_inputs import configs
    sample = configs.sample_rows(wl, rows)
    keys = configs.k_idx_bytes(wl, 0, np.arange(int(sample.max()) + 1))
    jobs = []
    for t in sample:
        r = oracle.prefill_row(wl, int(t), keys)
        sel = r["idx"][r["idx"] >= 0]
        jobs.append((configs.q_bf16(wl, [int(t)])[0], oracle.gather_kv(wl, 0, r["idx"]), r["scores"][sel]))
    t0 = time.perf_counter()
    for q, kv_rows, isc in jobs:
        oracle.indexer_kl_row(q, kv_rows, wl.scale, isc)
    dt = time.perf_counter() - t0
    return {"value": len(sample) / dt, "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(sample)} seeded-random query rows of {wl.name} (positions "
                      f"{int(sample.min())}..{int(sample.max())}), KL loss per row on the oracle's own "
                      f"selection, single-threaded C oracle in fp64, {dt:.1f} s"}


def bench_dense_kl(args, wl):
    """Dense warm-up indexer KL loss ("DeepSeek-V3.2" walk-through §2.3.1) over
    every query row of a prefill workload: one fused dsa_dense_warmup_loss call
    per step (indexer scores over row tiles, then the dense KL kernel on each
    tile), timed in the two phases of the prefill bench."""
    import numpy as np
    import torch

    import oracle
    import sparse_attention_long_08_amd as dsa
    from dsa_inputs import configs, device

    dsa.load()
    T, N, H = wl.T, wl.N, wl.H
    print(f"[bench] generating {wl.name} inputs on the GPU", file=sys.stderr, flush=True)
    inp = device.make_prefill_inputs(wl)
    stream = torch.cuda.current_stream()
    nb = dsa.dsa_dense_warmup_loss_workspace_bytes(T, N)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    kl = torch.empty((T,), dtype=torch.float32, device="cuda")

    def fused():
        dsa.dsa_dense_warmup_loss(inp["q_idx"], inp["w"], inp["k_idx"], inp["q"], inp["kv"], T, N, wl.H_I, wl.d_I, H,
                                  wl.D_qk, 0, wl.scale, kl, None, ws, nb)

    for _ in range(args.warmup):
        fused()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        fused()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    print(f"[bench] {args.steps} dense warm-up loss steps done: {ms_per_step:.1f} ms per step", file=sys.stderr,
          flush=True)
    rec_t, ev_ms_per_step = launch_times(dsa, torch, stream, fused, args.steps)
    stage_ms = {"indexer": rec_t["indexer"][0] / args.steps, "dense_kl": rec_t["dense_kl"][0] / args.steps}
    launches = rec_t["dense_kl"][1] // args.steps
    w = algorithmic_work(wl, T)
    # the loss needs every causal logit once (2*H*D_qk flop per pair); the kernel
    # computes them twice (once for the dense lse, once for the divergence)
    flops = w["pairs"] * 2 * H * wl.D_qk
    ach = flops / (stage_ms["dense_kl"] * 1e-3) / 1e12
    rec = {
        "metric": "DSA dense warm-up indexer KL loss query-tokens/s",
        "value": T / (ms_per_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "gpu_ms_per_step": e0.elapsed_time(e1) / args.steps,
        "ms_per_step_with_launch_events": ev_ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator, device-resident)",
        "config": {"workload": wl.name, "L": T, "H_I": wl.H_I, "H": H, "D_qk": wl.D_qk, "causal": True,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "dense_kl", "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                     "traffic": counter_traffic(wl.name, "dense_kl"), "launches_per_step": launches, "avg_launch_ms": stage_ms["dense_kl"] / max(launches, 1),
                     "mfma_issued_tflops": 2 * ach},
        "stages_ms": stage_ms,
    }
    del inp, ws, kl
    if args.no_cpu or args.fused_only:
        rec["cpu_baseline"] = None
    else:
        rows = configs.sample_rows(wl, max(1, args.cpu_rows // 15))
        keys = configs.k_idx_bytes(wl, 0, np.arange(int(rows.max()) + 1))
        print(f"[bench] CPU oracle baseline on {len(rows)} rows", file=sys.stderr, flush=True)
        t1 = time.perf_counter()
        for t in rows:
            oracle.dense_kl_row(wl, int(t), keys)
        dt = time.perf_counter() - t1
        rec["cpu_baseline"] = {"value": len(rows) / dt, "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{len(rows)} seeded-random query rows of {wl.name} (positions "
                                         f"{int(rows.min())}..{int(rows.max())}), indexer row + dense attention "
                                         f"lse + KL over all causal keys, single-threaded C oracle in fp64, "
                                         f"{dt:.1f} s"}
    print(json.dumps(rec))


def bench_bwd(args, wl):
    """Sparse MLA-MQA attention backward (the gradient the sparse training stage,
    "DeepSeek-V3.2" walk-through §2.3.2, takes through the attention of §2.1.2)
    over every query row of a prefill workload.  The selected sets, out and lse
    come from one fused forward call (untimed); each timed step is one
    dsa_sparse_mla_bwd call (dq kernel, then dkv kernel, per 8192-query tile),
    timed in the two phases of the prefill bench."""
    import torch

    import sparse_attention_long_08_amd as dsa
    from dsa_inputs import device, gen

    dsa.load()
    T, N, k, H = wl.T, wl.N, wl.k, wl.H
    print(f"[bench] generating {wl.name} inputs on the GPU", file=sys.stderr, flush=True)
    inp = device.make_prefill_inputs(wl)
    stream = torch.cuda.current_stream()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, wl.D_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    nbf = dsa.dsa_forward_prefill_workspace_bytes(T, N, H, wl.D_v, k)
    wsf = torch.empty(max(nbf, 256), dtype=torch.uint8, device="cuda")
    dsa.dsa_forward_prefill(inp["q_idx"], inp["w"], inp["k_idx"], inp["q"], inp["kv"], T, N, wl.H_I, wl.d_I, H,
                            wl.D_qk, wl.D_v, k, 0, wl.scale, idx, out, lse, wsf, nbf)
    del wsf
    dout = torch.empty((T, H, wl.D_v), dtype=torch.uint16, device="cuda")
    device.fill(dout, T, H * wl.D_v, device.BF16_NORMAL, wl.seed, gen.STREAM_DOUT)
    dq = torch.empty((T, H, wl.D_qk), dtype=torch.float32, device="cuda")
    dkv = torch.empty((N, wl.D_qk), dtype=torch.float32, device="cuda")
    nb = dsa.dsa_sparse_mla_bwd_workspace_bytes(T, N, H, k)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")

    def fused():
        dsa.dsa_sparse_mla_bwd(inp["q"], inp["kv"], idx, out, lse, dout, T, N, H, wl.D_qk, wl.D_v, k, wl.scale, dq,
                               dkv, ws, nb)

    for _ in range(args.warmup):
        fused()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        fused()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    print(f"[bench] {args.steps} backward steps done: {ms_per_step:.1f} ms per step", file=sys.stderr, flush=True)
    rec_t, ev_ms_per_step = launch_times(dsa, torch, stream, fused, args.steps)
    kinds = ("mla_bwd_dq", "mla_bwd_dkv", "mla_bwd_reduce")
    stage_ms = {kind: rec_t[kind][0] / args.steps for kind in kinds}
    w = algorithmic_work(wl, T)
    # per selected (query, entry) pair and head: the dq kernel forms the logits
    # (576), dP (512) and dq (576); the dkv kernel dS^T q (576) and P^T dO (512).
    # The row sums read each pair's bf16 addend row once and update dkv.
    flops = {"mla_bwd_dq": w["selected"] * 2 * H * (wl.D_qk + wl.D_v + wl.D_qk),
             "mla_bwd_dkv": w["selected"] * 2 * H * (wl.D_qk + wl.D_v)}
    red_bytes = w["selected"] * (wl.D_qk * 2 + 2 * 4 + 4)
    dom = max(stage_ms, key=stage_ms.get)
    launches = rec_t[dom][1] // args.steps
    if dom == "mla_bwd_reduce":
        bound, unit, peak = "hbm", "GB/s", PEAK_HBM_GBS
        ach = red_bytes / (stage_ms[dom] * 1e-3) / 1e9
    else:
        bound, unit, peak = "mfma", "TFLOP/s", PEAK_BF16_TFLOPS
        ach = flops[dom] / (stage_ms[dom] * 1e-3) / 1e12
    total_tf = sum(flops.values()) / (ms_per_step * 1e-3) / 1e12
    rec = {
        "metric": "DSA sparse MLA-MQA attention backward query-tokens/s",
        "value": T / (ms_per_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "gpu_ms_per_step": e0.elapsed_time(e1) / args.steps,
        "ms_per_step_with_launch_events": ev_ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator, device-resident; selection from the fused forward)",
        "config": {"workload": wl.name, "L": T, "k": k, "H": H, "D_qk": wl.D_qk, "D_v": wl.D_v, "causal": True,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": bound, "achieved": ach, "peak": peak, "unit": unit,
                     "frac": ach / peak, "traffic": counter_traffic(wl.name, dom),
                     "launches_per_step": launches, "avg_launch_ms": stage_ms[dom] / max(launches, 1)},
        "stages_ms": stage_ms,
        "step_tflops": total_tf,
    }
    del inp, ws, dq, dkv, out, lse, dout, idx
    rec["cpu_baseline"] = None if (args.no_cpu or args.fused_only) else bwd_cpu_baseline(wl, 50)
    print(json.dumps(rec))


def bwd_cpu_baseline(wl, rows: int):
    """The oracle (single thread) on `rows` seeded-random query rows of the
    backward: one query's gradient over its selected rows."""
    import numpy as np
    import oracle
    from dsa_inputs import configs
    pos = configs.sample_rows(wl, rows)
    q = configs.q_bf16(wl, pos)
    dO = configs.dout_bf16(wl, pos)
    sel = configs.random_selection(wl, pos)
    kvs = [configs.kv_bf16(wl, 0, s[s >= 0]) for s in sel]
    print(f"[bench] CPU oracle baseline on {len(pos)} rows", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(len(pos)):
        oracle.sparse_mla_bwd_row(q[i], kvs[i], dO[i], wl.scale)
    dt = time.perf_counter() - t0
    return {"value": len(pos) / dt, "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(pos)} seeded-random query rows of {wl.name} (positions {int(pos.min())}.."
                      f"{int(pos.max())}), gradient of one query over its selected rows (k = {wl.k}, H = {wl.H}), "
                      f"single-threaded C oracle in fp64, {dt:.1f} s"}


def bench_kl(args, wl):
    """Sparse-stage indexer KL loss over every query row of a prefill workload.  Per
    row tile the indexer scores and top-k are computed first (untimed); the
    attention LSE comes from one attention call over all rows (untimed); the
    timed part is the KL kernel over all tiles."""
    import numpy as np
    import torch

    import sparse_attention_long_08_amd as dsa
    from dsa_inputs import device

    dsa.load()
    T, N, k, H = wl.T, wl.N, wl.k, wl.H
    print(f"[bench] generating {wl.name} inputs on the GPU", file=sys.stderr, flush=True)
    inp = device.make_prefill_inputs(wl)
    stream = torch.cuda.current_stream()
    tile_rows, ld = dsa.dsa_forward_prefill_plan(T, N)
    n_tiles = (T + tile_rows - 1) // tile_rows
    scores = torch.empty((n_tiles, tile_rows, ld), dtype=torch.float32, device="cuda") if n_tiles * tile_rows * ld \
        * 4 <= (8 << 30) else None
    if scores is None:
        print("[bench] --kl keeps every score tile resident; this workload's tiles exceed 8 GiB", file=sys.stderr)
        sys.exit(2)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    for i in range(n_tiles):
        r0 = i * tile_rows
        tr = min(tile_rows, T - r0)
        dsa.dsa_indexer_scores(inp["q_idx"][r0:], inp["w"][r0:], inp["k_idx"], tr, N, wl.H_I, wl.d_I, r0,
                               scores[i], ld)
        dsa.dsa_topk(scores[i], ld, tr, N, r0, None, k, idx[r0:])
    out = torch.empty((T, H, wl.D_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    nb = dsa.dsa_sparse_mla_fwd_workspace_bytes(T, H, wl.D_v, k)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    dsa.dsa_sparse_mla_fwd(inp["q"], inp["kv"], idx, T, N, H, wl.D_qk, wl.D_v, k, wl.scale, out, lse, ws, nb)
    del out
    kl = torch.empty((T,), dtype=torch.float32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_tiles)]

    def step(record):
        for i in range(n_tiles):
            r0 = i * tile_rows
            tr = min(tile_rows, T - r0)
            if record:
                ev[2 * i].record(stream)
            dsa.dsa_indexer_kl_fwd(inp["q"][r0:], inp["kv"], idx[r0:], lse[r0:], scores[i], ld, tr, N, H,
                                   wl.D_qk, k, wl.scale, kl[r0:])
            if record:
                ev[2 * i + 1].record(stream)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    kl_ms = 0.0
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        kl_ms += sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n_tiles))
        print(f"[bench] KL step {s_ + 1}/{args.steps} done", file=sys.stderr, flush=True)
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kl_ms /= args.steps
    w = algorithmic_work(wl, T)
    flops = w["selected"] * 2 * H * wl.D_qk
    ach = flops / (kl_ms * 1e-3) / 1e12
    rec = {
        "metric": "DSA sparse-stage indexer KL loss query-tokens/s",
        "value": T / (kl_ms * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": kl_ms,
        "host_wall_ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator, device-resident)",
        "config": {"workload": wl.name, "L": T, "k": k, "H": H, "D_qk": wl.D_qk, "causal": True,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "indexer_kl", "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                     "traffic": counter_traffic(wl.name, "indexer_kl"), "launches_per_step": n_tiles,
                     "avg_launch_ms": kl_ms / n_tiles},
        "loss": float(kl.sum().item()),
    }
    if not args.no_cpu:
        print("[bench] CPU oracle baseline on 12 rows", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = kl_cpu_baseline(wl, 12)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


def decode_work(wl, ctx):
    """Algorithmic bytes of one decode step (every input read once, outputs written once)."""
    import numpy as np
    ctx = ctx.astype(np.float64)
    sel = np.minimum(ctx, wl.k).sum()
    idx_bytes = wl.B * (wl.H_I * wl.d_I + 4 * wl.H_I) + ctx.sum() * wl.d_I
    topk_bytes = wl.B * wl.k * 4
    mla_bytes = wl.B * (wl.H * wl.D_qk * 2 + wl.H * wl.D_v * 4 + wl.H * 4) + sel * wl.D_qk * 2
    idx_flops = ctx.sum() * 2 * wl.H_I * wl.d_I
    mla_flops = sel * 2 * wl.H * (wl.D_qk + wl.D_v)
    return dict(idx_bytes=idx_bytes, topk_bytes=topk_bytes, mla_bytes=mla_bytes, idx_flops=idx_flops,
                mla_flops=mla_flops, selected=sel, keys=ctx.sum())


def bench_decode(args, wl):
    import numpy as np
    import torch

    import sparse_attention_long_08_amd as dsa
    from dsa_inputs import configs, device

    dsa.load()
    B, k = wl.B, wl.k
    ctx = configs.ctx_lens(wl)
    max_ctx = int(ctx.max())
    print(f"[bench] generating {wl.name} inputs on the GPU", file=sys.stderr, flush=True)
    if wl.kind == "paged_decode":
        inp = device.make_paged_inputs(wl)
        k_pool, kv_pool, page_table, n_pages = inp["k_pool"], inp["kv_pool"], inp["page_table"], inp["n_pages"]
        max_pages = page_table.shape[1]
        nb = dsa.dsa_forward_decode_paged_workspace_bytes(B, max_ctx, wl.H, wl.D_v, k)
    else:
        inp = device.make_decode_inputs(wl)
        # the contiguous [B, N, dim] caches seen as pools of 64-token pages with an identity table
        max_pages = wl.N // wl.page
        n_pages = B * max_pages
        k_pool, kv_pool = inp["k_idx"], inp["kv"]
        page_table = torch.arange(n_pages, dtype=torch.int32, device="cuda").reshape(B, max_pages)
        nb = dsa.dsa_forward_decode_workspace_bytes(B, wl.N, wl.H, wl.D_v, k)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, wl.H, wl.D_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, wl.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def fused():
        if wl.kind == "paged_decode":
            dsa.dsa_forward_decode_paged(inp["q_idx"], inp["w"], k_pool, inp["q"], kv_pool, n_pages, page_table,
                                         max_pages, inp["ctx_len"], wl.page, B, max_ctx, wl.H_I, wl.d_I, wl.H,
                                         wl.D_qk, wl.D_v, k, wl.scale, idx, out, lse, ws, ws.numel())
        else:
            dsa.dsa_forward_decode(inp["q_idx"], inp["w"], inp["k_idx"], inp["q"], inp["kv"], inp["ctx_len"], B,
                                   wl.N, wl.H_I, wl.d_I, wl.H, wl.D_qk, wl.D_v, k, wl.scale, idx, out, lse, ws,
                                   ws.numel())

    # staged replay through the paged entry points, for per-kernel times
    ld = (max_ctx + 63) // 64 * 64
    scores = torch.empty((B, ld), dtype=torch.float32, device="cuda")
    s_idx = torch.empty_like(idx)
    s_out = torch.empty_like(out)
    s_lse = torch.empty_like(lse)
    mla_nb = dsa.dsa_sparse_mla_fwd_paged_workspace_bytes(B, wl.H, wl.D_v, k)
    mla_ws = torch.empty(max(mla_nb, 256), dtype=torch.uint8, device="cuda")

    def staged():
        dsa.dsa_indexer_scores_paged(inp["q_idx"], inp["w"], k_pool, n_pages, page_table, max_pages, inp["ctx_len"],
                                     wl.page, B, wl.H_I, wl.d_I, max_ctx, scores, ld)
        dsa.dsa_topk(scores, ld, B, max_ctx, 0, inp["ctx_len"], k, s_idx)
        dsa.dsa_sparse_mla_fwd_paged(inp["q"], kv_pool, n_pages, page_table, max_pages, inp["ctx_len"], wl.page,
                                     s_idx, B, wl.H, wl.D_qk, wl.D_v, k, wl.scale, s_out, s_lse, mla_ws, mla_nb)

    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()
    # phase A, the timed region: K fused calls
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        fused()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_per_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} fused decode steps done", file=sys.stderr, flush=True)
    # phase B: per-kernel-stage durations from the library's launch events
    rec_t, ev_ms_per_step = launch_times(dsa, torch, stream, fused, args.steps)
    stage_ms = {"indexer": rec_t["indexer"][0] / args.steps, "topk": rec_t["topk"][0] / args.steps,
                "sparse_mla": rec_t["attention"][0] / args.steps}
    graph = decode_graph_times(torch, stream, fused, (idx, out, lse), args.steps) if not args.no_graph else None

    # the same step through the single-stage paged calls (untimed) must give the same bits
    same = None
    if not args.fused_only:
        staged()
        torch.cuda.synchronize()
        same = bool(torch.equal(s_idx, idx) and torch.equal(s_out, out) and torch.equal(s_lse, lse))

    w = decode_work(wl, ctx)
    total_bytes = w["idx_bytes"] + w["topk_bytes"] + w["mla_bytes"]
    t_roof = max(total_bytes / (PEAK_HBM_GBS * 1e9),
                 w["idx_flops"] / (PEAK_FP8_TFLOPS * 1e12) + w["mla_flops"] / (PEAK_BF16_TFLOPS * 1e12))
    kernels = {
        "indexer": ("hbm", w["idx_bytes"] / (stage_ms["indexer"] * 1e-3) / 1e9),
        "topk": ("hbm", w["topk_bytes"] / (stage_ms["topk"] * 1e-3) / 1e9),
        "sparse_mla": ("hbm", w["mla_bytes"] / (stage_ms["sparse_mla"] * 1e-3) / 1e9),
    }
    dom = max(stage_ms, key=stage_ms.get)
    bound, ach = kernels[dom]
    rec = {
        "metric": "DSA decode query-tokens/s (indexer+topk+sparse MLA); %roofline",
        "value": B / (ms_per_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "host_wall_ms_per_step": wall_ms,
        "ms_per_step_with_launch_events": ev_ms_per_step,
        "hip_graph": graph,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator, device-resident)",
        "config": {"workload": wl.name, "B": B, "max_ctx": max_ctx, "mean_ctx": float(ctx.mean()), "k": k,
                   "H_I": wl.H_I, "H": wl.H, "paged": wl.kind == "paged_decode"},
        "roofline": {"kernel": dom, "bound": bound, "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach / PEAK_HBM_GBS, "traffic": counter_traffic(wl.name, dom), "launches_per_step": 1,
                     "avg_launch_ms": stage_ms[dom]},
        # every stage against the HBM peak: `achieved` from its algorithmic bytes, `counter_gbs` from the
        # bytes the HBM counters read for it (the key stream of the indexer, the gather of the attention)
        "stage_rooflines": {kk: {"bound": b, "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": a / PEAK_HBM_GBS, "traffic": counter_traffic(wl.name, kk),
                                 "counter_gbs": (None if counter_traffic(wl.name, kk) is None
                                                 else counter_traffic(wl.name, kk) / (stage_ms[kk] * 1e-3) / 1e9),
                                 "launches_per_step": 1}
                            for kk, (b, a) in kernels.items()},
        "stages_ms": stage_ms,
        "path_roofline": {"t_roof_ms": t_roof * 1e3, "algorithmic_bytes": total_bytes,
                          "frac": t_roof * 1e3 / ms_per_step},
        "staged_equals_fused": same,
        "cpu_baseline": None,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
