"""Benchmark of the DSA forward hot path on one MI355X.

One step = the whole path (lightning indexer -> top-k -> sparse MLA-MQA) over
all query rows of the 128K-context causal prefill (L = 131072, k = 2048,
H_I = 64 FP8 indexer heads, 128 MLA heads over 576-d bf16 latents), with
inputs already resident in HBM.  The step replays dsa_forward_prefill stage by
stage through the C ABI (same kernels, same row tiling, same stream), with HIP
events around every launch to time each kernel; the staged outputs are checked
bit-identical to one fused call.

Prints one JSON line: query-tokens/s, the dominant kernel's roofline, and the
CPU oracle's rate on a bounded sample of the same workload.
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
    """The oracle (single thread) on `rows` seeded-random query rows."""
    import numpy as np
    import oracle
    from dsa_inputs import configs
    sample = configs.sample_rows(wl, rows)
    keys = configs.k_idx_bytes(wl, 0, np.arange(int(sample.max()) + 1))
    t0 = time.perf_counter()
    for t in sample:
        oracle.prefill_row(wl, int(t), keys)
    dt = time.perf_counter() - t0
    return {"value": len(sample) / dt, "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(sample)} seeded-random query rows of {wl.name} (positions "
                      f"{int(sample.min())}..{int(sample.max())}), indexer+top-k+attention per row, "
                      f"single-threaded C oracle in fp64, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="prefill_L128k")
    ap.add_argument("--cpu-rows", type=int, default=6)
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the DSA path here is a single-GPU kernel library).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_long_08_amd as dsa
    from dsa_inputs import configs, device

    dsa.load()
    wl = configs.WORKLOADS[args.workload]
    assert wl.kind == "prefill"
    T, N, k = wl.T, wl.N, wl.k
    print(f"[bench] generating {wl.name} inputs on the GPU", file=sys.stderr, flush=True)
    inp = device.make_prefill_inputs(wl)
    stream = torch.cuda.current_stream()
    tile_rows, ld = dsa.dsa_forward_prefill_plan(T, N)
    scores = torch.empty((tile_rows, ld), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, wl.H, wl.D_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, wl.H), dtype=torch.float32, device="cuda")
    mla_ws_bytes = dsa.dsa_sparse_mla_fwd_workspace_bytes(T, wl.H, wl.D_v, k)
    mla_ws = torch.empty(max(mla_ws_bytes, 256), dtype=torch.uint8, device="cuda")
    n_tiles = (T + tile_rows - 1) // tile_rows

    ev = {name: [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_tiles)] for name in ("idx", "topk")}
    ev_mla = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def step(record: bool):
        for i in range(n_tiles):
            r0 = i * tile_rows
            tr = min(tile_rows, T - r0)
            if record:
                ev["idx"][2 * i].record(stream)
            dsa.dsa_indexer_scores(inp["q_idx"][r0:], inp["w"][r0:], inp["k_idx"], tr, N, wl.H_I, wl.d_I, r0,
                                   scores, ld)
            if record:
                ev["idx"][2 * i + 1].record(stream)
                ev["topk"][2 * i].record(stream)
            dsa.dsa_topk(scores, ld, tr, N, r0, None, k, idx[r0:])
            if record:
                ev["topk"][2 * i + 1].record(stream)
        if record:
            ev_mla[0].record(stream)
        dsa.dsa_sparse_mla_fwd(inp["q"], inp["kv"], idx, T, N, wl.H, wl.D_qk, wl.D_v, k, wl.scale, out, lse, mla_ws,
                               mla_ws_bytes)
        if record:
            ev_mla[1].record(stream)

    # one fused call: the staged replay must reproduce it bit for bit
    print("[bench] fused reference call", file=sys.stderr, flush=True)
    fws_bytes = dsa.dsa_forward_prefill_workspace_bytes(T, N, wl.H, wl.D_v, k)
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device="cuda")
    f_idx = torch.empty_like(idx)
    f_lse = torch.empty_like(lse)
    f_out = torch.empty_like(out)
    t0 = time.perf_counter()
    dsa.dsa_forward_prefill(inp["q_idx"], inp["w"], inp["k_idx"], inp["q"], inp["kv"], T, N, wl.H_I, wl.d_I, wl.H,
                            wl.D_qk, wl.D_v, k, 0, wl.scale, f_idx, f_out, f_lse, fws, fws_bytes)
    torch.cuda.synchronize()
    fused_ms = (time.perf_counter() - t0) * 1e3
    del fws
    print(f"[bench] fused call {fused_ms:.1f} ms; warmup {args.warmup}", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    stage_ms = {"indexer": 0.0, "topk": 0.0, "sparse_mla": 0.0}
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        stage_ms["indexer"] += sum(ev["idx"][2 * i].elapsed_time(ev["idx"][2 * i + 1]) for i in range(n_tiles))
        stage_ms["topk"] += sum(ev["topk"][2 * i].elapsed_time(ev["topk"][2 * i + 1]) for i in range(n_tiles))
        stage_ms["sparse_mla"] += ev_mla[0].elapsed_time(ev_mla[1])
        print(f"[bench] step {s + 1}/{args.steps} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    stage_ms = {kk: v / args.steps for kk, v in stage_ms.items()}

    same = bool(torch.equal(f_idx, idx) and torch.equal(f_lse, lse) and torch.equal(f_out, out))
    del f_out
    w = algorithmic_work(wl, T)
    t_roof = max(w["idx_flops"] / (PEAK_FP8_TFLOPS * 1e12) + w["mla_flops"] / (PEAK_BF16_TFLOPS * 1e12),
                 (w["idx_bytes"] + w["topk_bytes"] + w["mla_bytes"]) / (PEAK_HBM_GBS * 1e9))
    kernels = {
        "sparse_mla": ("mfma", w["mla_flops"] / (stage_ms["sparse_mla"] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
        "indexer": ("mfma", w["idx_flops"] / (stage_ms["indexer"] * 1e-3) / 1e12, PEAK_FP8_TFLOPS, "TFLOP/s"),
        "topk": ("hbm", w["topk_bytes"] / (stage_ms["topk"] * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"),
    }
    dom = max(stage_ms, key=stage_ms.get)
    bound, ach, peak, unit = kernels[dom]
    launches = 1 if dom == "sparse_mla" else n_tiles
    rec = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3(indexer)+bf16(attention), fp32 accumulate",
        "data": "synthetic (seeded counter-based generator, device-resident)",
        "config": {"workload": wl.name, "L": T, "k": k, "H_I": wl.H_I, "d_I": wl.d_I, "H": wl.H,
                   "D_qk": wl.D_qk, "D_v": wl.D_v, "causal": True, "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": bound, "achieved": ach, "peak": peak, "unit": unit,
                     "frac": ach / peak, "traffic": None, "launches_per_step": launches,
                     "avg_launch_ms": stage_ms[dom] / launches},
        "stages_ms": stage_ms,
        "path_roofline": {"t_roof_ms": t_roof * 1e3, "frac": t_roof * 1e3 / ms_per_step},
        "fused_call_ms": fused_ms,
        "staged_equals_fused": same,
    }
    if not args.no_cpu:
        print(f"[bench] CPU oracle baseline on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
