"""GPU parity of the sparse-stage indexer KL loss ("DeepSeek-V3.2" walk-through
§2.3.2) against the CPU oracle, on the GPU's own index sets, attention LSE
and indexer scores (stage isolation)."""
import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import configs, device, gen
from dsa_run import ws_tensor

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _check_kl(g, o, what):
    assert abs(g - o) <= 1e-4 + 1e-3 * abs(o), f"{what}: gpu {g} oracle {o}"


def _rand_idx(rng, T, k, n):
    idx = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        m = int(rng.integers(0, min(k, n) + 1)) if t % 5 else min(k, n)
        idx[t, :m] = np.sort(rng.choice(n, size=m, replace=False))
    idx[0, :] = -1  # an empty row
    return idx


@pytest.mark.parametrize("T,k,H", [(3, 2048, 128), (40, 300, 128), (17, 100, 8), (9, 70, 40)])
def test_indexer_kl_against_oracle(dsa, T, k, H):
    name = "tiny_prefill_L256" if H == 8 else "prefill_L32k"
    wl0 = configs.WORKLOADS[name]
    N = 4096
    wl = configs.Workload(**{**wl0.__dict__, "H": H, "N": N})
    _case(f"indexer_kl T={T} k={k} H={H} N={N}")
    rng = np.random.default_rng(T * 7 + k)
    q = torch.empty((T, H, 576), dtype=torch.uint16, device="cuda")
    kv = torch.empty((N, 576), dtype=torch.uint16, device="cuda")
    device.fill(q, T, H * 576, device.BF16_NORMAL, wl.seed, gen.STREAM_Q)
    device.fill(kv, N, 576, device.BF16_NORMAL, wl.seed, gen.STREAM_KV, div=wl.kv_div)
    idx = _rand_idx(rng, T, k, N)
    idx[1, 0] = N + 5  # out-of-range entries are skipped
    ld = N + 8
    scores = (rng.standard_normal((T, ld)) * 2.0).astype(np.float32)
    idx_d = torch.from_numpy(idx).cuda()
    out = torch.empty((T, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    nb = dsa.dsa_sparse_mla_fwd_workspace_bytes(T, H, 512, k)
    ws = ws_tensor(nb)
    dsa.dsa_sparse_mla_fwd(q, kv, idx_d, T, N, H, 576, 512, k, wl.scale, out, lse, ws, nb)
    kl = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_kl_fwd(q, kv, idx_d, lse, torch.from_numpy(scores).cuda(), ld, T, N, H, 576, k, wl.scale, kl)
    torch.cuda.synchronize()
    g = kl.cpu().numpy()
    qh = configs.q_bf16(wl, np.arange(T))
    for t in range(T):
        ok = (idx[t] >= 0) & (idx[t] < N)
        sel = idx[t][ok]
        o = oracle.indexer_kl_row(qh[t], configs.kv_bf16(wl, 0, sel), wl.scale, scores[t, sel].astype(np.float64))
        _check_kl(float(g[t]), o, f"row {t}")
    assert g[0] == 0.0  # empty row


@pytest.mark.parametrize("name,rows", [("tiny_prefill_L256", None), ("prefill_L32k", (30000, 256))])
def test_indexer_kl_chain(dsa, name, rows):
    """Indexer scores -> top-k -> attention LSE -> KL through the C ABI, each
    on the previous call's GPU output, checked row by row against the oracle."""
    wl = configs.WORKLOADS[name]
    r0, T = (0, wl.T) if rows is None else rows
    _case(f"indexer_kl chain {name} rows {r0}..{r0 + T}")
    inp = device.make_prefill_inputs(wl)
    N, k, H = wl.N, wl.k, wl.H
    ld = N + 8
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores(inp["q_idx"][r0:], inp["w"][r0:], inp["k_idx"], T, N, wl.H_I, wl.d_I, r0, scores, ld)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(scores, ld, T, N, r0, None, k, idx)
    out = torch.empty((T, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    nb = dsa.dsa_sparse_mla_fwd_workspace_bytes(T, H, 512, k)
    ws = ws_tensor(nb)
    q = inp["q"][r0:r0 + T].contiguous()
    dsa.dsa_sparse_mla_fwd(q, inp["kv"], idx, T, N, H, 576, 512, k, wl.scale, out, lse, ws, nb)
    kl = torch.empty((T,), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_kl_fwd(q, inp["kv"], idx, lse, scores, ld, T, N, H, 576, k, wl.scale, kl)
    torch.cuda.synchronize()
    g = kl.cpu().numpy()
    g_idx = idx.cpu().numpy()
    g_sc = scores.cpu().numpy()
    check = range(T) if rows is None else list(range(0, 8)) + list(range(T - 8, T))
    qh = configs.q_bf16(wl, r0 + np.asarray(list(check)))
    for i, t in enumerate(check):
        sel = g_idx[t][g_idx[t] >= 0]
        o = oracle.indexer_kl_row(qh[i], configs.kv_bf16(wl, 0, sel), wl.scale, g_sc[t, sel].astype(np.float64))
        _check_kl(float(g[t]), o, f"row {r0 + t}")
    assert np.all(np.isfinite(g)) and np.all(g >= -1e-5)


# ------------------------------------------------------------------ dense warm-up loss (§2.3.1)
def _dense_warmup(dsa, wl, inp):
    T, N = wl.T, wl.N
    nb = dsa.dsa_dense_warmup_loss_workspace_bytes(T, N)
    ws = ws_tensor(nb)
    kl = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((T, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_dense_warmup_loss(inp["q_idx"], inp["w"], inp["k_idx"], inp["q"], inp["kv"], T, N, wl.H_I, wl.d_I, wl.H,
                              wl.D_qk, 0, wl.scale, kl, lse, ws, nb)
    torch.cuda.synchronize()
    return kl.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny_prefill_L256", "prefill_L32k"])
def test_dense_warmup_loss_against_oracle(dsa, name):
    """The fused dense warm-up loss (indexer over row tiles, then the dense KL
    kernel) against the oracle: every row of the tiny workload, and the first,
    block-edge, tile-edge, last and seeded-random rows of the 32K prefill."""
    from oracle import jobs
    wl = configs.WORKLOADS[name]
    _case(f"dense warm-up loss {name}")
    inp = device.make_prefill_inputs(wl)
    g_kl, g_lse = _dense_warmup(dsa, wl, inp)
    del inp
    torch.cuda.empty_cache()
    if wl.T <= 256:
        rows = np.arange(wl.T)
    else:
        rows = np.unique(np.concatenate([configs.sample_rows(wl, 16), [0, 1, 31, 32, 33, 2047, 2048, 8191, 8192,
                                                                        wl.T - 1]]))
    results = jobs.run(jobs.dense_kl_job, [(name, int(t)) for t in rows])
    for t, r in zip(rows, results):
        _check_kl(float(g_kl[t]), r["kl"], f"{name} row {t}")
        assert np.max(np.abs(g_lse[t] - r["lse"])) <= 1e-3, f"{name} row {t} lse"
    print(f"[{name}] {len(rows)} dense warm-up rows checked", flush=True)


def test_dense_kl_equals_sparse_kl_over_all_keys(dsa):
    """With S_t = every causal key and the dense lse, the sparse-stage kernel
    computes the same loss as the dense kernel (two kernels, one definition)."""
    wl = configs.WORKLOADS["tiny_prefill_L256"]
    _case("dense KL vs sparse KL over all keys")
    T, N, H = wl.T, wl.N, wl.H
    inp = device.make_prefill_inputs(wl)
    ld = N
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores(inp["q_idx"], inp["w"], inp["k_idx"], T, N, wl.H_I, wl.d_I, 0, scores, ld)
    kl_d = torch.empty((T,), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_dense_kl_fwd(inp["q"], inp["kv"], scores, ld, T, N, 0, H, wl.D_qk, wl.scale, kl_d, lse)
    k = N
    idx = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        idx[t, : t + 1] = np.arange(t + 1)
    kl_s = torch.empty((T,), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_kl_fwd(inp["q"], inp["kv"], torch.from_numpy(idx).cuda(), lse, scores, ld, T, N, H, wl.D_qk, k,
                           wl.scale, kl_s)
    torch.cuda.synchronize()
    a, b = kl_d.cpu().numpy(), kl_s.cpu().numpy()
    assert np.all(np.abs(a - b) <= 1e-6 + 1e-5 * np.abs(b)), np.max(np.abs(a - b))


def test_dense_warmup_loss_chunk_matches_full_sequence(dsa):
    """The dense warm-up loss of rows q_pos0 .. T-1 computed as a chunk (queries
    starting at q_pos0 over the same keys) equals those rows of the full call."""
    wl = configs.WORKLOADS["tiny_prefill_L256"]
    _case("dense warm-up loss: chunk at q_pos0 = 100 against the full sequence")
    inp = device.make_prefill_inputs(wl)
    g_kl, g_lse = _dense_warmup(dsa, wl, inp)
    T, N, q0 = wl.T, wl.N, 100
    nb = dsa.dsa_dense_warmup_loss_workspace_bytes(T - q0, N)
    ws = ws_tensor(nb)
    kl = torch.empty((T - q0,), dtype=torch.float32, device="cuda")
    lse = torch.empty((T - q0, wl.H), dtype=torch.float32, device="cuda")
    dsa.dsa_dense_warmup_loss(inp["q_idx"][q0:], inp["w"][q0:], inp["k_idx"], inp["q"][q0:], inp["kv"], T - q0, N,
                              wl.H_I, wl.d_I, wl.H, wl.D_qk, q0, wl.scale, kl, lse, ws, nb)
    torch.cuda.synchronize()
    assert np.array_equal(kl.cpu().numpy(), g_kl[q0:])
    assert np.array_equal(lse.cpu().numpy(), g_lse[q0:])
