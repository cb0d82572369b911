"""Stage-level GPU parity: each C-ABI call against the CPU oracle on seeded
inputs, covering several tiles, ragged tails and edge cases."""
import numpy as np
import pytest
import torch

import oracle
from oracle import jobs
from dsa_inputs import configs, device, gen
from dsa_run import check_attention, check_scores, ws_tensor

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


# ------------------------------------------------------------------ generator
def test_device_generator_matches_host(dsa):
    for name in ("tiny_prefill_L256", "prefill_L32k"):
        wl = configs.WORKLOADS[name]
        _case(f"generator {name}")
        rows = 40
        inp = {}
        q_idx = torch.empty((rows, wl.H_I, wl.d_I), dtype=torch.uint8, device="cuda")
        w = torch.empty((rows, wl.H_I), dtype=torch.float32, device="cuda")
        k_idx = torch.empty((rows, wl.d_I), dtype=torch.uint8, device="cuda")
        q = torch.empty((rows, wl.H, wl.D_qk), dtype=torch.uint16, device="cuda")
        kv = torch.empty((rows, wl.D_qk), dtype=torch.uint16, device="cuda")
        device._fill_common(wl, q_idx, w, k_idx, q, kv, rows, rows)
        torch.cuda.synchronize()
        r = np.arange(rows)
        assert np.array_equal(q_idx.cpu().numpy(), configs.q_idx_bytes(wl, r))
        assert np.array_equal(w.cpu().numpy(), configs.w_f32(wl, r))
        assert np.array_equal(k_idx.cpu().numpy(), configs.k_idx_bytes(wl, 0, r))
        assert np.array_equal(q.cpu().numpy().view(np.uint16), configs.q_bf16(wl, r))
        assert np.array_equal(kv.cpu().numpy().view(np.uint16), configs.kv_bf16(wl, 0, r))
    # paged pools through a row map
    wl = configs.WORKLOADS["paged_decode_b32_ctx4k_128k"]
    _case("generator paged rowmap")
    rowmap = np.array([5 * wl.S + 7, 3, 2 * wl.S + 70000, 0], dtype=np.int64)
    kv = torch.empty((4, wl.D_qk), dtype=torch.uint16, device="cuda")
    device.fill(kv, 4, wl.D_qk, device.BF16_NORMAL, wl.seed, gen.STREAM_KV, div=wl.kv_div,
                rowmap=torch.from_numpy(rowmap).cuda())
    torch.cuda.synchronize()
    ref = np.stack([configs.kv_bf16(wl, int(r // wl.S), [int(r % wl.S)])[0] for r in rowmap])
    assert np.array_equal(kv.cpu().numpy().view(np.uint16), ref)


# ------------------------------------------------------------------ indexer
def test_indexer_tiny_exact(dsa):
    wl = configs.WORKLOADS["tiny_prefill_L256"]
    _case("indexer tiny L=256 exact")
    inp = device.make_prefill_inputs(wl)
    T, N = wl.T, wl.N
    ld = N + 4
    scores = torch.full((T, ld), 7.0, dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores(inp["q_idx"], inp["w"], inp["k_idx"], T, N, wl.H_I, wl.d_I, 0, scores, ld)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    keys = configs.k_idx_bytes(wl, 0, np.arange(N))
    for t in range(T):
        o = oracle.indexer_row(configs.q_idx_bytes(wl, [t])[0], configs.w_f32(wl, [t])[0], keys[: t + 1])
        assert np.array_equal(s[t, : t + 1].astype(np.float64), o), f"row {t}"
        assert np.all(np.isneginf(s[t, t + 1: N])), f"row {t} mask"
        assert np.all(s[t, N:] == 7.0), "wrote past N"


@pytest.mark.parametrize("H_I", [64, 20, 4])
def test_indexer_offset_rows_multi_chunk(dsa, H_I):
    base = configs.WORKLOADS["prefill_L32k"]
    wl = configs.Workload("idx_probe", "prefill", 3, B=1, N=9100, H_I=H_I, H=128, k=2048)
    wl = configs.Workload(**{**wl.__dict__, "cfg_no": base.cfg_no})
    q_pos0, T, N = 9000, 37, 9100  # ragged query block, 3 key chunks, causal cap at N
    _case(f"indexer offset rows H_I={H_I} q_pos0={q_pos0} T={T} N={N}")
    q_idx = torch.empty((q_pos0 + T, H_I, 128), dtype=torch.uint8, device="cuda")
    w = torch.empty((q_pos0 + T, H_I), dtype=torch.float32, device="cuda")
    k_idx = torch.empty((N, 128), dtype=torch.uint8, device="cuda")
    device.fill(q_idx, q_pos0 + T, H_I * 128, device.E4M3_NORMAL, wl.seed, gen.STREAM_Q_IDX)
    device.fill(w, q_pos0 + T, H_I, device.F32_UNIFORM, wl.seed, gen.STREAM_W)
    device.fill(k_idx, N, 128, device.E4M3_NORMAL, wl.seed, gen.STREAM_K_IDX)
    ld = 9152
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores(q_idx[q_pos0:], w[q_pos0:], k_idx, T, N, H_I, 128, q_pos0, scores, ld)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    keys = configs.k_idx_bytes(wl, 0, np.arange(N))
    for t in range(T):
        pos = q_pos0 + t
        n = min(pos + 1, N)
        o = oracle.indexer_row(configs.q_idx_bytes(wl, [pos])[0], configs.w_f32(wl, [pos])[0], keys[:n])
        check_scores(s[t, :n], o)
        assert np.all(np.isneginf(s[t, n:N]))


def test_indexer_paged(dsa):
    wl = configs.WORKLOADS["paged_decode_b32_ctx4k_128k"]
    ctx = np.array([1, 63, 64, 65, 3000, 200], dtype=np.int32)
    B = len(ctx)
    _case(f"indexer paged ctx={ctx.tolist()}")
    npg = (ctx + 63) // 64
    P = int(npg.sum()) + 3  # a few spare pages never referenced
    rng = np.random.default_rng(11)
    perm = rng.permutation(P)
    max_pages = int(npg.max()) + 2
    pt = np.full((B, max_pages), -1, dtype=np.int32)
    rowmap = np.zeros(P * 64, dtype=np.int64)
    f = 0
    for b in range(B):
        for lp in range(npg[b]):
            p = int(perm[f]); f += 1
            pt[b, lp] = p
            rowmap[p * 64:(p + 1) * 64] = b * wl.S + lp * 64 + np.arange(64)
    k_pool = torch.empty((P, 64, 128), dtype=torch.uint8, device="cuda")
    device.fill(k_pool, P * 64, 128, device.E4M3_NORMAL, wl.seed, gen.STREAM_K_IDX,
                rowmap=torch.from_numpy(rowmap).cuda())
    q_idx = torch.empty((B, 64, 128), dtype=torch.uint8, device="cuda")
    w = torch.empty((B, 64), dtype=torch.float32, device="cuda")
    device.fill(q_idx, B, 64 * 128, device.E4M3_NORMAL, wl.seed, gen.STREAM_Q_IDX)
    device.fill(w, B, 64, device.F32_UNIFORM, wl.seed, gen.STREAM_W)
    max_ctx = 3050
    ld = 3072
    scores = torch.empty((B, ld), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores_paged(q_idx, w, k_pool, P, torch.from_numpy(pt).cuda(), max_pages,
                                 torch.from_numpy(ctx).cuda(), 64, B, 64, 128, max_ctx, scores, ld)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    for b in range(B):
        keys = configs.k_idx_bytes(wl, b, np.arange(ctx[b]))
        o = oracle.indexer_row(configs.q_idx_bytes(wl, [b])[0], configs.w_f32(wl, [b])[0], keys)
        check_scores(s[b, : ctx[b]], o)
        assert np.all(np.isneginf(s[b, ctx[b]: max_ctx]))


def test_indexer_full_rows_128k(dsa):
    """The last 8 rows of the 128K prefill (q_pos0 = 131064) over all 131072
    keys: every one of the 16 key chunks, every candidate within 1e-5 |o| + 1e-6."""
    wl = configs.WORKLOADS["prefill_L128k"]
    T, N = 8, wl.N
    q_pos0 = N - T
    _case(f"indexer full rows q_pos0={q_pos0} T={T} N={N}")
    rows = torch.arange(q_pos0, q_pos0 + T, dtype=torch.int64, device="cuda")
    q_idx = torch.empty((T, wl.H_I, wl.d_I), dtype=torch.uint8, device="cuda")
    w = torch.empty((T, wl.H_I), dtype=torch.float32, device="cuda")
    k_idx = torch.empty((N, wl.d_I), dtype=torch.uint8, device="cuda")
    device.fill(q_idx, T, wl.H_I * wl.d_I, device.E4M3_NORMAL, wl.seed, gen.STREAM_Q_IDX, rowmap=rows)
    device.fill(w, T, wl.H_I, device.F32_UNIFORM, wl.seed, gen.STREAM_W, rowmap=rows)
    device.fill(k_idx, N, wl.d_I, device.E4M3_NORMAL, wl.seed, gen.STREAM_K_IDX)
    scores = torch.empty((T, N), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores(q_idx, w, k_idx, T, N, wl.H_I, wl.d_I, q_pos0, scores, N)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    ref = jobs.run(jobs.indexer_row_job, [(wl.name, q_pos0 + i) for i in range(T)])
    for i in range(T):
        n = q_pos0 + i + 1
        assert ref[i].shape[0] == n
        check_scores(s[i, :n], ref[i])
        assert np.all(np.isneginf(s[i, n:]))


def test_indexer_paged_identity_table_decode_rows(dsa):
    """The contiguous 64 x 32K decode keys addressed as a paged pool through an
    identity page table (sequence b's page p is pool page 512 b + p): whole
    score rows of three sequences within 1e-5 |o| + 1e-6 of the oracle."""
    wl = configs.WORKLOADS["decode_b64_ctx32k"]
    B, N = wl.B, wl.N
    _case(f"indexer paged identity table B={B} N={N}")
    q_idx = torch.empty((B, wl.H_I, wl.d_I), dtype=torch.uint8, device="cuda")
    w = torch.empty((B, wl.H_I), dtype=torch.float32, device="cuda")
    k_idx = torch.empty((B, N, wl.d_I), dtype=torch.uint8, device="cuda")
    device.fill(q_idx, B, wl.H_I * wl.d_I, device.E4M3_NORMAL, wl.seed, gen.STREAM_Q_IDX)
    device.fill(w, B, wl.H_I, device.F32_UNIFORM, wl.seed, gen.STREAM_W)
    device.fill(k_idx, B * N, wl.d_I, device.E4M3_NORMAL, wl.seed, gen.STREAM_K_IDX)
    pages = N // wl.page
    pt = torch.arange(B * pages, dtype=torch.int32, device="cuda").view(B, pages)
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    scores = torch.empty((B, N), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores_paged(q_idx, w, k_idx.view(B * pages, wl.page, wl.d_I), B * pages, pt, pages, ctx,
                                 wl.page, B, wl.H_I, wl.d_I, N, scores, N)
    torch.cuda.synchronize()
    seqs = [0, 37, B - 1]
    s = scores[seqs].cpu().numpy()
    ref = jobs.run(jobs.decode_indexer_row_job, [(wl.name, b) for b in seqs])
    for i in range(len(seqs)):
        assert ref[i].shape[0] == N
        check_scores(s[i], ref[i])


# ------------------------------------------------------------------ top-k
def _topk_rows():
    rng = np.random.default_rng(5)
    rows = []
    rows.append(("normal", rng.standard_normal(5000)))
    rows.append(("normal_long", rng.standard_normal(131072) * 30 + 150))
    rows.append(("int_ties", rng.integers(0, 10, 40000).astype(np.float64)))
    rows.append(("all_equal", np.full(20000, 3.5)))
    rows.append(("increasing", np.arange(9000, dtype=np.float64)))
    rows.append(("decreasing", np.arange(9000, dtype=np.float64)[::-1].copy()))
    z = rng.integers(0, 2, 6000).astype(np.float64) * 0.0
    z[rng.random(6000) < 0.5] = -0.0
    z[rng.random(6000) < 0.01] = 1.0
    rows.append(("signed_zeros", z))
    x = rng.standard_normal(7000)
    x[rng.random(7000) < 0.3] = -np.inf
    rows.append(("with_neg_inf", x))
    rows.append(("short", rng.standard_normal(100)))
    rows.append(("one", np.array([2.0])))
    rows.append(("quantised_ties", np.round(rng.standard_normal(65536) * 4) / 4))
    # rows built to mislead a 1-in-S chunk sample of the row (64-key chunks
    # S*j + (5*j % S), S = 32 for these fp32 rows and 16 for the fused
    # prefill's f16 rows): large values only inside, or only outside, those
    # chunks, so an estimated threshold is far too high or far too low
    n = 65536
    for S in (32, 16):
        inside = np.zeros(n, dtype=bool)
        for j in range(n // 64 // S):
            c = S * j + (5 * j) % S
            inside[64 * c:64 * c + 64] = True
        x = rng.standard_normal(n)
        rows.append((f"sample{S}_biased_high", np.where(inside, x + 100.0, x)))
        rows.append((f"sample{S}_biased_low", np.where(inside, x, x + 100.0)))
    return rows


@pytest.mark.parametrize("k", [1, 97, 2048])
def test_topk_host_rows(dsa, k):
    rows = _topk_rows()
    T = len(rows)
    N = max(len(r) for _, r in rows)
    ld = (N + 3) // 4 * 4
    host = np.full((T, ld), np.nan, dtype=np.float32)
    n_valid = np.zeros(T, dtype=np.int32)
    for i, (_, r) in enumerate(rows):
        host[i, : len(r)] = r.astype(np.float32)
        n_valid[i] = len(r)
    _case(f"topk host rows k={k} T={T} N={N}")
    scores = torch.from_numpy(host).cuda()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(scores, ld, T, N, 0, torch.from_numpy(n_valid).cuda(), k, idx)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    for i, (name, r) in enumerate(rows):
        o = oracle.topk_row(r.astype(np.float32).astype(np.float64), k)
        assert np.array_equal(g[i], o), f"row {name}"


def test_topk_causal_rule(dsa):
    # n_valid = NULL: row t has min(q_pos0 + t + 1, N) candidates
    rng = np.random.default_rng(8)
    T, N, k, q_pos0 = 40, 3000, 64, 2980
    host = rng.standard_normal((T, N)).astype(np.float32)
    _case("topk causal rule")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(torch.from_numpy(host).cuda(), N, T, N, q_pos0, None, k, idx)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    for t in range(T):
        n = min(q_pos0 + t + 1, N)
        assert np.array_equal(g[t], oracle.topk_row(host[t, :n].astype(np.float64), k))
    # rows with fewer candidates than k
    idx2 = torch.empty((3, k), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(torch.from_numpy(host[:3]).cuda(), N, 3, N, 0, None, k, idx2)
    torch.cuda.synchronize()
    for t in range(3):
        assert np.array_equal(idx2.cpu().numpy()[t], list(range(t + 1)) + [-1] * (k - t - 1))


# ------------------------------------------------------------------ attention
def _rand_idx(rng, T, k, n):
    idx = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        m = int(rng.integers(0, min(k, n) + 1)) if t % 5 else min(k, n)
        idx[t, :m] = np.sort(rng.choice(n, size=m, replace=False))
    idx[0, :] = -1  # an empty row
    return idx


# (3, 2048, 128): 8 splits per query merged by the combine kernel, (2, 4096,
# 128): the most, 16; (3, 1024, 40), (5, 2000, 96) and (2, 777, 8): 4, 7 and 3
# splits (the last two with a shorter last split) with head counts that leave
# waves partly or wholly idle
@pytest.mark.parametrize("T,k,H", [(3, 2048, 128), (2, 4096, 128), (40, 300, 128), (300, 64, 128), (17, 100, 8),
                                   (9, 70, 40), (3, 1024, 40), (5, 2000, 96), (2, 777, 8)])
def test_sparse_mla_against_oracle(dsa, T, k, H):
    name = "tiny_prefill_L256" if H == 8 else "prefill_L32k"
    wl0 = configs.WORKLOADS[name]
    N = 4096
    wl = configs.Workload(**{**wl0.__dict__, "H": H, "N": N})
    _case(f"sparse_mla T={T} k={k} H={H} N={N}")
    rng = np.random.default_rng(T * 1000 + k)
    q = torch.empty((T, H, 576), dtype=torch.uint16, device="cuda")
    kv = torch.empty((N, 576), dtype=torch.uint16, device="cuda")
    device.fill(q, T, H * 576, device.BF16_NORMAL, wl.seed, gen.STREAM_Q)
    device.fill(kv, N, 576, device.BF16_NORMAL, wl.seed, gen.STREAM_KV, div=wl.kv_div)
    idx = _rand_idx(rng, T, k, N)
    idx[1, 0] = N + 5  # out-of-range entries are skipped
    out = torch.empty((T, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    nb = dsa.dsa_sparse_mla_fwd_workspace_bytes(T, H, 512, k)
    ws = ws_tensor(nb)
    dsa.dsa_sparse_mla_fwd(q, kv, torch.from_numpy(idx).cuda(), T, N, H, 576, 512, k, wl.scale, out, lse, ws, nb)
    torch.cuda.synchronize()
    g_out, g_lse = out.cpu().numpy(), lse.cpu().numpy()
    qh = configs.q_bf16(wl, np.arange(T))
    for t in range(T):
        sel = idx[t][(idx[t] >= 0) & (idx[t] < N)]
        o_out, o_lse = oracle.sparse_mla_row(qh[t], configs.kv_bf16(wl, 0, sel), wl.scale, 512)
        check_attention(g_out[t], g_lse[t], o_out, o_lse)


def _bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_sparse_mla_large_logit_jump(dsa):
    """A selected row whose logit exceeds every earlier block's by far more
    than the softmax reference allows (~120 in log2 units): the query must be
    redone against the true max and still match the oracle.  Query 0 meets
    the large row in its fourth block, query 1 in its first."""
    T, H, N, k = 2, 32, 256, 128
    scale = 1.0 / np.sqrt(192.0)
    _case("sparse_mla large logit jump")
    qv = np.ones((T, H, 576), dtype=np.float32) * (1.0 + 0.25 * (np.arange(H) % 4))[None, :, None]
    kvv = np.full((N, 576), 2.0 ** -7, dtype=np.float32)
    kvv[200] = 2.0
    kvv[3, :512] = -(2.0 ** -6)  # a second, distinct small row
    q_h, kv_h = _bf16_bits(qv), _bf16_bits(kvv)
    idx = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    idx[0, 100] = 200
    idx[1, 5] = 200
    q = torch.from_numpy(q_h.view(np.int16)).cuda().view(torch.uint16)
    kv = torch.from_numpy(kv_h.view(np.int16)).cuda().view(torch.uint16)
    out = torch.empty((T, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    nb = dsa.dsa_sparse_mla_fwd_workspace_bytes(T, H, 512, k)
    ws = ws_tensor(nb)
    dsa.dsa_sparse_mla_fwd(q, kv, torch.from_numpy(idx).cuda(), T, N, H, 576, 512, k, scale, out, lse, ws, nb)
    torch.cuda.synchronize()
    g_out, g_lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(g_out)) and np.all(np.isfinite(g_lse))
    for t in range(T):
        o_out, o_lse = oracle.sparse_mla_row(q_h[t], kv_h[idx[t]], scale, 512)
        check_attention(g_out[t], g_lse[t], o_out, o_lse)


def test_sparse_mla_split_partials_of_large_values(dsa):
    """Split partials are stored in f16, each (split, head) row scaled by a
    power of two when its largest value passes 2^15.  With the latent rows
    times 2^20 and the queries times 2^-20 the logits are the same numbers, so
    the output must be exactly 2^20 times the plain one up to f16 subnormals
    (here within 2^-11 of the largest value) and the lse equal; the plain call
    also against the oracle.  8 queries x 2048 entries run 4 splits."""
    T, H, N, k = 8, 128, 4096, 2048
    scale = 1.0 / np.sqrt(192.0)
    _case("sparse_mla split partials of large values")
    rng = np.random.default_rng(11)
    qv = rng.standard_normal((T, H, 576)).astype(np.float32)
    kvv = rng.standard_normal((N, 576)).astype(np.float32)
    idx = np.stack([rng.permutation(N)[:k] for _ in range(T)]).astype(np.int32)
    res = {}
    for name, fq, fkv in (("plain", 1.0, 1.0), ("scaled", 2.0 ** -20, 2.0 ** 20)):
        q_h, kv_h = _bf16_bits(qv * fq), _bf16_bits(kvv * fkv)
        q = torch.from_numpy(q_h.view(np.int16)).cuda().view(torch.uint16)
        kv = torch.from_numpy(kv_h.view(np.int16)).cuda().view(torch.uint16)
        out = torch.empty((T, H, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
        nb = dsa.dsa_sparse_mla_fwd_workspace_bytes(T, H, 512, k)
        ws = ws_tensor(nb)
        dsa.dsa_sparse_mla_fwd(q, kv, torch.from_numpy(idx).cuda(), T, N, H, 576, 512, k, scale, out, lse, ws, nb)
        torch.cuda.synchronize()
        res[name] = (out.cpu().numpy().astype(np.float64), lse.cpu().numpy(), q_h, kv_h)
    p_out, p_lse, q_h, kv_h = res["plain"]
    s_out, s_lse = res["scaled"][0], res["scaled"][1]
    assert np.array_equal(p_lse, s_lse)
    assert np.max(np.abs(s_out * 2.0 ** -20 - p_out)) <= 2.0 ** -11 * np.max(np.abs(p_out))
    assert np.max(np.abs(s_out)) > 2.0 ** 15  # the scaled partials took the scaled store
    for t in (0, T - 1):
        o_out, o_lse = oracle.sparse_mla_row(q_h[t], kv_h[idx[t]], scale, 512)
        check_attention(p_out[t], p_lse[t], o_out, o_lse)


def test_sparse_mla_paged(dsa):
    wl = configs.WORKLOADS["paged_decode_b32_ctx4k_128k"]
    ctx = np.array([5, 700, 4096, 2000], dtype=np.int32)
    B, k, H = len(ctx), 512, 128
    _case("sparse_mla paged")
    npg = (ctx + 63) // 64
    P = int(npg.sum())
    rng = np.random.default_rng(12)
    perm = rng.permutation(P)
    max_pages = int(npg.max())
    pt = np.full((B, max_pages), -1, dtype=np.int32)
    rowmap = np.zeros(P * 64, dtype=np.int64)
    f = 0
    for b in range(B):
        for lp in range(npg[b]):
            p = int(perm[f]); f += 1
            pt[b, lp] = p
            rowmap[p * 64:(p + 1) * 64] = b * wl.S + lp * 64 + np.arange(64)
    kv_pool = torch.empty((P, 64, 576), dtype=torch.uint16, device="cuda")
    device.fill(kv_pool, P * 64, 576, device.BF16_NORMAL, wl.seed, gen.STREAM_KV, div=wl.kv_div,
                rowmap=torch.from_numpy(rowmap).cuda())
    q = torch.empty((B, H, 576), dtype=torch.uint16, device="cuda")
    device.fill(q, B, H * 576, device.BF16_NORMAL, wl.seed, gen.STREAM_Q)
    idx = np.full((B, k), -1, dtype=np.int32)
    for b in range(B):
        m = min(k, int(ctx[b]))
        idx[b, :m] = np.sort(rng.choice(int(ctx[b]), size=m, replace=False))
    idx[1, 3] = int(ctx[1]) + 10  # beyond the context: skipped
    out = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    nb = dsa.dsa_sparse_mla_fwd_paged_workspace_bytes(B, H, 512, k)
    ws = ws_tensor(nb)
    dsa.dsa_sparse_mla_fwd_paged(q, kv_pool, P, torch.from_numpy(pt).cuda(), max_pages, torch.from_numpy(ctx).cuda(),
                                 64, torch.from_numpy(idx).cuda(), B, H, 576, 512, k, wl.scale, out, lse, ws, nb)
    torch.cuda.synchronize()
    qh = configs.q_bf16(wl, np.arange(B))
    for b in range(B):
        sel = idx[b][(idx[b] >= 0) & (idx[b] < ctx[b])]
        o_out, o_lse = oracle.sparse_mla_row(qh[b], configs.kv_bf16(wl, b, sel), wl.scale, 512)
        check_attention(out.cpu().numpy()[b], lse.cpu().numpy()[b], o_out, o_lse)
