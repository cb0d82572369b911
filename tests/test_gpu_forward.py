"""End-to-end GPU parity of the fused calls on the five workloads: tiny exact
prefill (both k), 64 x 32K contiguous decode, 32K and 128K causal prefill
(sampled rows) and 32-sequence paged decode with 4K..128K contexts."""
import numpy as np
import pytest
import torch

import oracle
from oracle import jobs
from dsa_inputs import configs, device, gen
from dsa_run import check_attention, check_selection, decode, paged_decode, prefill, ws_tensor

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k", [32, 256])
def test_tiny_prefill_exact(dsa, k):
    wl = configs.WORKLOADS["tiny_prefill_L256"].with_k(k)
    _case(f"forward_prefill tiny L=256 k={k}")
    inp = device.make_prefill_inputs(wl)
    idx, out, lse = prefill(wl, inp)
    g_idx, g_out, g_lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    keys = configs.k_idx_bytes(wl, 0, np.arange(wl.N))
    kv_all = configs.kv_bf16(wl, 0, np.arange(wl.N))
    for t in range(wl.T):
        r = oracle.prefill_row(wl, t, keys)
        check_selection(g_idx[t], r["idx"], r["scores"], k, exact=True)
        check_attention(g_out[t], g_lse[t], r["out"], r["lse"])
        if k >= wl.N:  # every candidate selected: equals dense causal attention
            o_d, l_d = oracle.dense_mla_row(configs.q_bf16(wl, [t])[0], kv_all, t + 1, wl.scale, wl.D_v)
            check_attention(g_out[t], g_lse[t], o_d, l_d)


def _check_rows(name, rows, results, g_idx, g_out, g_lse, k, attn_on):
    """Selection rule per row; attention against the oracle's chain when the sets
    are equal, else against the oracle's attention on the GPU's own index set
    (attn_on(i, idx) -> (out, lse)), with every attention rule in both cases."""
    swapped = 0
    for i, r in enumerate(results):
        d = check_selection(g_idx[i], r["idx"], r["scores"], k, exact=False)
        swapped += d > 0
        if d:
            o_out, o_lse = attn_on(i, g_idx[i])
            check_attention(g_out[i], g_lse[i], o_out, o_lse)
        else:
            check_attention(g_out[i], g_lse[i], r["out"], r["lse"])
    print(f"[{name}] {len(rows)} rows checked, {swapped} with near-tie swaps", flush=True)
    assert swapped <= max(2, len(rows) // 20)


def _attn_on(wl, q_rows, seqs):
    """Oracle attention of query row i (generator row q_rows[i], sequence
    seqs[i]) over a given index set (-1 entries dropped)."""
    def f(i, idx):
        sel = idx[idx >= 0]
        return oracle.sparse_mla_row(configs.q_bf16(wl, [int(q_rows[i])])[0],
                                     configs.kv_bf16(wl, int(seqs[i]), sel), wl.scale, wl.D_v)
    return f


def _stage_isolation(name, g_idx, score_rows, ns, k):
    """The oracle's top-k run on the GPU's own fp32 score rows reproduces the
    fused call's selection bit for bit."""
    for i in range(len(g_idx)):
        o = oracle.topk_row(score_rows[i, : ns[i]].astype(np.float64), k)
        assert np.array_equal(g_idx[i], o), f"{name}: row {i}: selection differs from top-k of its own GPU scores"
    print(f"[{name}] stage isolation: {len(g_idx)} rows bit-exact", flush=True)


def _decode_score_rows(dsa, wl, q_idx, w, k_pool, n_pages, page_table, ctx):
    """The GPU's own score rows of a decode batch (dsa_indexer_scores_paged)."""
    B, max_pages = page_table.shape
    max_ctx = int(ctx.max().item())
    scores = torch.empty((B, max_ctx), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores_paged(q_idx, w, k_pool, n_pages, page_table, max_pages, ctx, wl.page, B, wl.H_I,
                                 wl.d_I, max_ctx, scores, max_ctx)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


def test_decode_b64_ctx32k(dsa):
    wl = configs.WORKLOADS["decode_b64_ctx32k"]
    _case("forward_decode B=64 N=32768")
    inp = device.make_decode_inputs(wl)
    idx, out, lse = decode(wl, inp)
    g_idx, g_out, g_lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    # the GPU's own score rows: the contiguous keys as a pool through an identity page table
    _case("decode B=64: GPU score rows for stage isolation")
    B, N, pages = wl.B, wl.N, wl.N // wl.page
    pt = torch.arange(B * pages, dtype=torch.int32, device="cuda").view(B, pages)
    srows = _decode_score_rows(dsa, wl, inp["q_idx"], inp["w"], inp["k_idx"].view(B * pages, wl.page, wl.d_I),
                               B * pages, pt, inp["ctx_len"])
    del inp, idx, out, lse
    _free()
    _stage_isolation(wl.name, g_idx, srows, configs.ctx_lens(wl), wl.k)
    rows = list(range(wl.B))
    results = jobs.run(jobs.decode_job, [(wl.name, b, None) for b in rows])
    _check_rows(wl.name, rows, results, g_idx, g_out, g_lse, wl.k, _attn_on(wl, rows, rows))


def test_paged_decode_b32(dsa):
    wl = configs.WORKLOADS["paged_decode_b32_ctx4k_128k"]
    _case("forward_decode_paged B=32 ctx 4K..128K")
    inp = device.make_paged_inputs(wl)
    idx, out, lse = paged_decode(wl, inp)
    g_idx, g_out, g_lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    _case("paged decode B=32: GPU score rows for stage isolation")
    srows = _decode_score_rows(dsa, wl, inp["q_idx"], inp["w"], inp["k_pool"], inp["n_pages"], inp["page_table"],
                               inp["ctx_len"])
    del inp, idx, out, lse
    _free()
    _stage_isolation(wl.name, g_idx, srows, configs.ctx_lens(wl), wl.k)
    rows = list(range(wl.B))
    results = jobs.run(jobs.decode_job, [(wl.name, b, None) for b in rows])
    _check_rows(wl.name, rows, results, g_idx, g_out, g_lse, wl.k, _attn_on(wl, rows, rows))


def _prefill_sampled(dsa, name, rows):
    wl = configs.WORKLOADS[name]
    _case(f"forward_prefill {name} T={wl.T}")
    inp = device.make_prefill_inputs(wl)
    idx, out, lse = prefill(wl, inp)
    ridx = torch.from_numpy(np.asarray(rows)).cuda()
    g_idx = idx[ridx].cpu().numpy()
    g_out = out[ridx].cpu().numpy()
    g_lse = lse[ridx].cpu().numpy()
    del idx, out, lse
    # the GPU's own fp32 score rows of the sampled rows (one dsa_indexer_scores call each)
    _case(f"{name}: GPU score rows of {len(rows)} sampled rows for stage isolation")
    N = wl.N
    scores = torch.empty((len(rows), N), dtype=torch.float32, device="cuda")
    for i, t in enumerate(rows):
        t = int(t)
        dsa.dsa_indexer_scores(inp["q_idx"][t:t + 1], inp["w"][t:t + 1], inp["k_idx"], 1, N, wl.H_I, wl.d_I, t,
                               scores[i:i + 1], N)
    torch.cuda.synchronize()
    srows = scores.cpu().numpy()
    del inp, scores
    _free()
    _stage_isolation(name, g_idx, srows, np.minimum(np.asarray(rows) + 1, N), wl.k)
    del srows
    results = jobs.run(jobs.prefill_job, [(wl.name, int(t), None) for t in rows])
    _check_rows(name, rows, results, g_idx, g_out, g_lse, wl.k, _attn_on(wl, rows, np.zeros(len(rows), int)))


def test_prefill_32k_sampled(dsa):
    wl = configs.WORKLOADS["prefill_L32k"]
    rows = np.unique(np.concatenate([configs.sample_rows(wl, wl.oracle_rows), np.arange(64),
                                     np.arange(wl.T - 64, wl.T), [2046, 2047, 2048, 2049]]))
    _prefill_sampled(dsa, wl.name, rows)


def test_prefill_128k_sampled(dsa):
    wl = configs.WORKLOADS["prefill_L128k"]
    rows = np.unique(np.concatenate([configs.sample_rows(wl, wl.oracle_rows), np.arange(8), [2047, 2048],
                                     [wl.T - 1]]))
    _prefill_sampled(dsa, wl.name, rows)


# Irregular shapes of the fused prefill against the oracle: a chunk of a
# sequence at a query offset with head counts that fill no MFMA tile (rows
# shorter and longer than k), long rows with few heads, k above every row's
# length (every candidate, in order), and rows over two 8192-key chunks of
# the scoring pass with 96 heads.
_SHAPES = [  # N, H_I, H, k, q_pos0, T, rows checked
    (700, 20, 40, 100, 400, 300, 300),
    (5000, 4, 8, 2048, 4870, 130, 130),
    (64, 64, 128, 4096, 0, 64, 64),
    (9000, 64, 96, 300, 8100, 900, 40),
]


@pytest.mark.parametrize("shape", _SHAPES, ids=[f"N{s[0]}_HI{s[1]}_H{s[2]}_k{s[3]}" for s in _SHAPES])
def test_fused_prefill_shapes(dsa, shape):
    N, H_I, H, k, q_pos0, T, n_check = shape
    wl = configs.Workload(f"prefill_N{N}_H{H}", "prefill", 20 + _SHAPES.index(shape), B=1, N=N, H_I=H_I, H=H, k=k)
    _case(f"forward_prefill N={N} H_I={H_I} H={H} k={k} rows {q_pos0}..{q_pos0 + T - 1}")
    inp = device.make_prefill_inputs(wl)  # rows of every position; the call takes rows q_pos0 ..
    part = dict(inp, q_idx=inp["q_idx"][q_pos0:q_pos0 + T].contiguous(), w=inp["w"][q_pos0:q_pos0 + T].contiguous(),
                q=inp["q"][q_pos0:q_pos0 + T].contiguous())
    idx, out, lse = prefill(wl, part, k=k, T=T, q_pos0=q_pos0)
    rows = np.arange(T)
    if n_check < T:
        rng = np.random.default_rng(N)
        rows = np.unique(np.concatenate([rng.choice(T, n_check - 4, replace=False), [0, 1, T - 2, T - 1]]))
    g_idx, g_out, g_lse = idx.cpu().numpy()[rows], out.cpu().numpy()[rows], lse.cpu().numpy()[rows]
    del inp, part, idx, out, lse
    _free()
    keys = configs.k_idx_bytes(wl, 0, np.arange(N))
    results = [oracle.prefill_row(wl, q_pos0 + int(i), keys, k) for i in rows]
    _check_rows(wl.name, rows, results, g_idx, g_out, g_lse, k,
                _attn_on(wl, q_pos0 + rows, np.zeros(len(rows), int)))


def test_decode_heavy_ties_and_mixed_lengths(dsa):
    """Long decode rows go through the multi-workgroup top-k.  Keys 0..4095 of
    every sequence are equal (one shared score) and the rest are zero (score 0),
    so a row's threshold bin holds thousands of equal scores.
    Sequences 0 and 3 have 4096 tied keys, more than the candidate list holds,
    and take the exact path; sequence 1 has 3000.  Contexts also cover a short
    row (n <= k) and a partial last chunk."""
    B, N, H_I, H, k = 4, 70000, 4, 8, 2048
    _case("decode heavy ties")
    ctx = np.array([70000, 66003, 1500, 65536], dtype=np.int32)
    key = np.zeros((B, N, 128), dtype=np.uint8)
    key[:, :4096, :] = 0x38  # 1.0 in every dim
    key[1, 3000:4096, :] = 0  # sequence 1: 3000 tied keys, few enough for the candidate list
    key[1, 5000:5100, :] = 0x40  # 2.0: a hundred larger scores in sequence 1
    q_idx = np.full((B, H_I, 128), 0x38, dtype=np.uint8)  # 1.0
    w = np.full((B, H_I), 0.5, dtype=np.float32)
    rng = np.random.default_rng(4)
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, H, 576)).astype(np.float32))
    kv = np.zeros((B, N, 576), dtype=np.uint16)  # the selection does not depend on it
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    nb = dsa.dsa_forward_decode_workspace_bytes(B, N, H, 512, k)
    ws = ws_tensor(nb)
    dsa.dsa_forward_decode(dev(q_idx), dev(w), dev(key), dev(q), dev(kv), dev(ctx), B, N, H_I, 128, H, 576, 512, k,
                           1.0 / np.sqrt(192.0), idx, out, lse, ws, nb)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    for b in range(B):
        n = int(ctx[b])
        keys_b = key[b, :n]
        o = oracle.topk_row(oracle.indexer_row(q_idx[b], w[b], keys_b), k)
        assert np.array_equal(g[b], o), f"sequence {b}"


def test_launch_timing_counts_and_leaves_results_unchanged(dsa):
    """With launch timing on, the fused prefill gives the same bits and one
    record per kernel stage: an indexer and a top-k per row tile, one attention."""
    wl = configs.WORKLOADS["prefill_L32k"]
    _case(f"{wl.name} fused prefill with and without launch timing")
    inp = device.make_prefill_inputs(wl)
    idx0, out0, lse0 = prefill(wl, inp)
    dsa.dsa_timing_begin()
    idx1, out1, lse1 = prefill(wl, inp)
    rec = dsa.dsa_timing_end()
    tile_rows, _ = dsa.dsa_forward_prefill_plan(wl.T, wl.N)
    n_tiles = (wl.T + tile_rows - 1) // tile_rows
    assert torch.equal(idx0, idx1) and torch.equal(out0, out1) and torch.equal(lse0, lse1)
    assert rec["indexer"][1] == n_tiles and rec["topk"][1] == n_tiles and rec["attention"][1] == 1
    assert rec["indexer_kl"] == (0.0, 0)
    assert all(rec[kk][0] > 0 for kk in ("indexer", "topk", "attention"))
    # records stop with dsa_timing_end
    prefill(wl, inp)
    assert dsa.dsa_timing_end() == {kind: (0.0, 0) for kind in dsa.TIMING_KINDS}
    del inp, idx0, out0, lse0, idx1, out1, lse1
    _free()


def test_paged_prefill_mixed(dsa):
    """Chunked prefill of four sequences into a paged cache in one call: a chunk
    after 7500 cached tokens, a whole 2100-token prompt, 256 new tokens after
    16128 and a one-token chunk.  Sequences 0 and 1 must equal the contiguous
    fused prefill of the same keys bit for bit (only the key addressing differs);
    sampled rows of every sequence are checked against the oracle."""
    wl = configs.WORKLOADS["paged_prefill_mixed"]
    _case(f"{wl.name}: forward_prefill_paged")
    inp = device.make_paged_prefill_inputs(wl)
    q_start, seq, pos = configs.chunk_rows(wl)
    T, k, ctx = wl.T, wl.k, inp["ctx_len"]
    pt = inp["page_table"]
    nb = dsa.dsa_forward_prefill_paged_workspace_bytes(T, int(ctx.max()), wl.H, wl.D_v, k)
    ws = ws_tensor(nb)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, wl.H, wl.D_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, wl.H), dtype=torch.float32, device="cuda")
    dsa.dsa_forward_prefill_paged(inp["q_idx"], inp["w"], inp["k_pool"], inp["q"], inp["kv_pool"], inp["n_pages"], pt,
                                  pt.shape[1], wl.page, q_start, ctx, wl.B, wl.H_I, wl.d_I, wl.H, wl.D_qk, wl.D_v, k,
                                  wl.scale, idx, out, lse, ws, nb)
    torch.cuda.synchronize()
    for b in (0, 1):
        _case(f"{wl.name}: sequence {b} against the contiguous fused prefill")
        n, q0, q1 = int(ctx[b]), int(q_start[b]), int(q_start[b + 1])
        s = np.arange(n)
        rows = torch.from_numpy(inp["page_table_host"][b][s // wl.page].astype(np.int64) * wl.page + s % wl.page).cuda()
        k_c = inp["k_pool"].view(-1, wl.d_I)[rows].contiguous()
        kv_c = inp["kv_pool"].view(torch.int16).view(-1, wl.D_qk)[rows].contiguous().view(torch.uint16)
        cnb = dsa.dsa_forward_prefill_workspace_bytes(q1 - q0, n, wl.H, wl.D_v, k)
        cws = ws_tensor(cnb)
        c_idx = torch.empty((q1 - q0, k), dtype=torch.int32, device="cuda")
        c_out = torch.empty((q1 - q0, wl.H, wl.D_v), dtype=torch.float32, device="cuda")
        c_lse = torch.empty((q1 - q0, wl.H), dtype=torch.float32, device="cuda")
        dsa.dsa_forward_prefill(inp["q_idx"][q0:q1], inp["w"][q0:q1], k_c, inp["q"][q0:q1], kv_c, q1 - q0, n, wl.H_I,
                                wl.d_I, wl.H, wl.D_qk, wl.D_v, k, n - (q1 - q0), wl.scale, c_idx, c_out, c_lse, cws,
                                cnb)
        torch.cuda.synchronize()
        assert torch.equal(idx[q0:q1], c_idx)
        assert torch.equal(out[q0:q1], c_out) and torch.equal(lse[q0:q1], c_lse)
        del k_c, kv_c, cws, c_idx, c_out, c_lse
    g_idx, g_out, g_lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    del inp, idx, out, lse, ws
    _free()
    ends = np.concatenate([q_start[:-1], q_start[1:] - 1])
    rows = np.unique(np.concatenate([configs.sample_rows(wl, wl.oracle_rows), ends]))
    results = jobs.run(jobs.paged_prefill_job, [(wl.name, int(seq[r]), int(pos[r]), None) for r in rows])
    _check_rows(wl.name, rows, results, g_idx[rows], g_out[rows], g_lse[rows], wl.k,
                _attn_on(wl, seq[rows] * wl.S + pos[rows], seq[rows]))


def test_paged_prefill_empty_chunk_and_page_multiple(dsa):
    """A call whose sequences include an empty chunk and a context that ends on a
    page boundary: the empty sequence contributes no rows, and every other row
    equals the same rows of the mixed workload computed alone."""
    wl = configs.WORKLOADS["paged_prefill_mixed"]
    _case(f"{wl.name}: empty chunk and a page-multiple context")
    inp = device.make_paged_prefill_inputs(wl)
    q_start, seq, pos = configs.chunk_rows(wl)
    T, k, ctx, pt = wl.T, wl.k, inp["ctx_len"], inp["page_table"]

    def call(qs, cl, rows, table):
        nbytes = dsa.dsa_forward_prefill_paged_workspace_bytes(len(rows), int(max(cl)), wl.H, wl.D_v, k)
        ws = ws_tensor(nbytes)
        idx = torch.empty((len(rows), k), dtype=torch.int32, device="cuda")
        out = torch.empty((len(rows), wl.H, wl.D_v), dtype=torch.float32, device="cuda")
        lse = torch.empty((len(rows), wl.H), dtype=torch.float32, device="cuda")
        r = torch.from_numpy(np.asarray(rows, dtype=np.int64)).cuda()
        dsa.dsa_forward_prefill_paged(inp["q_idx"][r].contiguous(), inp["w"][r].contiguous(), inp["k_pool"],
                                      inp["q"].view(torch.int16)[r].contiguous().view(torch.uint16), inp["kv_pool"],
                                      inp["n_pages"], table, table.shape[1], wl.page, qs, cl, len(cl), wl.H_I, wl.d_I,
                                      wl.H, wl.D_qk, wl.D_v, k, wl.scale, idx, out, lse, ws, nbytes)
        torch.cuda.synchronize()
        return idx, out, lse

    full = call(q_start, ctx, np.arange(T), pt)
    # sequence 2 (16384 = 256 pages of context) keeps its 256-row chunk; sequence 0 gets an empty chunk
    rows2 = np.arange(q_start[2], q_start[3])
    qs = [0, 0, len(rows2)]
    sub = call(qs, [int(ctx[0]), int(ctx[2])], rows2, pt[[0, 2]].contiguous())
    for a, b in zip(sub, full):
        assert torch.equal(a, b[q_start[2]:q_start[3]])
    del inp
    _free()
