"""The fused prefill's selection path: the FP8 scoring pass plus the band
top-k must select exactly what the exact scores select.  Every row of each
case is compared bit for bit with the staged path (dsa_indexer_scores, whose
scores the oracle pins at 1e-5, then dsa_topk), and sampled rows with the
oracle's own chain.  Cases cover several indexer head counts, inputs scaled
towards the E4M3 range's ends (large products, subnormals), rows whose
weights send them down the exact route (a negative weight, all weights zero)
and a query offset with a ragged last tile.  At scale 24 every row's dot
products could leave f16's range, so every row takes the exact route."""
import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import gen
from dsa_run import check_selection, ws_tensor

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _inputs(seed, T, N, H_I, scale=1.0, w_mode="uniform"):
    rng = np.random.default_rng(seed)
    q_idx = gen.f32_to_e4m3_bits((rng.standard_normal((T, H_I, 128)) * scale).astype(np.float32))
    k_idx = gen.f32_to_e4m3_bits((rng.standard_normal((N, 128)) * scale).astype(np.float32))
    w = rng.random((T, H_I)).astype(np.float32)
    if w_mode == "flagged":
        w[3::7, min(5, H_I - 1)] = -0.25  # a negative weight: the row takes the exact route
        w[5::11, :] = 0.0      # every weight zero: all scores 0, every candidate tied
    return q_idx, w, k_idx


def _fused_vs_staged(dsa, q_idx, w, k_idx, T, N, H_I, k, q_pos0):
    H, D_qk, D_v = 8, 576, 512
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    qi, wd, ki = dev(q_idx), dev(w), dev(k_idx)
    # attention inputs are irrelevant to the selection; small and zero
    q = torch.zeros((T, H, D_qk), dtype=torch.uint16, device="cuda")
    kv = torch.zeros((N, D_qk), dtype=torch.uint16, device="cuda")
    nb = dsa.dsa_forward_prefill_workspace_bytes(T, N, H, D_v, k)
    ws = ws_tensor(nb)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, D_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dsa.dsa_forward_prefill(qi, wd, ki, q, kv, T, N, H_I, 128, H, D_qk, D_v, k, q_pos0, 1.0 / np.sqrt(192.0), idx,
                            out, lse, ws, nb)
    ld = (N + 63) // 64 * 64
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores(qi, wd, ki, T, N, H_I, 128, q_pos0, scores, ld)
    idx2 = torch.empty_like(idx)
    dsa.dsa_topk(scores, ld, T, N, q_pos0, None, k, idx2)
    torch.cuda.synchronize()
    g, s = idx.cpu().numpy(), idx2.cpu().numpy()
    bad = np.nonzero(~np.all(g == s, axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ from the staged exact selection, first row {bad[0]}"
    return g, scores.cpu().numpy()


@pytest.mark.parametrize("H_I,scale,w_mode", [(64, 1.0, "uniform"), (20, 1.0, "uniform"), (64, 6.0, "uniform"),
                                              (64, 24.0, "uniform"), (64, 1.0 / 64, "uniform"), (64, 1.0, "flagged"),
                                              (4, 3.0, "flagged")])
def test_fused_selection_equals_exact(dsa, H_I, scale, w_mode):
    T, N, k, q_pos0 = 1500, 12000, 512, 10700
    _case(f"fused vs staged H_I={H_I} scale={scale} w={w_mode} T={T} N={N} k={k} q_pos0={q_pos0}")
    q_idx, w, k_idx = _inputs(17 + H_I, T, N, H_I, scale, w_mode)
    g, _ = _fused_vs_staged(dsa, q_idx, w, k_idx, T, N, H_I, k, q_pos0)
    # oracle chain on sampled rows (exact E4M3 arithmetic in fp64)
    rng = np.random.default_rng(3)
    for t in np.unique(np.concatenate([rng.choice(T, 6, replace=False), [0, T - 1, 3, 5]])):
        n = min(q_pos0 + t + 1, N)
        o_s = oracle.indexer_row(q_idx[t], w[t], k_idx[:n])
        check_selection(g[t], oracle.topk_row(o_s, k), o_s, k, exact=False)


def test_fused_selection_long_rows_and_tiles(dsa):
    """Rows of 40000..41023 keys (the sampled estimate's regime) with k = 2048,
    one tile; a second call over the same rows split at q_pos0 gives the same
    selection."""
    T, N, k, H_I = 1024, 41024, 2048, 64
    q_pos0 = N - T
    _case(f"fused vs staged long rows T={T} N={N} k={k}")
    q_idx, w, k_idx = _inputs(99, T, N, H_I)
    g, _ = _fused_vs_staged(dsa, q_idx, w, k_idx, T, N, H_I, k, q_pos0)
    h = 300
    g1, _ = _fused_vs_staged(dsa, q_idx[h:], w[h:], k_idx, T - h, N, H_I, k, q_pos0 + h)
    assert np.array_equal(g[h:], g1)


@pytest.mark.parametrize("where", ["query", "key"])
def test_fused_selection_with_nan_codes(dsa, where):
    """E4M3 NaN codes (S.1111.111): a query row holding one takes the exact
    route; a key holding one sends every row of the call down the exact
    route.  The selection still equals the staged exact one, whose scores
    are NaN wherever such a code meets a candidate."""
    T, N, k, H_I = 600, 5000, 256, 64
    q_pos0 = N - T
    _case(f"fused vs staged with NaN codes in the {where}s")
    q_idx, w, k_idx = _inputs(5, T, N, H_I)
    if where == "query":
        q_idx[7::50, 3, 17] = 0x7F
        q_idx[11, 0, 0] = 0xFF
    else:
        k_idx[1234, 5] = 0x7F
    g, scores = _fused_vs_staged(dsa, q_idx, w, k_idx, T, N, H_I, k, q_pos0)
    nan_rows = np.isnan(scores[:, :N]).any(axis=1)
    assert nan_rows.sum() == (13 if where == "query" else T)
