"""Pins for the CPU oracle: each check is fixed by hand arithmetic, a closed
form, an independent library routine or a brute-force algorithm, so that a
dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import configs, gen


# --------------------------------------------------------------- storage formats
def test_e4m3_hand_values():
    assert oracle.e4m3_to_f64(0x38) == 1.0
    assert oracle.e4m3_to_f64(0xB8) == -1.0
    assert oracle.e4m3_to_f64(0x7E) == 448.0
    assert oracle.e4m3_to_f64(0x01) == 2.0 ** -9
    assert oracle.e4m3_to_f64(0x08) == 2.0 ** -6
    assert oracle.e4m3_to_f64(0x44) == 3.0
    assert math.isnan(oracle.e4m3_to_f64(0x7F))


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_bf16_codes_match_torch():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 1 << 16, size=4000).astype(np.uint16)
    codes = codes[((codes >> 7) & 0xFF) != 0xFF]  # finite only
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = np.array([oracle.bf16_to_f64(c) for c in codes])
    assert np.array_equal(mine, ref)


# --------------------------------------------------------------- indexer
def _e4m3(vals):
    return gen.f32_to_e4m3_bits(np.asarray(vals, dtype=np.float32))


def test_indexer_hand_case():
    # H_I = 2 heads, d_I = 2; scores worked out by hand:
    #   head dot products q_j . k_s, ReLU, then weighted by w_j and summed.
    q = _e4m3([[1, 2], [-1, 3]])
    k = _e4m3([[1, 1], [2, 1], [-1, -1], [0.5, -0.25]])
    w = np.array([0.5, 2.0], dtype=np.float32)
    # s0: dots (3, 2)    -> 0.5*3 + 2*2 = 5.5
    # s1: dots (4, 1)    -> 0.5*4 + 2*1 = 4.0
    # s2: dots (-3, -2)  -> 0
    # s3: dots (0, -1.25)-> 0
    assert np.array_equal(oracle.indexer_row(q, w, k), [5.5, 4.0, 0.0, 0.0])


def test_indexer_relu_comes_before_weight():
    # a negative weight must scale the rectified dot product (not be rectified)
    q = _e4m3([[1, 2], [-1, 3]])
    k = _e4m3([[1, 1], [2, 1]])
    w = np.array([0.5, -2.0], dtype=np.float32)
    # s0: 0.5*3 + (-2)*2 = -2.5 ; s1: 0.5*4 + (-2)*1 = 0
    assert np.array_equal(oracle.indexer_row(q, w, k), [-2.5, 0.0])


def test_indexer_onehot_zero_and_scaling():
    rng = np.random.default_rng(1)
    H_I, d, n = 4, 128, 37
    q = _e4m3(rng.integers(-4, 5, size=(H_I, d)))
    k = _e4m3(rng.integers(-4, 5, size=(n, d)))
    base = oracle.indexer_row(q, np.ones(H_I, np.float32), k)
    # zero weights -> zero scores
    assert np.all(oracle.indexer_row(q, np.zeros(H_I, np.float32), k) == 0.0)
    # power-of-two scaling of all weights scales the scores exactly
    assert np.array_equal(oracle.indexer_row(q, np.full(H_I, 4.0, np.float32), k), 4.0 * base)
    # one-hot weights isolate one head; summing them recovers the all-ones score
    parts = []
    for j in range(H_I):
        wj = np.zeros(H_I, np.float32)
        wj[j] = 1.0
        parts.append(oracle.indexer_row(q, wj, k))
    assert np.array_equal(np.sum(parts, axis=0), base)
    # a head alone is the rectified integer dot product (inputs are small integers)
    qv = np.array([[oracle.e4m3_to_f64(b) for b in row] for row in q])
    kv = np.array([[oracle.e4m3_to_f64(b) for b in row] for row in k])
    dots = kv @ qv[0]
    assert np.array_equal(parts[0], np.maximum(dots, 0.0))
    # permuting heads together with their weights changes nothing
    perm = [2, 0, 3, 1]
    w = np.array([0.25, 0.5, 1.0, 2.0], np.float32)
    assert np.array_equal(oracle.indexer_row(q[perm], w[perm], k), oracle.indexer_row(q, w, k))


def test_indexer_tiny_workload_scores_are_exact_quarters():
    wl = configs.WORKLOADS["tiny_prefill_L256"]
    keys = configs.k_idx_bytes(wl, 0, np.arange(wl.N))
    for t in (0, 1, 100, 255):
        s = oracle.indexer_row(configs.q_idx_bytes(wl, [t])[0], configs.w_f32(wl, [t])[0], keys[: t + 1])
        assert s.shape == (t + 1,)
        assert np.all(s >= 0.0)
        assert np.array_equal(s * 4.0, np.round(s * 4.0))


# --------------------------------------------------------------- top-k
def _brute_topk(scores, k):
    """Rank counting: s is selected iff fewer than k candidates beat it
    (a larger score, or an equal score at a lower index)."""
    n = len(scores)
    sel = []
    for s in range(n):
        beats = sum(1 for u in range(n) if scores[u] > scores[s] or (scores[u] == scores[s] and u < s))
        if beats < k:
            sel.append(s)
    return np.array(sel + [-1] * (k - len(sel)), dtype=np.int32)


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_rank_counting_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    k = int(rng.integers(1, 40))
    scores = rng.integers(0, 6, size=n).astype(np.float64) * 0.5  # many ties
    assert np.array_equal(oracle.topk_row(scores, k), _brute_topk(scores, k))


def test_topk_special_rows():
    n, k = 50, 8
    assert np.array_equal(oracle.topk_row(np.zeros(n), k), np.arange(k))          # all equal
    assert np.array_equal(oracle.topk_row(np.arange(n, dtype=float), k), np.arange(n - k, n))  # increasing
    assert np.array_equal(oracle.topk_row(np.arange(n, dtype=float)[::-1].copy(), k), np.arange(k))
    r = oracle.topk_row(np.ones(5), 8)                                              # fewer candidates
    assert np.array_equal(r, [0, 1, 2, 3, 4, -1, -1, -1])
    assert np.array_equal(oracle.topk_row(np.array([-0.0, 0.0, -0.0]), 2), [0, 1])  # -0 == +0
    assert np.array_equal(oracle.topk_row(np.array([1.0, 3.0, 2.0, 3.0]), 1), [1])  # k = 1, tie to lower


def test_topk_random_rows_invariants():
    rng = np.random.default_rng(7)
    for _ in range(20):
        n = int(rng.integers(1, 3000))
        k = int(rng.integers(1, 300))
        s = rng.standard_normal(n)
        r = oracle.topk_row(s, k)
        m = min(n, k)
        sel = r[:m]
        assert np.all(r[m:] == -1)
        assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < n
        if n > k:
            thr = np.sort(s)[::-1][k - 1]
            assert np.all(s[sel] >= thr)
            assert np.sum(s > thr) <= k


# --------------------------------------------------------------- attention
def test_attention_hand_case():
    # one head, D_qk = 2, D_v = 1, scale 1: logits (0, 1) -> softmax (1, e)/(1+e)
    q = gen.f32_to_bf16_bits(np.array([[1.0, 0.0]], np.float32))
    kv = gen.f32_to_bf16_bits(np.array([[0.0, 2.0], [1.0, 4.0]], np.float32))
    out, lse = oracle.sparse_mla_row(q, kv, 1.0, 1)
    e = math.e
    assert out[0, 0] == pytest.approx(e / (1 + e), rel=1e-15)
    assert lse[0] == pytest.approx(math.log(1 + e), rel=1e-15)


def _rand_bf16(rng, shape, sd=1.0):
    return gen.f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))


def _bf16_to_np(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_dense_matches_torch_sdpa():
    rng = np.random.default_rng(3)
    H, D_qk, D_v, N = 3, 24, 16, 11
    q = _rand_bf16(rng, (H, D_qk))
    kv = _rand_bf16(rng, (N, D_qk))
    scale = 0.3
    qt = torch.from_numpy(_bf16_to_np(q))[None, :, None, :]          # [1, H, 1, D]
    kt = torch.from_numpy(_bf16_to_np(kv))[None, None].expand(1, H, N, D_qk)
    vt = torch.from_numpy(_bf16_to_np(kv)[:, :D_v])[None, None].expand(1, H, N, D_v)
    for n in (1, 5, N):
        mask = torch.zeros(1, 1, 1, N, dtype=torch.bool)
        mask[..., :n] = True
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        out, lse = oracle.dense_mla_row(q, kv, n, scale, D_v)
        np.testing.assert_allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-13)
        logits = (qt[0, :, 0] @ kt[0, 0, :n].T) * scale
        np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), rtol=1e-13)


def test_sparse_with_all_candidates_equals_dense():
    wl = configs.WORKLOADS["tiny_prefill_L256"]
    kv = configs.kv_bf16(wl, 0, np.arange(wl.N))
    for t in (0, 7, 130, 255):
        q = configs.q_bf16(wl, [t])[0]
        o_s, l_s = oracle.sparse_mla_row(q, kv[: t + 1], wl.scale, wl.D_v)
        o_d, l_d = oracle.dense_mla_row(q, kv, t + 1, wl.scale, wl.D_v)
        np.testing.assert_allclose(o_s, o_d, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l_s, l_d, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(5)
    H, D_qk, D_v, m = 4, 576, 512, 9
    q = _rand_bf16(rng, (H, D_qk))
    kv = _rand_bf16(rng, (m, D_qk))
    kvd = _bf16_to_np(kv)
    # one selected row: the output is that row's value part, lse its logit
    out, lse = oracle.sparse_mla_row(q, kv[:1], 0.1, D_v)
    assert np.array_equal(out, np.broadcast_to(kvd[0, :D_v], (H, D_v)))
    np.testing.assert_allclose(lse, 0.1 * (_bf16_to_np(q) @ kvd[0]), rtol=1e-13)
    # zero query: uniform weights -> mean of the values, lse = ln m
    out, lse = oracle.sparse_mla_row(np.zeros((H, D_qk), np.uint16), kv, 0.1, D_v)
    np.testing.assert_allclose(out, np.broadcast_to(kvd[:, :D_v].mean(0), (H, D_v)), rtol=1e-13, atol=1e-15)
    assert np.all(lse == math.log(m))
    # empty selection
    out, lse = oracle.sparse_mla_row(q, kv[:0], 0.1, D_v)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))
    # values are the first D_v latent dims only: with the query's trailing
    # (rope) dims at zero, the rows' trailing dims cannot change the output,
    # while the logits do use every one of the D_qk dims
    q0 = q.copy()
    q0[:, D_v:] = 0
    kv2 = kv.copy()
    kv2[:, D_v:] = gen.f32_to_bf16_bits(np.full((m, D_qk - D_v), 3.0, np.float32))
    o_a, l_a = oracle.sparse_mla_row(q0, kv, 0.1, D_v)
    o_b, l_b = oracle.sparse_mla_row(q0, kv2, 0.1, D_v)
    assert np.array_equal(o_a, o_b) and np.array_equal(l_a, l_b)
    _, l_c = oracle.sparse_mla_row(q, kv2, 0.1, D_v)
    _, l_d = oracle.sparse_mla_row(q, kv, 0.1, D_v)
    assert not np.allclose(l_c, l_d)


def test_attention_heads_are_independent_and_share_kv():
    rng = np.random.default_rng(6)
    H, D_qk, D_v, m = 5, 64, 32, 13
    q = _rand_bf16(rng, (H, D_qk))
    kv = _rand_bf16(rng, (m, D_qk))
    out, lse = oracle.sparse_mla_row(q, kv, 0.2, D_v)
    for h in range(H):
        o1, l1 = oracle.sparse_mla_row(q[h:h + 1], kv, 0.2, D_v)
        assert np.array_equal(o1[0], out[h]) and l1[0] == lse[h]
    # selection order does not matter
    perm = rng.permutation(m)
    o2, l2 = oracle.sparse_mla_row(q, kv[perm], 0.2, D_v)
    np.testing.assert_allclose(o2, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, lse, rtol=1e-13)


# --------------------------------------------------------------- chain
def test_tiny_chain_invariants_and_k_covering_all():
    wl = configs.WORKLOADS["tiny_prefill_L256"]
    keys = configs.k_idx_bytes(wl, 0, np.arange(wl.N))
    kv = configs.kv_bf16(wl, 0, np.arange(wl.N))
    for t in (0, 31, 32, 200, 255):
        r = oracle.prefill_row(wl, t, keys)
        m = min(t + 1, wl.k)
        sel = r["idx"][:m]
        assert np.all(r["idx"][m:] == -1)
        assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] <= t
        # k = 256 >= every candidate count: sparse attention is dense causal attention
        r2 = oracle.prefill_row(wl, t, keys, k=256)
        assert np.array_equal(r2["idx"][: t + 1], np.arange(t + 1))
        o_d, l_d = oracle.dense_mla_row(configs.q_bf16(wl, [t])[0], kv, t + 1, wl.scale, wl.D_v)
        np.testing.assert_allclose(r2["out"], o_d, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r2["lse"], l_d, rtol=1e-12, atol=1e-12)
    # row 0 closed form: the only candidate is token 0
    r0 = oracle.prefill_row(wl, 0, keys)
    kvd = _bf16_to_np(kv[0])
    assert np.array_equal(r0["out"], np.broadcast_to(kvd[: wl.D_v], (wl.H, wl.D_v)))


# ------------------------------------------------------------------ indexer KL loss
# "DeepSeek-V3.2" walk-through §2.3.2: KL(p_{t,S_t} || Softmax(I_{t,S_t})), with p the
# attention scores summed over heads and L1-normalised along the selected tokens (§2.3.1).

def test_indexer_kl_hand_cases():
    # one head, D_qk = 2, scale 1, two selected rows with logits (0, 1):
    # p = (1, e)/(1+e).  Against I = (0, 0), r = (1/2, 1/2) and
    # KL = sum p ln(2p) = ln 2 + p0 ln p0 + p1 ln p1.
    q = gen.f32_to_bf16_bits(np.array([[1.0, 0.0]], np.float32))
    kv = gen.f32_to_bf16_bits(np.array([[0.0, 2.0], [1.0, 4.0]], np.float32))
    e = math.e
    p0, p1 = 1 / (1 + e), e / (1 + e)
    want = math.log(2) + p0 * math.log(p0) + p1 * math.log(p1)
    assert oracle.indexer_kl_row(q, kv, 1.0, np.array([0.0, 0.0])) == pytest.approx(want, rel=1e-14)
    # an indexer that reproduces the logits up to a constant has zero loss
    assert abs(oracle.indexer_kl_row(q, kv, 1.0, np.array([3.0, 4.0]))) < 1e-15
    # with I = (1, 0) the model distribution is r = (e, 1)/(1+e): KL = sum p ln(p/r)
    r0, r1 = e / (1 + e), 1 / (1 + e)
    want = p0 * math.log(p0 / r0) + p1 * math.log(p1 / r1)
    assert oracle.indexer_kl_row(q, kv, 1.0, np.array([1.0, 0.0])) == pytest.approx(want, rel=1e-13)


def test_indexer_kl_heads_are_summed_then_normalised():
    # two heads with logits (0, 1) and (1, 0): their probabilities sum to (1, 1) per
    # position, so the L1-normalised target is uniform whatever the per-head shapes
    q = gen.f32_to_bf16_bits(np.array([[1.0, 0.0], [0.0, 1.0]], np.float32))
    kv = gen.f32_to_bf16_bits(np.array([[0.0, 1.0], [1.0, 0.0]], np.float32))
    iscore = np.array([0.25, -1.5])
    r = np.exp(iscore) / np.exp(iscore).sum()
    want = float(np.sum(0.5 * np.log(0.5 / r)))
    assert oracle.indexer_kl_row(q, kv, 1.0, iscore) == pytest.approx(want, rel=1e-13)


def test_indexer_kl_single_row_and_empty_are_zero():
    rng = np.random.default_rng(5)
    q = _rand_bf16(rng, (4, 16))
    kv = _rand_bf16(rng, (1, 16))
    assert oracle.indexer_kl_row(q, kv, 0.4, np.array([2.5])) == 0.0
    assert oracle.indexer_kl_row(q, kv[:0], 0.4, np.zeros(0)) == 0.0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_indexer_kl_matches_torch_kl_div(seed):
    # an independent route: torch's fp64 softmax per head and its kl_div
    rng = np.random.default_rng(10 + seed)
    H, D_qk, m = 5, 40, 23
    q = _rand_bf16(rng, (H, D_qk))
    kv = _rand_bf16(rng, (m, D_qk))
    iscore = rng.standard_normal(m) * 3
    scale = 0.2
    z = torch.from_numpy(_bf16_to_np(q)) @ torch.from_numpy(_bf16_to_np(kv)).T * scale   # [H, m]
    target = torch.softmax(z, dim=1).sum(0)
    target = target / target.sum()
    log_r = torch.log_softmax(torch.from_numpy(iscore), dim=0)
    want = torch.nn.functional.kl_div(log_r, target, reduction="sum").item()
    got = oracle.indexer_kl_row(q, kv, scale, iscore)
    assert got == pytest.approx(want, rel=1e-12, abs=1e-14)
    assert got >= 0.0
    # invariant under a shift of every indexer score
    assert oracle.indexer_kl_row(q, kv, scale, iscore + 7.0) == pytest.approx(got, rel=1e-10, abs=1e-13)


def test_dense_kl_row_matches_torch_from_raw_inputs():
    """The dense warm-up loss driver end to end on the tiny workload against an
    independent torch fp64 route from the generator's raw bytes (float8_e4m3fn and
    bfloat16 decoding by torch): indexer scores, per-head softmax over all causal
    keys, the L1-normalised head sum, and kl_div against the indexer softmax."""
    wl = configs.WORKLOADS["tiny_prefill_L256"]
    keys = configs.k_idx_bytes(wl, 0, np.arange(wl.N))
    f8 = lambda b: torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).to(torch.float64)
    bf = lambda u: torch.from_numpy(np.ascontiguousarray(u).astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    for t in (0, 1, 37, 255):
        got = oracle.dense_kl_row(wl, t, keys)
        n = t + 1
        qi = f8(configs.q_idx_bytes(wl, [t])[0])                   # [H_I, d]
        w = torch.from_numpy(configs.w_f32(wl, [t])[0]).to(torch.float64)
        ki = f8(keys[:n])                                            # [n, d]
        scores = (torch.relu(qi @ ki.T) * w[:, None]).sum(0)         # [n]
        q = bf(configs.q_bf16(wl, [t])[0])                           # [H, 576]
        kv = bf(configs.kv_bf16(wl, 0, np.arange(n)))                # [n, 576]
        z = q @ kv.T * wl.scale                                      # [H, n]
        target = torch.softmax(z, dim=1).mean(0)
        want = torch.nn.functional.kl_div(torch.log_softmax(scores, dim=0), target, reduction="sum").item()
        assert np.allclose(got["scores"], scores.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(got["lse"], torch.logsumexp(z, dim=1).numpy(), rtol=1e-12, atol=1e-12)
        assert got["kl"] == pytest.approx(want, rel=1e-10, abs=1e-13)


# --------------------------------------------------------------- sparse attention backward
def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to bf16 (nearest even) and return the bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bits_f64(u: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("seed,H,D_qk,D_v,m", [(0, 3, 16, 8, 5), (1, 2, 24, 16, 1), (2, 4, 12, 12, 9)])
def test_sparse_mla_bwd_matches_autograd(seed, H, D_qk, D_v, m):
    """dq and dkv against torch autograd (fp64) of the plain forward
    softmax(scale q K^T) V with V the first D_v dims of each latent row: the
    gradient is derived by the library, not retyped here."""
    rng = np.random.default_rng(seed)
    q = _bf16_bits(rng.standard_normal((H, D_qk)))
    kv = _bf16_bits(rng.standard_normal((m, D_qk)))
    dO = _bf16_bits(rng.standard_normal((H, D_v)))
    scale = 0.37
    dq, dkv = oracle.sparse_mla_bwd_row(q, kv, dO, scale)
    qt = torch.tensor(_bits_f64(q), requires_grad=True)
    kt = torch.tensor(_bits_f64(kv), requires_grad=True)
    out = torch.softmax(scale * qt @ kt.T, dim=-1) @ kt[:, :D_v]
    out.backward(torch.tensor(_bits_f64(dO)))
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dkv, kt.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_sparse_mla_bwd_matches_finite_differences():
    """Central differences of the oracle's own forward (fp64) along random
    directions agree with the directional derivative from dq and dkv."""
    rng = np.random.default_rng(7)
    H, D_qk, D_v, m, scale = 2, 8, 4, 4, 0.5
    q0 = _bits_f64(_bf16_bits(rng.standard_normal((H, D_qk))))
    kv0 = _bits_f64(_bf16_bits(rng.standard_normal((m, D_qk))))
    dO = _bf16_bits(rng.standard_normal((H, D_v)))
    g = _bits_f64(dO)
    dq, dkv = oracle.sparse_mla_bwd_row(_bf16_bits(q0), _bf16_bits(kv0), dO, scale)

    def loss(q, kv):  # sum dO . out, forward written out in numpy fp64
        z = scale * q @ kv.T
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        return float((g * (p @ kv[:, :D_v])).sum())

    for _ in range(3):
        uq, uk = rng.standard_normal(q0.shape), rng.standard_normal(kv0.shape)
        eps = 1e-5
        fd = (loss(q0 + eps * uq, kv0 + eps * uk) - loss(q0 - eps * uq, kv0 - eps * uk)) / (2 * eps)
        an = float((dq * uq).sum() + (dkv * uk).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_sparse_mla_bwd_closed_forms():
    rng = np.random.default_rng(3)
    H, D_qk, D_v = 3, 10, 6
    q = _bf16_bits(rng.standard_normal((H, D_qk)))
    dO = _bf16_bits(rng.standard_normal((H, D_v)))
    g = _bits_f64(dO)
    # one entry: P = 1, so the softmax Jacobian vanishes; the row gets sum_h dO[h]
    kv1 = _bf16_bits(rng.standard_normal((1, D_qk)))
    dq, dkv = oracle.sparse_mla_bwd_row(q, kv1, dO, 0.3)
    assert np.all(dq == 0.0)
    np.testing.assert_allclose(dkv[0, :D_v], g.sum(axis=0), rtol=1e-15)
    assert np.all(dkv[0, D_v:] == 0.0)
    # m copies of one row: P = 1/m, dZ = 0, each row gets sum_h dO[h] / m
    kv4 = np.repeat(kv1, 4, axis=0)
    dq, dkv = oracle.sparse_mla_bwd_row(q, kv4, dO, 0.3)
    assert np.abs(dq).max() < 1e-14
    np.testing.assert_allclose(dkv[:, :D_v], np.tile(g.sum(axis=0) / 4, (4, 1)), rtol=1e-13, atol=1e-15)
    # zero upstream gradient, and no entries at all
    dq, dkv = oracle.sparse_mla_bwd_row(q, kv4, np.zeros_like(dO), 0.3)
    assert not dq.any() and not dkv.any()
    dq, dkv = oracle.sparse_mla_bwd_row(q, kv4[:0], dO, 0.3)
    assert not dq.any() and dkv.shape == (0, D_qk)


def test_sparse_mla_bwd_magnitudes_bound_values():
    rng = np.random.default_rng(4)
    q = _bf16_bits(rng.standard_normal((3, 16)))
    kv = _bf16_bits(rng.standard_normal((6, 16)))
    dO = _bf16_bits(rng.standard_normal((3, 8)))
    dq, dkv, mq, mk = oracle.sparse_mla_bwd_row(q, kv, dO, 0.25, magnitudes=True)
    assert np.all(np.abs(dq) <= mq * (1 + 1e-12)) and np.all(np.abs(dkv) <= mk * (1 + 1e-12))
    assert mq.max() > 0 and mk.max() > 0


def test_sparse_mla_bwd_magnitude_scale_hand_values():
    """The magnitude scale that sets the backward's per-element tolerance, at a
    hand-computed case (pinned from both sides, so a scale that is too large
    fails as well as one that is too small).  H = 1, two rows, D_qk = 2, D_v = 1,
    scale 1/2: q = (1, 0), kv = (1, 2) and (1, -4), dO = (2).  Both logits are
    1/2, so P = (1/2, 1/2); A(s) = |dO|.|kv_s[:1]| = 2 for both rows and
    sum_s P A = 2, so each row's |dP - D| stand-in is P (A + sum P A) = 2.
    mag_dq[c] = sum_s scale * 2 * |kv_s,c| = (1 + 1, 2 + 4) = (2, 6);
    mag_dkv[s] = scale * 2 * |q| + P |dO| on the value dim = (1 + 1, 0) = (2, 0).
    The gradient itself: dP = 2 = D for both rows, so dq = 0 and each row
    gets P dO = 1 on its value dim."""
    q = _bf16_bits(np.array([[1.0, 0.0]]))
    kv = _bf16_bits(np.array([[1.0, 2.0], [1.0, -4.0]]))
    dO = _bf16_bits(np.array([[2.0]]))
    dq, dkv, mq, mk = oracle.sparse_mla_bwd_row(q, kv, dO, 0.5, magnitudes=True)
    np.testing.assert_allclose(mq, [[2.0, 6.0]], rtol=1e-15)
    np.testing.assert_allclose(mk, [[2.0, 0.0], [2.0, 0.0]], rtol=1e-15)
    np.testing.assert_allclose(dq, [[0.0, 0.0]], atol=1e-15)
    np.testing.assert_allclose(dkv, [[1.0, 0.0], [1.0, 0.0]], rtol=1e-15, atol=1e-15)
    # one row: P = 1, A = sum P A = |dO| |kv[:1]| = 2 * 3 = 6, stand-in 12;
    # mag_dq = scale * 12 * |kv| = (18, 3), mag_dkv = scale * 12 * |q| + (2, 0) = (8, 0)
    kv1 = _bf16_bits(np.array([[-3.0, 0.5]]))
    dq, dkv, mq, mk = oracle.sparse_mla_bwd_row(q, kv1, dO, 0.5, magnitudes=True)
    np.testing.assert_allclose(mq, [[18.0, 3.0]], rtol=1e-15)
    np.testing.assert_allclose(mk, [[8.0, 0.0]], rtol=1e-15)


@pytest.mark.parametrize("kind", ["decode", "paged_decode"])
def test_decode_row_candidates_are_the_whole_context(kind):
    """A decode query sits at position ctx_len - 1 and its own key is already in
    the cache, so it has exactly ctx_len candidates, 0 .. ctx_len - 1.  With
    k >= ctx_len the oracle therefore selects every one of them (its own
    position included) and pads the rest; with k = ctx_len - 1 it drops exactly
    one candidate, the lowest-scoring one (lowest position among equals)."""
    if kind == "decode":
        wl = configs.Workload("pin_decode", "decode", 2, B=3, N=37, H_I=4, H=8, k=40)
    else:
        wl = configs.Workload("pin_paged", "paged_decode", 5, B=3, N=128, H_I=4, H=8, k=200, ctx_lo=20, ctx_hi=70)
    ctx = configs.ctx_lens(wl)
    for b in range(wl.B):
        n = int(ctx[b])
        r = oracle.decode_row(wl, b)
        assert r["scores"].shape == (n,)
        assert np.array_equal(r["idx"][:n], np.arange(n)) and np.all(r["idx"][n:] == -1)
        r1 = oracle.decode_row(wl, b, k=n - 1)
        s = r["scores"]
        drop = int(np.flatnonzero(s == s.min())[-1])  # ties keep the lowest positions
        assert np.array_equal(r1["idx"], np.delete(np.arange(n), drop))
