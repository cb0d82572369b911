"""GPU parity of the sparse MLA-MQA attention backward (the gradient the sparse
training stage of the "DeepSeek-V3.2" walk-through, §2.3.2, takes through the
attention of §2.1.2) against the CPU oracle.  The forward's out and lse come
from the GPU forward of the same inputs (they are inputs of the backward
kernels); the oracle recomputes the whole gradient from q, kv, idx and dO.

Tolerance: P and dS enter the gradient products as bf16 (relative error at
most 2^-9 each), and D = dO . out inherits the forward's bf16 probabilities
(at most 2^-9 of sum_s P A(s)).  The oracle returns, for every output element,
the same sum over absolute values with |dP - D| replaced by A(s) + sum_s P A
(A(s) = sum_c |dO_c| |kv_s,c|), so each element must lie within 2^-7 (four
units of 2^-9) of that scale; elements whose scale is 0 must be exactly 0.
Each tensor must also match in the Frobenius norm to 2^-7 relative: the
rounding errors above have random sign, and the normwise error measured on
these cases is about 1.6e-3 (dS sums to zero over the entries of a head, so
the errors of its terms do not average out against the sum); a misplaced or
wrong term shows up as an error of the order of the norm itself."""
import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import configs, device, gen
from dsa_run import ws_tensor

pytestmark = pytest.mark.gpu

TOL = 2.0 ** -7


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _bwd_on_gpu(dsa, q, kv, idx, dO, T, N, H, k, scale):
    """Forward (for out and lse), then the backward; returns dq, dkv on the host."""
    q_d = torch.from_numpy(q.view(np.int16)).cuda().view(torch.uint16) if isinstance(q, np.ndarray) else q
    kv_d = torch.from_numpy(kv.view(np.int16)).cuda().view(torch.uint16) if isinstance(kv, np.ndarray) else kv
    idx_d = torch.from_numpy(idx).cuda()
    do_d = torch.from_numpy(dO.view(np.int16)).cuda().view(torch.uint16)
    out = torch.empty((max(T, 1), H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((max(T, 1), H), dtype=torch.float32, device="cuda")
    if T > 0:
        nb = dsa.dsa_sparse_mla_fwd_workspace_bytes(T, H, 512, k)
        ws = ws_tensor(nb)
        dsa.dsa_sparse_mla_fwd(q_d, kv_d, idx_d, T, N, H, 576, 512, k, scale, out, lse, ws, nb)
    dq = torch.full((max(T, 1), H, 576), float("nan"), dtype=torch.float32, device="cuda")
    dkv = torch.full((N, 576), float("nan"), dtype=torch.float32, device="cuda")
    nbb = dsa.dsa_sparse_mla_bwd_workspace_bytes(T, N, H, k)
    wsb = ws_tensor(nbb)
    dsa.dsa_sparse_mla_bwd(q_d, kv_d, idx_d, out, lse, do_d, T, N, H, 576, 512, k, scale, dq, dkv, wsb, nbb)
    torch.cuda.synchronize()
    return dq.cpu().numpy()[:T], dkv.cpu().numpy()


def _oracle(q, kv_rows_of, idx, dO, N, scale):
    """dq [T, H, 576], dkv [N, 576] and their magnitude scales from the oracle."""
    T, H, _ = q.shape
    dq = np.zeros((T, H, 576))
    mq = np.zeros_like(dq)
    dkv = np.zeros((N, 576))
    mk = np.zeros_like(dkv)
    for t in range(T):
        sel = idx[t][(idx[t] >= 0) & (idx[t] < N)]
        d, rows, m1, m2 = oracle.sparse_mla_bwd_row(q[t], kv_rows_of(sel), dO[t], scale, magnitudes=True)
        dq[t], mq[t] = d, m1
        np.add.at(dkv, sel, rows)
        np.add.at(mk, sel, m2)
    return dq, mq, dkv, mk


def _check(g, ref, mag, what):
    """Every element within TOL of its scale, and the whole tensor within 2^-7
    of the oracle in the Frobenius norm (the elementwise scales are worst-case
    sums; the normwise bound catches errors that stay below them)."""
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    diff = g.astype(np.float64) - ref
    rn = float(np.linalg.norm(diff)) / max(float(np.linalg.norm(ref)), 1e-300)
    assert rn <= 2.0 ** -7, f"{what}: relative Frobenius error {rn:.3e}"
    err = np.abs(diff)
    bad = err > TOL * mag
    if bad.any():
        i = np.unravel_index(np.argmax(err - TOL * mag), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; worst at {i}: gpu {g[i]} "
                             f"oracle {ref[i]} scale {mag[i]}")


def _rand_idx(rng, T, k, n):
    idx = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        m = int(rng.integers(1, min(k, n) + 1)) if t % 4 else min(k, n)
        idx[t, :m] = np.sort(rng.choice(n, size=m, replace=False))
    return idx


@pytest.mark.parametrize("T,k,H,N", [(40, 72, 8, 256), (24, 100, 128, 512), (9, 70, 40, 300), (7, 130, 96, 400),
                                     (5, 2048, 128, 4096)])
def test_sparse_mla_bwd_against_oracle(dsa, T, k, H, N):
    """Several 32-entry blocks with a ragged tail, padded rows, an all-padding
    row, an out-of-range entry, a repeated index, head counts below 128
    (padded heads)."""
    _case(f"sparse_mla_bwd T={T} k={k} H={H} N={N}")
    wl = configs.Workload(**{**configs.WORKLOADS["prefill_L32k"].__dict__, "H": H, "N": N})
    rng = np.random.default_rng(T * 31 + k + H)
    q = configs.q_bf16(wl, np.arange(T))
    kv = configs.kv_bf16(wl, 0, np.arange(N))
    dO = gen.f32_to_bf16_bits(rng.standard_normal((T, H, 512)).astype(np.float32))
    idx = _rand_idx(rng, T, k, N)
    idx[0, :] = -1          # no valid entry: dq = 0, nothing scattered
    idx[1, -1] = N + 5      # out-of-range entries are skipped
    if T > 2 and k >= 3:
        idx[2, 1:3] = idx[2, 0]  # a repeated index counts once per occurrence, as in the forward
    dq, dkv = _bwd_on_gpu(dsa, q, kv, idx, dO, T, N, H, k, wl.scale)
    rdq, mq, rdkv, mk = _oracle(q, lambda sel: kv[sel], idx, dO, N, wl.scale)
    assert np.all(dq[0] == 0.0)
    _check(dq, rdq, mq, "dq")
    _check(dkv, rdkv, mk, "dkv")


def test_sparse_mla_bwd_several_query_tiles(dsa):
    """4100 queries: the call works through query tiles of 2048 (the last one
    ragged), so dq is written per tile and dkv sums contributions across
    tiles; every element is compared."""
    T, k, H, N = 4100, 40, 8, 300
    _case(f"sparse_mla_bwd T={T} k={k} H={H} N={N} (three query tiles)")
    wl = configs.Workload(**{**configs.WORKLOADS["tiny_prefill_L256"].__dict__, "H": H, "N": N})
    rng = np.random.default_rng(4100)
    q = configs.q_bf16(wl, np.arange(T))
    kv = configs.kv_bf16(wl, 0, np.arange(N))
    dO = gen.f32_to_bf16_bits(rng.standard_normal((T, H, 512)).astype(np.float32))
    idx = _rand_idx(rng, T, k, N)
    dq, dkv = _bwd_on_gpu(dsa, q, kv, idx, dO, T, N, H, k, wl.scale)
    rdq, mq, rdkv, mk = _oracle(q, lambda sel: kv[sel], idx, dO, N, wl.scale)
    _check(dq, rdq, mq, "dq")
    _check(dkv, rdkv, mk, "dkv")


def test_sparse_mla_bwd_full_size_sampled_rows(dsa):
    """The 32K-token workload's shapes (N = 32768 cached rows, k = 2048, 128
    heads) in the launch configuration of a full run, on 12 seeded-random query
    positions plus two early ones with fewer than k candidates; every element of
    dq and dkv is compared."""
    wl = configs.WORKLOADS["prefill_L32k"]
    pos = np.concatenate([[0, 700], configs.sample_rows(wl, 12)]).astype(np.int64)
    T, N, H, k = len(pos), wl.N, wl.H, wl.k
    _case(f"sparse_mla_bwd full size T={T} N={N} k={k}")
    q = configs.q_bf16(wl, pos)
    kv_d = torch.empty((N, 576), dtype=torch.uint16, device="cuda")
    device.fill(kv_d, N, 576, device.BF16_NORMAL, wl.seed, gen.STREAM_KV, div=wl.kv_div)
    dO = configs.dout_bf16(wl, pos)
    idx = configs.random_selection(wl, pos)
    dq, dkv = _bwd_on_gpu(dsa, q, kv_d, idx, dO, T, N, H, k, wl.scale)
    rdq, mq, rdkv, mk = _oracle(q, lambda sel: configs.kv_bf16(wl, 0, sel), idx, dO, N, wl.scale)
    _check(dq, rdq, mq, "dq")
    _check(dkv, rdkv, mk, "dkv")


def test_sparse_mla_bwd_empty_batch_clears_dkv(dsa):
    _case("sparse_mla_bwd T=0")
    N, H, k = 100, 8, 16
    q = np.zeros((0, H, 576), dtype=np.uint16)
    kv = np.zeros((N, 576), dtype=np.uint16)
    dO = np.zeros((0, H, 512), dtype=np.uint16)
    idx = np.zeros((0, k), dtype=np.int32)
    q_d = torch.empty((1, H, 576), dtype=torch.uint16, device="cuda")
    kv_d = torch.from_numpy(kv.view(np.int16)).cuda().view(torch.uint16)
    dkv = torch.full((N, 576), float("nan"), dtype=torch.float32, device="cuda")
    dq = torch.empty((1, H, 576), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_mla_bwd(q_d, kv_d, torch.empty((1, k), dtype=torch.int32, device="cuda"),
                           torch.empty((1, H, 512), device="cuda"), torch.empty((1, H), device="cuda"),
                           torch.empty((1, H, 512), dtype=torch.uint16, device="cuda"), 0, N, H, 576, 512, k, 0.1,
                           dq, dkv, None, 0)
    torch.cuda.synchronize()
    assert torch.all(dkv == 0).item()
    del q, dO, idx
