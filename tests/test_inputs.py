"""Host-side checks of the seeded input generator (CPU only)."""
import numpy as np
import torch

from dsa_inputs import configs, gen


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-3).astype(np.float32),
                        # exact ties between two bf16 neighbours
                        (np.arange(1, 200, dtype=np.float32) + np.float32(2.0 ** -8)) * np.float32(1.0)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.f32_to_bf16_bits(x), ref)


def test_e4m3_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 3,
                        rng.uniform(-2 ** -5, 2 ** -5, 5000).astype(np.float32),   # subnormal range
                        np.array([0.0, -0.0, 448.0, -448.0, 1.0625, 1.1875, 2 ** -10, 3 * 2 ** -10,
                                  400.0, 440.0, 447.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(gen.f32_to_e4m3_bits(x), ref)
    # saturation beyond the largest finite value
    assert np.array_equal(gen.f32_to_e4m3_bits(np.array([500.0, -1e6], np.float32)), [0x7E, 0xFE])


def test_integer_e4m3_codes():
    assert np.array_equal(gen.int_to_e4m3_bits(np.arange(-4, 5)),
                          [0xC8, 0xC4, 0xC0, 0xB8, 0x00, 0x38, 0x40, 0x44, 0x48])


def test_normal_and_uniform_moments():
    x = gen.normal_f32(1, 99, np.arange(200000))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    assert np.all(np.abs(x) <= 6.0)
    # exact fp32 values on the 2^-16 grid
    assert np.array_equal(x * 65536, np.round(x * 65536))
    u = gen.uniform01_f32(1, 98, np.arange(100000))
    assert u.min() >= 0.0 and u.max() < 1.0 and abs(u.mean() - 0.5) < 0.01
    p = gen.pow2_quarter_f32(1, 97, np.arange(1000))
    assert set(np.unique(p)) == {0.25, 0.5, 1.0, 2.0}
    # streams and seeds are distinct
    assert not np.array_equal(gen.draws(1, 1, np.arange(8)), gen.draws(1, 2, np.arange(8)))
    assert not np.array_equal(gen.draws(1, 1, np.arange(8)), gen.draws(2, 1, np.arange(8)))


def test_rows_are_independent_of_slicing():
    wl = configs.WORKLOADS["prefill_L32k"]
    a = configs.q_idx_bytes(wl, [5, 6, 7])
    b = configs.q_idx_bytes(wl, [6])
    assert np.array_equal(a[1], b[0])
    ka = configs.kv_bf16(wl, 0, np.arange(10))
    kb = configs.kv_bf16(wl, 0, [3, 9])
    assert np.array_equal(ka[[3, 9]], kb)


def test_paged_layout_is_a_bijection_and_reads_back_logical_rows():
    wl = configs.WORKLOADS["paged_decode_b32_ctx4k_128k"]
    ctx = configs.ctx_lens(wl)
    assert ctx.min() >= 4096 and ctx.max() <= 131072 and len(ctx) == 32
    pt, P = configs.page_layout(wl)
    used = pt[pt >= 0]
    assert len(used) == P and np.array_equal(np.sort(used), np.arange(P))
    npg = (ctx + 63) // 64
    assert np.array_equal((pt >= 0).sum(1), npg)
    # build a small slice of the physical pool on the host through the row map
    rowmap = configs.pool_rowmap(wl, pt, P)
    b = 3
    s = np.array([0, 1, 63, 64, 1000, int(ctx[b]) - 1])
    phys = pt[b, s // 64].astype(np.int64) * 64 + s % 64
    logical = rowmap[phys]
    assert np.array_equal(logical, b * wl.S + s)
    # values in the pool at those physical rows equal the logical rows' values
    tok_vals = configs.k_idx_bytes(wl, b, s)
    pool_vals = np.stack([configs.k_idx_bytes(wl, int(lr // wl.S), [int(lr % wl.S)])[0] for lr in logical])
    assert np.array_equal(tok_vals, pool_vals)


def test_sample_rows():
    wl = configs.WORKLOADS["prefill_L128k"]
    r = configs.sample_rows(wl, 256)
    assert len(r) == 256 and len(np.unique(r)) == 256 and r.min() >= 0 and r.max() < wl.T
    assert np.array_equal(r, configs.sample_rows(wl, 256))


def test_chunk_rows_layout():
    """Paged-prefill rows: chunk b's rows are the last chunks[b] positions of
    sequence b, in order, and q_start delimits them."""
    wl = configs.WORKLOADS["paged_prefill_mixed"]
    q_start, seq, pos = configs.chunk_rows(wl)
    assert q_start[0] == 0 and q_start[-1] == wl.T == len(seq) == len(pos)
    for b, (c, n) in enumerate(zip(wl.ctxs, wl.chunks)):
        sl = slice(q_start[b], q_start[b + 1])
        assert np.all(seq[sl] == b)
        assert np.array_equal(pos[sl], np.arange(c - n, c))
    assert list(configs.ctx_lens(wl)) == list(wl.ctxs)
    pt, P = configs.page_layout(wl)
    assert P == sum((c + wl.page - 1) // wl.page for c in wl.ctxs)
    assert sorted(pt[pt >= 0].tolist()) == list(range(P))
