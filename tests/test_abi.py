"""The C-ABI library loads, exports every entry point include/dsa.h declares,
and rejects bad arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

import sparse_attention_long_08_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    declared = _declared()
    assert declared, "no declarations parsed"
    assert sorted(dsa.SIGNATURES) == declared


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dsa.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = dsa.load()
    assert lib.dsa_abi_version() == 2
    for s in range(5):
        assert lib.dsa_status_string(s)
    assert lib.dsa_status_string(99) == b"unknown status"


FAKE = 0x100000  # an aligned non-null address; validation fails before any use


@pytest.mark.parametrize("args,status,needle", [
    # d_I must be 128
    ((FAKE, FAKE, FAKE, 4, 8, 4, 64, 0, FAKE, 8, 0), 2, "d_I"),
    # H_I range
    ((FAKE, FAKE, FAKE, 4, 8, 65, 128, 0, FAKE, 8, 0), 2, "H_I"),
    # ld < N
    ((FAKE, FAKE, FAKE, 4, 8, 4, 128, 0, FAKE, 7, 0), 1, "ld"),
    # null pointer
    ((0, FAKE, FAKE, 4, 8, 4, 128, 0, FAKE, 8, 0), 1, "q_idx"),
    # misaligned pointer
    ((FAKE + 4, FAKE, FAKE, 4, 8, 4, 128, 0, FAKE, 8, 0), 1, "aligned"),
])
def test_indexer_validation(args, status, needle):
    lib = dsa.load()
    st = lib.dsa_indexer_scores(*args)
    assert st == status
    assert needle in lib.dsa_last_error_message().decode()


def test_topk_and_attention_validation():
    lib = dsa.load()
    assert lib.dsa_topk(FAKE, 8, 2, 8, 0, 0, 0, FAKE, 0) == 2          # k = 0
    assert lib.dsa_topk(FAKE, 8, 2, 8, 0, 0, 5000, FAKE, 0) == 2       # k too large
    assert lib.dsa_topk(FAKE, 300000, 2, 300000, 0, 0, 8, FAKE, 0) == 2  # row longer than supported
    assert lib.dsa_topk(FAKE, 8, 0, 8, 0, 0, 4, FAKE, 0) == 0          # empty call is a no-op
    # attention: D_qk / D_v / H / scale / workspace
    assert lib.dsa_sparse_mla_fwd(FAKE, FAKE, FAKE, 4, 8, 8, 512, 512, 4, 0.1, FAKE, FAKE, 0, 0, 0) == 2
    assert lib.dsa_sparse_mla_fwd(FAKE, FAKE, FAKE, 4, 8, 8, 576, 256, 4, 0.1, FAKE, FAKE, 0, 0, 0) == 2
    assert lib.dsa_sparse_mla_fwd(FAKE, FAKE, FAKE, 4, 8, 200, 576, 512, 4, 0.1, FAKE, FAKE, 0, 0, 0) == 2
    assert lib.dsa_sparse_mla_fwd(FAKE, FAKE, FAKE, 4, 8, 8, 576, 512, 4, -1.0, FAKE, FAKE, 0, 0, 0) == 1
    need = lib.dsa_sparse_mla_fwd_workspace_bytes(4, 128, 512, 2048)
    assert need > 0  # few queries: split partials need scratch
    assert lib.dsa_sparse_mla_fwd(FAKE, FAKE, FAKE, 4, 8, 128, 576, 512, 2048, 0.1, FAKE, FAKE, FAKE, need - 1,
                                  0) == 3
    assert lib.dsa_sparse_mla_fwd_workspace_bytes(100000, 128, 512, 2048) == 0


def test_fused_validation():
    lib = dsa.load()
    need = lib.dsa_forward_prefill_workspace_bytes(1024, 1024, 128, 512, 64)
    assert need >= 1024 * 1024 * 4
    st = lib.dsa_forward_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, 1024, 1024, 64, 128, 128, 576, 512, 64, 0, 0.07, 0,
                                 FAKE, FAKE, FAKE, need - 1, 0)
    assert st == 3 and "workspace" in lib.dsa_last_error_message().decode()
    # paged decode: page size and context bound
    st = lib.dsa_forward_decode_paged(FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, 4, FAKE, 32, 2, 100, 64, 128, 128, 576,
                                      512, 64, 0.07, 0, FAKE, FAKE, FAKE, 1 << 30, 0)
    assert st == 2 and "page_size" in lib.dsa_last_error_message().decode()
    st = lib.dsa_forward_decode_paged(FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, 4, FAKE, 64, 2, 300, 64, 128, 128, 576,
                                      512, 64, 0.07, 0, FAKE, FAKE, FAKE, 1 << 30, 0)
    assert st == 1 and "max_ctx" in lib.dsa_last_error_message().decode()


def test_binding_raises():
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_indexer_scores(FAKE, FAKE, FAKE, 4, 8, 4, 64, 0, FAKE, 8, stream=0)
    assert e.value.status == 2


def test_timing_end_validation():
    """dsa_timing_end rejects a bad kind count or missing arrays; with nothing
    recorded it returns zeros (no HIP call is made)."""
    n = len(dsa.TIMING_KINDS)
    lib = dsa.load()
    assert lib.dsa_timing_begin() == 0
    ms = (ctypes.c_double * 8)()
    launches = (ctypes.c_int64 * 8)()
    assert lib.dsa_timing_end(ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(launches, ctypes.c_void_p), n + 1) == 1
    assert "n_kinds" in lib.dsa_last_error_message().decode()
    assert lib.dsa_timing_end(None, None, n) == 1
    assert lib.dsa_timing_end(None, None, 0) == 0
    assert lib.dsa_timing_begin() == 0
    assert dsa.dsa_timing_end() == {kind: (0.0, 0) for kind in dsa.TIMING_KINDS}


@pytest.mark.parametrize("q_start,ctx,page_size,status,needle", [
    ([1, 4], [8], 64, 1, "q_start[0]"),
    ([0, 4, 2], [8, 8], 64, 1, "non-decreasing"),
    ([0, 9], [8], 64, 1, "ctx_len[0]"),            # more new rows than tokens
    ([0, 4], [64 * 4 + 1], 64, 1, "ctx_len[0]"),   # beyond max_pages * page_size
    ([0, 4], [8], 32, 2, "page_size"),
])
def test_paged_prefill_validation(q_start, ctx, page_size, status, needle):
    B = len(ctx)
    qs = (ctypes.c_int64 * (B + 1))(*q_start)
    cl = (ctypes.c_int64 * B)(*ctx)
    lib = dsa.load()
    st = lib.dsa_forward_prefill_paged(FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, page_size,
                                       ctypes.cast(qs, ctypes.c_void_p), ctypes.cast(cl, ctypes.c_void_p), B, 64,
                                       128, 8, 576, 512, 32, 0.07, 0, FAKE, FAKE, FAKE, 1 << 30, 0)
    assert st == status
    assert needle in lib.dsa_last_error_message().decode()


@pytest.mark.parametrize("args,status,needle", [
    ((FAKE, FAKE, FAKE, 7, 4, 8, 0, 8, 576, 0.07, FAKE, 0, 0), 1, "ld"),
    ((FAKE, FAKE, FAKE, 8, 4, 8, -1, 8, 576, 0.07, FAKE, 0, 0), 1, "q_pos0"),
    ((FAKE, FAKE, FAKE, 8, 4, 8, 0, 8, 512, 0.07, FAKE, 0, 0), 2, "D_qk"),
    ((FAKE, FAKE, FAKE, 8, 4, 8, 0, 129, 576, 0.07, FAKE, 0, 0), 2, "H"),
    ((FAKE, FAKE, 0, 8, 4, 8, 0, 8, 576, 0.07, FAKE, 0, 0), 1, "scores"),
])
def test_dense_kl_validation(args, status, needle):
    lib = dsa.load()
    assert lib.dsa_indexer_dense_kl_fwd(*args) == status
    assert needle in lib.dsa_last_error_message().decode()


def test_dense_warmup_workspace_validation():
    lib = dsa.load()
    nb = lib.dsa_dense_warmup_loss_workspace_bytes(8, 16)
    assert nb >= 8 * 64 * 4
    st = lib.dsa_dense_warmup_loss(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 4, 128, 8, 576, 0, 0.07, FAKE, 0, FAKE,
                                   nb - 1, 0)
    assert st == 3 and "workspace" in lib.dsa_last_error_message().decode()


# dsa_sparse_mla_bwd(q, kv, idx, out, lse, dout, T, N, H, D_qk, D_v, k, scale, dq, dkv, ws, ws_bytes, stream)
@pytest.mark.parametrize("args,status,needle", [
    ((FAKE,) * 6 + (4, 0, 8, 576, 512, 16, 0.07, FAKE, FAKE, FAKE, 1 << 30, 0), 1, "N"),
    ((FAKE,) * 6 + (4, 64, 8, 576, 256, 16, 0.07, FAKE, FAKE, FAKE, 1 << 30, 0), 2, "D_v"),
    ((FAKE,) * 6 + (4, 64, 0, 576, 512, 16, 0.07, FAKE, FAKE, FAKE, 1 << 30, 0), 2, "H"),
    ((FAKE,) * 6 + (4, 64, 8, 576, 512, 5000, 0.07, FAKE, FAKE, FAKE, 1 << 30, 0), 2, "k"),
    ((FAKE,) * 6 + (4, 64, 8, 576, 512, 16, -1.0, FAKE, FAKE, FAKE, 1 << 30, 0), 1, "scale"),
    ((FAKE,) * 6 + (4, 64, 8, 576, 512, 16, 0.07, FAKE, 0, FAKE, 1 << 30, 0), 1, "dkv"),
    ((FAKE,) * 5 + (0,) + (4, 64, 8, 576, 512, 16, 0.07, FAKE, FAKE, FAKE, 1 << 30, 0), 1, "dout"),
    ((FAKE,) * 6 + (4, 64, 8, 576, 512, 16, 0.07, FAKE + 4, FAKE, FAKE, 1 << 30, 0), 1, "aligned"),
])
def test_sparse_mla_bwd_validation(args, status, needle):
    lib = dsa.load()
    assert lib.dsa_sparse_mla_bwd(*args) == status
    assert needle in lib.dsa_last_error_message().decode()


def _bwd_ws_bytes(T, N, H, k):
    """The documented layout: P and dS (bf16 [tile, k rounded up to 32, H
    rounded up to 64]), bf16 addend rows [tile, k, 576], row counts [N], row
    offsets [N+1] and the entry list [tile * k] (int32), each region 256-byte
    aligned; tile = min(T, 2048)."""
    al = lambda x: (x + 255) // 256 * 256
    ent = min(T, 2048) * k
    ent_p = min(T, 2048) * ((k + 31) // 32 * 32)
    hs = (H + 63) // 64 * 64
    return 2 * al(ent_p * hs * 2) + al(ent * 576 * 2) + al(N * 4) + al((N + 1) * 4) + al(ent * 4)


def test_sparse_mla_bwd_workspace():
    lib = dsa.load()
    for T, N, H, k in [(4, 64, 8, 16), (32768, 32768, 128, 2048), (3000, 5000, 96, 100)]:
        assert lib.dsa_sparse_mla_bwd_workspace_bytes(T, N, H, k) == _bwd_ws_bytes(T, N, H, k)
    assert lib.dsa_sparse_mla_bwd_workspace_bytes(32768, 32768, 128, 2048) < 7 * 2 ** 30
    assert lib.dsa_sparse_mla_bwd_workspace_bytes(0, 64, 128, 2048) == 0
    nb = lib.dsa_sparse_mla_bwd_workspace_bytes(4, 64, 8, 16)
    st = lib.dsa_sparse_mla_bwd(*((FAKE,) * 6), 4, 64, 8, 576, 512, 16, 0.07, FAKE, FAKE, FAKE, nb - 1, 0)
    assert st == 3 and "ws_bytes" in lib.dsa_last_error_message().decode()


def test_noalloc_decode_rejects_oversized_calls():
    """The allocation-free paged decode validates like the workspace call, and
    refuses (before any launch) a shape whose scratch exceeds its 96 MiB."""
    lib = dsa.load()
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, 4096, FAKE, 64, 64, 262144, 64, 128, 128, 576, 512, 2048, 0.07,
            FAKE, FAKE, FAKE, 0]
    need = lib.dsa_forward_decode_paged_workspace_bytes(64, 262144, 128, 512, 2048)
    assert need > 96 << 20
    assert lib.dsa_forward_decode_paged_noalloc(*args) == 2
    assert "maximum" in lib.dsa_last_error_message().decode()
    bad = list(args)
    bad[9] = 32  # page size
    assert lib.dsa_forward_decode_paged_noalloc(*bad) == 2
    bad = list(args)
    bad[2] = 0  # k_pool
    assert lib.dsa_forward_decode_paged_noalloc(*bad) == 1
    bad = list(args)
    bad[10] = 0  # B = 0 is a no-op
    assert lib.dsa_forward_decode_paged_noalloc(*bad) == 0
