"""Python binding of libdsa.so, the gfx950 DeepSeek Sparse Attention forward
library.

Argument marshalling only: each function has the name of the C-ABI entry
point it calls (see include/dsa.h), takes torch CUDA tensors for device
buffers and raises ``DsaError`` on a non-OK status.  Every step of the path
runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# DSA_LIB_PATH selects another build of the library (e.g. a sanitizer build of its host code)
LIB_PATH = os.environ.get("DSA_LIB_PATH") or os.path.join(_HERE, "libdsa.so")
_lib = None

_c_i32, _c_i64, _c_f32, _c_sz, _c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

# argument type lists of every exported entry point (mirrors include/dsa.h)
SIGNATURES = {
    "dsa_abi_version": (_c_i32, []),
    "dsa_status_string": (ctypes.c_char_p, [_c_i32]),
    "dsa_last_error_message": (ctypes.c_char_p, []),
    "dsa_timing_begin": (_c_i32, []),
    "dsa_timing_end": (_c_i32, [_c_p, _c_p, _c_i32]),
    "dsa_indexer_scores": (_c_i32, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i64, _c_p, _c_i64, _c_p]),
    "dsa_indexer_scores_paged": (_c_i32, [_c_p, _c_p, _c_p, _c_i64, _c_p, _c_i32, _c_p, _c_i32, _c_i64, _c_i32,
                                          _c_i32, _c_i64, _c_p, _c_i64, _c_p]),
    "dsa_topk": (_c_i32, [_c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_i32, _c_p, _c_p]),
    "dsa_sparse_mla_fwd_workspace_bytes": (_c_sz, [_c_i64, _c_i32, _c_i32, _c_i32]),
    "dsa_sparse_mla_fwd": (_c_i32, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _c_p,
                                    _c_p, _c_p, _c_sz, _c_p]),
    "dsa_sparse_mla_bwd_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i32, _c_i32]),
    "dsa_sparse_mla_bwd": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                    _c_i32, _c_f32, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "dsa_sparse_mla_fwd_paged_workspace_bytes": (_c_sz, [_c_i64, _c_i32, _c_i32, _c_i32]),
    "dsa_sparse_mla_fwd_paged": (_c_i32, [_c_p, _c_p, _c_i64, _c_p, _c_i32, _c_p, _c_i32, _c_p, _c_i64, _c_i32,
                                          _c_i32, _c_i32, _c_i32, _c_f32, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "dsa_indexer_kl_fwd": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                    _c_f32, _c_p, _c_p]),
    "dsa_indexer_dense_kl_fwd": (_c_i32, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_f32,
                                          _c_p, _c_p, _c_p]),
    "dsa_dense_warmup_loss_workspace_bytes": (_c_sz, [_c_i64, _c_i64]),
    "dsa_dense_warmup_loss": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                       _c_i64, _c_f32, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "dsa_forward_prefill_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32]),
    "dsa_forward_prefill": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                     _c_i32, _c_i32, _c_i64, _c_f32, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "dsa_forward_prefill_plan": (_c_i32, [_c_i64, _c_i64, _c_p, _c_p]),
    "dsa_forward_prefill_paged_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32]),
    "dsa_forward_prefill_paged": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i32, _c_i32, _c_p, _c_p,
                                           _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _c_p,
                                           _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "dsa_forward_decode_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32]),
    "dsa_forward_decode": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                    _c_i32, _c_i32, _c_i32, _c_f32, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "dsa_forward_decode_paged_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32]),
    "dsa_forward_decode_paged": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i32, _c_p, _c_i32,
                                          _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32,
                                          _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "dsa_forward_decode_paged_noalloc": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i32, _c_p, _c_i32,
                                                  _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                  _c_f32, _c_p, _c_p, _c_p, _c_p]),
}


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def build() -> str:
    from . import _builder
    return _builder.build()


def load():
    """Load libdsa.so (building it first only when no built library exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name: str, *args) -> None:
    lib = load()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise DsaError(name, st, lib.dsa_last_error_message().decode())


def dsa_abi_version() -> int:
    return load().dsa_abi_version()


# stage kinds of dsa_timing_end
TIMING_KINDS = ("indexer", "topk", "attention", "indexer_kl", "dense_kl", "mla_bwd_dq", "mla_bwd_dkv",
                "mla_bwd_reduce")


def dsa_timing_begin() -> None:
    _call("dsa_timing_begin")


def dsa_timing_end():
    """Stops launch timing; returns {kind: (summed ms, launches)} for TIMING_KINDS."""
    n = len(TIMING_KINDS)
    ms = (ctypes.c_double * n)()
    launches = (ctypes.c_int64 * n)()
    _call("dsa_timing_end", ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(launches, ctypes.c_void_p), n)
    return {kind: (ms[i], launches[i]) for i, kind in enumerate(TIMING_KINDS)}


def dsa_indexer_scores(q_idx, w, k_idx, T, N, H_I, d_I, q_pos0, scores, ld, stream=None):
    _call("dsa_indexer_scores", _ptr(q_idx), _ptr(w), _ptr(k_idx), T, N, H_I, d_I, q_pos0, _ptr(scores), ld,
          _stream(stream))


def dsa_indexer_scores_paged(q_idx, w, k_pool, n_pages, page_table, max_pages, ctx_len, page_size, B, H_I, d_I,
                             max_ctx, scores, ld, stream=None):
    _call("dsa_indexer_scores_paged", _ptr(q_idx), _ptr(w), _ptr(k_pool), n_pages, _ptr(page_table), max_pages,
          _ptr(ctx_len), page_size, B, H_I, d_I, max_ctx, _ptr(scores), ld, _stream(stream))


def dsa_topk(scores, ld, T, N, q_pos0, n_valid, k, idx, stream=None):
    _call("dsa_topk", _ptr(scores), ld, T, N, q_pos0, _ptr(n_valid), k, _ptr(idx), _stream(stream))


def dsa_sparse_mla_fwd_workspace_bytes(T, H, D_v, k) -> int:
    return load().dsa_sparse_mla_fwd_workspace_bytes(T, H, D_v, k)


def dsa_sparse_mla_fwd(q, kv, idx, T, N, H, D_qk, D_v, k, scale, out, lse, ws, ws_bytes, stream=None):
    _call("dsa_sparse_mla_fwd", _ptr(q), _ptr(kv), _ptr(idx), T, N, H, D_qk, D_v, k, scale, _ptr(out), _ptr(lse),
          _ptr(ws), ws_bytes, _stream(stream))


def dsa_sparse_mla_bwd_workspace_bytes(T, N, H, k) -> int:
    return load().dsa_sparse_mla_bwd_workspace_bytes(T, N, H, k)


def dsa_sparse_mla_bwd(q, kv, idx, out, lse, dout, T, N, H, D_qk, D_v, k, scale, dq, dkv, ws, ws_bytes,
                       stream=None):
    _call("dsa_sparse_mla_bwd", _ptr(q), _ptr(kv), _ptr(idx), _ptr(out), _ptr(lse), _ptr(dout), T, N, H, D_qk, D_v,
          k, scale, _ptr(dq), _ptr(dkv), _ptr(ws), ws_bytes, _stream(stream))


def dsa_sparse_mla_fwd_paged_workspace_bytes(B, H, D_v, k) -> int:
    return load().dsa_sparse_mla_fwd_paged_workspace_bytes(B, H, D_v, k)


def dsa_sparse_mla_fwd_paged(q, kv_pool, n_pages, page_table, max_pages, ctx_len, page_size, idx, B, H, D_qk, D_v,
                             k, scale, out, lse, ws, ws_bytes, stream=None):
    _call("dsa_sparse_mla_fwd_paged", _ptr(q), _ptr(kv_pool), n_pages, _ptr(page_table), max_pages, _ptr(ctx_len),
          page_size, _ptr(idx), B, H, D_qk, D_v, k, scale, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
          _stream(stream))


def dsa_indexer_kl_fwd(q, kv, idx, lse, scores, ld, T, N, H, D_qk, k, scale, kl, stream=None):
    _call("dsa_indexer_kl_fwd", _ptr(q), _ptr(kv), _ptr(idx), _ptr(lse), _ptr(scores), ld, T, N, H, D_qk, k, scale,
          _ptr(kl), _stream(stream))


def dsa_indexer_dense_kl_fwd(q, kv, scores, ld, T, N, q_pos0, H, D_qk, scale, kl, lse=None, stream=None):
    _call("dsa_indexer_dense_kl_fwd", _ptr(q), _ptr(kv), _ptr(scores), ld, T, N, q_pos0, H, D_qk, scale, _ptr(kl),
          _ptr(lse), _stream(stream))


def dsa_dense_warmup_loss_workspace_bytes(T, N) -> int:
    return load().dsa_dense_warmup_loss_workspace_bytes(T, N)


def dsa_dense_warmup_loss(q_idx, w, k_idx, q, kv, T, N, H_I, d_I, H, D_qk, q_pos0, scale, kl, lse, ws, ws_bytes,
                          stream=None):
    _call("dsa_dense_warmup_loss", _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(q), _ptr(kv), T, N, H_I, d_I, H, D_qk,
          q_pos0, scale, _ptr(kl), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream))


def dsa_forward_prefill_workspace_bytes(T, N, H, D_v, k) -> int:
    return load().dsa_forward_prefill_workspace_bytes(T, N, H, D_v, k)


def dsa_forward_prefill(q_idx, w, k_idx, q, kv, T, N, H_I, d_I, H, D_qk, D_v, k, q_pos0, scale, idx, out, lse, ws,
                        ws_bytes, stream=None):
    _call("dsa_forward_prefill", _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(q), _ptr(kv), T, N, H_I, d_I, H, D_qk,
          D_v, k, q_pos0, scale, _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream))


def dsa_forward_prefill_paged_workspace_bytes(total_q, max_ctx, H, D_v, k) -> int:
    return load().dsa_forward_prefill_paged_workspace_bytes(total_q, max_ctx, H, D_v, k)


def dsa_forward_prefill_paged(q_idx, w, k_pool, q, kv_pool, n_pages, page_table, max_pages, page_size, q_start,
                              ctx_len, B, H_I, d_I, H, D_qk, D_v, k, scale, idx, out, lse, ws, ws_bytes,
                              stream=None):
    """q_start ([B+1]) and ctx_len ([B]) are host sequences of ints."""
    qs = (ctypes.c_int64 * (B + 1))(*[int(x) for x in q_start])
    cl = (ctypes.c_int64 * max(B, 1))(*[int(x) for x in ctx_len])
    _call("dsa_forward_prefill_paged", _ptr(q_idx), _ptr(w), _ptr(k_pool), _ptr(q), _ptr(kv_pool), n_pages,
          _ptr(page_table), max_pages, page_size, ctypes.cast(qs, ctypes.c_void_p), ctypes.cast(cl, ctypes.c_void_p),
          B, H_I, d_I, H, D_qk, D_v, k, scale, _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream))


def dsa_forward_prefill_plan(T, N):
    """Returns (tile_rows, score_ld) of the fused prefill's row tiling."""
    tr, ld = ctypes.c_int64(0), ctypes.c_int64(0)
    _call("dsa_forward_prefill_plan", T, N, ctypes.byref(tr), ctypes.byref(ld))
    return tr.value, ld.value


def dsa_forward_decode_workspace_bytes(B, N, H, D_v, k) -> int:
    return load().dsa_forward_decode_workspace_bytes(B, N, H, D_v, k)


def dsa_forward_decode(q_idx, w, k_idx, q, kv, ctx_len, B, N, H_I, d_I, H, D_qk, D_v, k, scale, idx, out, lse, ws,
                       ws_bytes, stream=None):
    _call("dsa_forward_decode", _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(q), _ptr(kv), _ptr(ctx_len), B, N, H_I,
          d_I, H, D_qk, D_v, k, scale, _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream))


def dsa_forward_decode_paged_workspace_bytes(B, max_ctx, H, D_v, k) -> int:
    return load().dsa_forward_decode_paged_workspace_bytes(B, max_ctx, H, D_v, k)


def dsa_forward_decode_paged(q_idx, w, k_pool, q, kv_pool, n_pages, page_table, max_pages, ctx_len, page_size, B,
                             max_ctx, H_I, d_I, H, D_qk, D_v, k, scale, idx, out, lse, ws, ws_bytes, stream=None):
    _call("dsa_forward_decode_paged", _ptr(q_idx), _ptr(w), _ptr(k_pool), _ptr(q), _ptr(kv_pool), n_pages,
          _ptr(page_table), max_pages, _ptr(ctx_len), page_size, B, max_ctx, H_I, d_I, H, D_qk, D_v, k, scale,
          _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream))


def dsa_forward_decode_paged_noalloc(q_idx, w, k_pool, q, kv_pool, n_pages, page_table, max_pages, ctx_len, page_size,
                                     B, max_ctx, H_I, d_I, H, D_qk, D_v, k, scale, idx, out, lse, stream=None):
    _call("dsa_forward_decode_paged_noalloc", _ptr(q_idx), _ptr(w), _ptr(k_pool), _ptr(q), _ptr(kv_pool), n_pages,
          _ptr(page_table), max_pages, _ptr(ctx_len), page_size, B, max_ctx, H_I, d_I, H, D_qk, D_v, k, scale,
          _ptr(idx), _ptr(out), _ptr(lse), _stream(stream))
