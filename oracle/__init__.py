"""CPU oracle for the DSA forward path (test infrastructure only).

Thin ctypes wrapper over ``dsa_oracle.c`` (plain single-threaded C, double
precision) plus row-level drivers that regenerate a workload's inputs on the
host with ``dsa_inputs`` and run indexer -> top-k -> sparse attention for the
requested query rows.  Only the tests, the smoke check and the bench's
CPU-baseline leg use this package; the GPU library never does.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
# DSA_ORACLE_LIB selects another build of the oracle (e.g. a sanitizer build), used as it is
_LIB_OVERRIDE = os.environ.get("DSA_ORACLE_LIB")
_LIB = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


def build(out: str | None = None, extra=()) -> str:
    """Compile the oracle with gcc (no fast-math, so double arithmetic is IEEE)
    into `out` (default: the in-tree library)."""
    out = out or os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-fno-fast-math", *extra, _SRC, "-o", tmp, "-lm"],
                   check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is None:
        if not _LIB_OVERRIDE and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_e4m3_to_double.restype = ctypes.c_double
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_indexer_row.restype = None
        lib.oracle_indexer_row.argtypes = [_u8p, _f32p, _u8p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           _f64p]
        lib.oracle_topk_row.restype = ctypes.c_int32
        lib.oracle_topk_row.argtypes = [_f64p, ctypes.c_int64, ctypes.c_int32, _i32p]
        lib.oracle_sparse_mla_row.restype = None
        lib.oracle_sparse_mla_row.argtypes = [_u16p, _u16p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_double, _f64p, _f64p]
        lib.oracle_dense_mla_row.restype = None
        lib.oracle_dense_mla_row.argtypes = [_u16p, _u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_double, _f64p, _f64p]
        lib.oracle_indexer_kl_row.restype = ctypes.c_double
        lib.oracle_indexer_kl_row.argtypes = [_u16p, _u16p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_double, _f64p]
        _f64p_opt = ctypes.c_void_p
        lib.oracle_sparse_mla_bwd_row.restype = None
        lib.oracle_sparse_mla_bwd_row.argtypes = [_u16p, _u16p, _u16p, ctypes.c_int64, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_double, _f64p, _f64p,
                                                  _f64p_opt, _f64p_opt]
        _lib = lib
    return _lib


# ------------------------------------------------------------------ primitives
def e4m3_to_f64(b: int) -> float:
    return _load().oracle_e4m3_to_double(int(b))


def bf16_to_f64(u: int) -> float:
    return _load().oracle_bf16_to_double(int(u))


def indexer_row(q_row: np.ndarray, w_row: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Index scores of one query over key rows ``k`` [n, d] (token s = row s)."""
    q_row = np.ascontiguousarray(q_row, dtype=np.uint8)
    w_row = np.ascontiguousarray(w_row, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.uint8)
    H_I, d = q_row.shape
    n = k.shape[0]
    assert k.shape[1] == d and w_row.shape == (H_I,)
    out = np.empty(n, dtype=np.float64)
    _load().oracle_indexer_row(q_row, w_row, k, n, H_I, d, out)
    return out


def topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """Top-k of one score row: ascending token indices, -1 padded to k."""
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    out = np.empty(k, dtype=np.int32)
    _load().oracle_topk_row(scores, scores.shape[0], k, out)
    return out


def sparse_mla_row(q: np.ndarray, kv_rows: np.ndarray, scale: float, D_v: int):
    """MQA attention of q [H, D_qk] over gathered latent rows [m, D_qk]."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kv_rows = np.ascontiguousarray(kv_rows, dtype=np.uint16).reshape(-1, q.shape[1])
    H, D_qk = q.shape
    out = np.empty((H, D_v), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    _load().oracle_sparse_mla_row(q, kv_rows, kv_rows.shape[0], H, D_qk, D_v, float(scale), out, lse)
    return out, lse


def dense_mla_row(q: np.ndarray, kv: np.ndarray, n: int, scale: float, D_v: int):
    """Dense causal attention of q [H, D_qk] over kv [N, D_qk], first n rows visible."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    H, D_qk = q.shape
    out = np.empty((H, D_v), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    _load().oracle_dense_mla_row(q, kv, kv.shape[0], n, H, D_qk, D_v, float(scale), out, lse)
    return out, lse


def indexer_kl_row(q: np.ndarray, kv_rows: np.ndarray, scale: float, iscore: np.ndarray) -> float:
    """Indexer KL loss of one query over its selected rows [m, D_qk] with indexer
    scores iscore [m] ("DeepSeek-V3.2" walk-through §2.3.2)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kv_rows = np.ascontiguousarray(kv_rows, dtype=np.uint16).reshape(-1, q.shape[1])
    iscore = np.ascontiguousarray(iscore, dtype=np.float64)
    assert iscore.shape[0] == kv_rows.shape[0]
    H, D_qk = q.shape
    return float(_load().oracle_indexer_kl_row(q, kv_rows, kv_rows.shape[0], H, D_qk, float(scale), iscore))


def sparse_mla_bwd_row(q: np.ndarray, kv_rows: np.ndarray, dO: np.ndarray, scale: float, magnitudes: bool = False):
    """Gradient of the MQA attention of q [H, D_qk] over gathered latent rows
    [m, D_qk] for the upstream gradient dO [H, D_v] (bf16 bits): returns
    (dq [H, D_qk], dkv_rows [m, D_qk]) and, with magnitudes=True, the two
    absolute-value sums that bound their rounding ("DeepSeek-V3.2" walk-through
    §2.1.2 attention equation, §2.3.2 sparse training stage)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kv_rows = np.ascontiguousarray(kv_rows, dtype=np.uint16).reshape(-1, q.shape[1])
    dO = np.ascontiguousarray(dO, dtype=np.uint16)
    H, D_qk = q.shape
    D_v = dO.shape[1]
    assert dO.shape[0] == H and D_v <= D_qk
    m = kv_rows.shape[0]
    dq = np.empty((H, D_qk), dtype=np.float64)
    dkv = np.empty((m, D_qk), dtype=np.float64)
    mq = np.empty_like(dq) if magnitudes else None
    mk = np.empty_like(dkv) if magnitudes else None
    _load().oracle_sparse_mla_bwd_row(q, kv_rows, dO, m, H, D_qk, D_v, float(scale), dq, dkv,
                                      None if mq is None else mq.ctypes.data,
                                      None if mk is None else mk.ctypes.data)
    return (dq, dkv, mq, mk) if magnitudes else (dq, dkv)


# ------------------------------------------------------------------ row drivers
def gather_kv(wl, seq: int, idx: np.ndarray) -> np.ndarray:
    """Latent rows of the selected tokens (entries < 0 are padding, dropped)."""
    from dsa_inputs import configs
    sel = idx[idx >= 0]
    return configs.kv_bf16(wl, seq, sel)


def prefill_row(wl, t: int, k_all: np.ndarray, k: int | None = None):
    """Oracle chain for prefill query row t (position t, candidates 0..t).

    ``k_all`` holds the key rows of the sequence (at least t+1 of them).
    Returns dict(scores, idx, out, lse).
    """
    from dsa_inputs import configs
    k = wl.k if k is None else k
    q_i = configs.q_idx_bytes(wl, [t])[0]
    w = configs.w_f32(wl, [t])[0]
    scores = indexer_row(q_i, w, k_all[: t + 1])
    idx = topk_row(scores, k)
    q = configs.q_bf16(wl, [t])[0]
    out, lse = sparse_mla_row(q, gather_kv(wl, 0, idx), wl.scale, wl.D_v)
    return dict(scores=scores, idx=idx, out=out, lse=lse)


def decode_row(wl, b: int, k: int | None = None):
    """Oracle chain for the decode query of sequence b (position ctx_b - 1).

    Keys and latent rows are regenerated by logical token position; paged
    layouts therefore do not enter the oracle at all.
    """
    from dsa_inputs import configs
    k = wl.k if k is None else k
    n = int(configs.ctx_lens(wl)[b])
    q_i = configs.q_idx_bytes(wl, [b])[0]
    w = configs.w_f32(wl, [b])[0]
    keys = configs.k_idx_bytes(wl, b, np.arange(n))
    scores = indexer_row(q_i, w, keys)
    idx = topk_row(scores, k)
    q = configs.q_bf16(wl, [b])[0]
    out, lse = sparse_mla_row(q, gather_kv(wl, b, idx), wl.scale, wl.D_v)
    return dict(scores=scores, idx=idx, out=out, lse=lse)


def paged_prefill_row(wl, b: int, pos: int, keys: np.ndarray | None = None, k: int | None = None):
    """Oracle chain for the chunked-prefill query of sequence b at position pos:
    the prefill chain over keys 0..pos of sequence b (row index b*S + pos for
    the generated query values).  ``keys`` may hold the sequence's key rows
    (at least pos+1 of them).  The paged layout does not enter the oracle."""
    from dsa_inputs import configs
    k = wl.k if k is None else k
    row = b * wl.S + pos
    if keys is None:
        keys = configs.k_idx_bytes(wl, b, np.arange(pos + 1))
    q_i = configs.q_idx_bytes(wl, [row])[0]
    w = configs.w_f32(wl, [row])[0]
    scores = indexer_row(q_i, w, keys[: pos + 1])
    idx = topk_row(scores, k)
    q = configs.q_bf16(wl, [row])[0]
    out, lse = sparse_mla_row(q, gather_kv(wl, b, idx), wl.scale, wl.D_v)
    return dict(scores=scores, idx=idx, out=out, lse=lse)


def dense_kl_row(wl, t: int, k_all: np.ndarray):
    """Oracle of the dense warm-up loss for prefill query row t ("DeepSeek-V3.2"
    walk-through §2.3.1): the indexer scores over every causal key 0..t, the
    dense attention's per-head log-sum-exp over the same keys, and the KL of the
    head-averaged dense attention against the indexer softmax (indexer_kl_row
    over all causal rows).  Returns dict(kl, lse, scores)."""
    from dsa_inputs import configs
    n = t + 1
    q_i = configs.q_idx_bytes(wl, [t])[0]
    w = configs.w_f32(wl, [t])[0]
    scores = indexer_row(q_i, w, k_all[:n])
    q = configs.q_bf16(wl, [t])[0]
    kv = configs.kv_bf16(wl, 0, np.arange(n))
    _, lse = dense_mla_row(q, kv, n, wl.scale, wl.D_v)
    return dict(kl=indexer_kl_row(q, kv, wl.scale, scores), lse=lse, scores=scores)
