"""Device-side fills of the synthetic workloads (wraps libdsagen.so).

Produces the same values as the host slices in ``configs.py`` (bit for bit),
directly in GPU memory, so the 128K-context inputs (tens of GB) never cross
PCIe.  Test and bench infrastructure.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import gen
from .configs import Workload, ctx_lens, page_layout, pool_rowmap

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdsagen.so")
_lib = None

E4M3_NORMAL, E4M3_INT, F32_UNIFORM, F32_POW2Q, BF16_NORMAL = 0, 1, 2, 3, 4


def build() -> str:
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "gen_device.hip"), "-o", _LIB_PATH + ".tmp"]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.dsagen_fill.restype = ctypes.c_int
        lib.dsagen_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                    ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        _lib = lib
    return _lib


def fill(t, rows: int, dim: int, recipe: int, seed: int, stream: int, div: float = 1.0,
         lo: int = 0, hi: int = 0, rowmap=None) -> None:
    import torch
    lib = _load()
    s = torch.cuda.current_stream().cuda_stream
    rc = lib.dsagen_fill(ctypes.c_void_p(t.data_ptr()), rows, dim,
                         ctypes.c_void_p(rowmap.data_ptr() if rowmap is not None else 0),
                         recipe, seed, stream, float(div), lo, hi, ctypes.c_void_p(s))
    if rc != 0:
        raise RuntimeError(f"dsagen_fill failed with hip error {rc}")


def make_prefill_inputs(wl: Workload, device="cuda"):
    """All inputs of a prefill workload (one sequence), resident on the GPU."""
    import torch
    T, N = wl.T, wl.N
    q_idx = torch.empty((T, wl.H_I, wl.d_I), dtype=torch.uint8, device=device)
    w = torch.empty((T, wl.H_I), dtype=torch.float32, device=device)
    k_idx = torch.empty((N, wl.d_I), dtype=torch.uint8, device=device)
    q = torch.empty((T, wl.H, wl.D_qk), dtype=torch.uint16, device=device)
    kv = torch.empty((N, wl.D_qk), dtype=torch.uint16, device=device)
    _fill_common(wl, q_idx, w, k_idx, q, kv, T, N)
    return dict(q_idx=q_idx, w=w, k_idx=k_idx, q=q, kv=kv)


def _fill_common(wl, q_idx, w, k_idx, q, kv, rows, tokens, rowmap=None):
    if wl.integer_fp8:
        fill(q_idx, rows, wl.H_I * wl.d_I, E4M3_INT, wl.seed, gen.STREAM_Q_IDX, lo=-4, hi=4)
        fill(k_idx, tokens, wl.d_I, E4M3_INT, wl.seed, gen.STREAM_K_IDX, lo=-4, hi=4, rowmap=rowmap)
        fill(w, rows, wl.H_I, F32_POW2Q, wl.seed, gen.STREAM_W)
    else:
        fill(q_idx, rows, wl.H_I * wl.d_I, E4M3_NORMAL, wl.seed, gen.STREAM_Q_IDX)
        fill(k_idx, tokens, wl.d_I, E4M3_NORMAL, wl.seed, gen.STREAM_K_IDX, rowmap=rowmap)
        fill(w, rows, wl.H_I, F32_UNIFORM, wl.seed, gen.STREAM_W)
    fill(q, rows, wl.H * wl.D_qk, BF16_NORMAL, wl.seed, gen.STREAM_Q)
    fill(kv, tokens, wl.D_qk, BF16_NORMAL, wl.seed, gen.STREAM_KV, div=wl.kv_div, rowmap=rowmap)


def make_decode_inputs(wl: Workload, device="cuda"):
    """Contiguous decode: k_idx [B, N, d_I], kv [B, N, D_qk]."""
    import torch
    B, N = wl.B, wl.N
    q_idx = torch.empty((B, wl.H_I, wl.d_I), dtype=torch.uint8, device=device)
    w = torch.empty((B, wl.H_I), dtype=torch.float32, device=device)
    k_idx = torch.empty((B, N, wl.d_I), dtype=torch.uint8, device=device)
    q = torch.empty((B, wl.H, wl.D_qk), dtype=torch.uint16, device=device)
    kv = torch.empty((B, N, wl.D_qk), dtype=torch.uint16, device=device)
    _fill_common(wl, q_idx, w, k_idx, q, kv, B, B * N)
    ctx = torch.from_numpy(ctx_lens(wl)).to(device)
    return dict(q_idx=q_idx, w=w, k_idx=k_idx, q=q, kv=kv, ctx_len=ctx)


def make_paged_inputs(wl: Workload, device="cuda"):
    """Paged decode: pools [P, page, dim] addressed through a shuffled page table."""
    import torch
    B = wl.B
    pt, P = page_layout(wl)
    rowmap = torch.from_numpy(pool_rowmap(wl, pt, P)).to(device)
    q_idx = torch.empty((B, wl.H_I, wl.d_I), dtype=torch.uint8, device=device)
    w = torch.empty((B, wl.H_I), dtype=torch.float32, device=device)
    k_pool = torch.empty((P, wl.page, wl.d_I), dtype=torch.uint8, device=device)
    q = torch.empty((B, wl.H, wl.D_qk), dtype=torch.uint16, device=device)
    kv_pool = torch.empty((P, wl.page, wl.D_qk), dtype=torch.uint16, device=device)
    _fill_common(wl, q_idx, w, k_pool, q, kv_pool, B, P * wl.page, rowmap=rowmap)
    del rowmap
    return dict(q_idx=q_idx, w=w, k_pool=k_pool, q=q, kv_pool=kv_pool,
                page_table=torch.from_numpy(pt).to(device), ctx_len=torch.from_numpy(ctx_lens(wl)).to(device),
                n_pages=P, page_table_host=pt)


def make_paged_prefill_inputs(wl: Workload, device="cuda"):
    """Chunked paged prefill: query rows [T, ...] (row r = token seq*S + pos of
    the chunks), key/latent pools [P, page, dim] through a shuffled page table."""
    import torch
    from .configs import chunk_rows
    pt, P = page_layout(wl)
    q_start, seq, pos = chunk_rows(wl)
    T = int(q_start[-1])
    qmap = torch.from_numpy(seq * wl.S + pos).to(device)
    rowmap = torch.from_numpy(pool_rowmap(wl, pt, P)).to(device)
    q_idx = torch.empty((T, wl.H_I, wl.d_I), dtype=torch.uint8, device=device)
    w = torch.empty((T, wl.H_I), dtype=torch.float32, device=device)
    k_pool = torch.empty((P, wl.page, wl.d_I), dtype=torch.uint8, device=device)
    q = torch.empty((T, wl.H, wl.D_qk), dtype=torch.uint16, device=device)
    kv_pool = torch.empty((P, wl.page, wl.D_qk), dtype=torch.uint16, device=device)
    fill(q_idx, T, wl.H_I * wl.d_I, E4M3_NORMAL, wl.seed, gen.STREAM_Q_IDX, rowmap=qmap)
    fill(w, T, wl.H_I, F32_UNIFORM, wl.seed, gen.STREAM_W, rowmap=qmap)
    fill(q, T, wl.H * wl.D_qk, BF16_NORMAL, wl.seed, gen.STREAM_Q, rowmap=qmap)
    fill(k_pool, P * wl.page, wl.d_I, E4M3_NORMAL, wl.seed, gen.STREAM_K_IDX, rowmap=rowmap)
    fill(kv_pool, P * wl.page, wl.D_qk, BF16_NORMAL, wl.seed, gen.STREAM_KV, div=wl.kv_div, rowmap=rowmap)
    del rowmap, qmap
    return dict(q_idx=q_idx, w=w, k_pool=k_pool, q=q, kv_pool=kv_pool, page_table=torch.from_numpy(pt).to(device),
                n_pages=P, page_table_host=pt, q_start=q_start, ctx_len=ctx_lens(wl).astype(np.int64))
