"""The five synthetic workloads and host-side (numpy) input slices.

Every tensor value is a pure function of (workload seed, tensor stream,
logical element index), so any row can be regenerated on its own.  Logical
element index conventions (``S`` is the per-sequence logical stride):

* ``q_idx``  [rows, H_I, d_I]  e4m3 bytes      index = (row*H_I + j)*d_I + i
* ``w``      [rows, H_I]       fp32            index = row*H_I + j
* ``k_idx``  token (b, s)      e4m3 [d_I]      index = (b*S + s)*d_I + i
* ``q``      [rows, H, D_qk]   bf16 bits       index = (row*H + h)*D_qk + c
* ``kv``     token (b, s)      bf16 [D_qk]     index = (b*S + s)*D_qk + c

A "row" is a query token: its position in the sequence for prefill, the
sequence number for decode.  Paged pools store token (b, s) of logical page
``s // page`` at the physical page the page table assigns to it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import gen


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" | "decode" | "paged_decode"
    cfg_no: int
    B: int                    # sequences
    N: int                    # keys per sequence (max context for paged decode)
    H_I: int
    H: int
    k: int
    integer_fp8: bool = False  # tiny exact recipe: small integers, power-of-two weights
    kv_div: float = 24.0       # kv ~ N(0,1)/kv_div
    d_I: int = 128
    D_qk: int = 576
    D_v: int = 512
    page: int = 64
    ctx_lo: int = 0            # paged decode: context lengths uniform in [ctx_lo, ctx_hi]
    ctx_hi: int = 0
    oracle_rows: int = 0       # seeded random rows checked by the oracle (prefill)
    ctxs: tuple = ()           # paged prefill: tokens of each sequence in the cache, chunk included
    chunks: tuple = ()         # paged prefill: new query tokens of each sequence (its last ones)

    @property
    def seed(self) -> int:
        return 0xD5A0 + self.cfg_no

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(192.0)

    @property
    def S(self) -> int:
        """Per-sequence logical stride of token indices."""
        return self.N

    @property
    def T(self) -> int:
        """Number of query rows."""
        if self.kind == "paged_prefill":
            return int(sum(self.chunks))
        return self.N if self.kind == "prefill" else self.B

    def with_k(self, k: int) -> "Workload":
        d = dict(self.__dict__)
        d["k"] = k
        return Workload(**d)


WORKLOADS = {
    "tiny_prefill_L256": Workload("tiny_prefill_L256", "prefill", 1, B=1, N=256, H_I=4, H=8, k=32,
                                  integer_fp8=True, kv_div=1.0, oracle_rows=256),
    "decode_b64_ctx32k": Workload("decode_b64_ctx32k", "decode", 2, B=64, N=32768, H_I=64, H=128, k=2048),
    "prefill_L32k": Workload("prefill_L32k", "prefill", 3, B=1, N=32768, H_I=64, H=128, k=2048,
                             oracle_rows=512),
    "prefill_L128k": Workload("prefill_L128k", "prefill", 4, B=1, N=131072, H_I=64, H=128, k=2048,
                              oracle_rows=256),
    "paged_decode_b32_ctx4k_128k": Workload("paged_decode_b32_ctx4k_128k", "paged_decode", 5, B=32,
                                            N=131072, H_I=64, H=128, k=2048, ctx_lo=4096, ctx_hi=131072),
    # chunked prefill into a paged cache, several sequences per call: a chunk
    # after earlier context, a whole prompt, a short chunk after a long
    # context and a one-token chunk
    "paged_prefill_mixed": Workload("paged_prefill_mixed", "paged_prefill", 6, B=4, N=16384, H_I=64, H=128,
                                    k=2048, ctxs=(9000, 2100, 16384, 700), chunks=(1500, 2100, 256, 1),
                                    oracle_rows=40),
    # the same call at serving size: 4 sequences of 32K tokens, the last 8K new
    "paged_prefill_b4_ctx32k_q8k": Workload("paged_prefill_b4_ctx32k_q8k", "paged_prefill", 7, B=4, N=32768,
                                            H_I=64, H=128, k=2048, ctxs=(32768,) * 4, chunks=(8192,) * 4),
}


# ------------------------------------------------------------------ host slices
def _rows(rows) -> np.ndarray:
    return np.asarray(rows, dtype=np.int64).reshape(-1)


def q_idx_bytes(wl: Workload, rows) -> np.ndarray:
    rows = _rows(rows)
    idx = (rows[:, None] * (wl.H_I * wl.d_I) + np.arange(wl.H_I * wl.d_I)[None, :]).reshape(-1)
    if wl.integer_fp8:
        v = gen.int_range(wl.seed, gen.STREAM_Q_IDX, idx, -4, 4).astype(np.float32)
    else:
        v = gen.normal_f32(wl.seed, gen.STREAM_Q_IDX, idx)
    return gen.f32_to_e4m3_bits(v).reshape(len(rows), wl.H_I, wl.d_I)


def w_f32(wl: Workload, rows) -> np.ndarray:
    rows = _rows(rows)
    idx = (rows[:, None] * wl.H_I + np.arange(wl.H_I)[None, :]).reshape(-1)
    if wl.integer_fp8:
        v = gen.pow2_quarter_f32(wl.seed, gen.STREAM_W, idx)
    else:
        v = gen.uniform01_f32(wl.seed, gen.STREAM_W, idx)
    return v.reshape(len(rows), wl.H_I)


def k_idx_bytes(wl: Workload, seq: int, positions) -> np.ndarray:
    pos = _rows(positions)
    tok = seq * wl.S + pos
    idx = (tok[:, None] * wl.d_I + np.arange(wl.d_I)[None, :]).reshape(-1)
    if wl.integer_fp8:
        v = gen.int_range(wl.seed, gen.STREAM_K_IDX, idx, -4, 4).astype(np.float32)
    else:
        v = gen.normal_f32(wl.seed, gen.STREAM_K_IDX, idx)
    return gen.f32_to_e4m3_bits(v).reshape(len(pos), wl.d_I)


def q_bf16(wl: Workload, rows) -> np.ndarray:
    rows = _rows(rows)
    idx = (rows[:, None] * (wl.H * wl.D_qk) + np.arange(wl.H * wl.D_qk)[None, :]).reshape(-1)
    v = gen.normal_f32(wl.seed, gen.STREAM_Q, idx)
    return gen.f32_to_bf16_bits(v).reshape(len(rows), wl.H, wl.D_qk)


def kv_bf16(wl: Workload, seq: int, positions) -> np.ndarray:
    pos = _rows(positions)
    tok = seq * wl.S + pos
    idx = (tok[:, None] * wl.D_qk + np.arange(wl.D_qk)[None, :]).reshape(-1)
    v = gen.normal_f32(wl.seed, gen.STREAM_KV, idx)
    if wl.kv_div != 1.0:
        v = (v / np.float32(wl.kv_div)).astype(np.float32)
    return gen.f32_to_bf16_bits(v).reshape(len(pos), wl.D_qk)


def ctx_lens(wl: Workload) -> np.ndarray:
    """Context length of each sequence; the (last) query sits at position ctx-1."""
    if wl.kind == "paged_prefill":
        return np.array(wl.ctxs, dtype=np.int32)
    if wl.kind == "paged_decode":
        return gen.int_range(wl.seed, gen.STREAM_CTX, np.arange(wl.B), wl.ctx_lo, wl.ctx_hi).astype(np.int32)
    if wl.kind == "decode":
        return np.full(wl.B, wl.N, dtype=np.int32)
    return np.array([wl.N], dtype=np.int32)


def chunk_rows(wl: Workload):
    """Paged prefill query rows: ``(q_start [B+1], seq [T], pos [T])``.  Row r is
    the query of sequence seq[r] at position pos[r]; its generated values use the
    logical token index ``seq*S + pos`` as the row index."""
    ctx = np.array(wl.ctxs, dtype=np.int64)
    nq = np.array(wl.chunks, dtype=np.int64)
    q_start = np.concatenate([[0], np.cumsum(nq)]).astype(np.int64)
    seq = np.repeat(np.arange(wl.B, dtype=np.int64), nq)
    pos = np.concatenate([np.arange(c - n, c, dtype=np.int64) for c, n in zip(ctx, nq)])
    return q_start, seq, pos


def page_layout(wl: Workload):
    """Seeded paged layout.

    Returns ``(page_table [B, max_pages] int32, n_pages)``.  Logical pages
    are numbered in (sequence, page) order; their physical ids are a
    Fisher-Yates shuffle of 0..P-1 driven by the permutation stream.
    Entries past a sequence's last page are -1.
    """
    ctx = ctx_lens(wl).astype(np.int64)
    npg = (ctx + wl.page - 1) // wl.page
    P = int(npg.sum())
    max_pages = wl.N // wl.page
    perm = np.arange(P, dtype=np.int64)
    if P > 1:
        h = gen.draws(wl.seed, gen.STREAM_PERM, np.arange(P, dtype=np.int64))
        for i in range(P - 1, 0, -1):
            j = int(h[i] % np.uint64(i + 1))
            perm[i], perm[j] = perm[j], perm[i]
    pt = np.full((wl.B, max_pages), -1, dtype=np.int32)
    flat = 0
    for b in range(wl.B):
        pt[b, : npg[b]] = perm[flat: flat + npg[b]]
        flat += int(npg[b])
    return pt, P


def pool_rowmap(wl: Workload, page_table: np.ndarray, n_pages: int) -> np.ndarray:
    """For each physical pool row, the logical token index ``b*S + s``."""
    rowmap = np.zeros(n_pages * wl.page, dtype=np.int64)
    B, mp = page_table.shape
    for b in range(B):
        for lp in range(mp):
            p = int(page_table[b, lp])
            if p < 0:
                break
            rowmap[p * wl.page: (p + 1) * wl.page] = b * wl.S + lp * wl.page + np.arange(wl.page)
    return rowmap


def sample_rows(wl: Workload, count: int) -> np.ndarray:
    """``count`` distinct seeded-random query rows (prefill workloads)."""
    if count >= wl.T:
        return np.arange(wl.T, dtype=np.int64)
    h = gen.draws(wl.seed, gen.STREAM_ROWS, np.arange(4 * count + 64, dtype=np.int64))
    cand = (h % np.uint64(wl.T)).astype(np.int64)
    _, first = np.unique(cand, return_index=True)
    rows = cand[np.sort(first)][:count]
    return np.sort(rows)


def dout_bf16(wl: Workload, rows) -> np.ndarray:
    """Upstream gradient of the attention output for query rows: bf16 bits,
    standard normal values, [len(rows), H, D_v]."""
    rows = _rows(rows)
    idx = (rows[:, None] * (wl.H * wl.D_v) + np.arange(wl.H * wl.D_v)[None, :]).reshape(-1)
    v = gen.normal_f32(wl.seed, gen.STREAM_DOUT, idx)
    return gen.f32_to_bf16_bits(v).reshape(len(rows), wl.H, wl.D_v)


def random_selection(wl: Workload, positions, k: int | None = None) -> np.ndarray:
    """A seeded stand-in for a top-k result, for tests that take the selected
    set as an input: for a query at position p with n = min(p + 1, N)
    candidates, all of 0..n-1 when n <= k, else k distinct candidates drawn
    uniformly; ascending, padded with -1.  int32 [len(positions), k]."""
    k = wl.k if k is None else k
    pos = _rows(positions)
    out = np.full((len(pos), k), -1, dtype=np.int32)
    for i, p_ in enumerate(pos):
        n = int(min(p_ + 1, wl.N))
        if n <= k:
            out[i, :n] = np.arange(n, dtype=np.int32)
            continue
        h = gen.draws(wl.seed, gen.STREAM_SEL, int(p_) * wl.N + np.arange(n, dtype=np.int64))
        out[i] = np.sort(np.argsort(h, kind="stable")[:k]).astype(np.int32)
    return out
