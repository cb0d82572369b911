"""Seeded, counter-based synthetic input generator (host side, numpy).

This module is shared test/bench infrastructure.  It produces the input
tensors of the sparse-attention workloads and holds none of the method's
arithmetic: it only draws numbers and rounds them to the storage formats.
The same definition is implemented for the GPU in ``gen_device.hip``; the two
are required to agree bit for bit (checked by the GPU tests), so large inputs
can be made on the device while the oracle regenerates, on the host, exactly
the rows it checks.

Definition (all arithmetic on unsigned 64-bit integers, wrapping):

* ``mix64`` is the SplitMix64 output function (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014, in the
  form popularised by Vigna): ``z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
  z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31``.
* a stream key is ``mix64((seed << 32) ^ stream)``;
* draw number ``c`` of a stream is ``mix64(key + (c + 1) * 0x9E3779B97F4A7C15)``.

Value recipes, element ``i`` of a tensor stream:

* ``normal``: Irwin-Hall sum of twelve 16-bit uniforms taken from draws
  ``3i, 3i+1, 3i+2`` (four 16-bit fields each).  With ``S`` the integer sum,
  ``x = (S - 393210) / 65536`` exactly in fp32 (mean 0, variance ~1).
* ``uniform01``: ``(draw_i >> 40) * 2^-24`` (exact fp32 in [0, 1)).
* ``int_range(lo, hi)``: ``lo + draw_i mod (hi - lo + 1)``.
* ``pow2_quarter``: ``2^((draw_i & 3) - 2)``, i.e. one of {1/4, 1/2, 1, 2}.

Storage rounding: fp32 -> bfloat16 round-to-nearest-even on the bit pattern;
fp32 -> OCP FP8 E4M3FN round-to-nearest-even with saturation to +-448.
Division by a constant (e.g. ``/24``) is a single correctly rounded fp32
division on both sides.
"""
from __future__ import annotations

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_U64 = np.uint64

# tensor stream ids (shared with gen_device.hip)
STREAM_Q_IDX = 1
STREAM_W = 2
STREAM_K_IDX = 3
STREAM_Q = 4
STREAM_KV = 5
STREAM_CTX = 6
STREAM_PERM = 7
STREAM_ROWS = 8
STREAM_DOUT = 9
STREAM_SEL = 10


def mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> _U64(30))) * _M1
        z = (z ^ (z >> _U64(27))) * _M2
    return z ^ (z >> _U64(31))


def stream_key(seed: int, stream: int) -> np.uint64:
    x = np.array([((int(seed) << 32) ^ int(stream)) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    return mix64(x)[0]


def draws(seed: int, stream: int, counters) -> np.ndarray:
    """Draw numbers ``counters`` (int64/uint64 array) of one stream."""
    c = np.asarray(counters, dtype=np.uint64)
    key = stream_key(seed, stream)
    with np.errstate(over="ignore"):
        z = key + (c + _U64(1)) * _U64(GOLDEN)
    return mix64(z)


# ---------------------------------------------------------------- value recipes
def normal_f32(seed: int, stream: int, idx) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.uint64)
    s = np.zeros(idx.shape, dtype=np.int64)
    for r in range(3):
        h = draws(seed, stream, idx * _U64(3) + _U64(r))
        for f in range(4):
            s += ((h >> _U64(16 * f)) & _U64(0xFFFF)).astype(np.int64)
    return (s - 393210).astype(np.float32) * np.float32(1.0 / 65536.0)


def uniform01_f32(seed: int, stream: int, idx) -> np.ndarray:
    h = draws(seed, stream, idx)
    return (h >> _U64(40)).astype(np.float32) * np.float32(2.0 ** -24)


def int_range(seed: int, stream: int, idx, lo: int, hi: int) -> np.ndarray:
    h = draws(seed, stream, idx)
    return (h % _U64(hi - lo + 1)).astype(np.int64) + lo


def pow2_quarter_f32(seed: int, stream: int, idx) -> np.ndarray:
    h = draws(seed, stream, idx)
    e = (h & _U64(3)).astype(np.int32) - 2
    return np.ldexp(np.float32(1.0), e).astype(np.float32)


# ---------------------------------------------------------------- storage rounding
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (inputs are finite)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + _U64(0x7FFF) + ((u >> _U64(16)) & _U64(1))) >> _U64(16)
    return r.astype(np.uint16)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E4M3FN byte, round to nearest even, saturating to +-448."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.int64)
    sign = ((u >> 31) & 1).astype(np.uint8) << 7
    a = u & 0x7FFFFFFF
    out = np.zeros(x.shape, dtype=np.uint8)
    exp32 = a >> 23
    # subnormal range of e4m3: |x| < 2^-6 -> multiples of 2^-9, RNE via the
    # 2^23 magic-number trick (exact fp32 adds)
    small = exp32 < 121
    if np.any(small):
        q = np.abs(x[small]) * np.float32(512.0)
        magic = np.float32(8388608.0)
        r = (q + magic) - magic
        out[small] = r.astype(np.int64).astype(np.uint8)
    big = ~small
    if np.any(big):
        ab = a[big]
        e = (ab >> 23) - 127
        m23 = ab & 0x7FFFFF
        keep = m23 >> 20
        rem = m23 & 0xFFFFF
        up = (rem > 0x80000) | ((rem == 0x80000) & ((keep & 1) == 1))
        keep = keep + up.astype(np.int64)
        carry = keep == 8
        keep = np.where(carry, 0, keep)
        e = e + carry.astype(np.int64)
        code = ((e + 7) << 3) | keep
        code = np.where((ab >= 0x43E80000) | (code > 0x7E), 0x7E, code)  # |x| >= 464 -> 448
        out[big] = code.astype(np.uint8)
    return out | sign


def int_to_e4m3_bits(v: np.ndarray) -> np.ndarray:
    return f32_to_e4m3_bits(np.asarray(v, dtype=np.float32))
