"""Quantized draft-KV rows (test infrastructure).

memra_engine `eagle.rs` (`Eagle3Scratch` doc and `attn`): the draft layer appends
each K/V row in a quantized layout and decode attention reads the quantized
views; K is q8_0 and V is q5_1 by default, blocks of 32 values of 34 and 24
bytes, and head_dim must be a multiple of 32.  The pages name the formats and
block sizes only.  Our reading, block by block along head_dim:
  * q8_0: d = max|x| / 127 in fp32, stored as fp16 D (round to nearest even);
    codes q = clamp(rint(x / D), -127, 127) (ties to even); value D * q;
    (2-byte scale + 32 int8 codes = 34 bytes);
  * q5_1: d = (max x - min x) / 31 in fp32, stored as fp16 D, the minimum stored
    as fp16 M; codes q = clamp(rint((x - M) / D), 0, 31); value D * q + M
    (2 + 2 bytes of scale and minimum, 32 x 5 bits of codes = 24 bytes);
  * a block whose D is 0 has codes 0 (q8_0 value 0, q5_1 value M);
  * every rounding decision is taken in fp32 on fp32 inputs: the differences
    and divisions are IEEE fp32 operations, so a GPU quantizer fed the same
    fp32 row makes the same codes.
Values must stay within fp16 range after the division (|x| < 127 * 65504).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32


def _blocks(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] % BLOCK == 0, "head_dim must be a multiple of 32"
    return x.reshape(*x.shape[:-1], x.shape[-1] // BLOCK, BLOCK)


def q8_0(x: np.ndarray):
    """fp32 rows [..., hd] -> (codes int8 [..., hd], fp16 scales [..., hd / 32])."""
    b = _blocks(x)
    amax = np.abs(b).max(axis=-1)
    D = (amax / np.float32(127)).astype(np.float16)
    Df = D.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(b / Df)
    q = np.where(Df > 0, np.clip(q, -127, 127), 0).astype(np.int8)
    return q.reshape(np.shape(x)), D


def q8_0_values(codes: np.ndarray, D: np.ndarray) -> np.ndarray:
    """D * q in fp64 (exact)."""
    q = _blocks(codes.astype(np.float32)).astype(np.float64)
    return (q * D.astype(np.float64)[..., None]).reshape(codes.shape)


def q5_1(x: np.ndarray):
    """fp32 rows [..., hd] -> (codes uint8 [..., hd] in [0, 31], fp16 D, fp16 M)."""
    b = _blocks(x)
    mn = b.min(axis=-1)
    mx = b.max(axis=-1)
    D = ((mx - mn) / np.float32(31)).astype(np.float16)
    M = mn.astype(np.float16)
    Df = D.astype(np.float32)[..., None]
    Mf = M.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((b - Mf) / Df)
    q = np.where(Df > 0, np.clip(q, 0, 31), 0).astype(np.uint8)
    return q.reshape(np.shape(x)), D, M


def q5_1_values(codes: np.ndarray, D: np.ndarray, M: np.ndarray) -> np.ndarray:
    """D * q + M in fp64 (exact for the fp16 D and M)."""
    q = _blocks(codes.astype(np.float32)).astype(np.float64)
    return (q * D.astype(np.float64)[..., None] + M.astype(np.float64)[..., None]).reshape(codes.shape)


def k_stored(k: np.ndarray) -> np.ndarray:
    """The K row the cache holds for the row k (fp64 values of its q8_0 form)."""
    return q8_0_values(*q8_0(np.asarray(k, dtype=np.float64).astype(np.float32)))


def v_stored(v: np.ndarray) -> np.ndarray:
    """The V row the cache holds for the row v (fp64 values of its q5_1 form)."""
    return q5_1_values(*q5_1(np.asarray(v, dtype=np.float64).astype(np.float32)))


def block_bytes() -> tuple:
    """Bytes per block of 32 values: (q8_0, q5_1)."""
    return (2 + BLOCK, 2 + 2 + BLOCK * 5 // 8)
