"""Group-wise int4 drafter weights (test infrastructure).

ExecuTorch's EAGLE-3 stack adds a weight-stationary INT4 GEMM for small M (PR
#20154, named in the stack lists of ExecuTorch PRs #20153 and #20156); the pages
give its title only, not the format.  Our reading, chosen for the drafter's
projection weights:
  * symmetric signed int4 along the input dimension, one scale per group of 32
    consecutive weights of a row (input widths must be multiples of 32);
  * scale = bf16(max|w| / 7) (round to nearest even), codes
    q = clamp(rint(w / scale), -7, 7) (ties to even); a group of zeros has
    scale 0 and codes 0;
  * the weight used is scale * q, exact in fp32;
  * both divisions are IEEE fp32 divisions (correctly rounded), so the codes are
    decided in fp32 on both sides;
  * storage: two codes a byte, element 2i in the low nibble, each stored as
    q + 8; scales as bf16 bit patterns, [rows][width / 32].
Norm weights and the token embedding are not quantized.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_bits_to_f64

GROUP = 32
QMAX = 7

# the projection weights the int4 mode quantizes
I4_WEIGHTS = ("fc", "q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj",
              "down_proj", "lm_head")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); finite inputs."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def quantize(w_bits: np.ndarray):
    """bf16 weight bit patterns [rows, width] -> (codes int8 [rows, width] in
    [-7, 7], scale bits uint16 [rows, width / 32])."""
    w = bf16_bits_to_f64(w_bits).astype(np.float32)
    rows, width = w.shape
    assert width % GROUP == 0, "int4 weights need input widths divisible by 32"
    g = w.reshape(rows, width // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    s_bits = f32_to_bf16_bits(amax / np.float32(QMAX))
    s = bf16_bits_to_f64(s_bits).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(g / s[..., None])
    q = np.where(s[..., None] > 0, np.clip(q, -QMAX, QMAX), 0).astype(np.int8)
    return q.reshape(rows, width), s_bits


def dequantize(codes: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """scale * q in fp64 (exact)."""
    rows, width = codes.shape
    s = bf16_bits_to_f64(s_bits)
    return (codes.reshape(rows, width // GROUP, GROUP).astype(np.float64) * s[..., None]).reshape(rows, width)


def pack(codes: np.ndarray) -> np.ndarray:
    """codes [rows, width] -> bytes [rows, width / 2]: (q[2i] + 8) | (q[2i+1] + 8) << 4."""
    u = (codes.astype(np.int16) + 8).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack(packed: np.ndarray) -> np.ndarray:
    lo = (packed & 0x0F).astype(np.int8) - 8
    hi = (packed >> 4).astype(np.int8) - 8
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def int4_weights(weights: dict) -> dict:
    """A copy of a drafter weight dict whose projection weights are replaced by
    their int4 values (fp64 arrays, scale * q); other entries are kept."""
    out = dict(weights)
    for k in I4_WEIGHTS:
        w = weights[k]
        bits = w if isinstance(w, np.ndarray) else \
            w.detach().cpu().contiguous().view(__import__("torch").int16).numpy().view(np.uint16)
        q, s = quantize(bits)
        out[k] = dequantize(q, s)
    return out
