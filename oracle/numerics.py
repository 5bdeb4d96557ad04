"""Elementary operations of the drafter layer, written out from their plain
definitions (test infrastructure; see the package docstring).

Readings of the pages used here (the pages name these ops but do not define
them):
  * RMSNorm: y = w * x / sqrt(mean(x^2) + eps); the weight multiplies x/rms.
  * NeoX partial rotary embedding: the first `rot` dims of a head are rotated
    in halves (i, i + rot/2) with angle pos * theta^(-2i/rot); dims >= rot pass
    through unchanged.  The memra listing (`attn`, the `rope_neox` call with a
    rotated-dims count of 64 of 256 and theta 1e7; the rope-width tests'
    "pass-through band 64..256") fixes the NeoX style and the band; the
    frequency denominator `rot` is our reading.
  * Attention: softmax(q . k / sqrt(head_dim)) over the rows of the draft KV
    up to and including the current row; query head h reads KV head
    floor(h * n_kv / n_head) (contiguous GQA groups; memra `attn`: "GQA
    broadcast in fa_decode", scale 1/sqrt(head_dim)).
  * argmax: the lowest index among equal maxima.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _float(x) -> np.ndarray:
    """x as a float array: float32 stays float32 (the oracle's timing mode),
    everything else becomes float64."""
    x = np.asarray(x)
    return x if x.dtype == np.float32 else x.astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (8 significant bits), ties to
    even, returned as fp64.  Exact for the normal bf16 range: with x = m * 2^e and
    0.5 <= |m| < 1, the kept significand is rint(m * 2^8) (rint rounds half to
    even) and the value is that times 2^(e - 8)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def round_f16(x) -> np.ndarray:
    """Round to the nearest IEEE half-precision value (11 significant bits, ties
    to even; numpy's float16 conversion), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (memra module doc: the four RMSNorms of the
    op-sequence; formula per the reading in the module docstring)."""
    x = _float(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return w * (x / np.sqrt(ms + eps))


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) (memra `draft_token`: the `silu_mul` of the MLP)."""
    return x / (1.0 + np.exp(-x))


def rope_neox_partial(x: np.ndarray, pos, rot: int, theta: float) -> np.ndarray:
    """Rotate the first `rot` dims of every head of x [..., heads, head_dim] at
    position(s) `pos` (scalar, or an array broadcastable to x[..., 0, 0])."""
    x = _float(x)
    assert rot % 2 == 0 and 0 < rot <= x.shape[-1]
    half = rot // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / rot)
    p = np.asarray(pos, dtype=np.float64)
    ang = p[..., None, None] * inv_freq          # [..., 1, half]
    c, s = np.cos(ang).astype(x.dtype), np.sin(ang).astype(x.dtype)
    out = x.copy()
    a, b = x[..., :half], x[..., half:rot]
    out[..., :half] = a * c - b * s
    out[..., half:rot] = b * c + a * s
    return out


def argmax_first(v: np.ndarray) -> int:
    """Index of the maximum; the lowest index wins a tie."""
    return int(np.argmax(v))


def _kv_head(h: int, n_head: int, n_head_kv: int) -> int:
    return (h * n_head_kv) // n_head


def attention_decode(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """One query row per head against every KV row.

    q [n_head, hd]; K, V [T, n_head_kv, hd]  ->  o [n_head, hd]
    """
    n_head, hd = q.shape
    n_kv = K.shape[1]
    out = np.empty_like(q, dtype=np.result_type(q, K, V))
    for h in range(n_head):
        g = _kv_head(h, n_head, n_kv)
        s = (K[:, g, :] @ q[h]) / float(np.sqrt(hd))
        p = np.exp(s - s.max())
        out[h] = (p / p.sum()) @ V[:, g, :]
    return out


def attention_causal(Q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Causal self-attention over T rows: row t sees rows 0..t inclusive.

    Q [T, n_head, hd]; K, V [T, n_head_kv, hd]  ->  O [T, n_head, hd]
    """
    T = Q.shape[0]
    out = np.empty_like(Q, dtype=np.result_type(Q, K, V))
    for t in range(T):
        out[t] = attention_decode(Q[t], K[: t + 1], V[: t + 1])
    return out


def attention_verify(Q: np.ndarray, K: np.ndarray, V: np.ndarray, ctx: int) -> np.ndarray:
    """Verify-window attention (ExecuTorch PR #20344 "split-K mid-M SDPA ... for
    EAGLE-3 target_verify at long context"; PR #20156 description: one target
    forward per round over the K-token verify window): M query rows whose K/V are
    rows ctx..ctx+M-1 of the cache; query row m sees rows 0..ctx+m inclusive.

    Q [M, n_head, hd]; K, V [>= ctx + M, n_head_kv, hd]  ->  O [M, n_head, hd]
    """
    M = Q.shape[0]
    out = np.empty_like(Q, dtype=np.result_type(Q, K, V))
    for m in range(M):
        out[m] = attention_decode(Q[m], K[: ctx + m + 1], V[: ctx + m + 1])
    return out
