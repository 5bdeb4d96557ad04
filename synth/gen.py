"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

Every value is a pure function of (cfg_id, tensor_id, element index), computed
with a counter-based integer hash written in plain torch integer ops.  The
same code therefore yields bit-identical tensors on the host and on a GPU, and
any slice (for example a handful of embedding rows) can be generated on its own
without materialising the whole table.

Distributions (the stand-in for the pages' checkpoints, which are not
available):
  * matrices and the embedding table: approximately N(0, 0.02^2);
  * norm weights: 1 + approximately N(0, 0.01^2);
  * aux taps: approximately N(0, 1) in fp32;
  * token ids: uniform on [0, V);
  * d2t: a seeded sorted subset of the target vocabulary stored as offsets.

"Approximately normal" is the Irwin-Hall sum of four 16-bit uniforms, centred
and scaled to the requested mean and standard deviation.  It is produced by one
exact integer sum and one fp32 multiply (plus one fp32 add for the norm
weights), so host and device agree to the bit.  Weights are then rounded to
bfloat16 with round-to-nearest-even; the resulting bit patterns are the weights
both implementations read.

This module holds no arithmetic of the drafter itself.
"""
from __future__ import annotations

import math
from typing import List, Dict, Iterable, Optional, Sequence

import torch

from .configs import DrafterConfig

M32 = 0xFFFFFFFF
_CHUNK = 1 << 24
_IH_MEAN = 2 * 65535                       # mean of the sum of four U{0..65535}
_IH_STD = math.sqrt(4 * (65536.0 ** 2 - 1) / 12.0)

# tensor ids of the drafter weights (fixed forever: they seed the values)
TID = {
    "fc": 1, "input_layernorm": 2, "hidden_norm": 3, "q_proj": 4, "k_proj": 5,
    "v_proj": 6, "o_proj": 7, "post_attention_layernorm": 8, "gate_proj": 9,
    "up_proj": 10, "down_proj": 11, "norm": 12, "lm_head": 13, "embed": 14,
    "d2t": 15,
}
NORM_NAMES = ("input_layernorm", "hidden_norm", "post_attention_layernorm", "norm")


def _mix32_py(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x1B873593) & M32
    x ^= x >> 16
    return x


def _mix32(x: torch.Tensor) -> torch.Tensor:
    """Bijective 32-bit mixer on int64 tensors holding values in [0, 2^32).
    Every product stays below 2^63, so no signed overflow occurs."""
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & M32
    x = x ^ (x >> 15)
    x = (x * 0x1B873593) & M32
    x = x ^ (x >> 16)
    return x


def _seeds(cfg_id: int, tensor_id: int) -> Sequence[int]:
    base = _mix32_py(0x2026_1202 ^ _mix32_py(cfg_id * 0x9E3779B1 + 17))
    base = _mix32_py(base ^ _mix32_py(tensor_id * 0x85EBCA77 + 91))
    return [_mix32_py(base + k * 0x632BE5AB) for k in range(4)]


def _hash_pair(idx: torch.Tensor, s: Sequence[int]):
    h1 = _mix32(_mix32(idx ^ s[0]) ^ s[1])
    h2 = _mix32(_mix32(idx ^ s[2]) ^ s[3])
    return h1, h2


def _normal_from_index(idx: torch.Tensor, s: Sequence[int], std: float,
                       mean: Optional[float]) -> torch.Tensor:
    h1, h2 = _hash_pair(idx, s)
    tot = (h1 & 0xFFFF) + (h1 >> 16) + (h2 & 0xFFFF) + (h2 >> 16) - _IH_MEAN
    z = tot.to(torch.float32) * torch.tensor(std / _IH_STD, dtype=torch.float32,
                                             device=idx.device)
    if mean is not None:
        z = z + torch.tensor(mean, dtype=torch.float32, device=idx.device)
    return z


def normal(cfg_id: int, tensor_id: int, shape: Sequence[int], std: float,
           mean: Optional[float] = None, device="cpu",
           dtype=torch.float32) -> torch.Tensor:
    """Approximately N(mean, std^2) tensor, generated in chunks."""
    numel = 1
    for d in shape:
        numel *= int(d)
    assert numel < (1 << 32), "element index must fit 32 bits"
    s = _seeds(cfg_id, tensor_id)
    out = torch.empty(numel, dtype=dtype, device=device)
    for c0 in range(0, numel, _CHUNK):
        c1 = min(numel, c0 + _CHUNK)
        idx = torch.arange(c0, c1, dtype=torch.int64, device=device)
        out[c0:c1] = _normal_from_index(idx, s, std, mean).to(dtype)
    return out.view(*shape)


def normal_rows(cfg_id: int, tensor_id: int, row_len: int,
                rows: torch.Tensor, std: float, device="cpu",
                dtype=torch.float32) -> torch.Tensor:
    """Rows `rows` of the matrix normal(cfg_id, tensor_id, [*, row_len], std),
    generated without materialising the other rows."""
    rows = rows.to(device=device, dtype=torch.int64).reshape(-1)
    s = _seeds(cfg_id, tensor_id)
    idx = rows[:, None] * row_len + torch.arange(row_len, dtype=torch.int64,
                                                 device=device)[None, :]
    return _normal_from_index(idx, s, std, None).to(dtype)


def uniform_int(cfg_id: int, tensor_id: int, count: int, high: int,
                device="cpu") -> torch.Tensor:
    """count integers uniform on [0, high), int32."""
    assert 0 < high < (1 << 30)
    s = _seeds(cfg_id, tensor_id)
    idx = torch.arange(count, dtype=torch.int64, device=device)
    h1, _ = _hash_pair(idx, s)
    return ((h1 * high) >> 32).to(torch.int32)


def sorted_subset(cfg_id: int, tensor_id: int, universe: int, k: int,
                  device="cpu") -> torch.Tensor:
    """A seeded k-element subset of [0, universe), ascending, int64."""
    s = _seeds(cfg_id, tensor_id)
    idx = torch.arange(universe, dtype=torch.int64, device=device)
    h1, _ = _hash_pair(idx, s)             # a bijection of idx: no ties
    pick = torch.sort(h1, stable=True).indices[:k]
    return torch.sort(pick).values


# ----------------------------------------------------------------------------
# drafter weight set
# ----------------------------------------------------------------------------

def weight_shapes(cfg: DrafterConfig) -> Dict[str, tuple]:
    n, q, kv, ff = cfg.n_embd, cfg.q_dim, cfg.kv_dim, cfg.n_ff
    return {
        "fc": (n, cfg.n_aux * n),
        "input_layernorm": (n,), "hidden_norm": (n,),
        "q_proj": (q, 2 * n), "k_proj": (kv, 2 * n), "v_proj": (kv, 2 * n),
        "o_proj": (n, q), "post_attention_layernorm": (n,),
        "gate_proj": (ff, n), "up_proj": (ff, n), "down_proj": (n, ff),
        "norm": (n,), "lm_head": (cfg.draft_vocab, n),
        "embed": (cfg.target_vocab, n),
    }


def drafter_weights(cfg: DrafterConfig, device="cpu",
                    with_embed: bool = True,
                    names: Optional[Iterable[str]] = None) -> Dict[str, torch.Tensor]:
    """bf16 weights of the drafter (PyTorch [out, in] layout) and int64 d2t."""
    out: Dict[str, torch.Tensor] = {}
    shapes = weight_shapes(cfg)
    for name, shape in shapes.items():
        if names is not None and name not in names:
            continue
        if name == "embed" and not with_embed:
            continue
        if name in NORM_NAMES:
            out[name] = normal(cfg.cfg_id, TID[name], shape, 0.01, mean=1.0,
                               device=device, dtype=torch.bfloat16)
        else:
            out[name] = normal(cfg.cfg_id, TID[name], shape, 0.02,
                               device=device, dtype=torch.bfloat16)
    if names is None or "d2t" in names:
        out["d2t"] = d2t(cfg, device=device)
    return out


def d2t(cfg: DrafterConfig, device="cpu") -> torch.Tensor:
    sub = sorted_subset(cfg.cfg_id, TID["d2t"], cfg.target_vocab,
                        cfg.draft_vocab, device=device)
    return sub - torch.arange(cfg.draft_vocab, dtype=torch.int64, device=device)


def embed_rows(cfg: DrafterConfig, tokens, device="cpu") -> torch.Tensor:
    """bf16 rows of the embedding table for the given target ids."""
    t = torch.as_tensor(tokens, dtype=torch.int64)
    return normal_rows(cfg.cfg_id, TID["embed"], cfg.n_embd, t, 0.02,
                       device=device, dtype=torch.bfloat16)


# ----------------------------------------------------------------------------
# activations: aux taps, tokens
# ----------------------------------------------------------------------------

def aux_taps(cfg: DrafterConfig, stream: int, rows: int, device="cpu"):
    """Three fp32 [rows, n_embd] tap streams, approximately N(0,1)."""
    return [normal(cfg.cfg_id, 10_000 + 8 * stream + j, (rows, cfg.n_embd), 1.0,
                   device=device) for j in range(cfg.n_aux)]


def tokens(cfg: DrafterConfig, stream: int, count: int, device="cpu") -> torch.Tensor:
    """int32 target ids uniform on [0, target_vocab)."""
    return uniform_int(cfg.cfg_id, 20_000 + stream, count, cfg.target_vocab,
                       device=device)


def lengths(cfg: DrafterConfig, stream: int, count: int, lo: int, hi: int) -> torch.Tensor:
    """int32 lengths uniform on [lo, hi] (inclusive)."""
    return uniform_int(cfg.cfg_id, 30_000 + stream, count, hi - lo + 1) + lo


def batch_lengths(cfg: DrafterConfig) -> List[int]:
    """Committed lengths of the batched workload: L_b uniform on [512, context] for
    max_seqs sequences, sequences 0 and 1 at the full context (the capacity edge)."""
    L = [int(x) for x in lengths(cfg, 0, cfg.max_seqs, 512, cfg.context)]
    for b in range(min(2, len(L))):
        L[b] = cfg.context
    return L


# ----------------------------------------------------------------------------
# target trunk (only the tiny workload has one)
# ----------------------------------------------------------------------------

TRUNK_NAMES = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate",
               "w_up", "w_down")


def trunk_weights(cfg: DrafterConfig, device="cpu") -> Dict[str, torch.Tensor]:
    """A random-init Llama-style trunk of the drafter's width (bf16)."""
    n, q, kv, ff = cfg.n_embd, cfg.q_dim, cfg.kv_dim, cfg.n_ff
    shapes = {"attn_norm": (n,), "wq": (q, n), "wk": (kv, n), "wv": (kv, n),
              "wo": (n, q), "mlp_norm": (n,), "w_gate": (ff, n), "w_up": (ff, n),
              "w_down": (n, ff)}
    out = {}
    for layer in range(cfg.trunk_layers):
        for k, name in enumerate(TRUNK_NAMES):
            tid = 100 + 16 * layer + k
            if name.endswith("norm"):
                t = normal(cfg.cfg_id, tid, shapes[name], 0.01, mean=1.0,
                           device=device, dtype=torch.bfloat16)
            else:
                t = normal(cfg.cfg_id, tid, shapes[name], 0.02, device=device,
                           dtype=torch.bfloat16)
            out[f"layers.{layer}.{name}"] = t
    out["final_norm"] = normal(cfg.cfg_id, 98, (n,), 0.01, mean=1.0,
                               device=device, dtype=torch.bfloat16)
    out["lm_head"] = normal(cfg.cfg_id, 99, (cfg.target_vocab, n), 0.02,
                            device=device, dtype=torch.bfloat16)
    return out


def bf16_bits(t: torch.Tensor):
    """The raw uint16 bit patterns of a bf16 tensor as a numpy array."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
