"""Shared test helpers: build the oracle and inputs for a workload."""
from __future__ import annotations

import numpy as np
import torch

from synth import gen
from synth.configs import DrafterConfig


def make_oracle(cfg: DrafterConfig, weights=None, max_ctx: int = 0, max_seqs: int = 1,
                max_gamma: int = 16, lazy_embed: bool = False, kv_format: str = "exact",
                dtype=np.float64, append_act: str = "exact"):
    from oracle import DrafterOracle
    if weights is None:
        weights = gen.drafter_weights(cfg, with_embed=not lazy_embed)
    if lazy_embed or "embed" not in weights:
        embed = lambda toks: gen.bf16_bits(gen.embed_rows(cfg, torch.as_tensor(toks)))
    else:
        embed = weights["embed"]
    return DrafterOracle(cfg, weights, embed, weights["d2t"],
                         max_ctx=max_ctx or cfg.max_ctx_eff, max_seqs=max_seqs,
                         max_gamma=max_gamma, kv_format=kv_format, dtype=dtype,
                         append_act=append_act)


def aux_np(cfg: DrafterConfig, stream: int, rows: int):
    return [a.numpy().astype(np.float64) for a in gen.aux_taps(cfg, stream, rows)]


def toks_np(cfg: DrafterConfig, stream: int, count: int):
    return gen.tokens(cfg, stream, count).numpy()


def row_slice(aux, i0, i1):
    return [a[i0:i1] for a in aux]
