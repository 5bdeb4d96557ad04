"""A tiny random-init Llama-style target trunk in fp64 (test infrastructure).

It stands in for the target model of the greedy speculative loop.  The loop's
invariant (memra_engine `eagle.rs` module doc: greedy speculative decoding is
token-for-token identical to plain greedy generation; ExecuTorch PR #20153 tests
that the whole shifted speculative loop gives the greedy tokens) is only exact
if a row's result does not depend on whether it was computed alone or inside a
verify batch.  So every token goes through the same one-row code path, in the
same order, whichever way it is fed.

Layer: x -> x + o.attn(RMSNorm(x)) -> h + down.(silu(gate.z) * up.z) with
z = RMSNorm(h); full NeoX rope; GQA; final RMSNorm; untied lm_head; the token
embedding table is the drafter's (shared, as the memra listing does).

Aux taps (memra `generate_spec_eagle` captures three residual hiddens in
ascending layer order; a two-layer trunk has no layers 1/15/28, so our reading
is): the residual stream entering layer 0 (the embedding), entering layer 1,
and leaving layer 1 before the final norm.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Tuple

import numpy as np

from .numerics import (argmax_first, attention_decode, bf16_bits_to_f64, rms_norm,
                       rope_neox_partial, silu)
from .drafter import _bits


class TrunkOracle:
    def __init__(self, geom, weights: Dict[str, object], embed_table, n_layers: int):
        self.n = geom.n_embd
        self.nh = geom.n_head
        self.nkv = geom.n_head_kv
        self.hd = geom.head_dim
        self.theta = float(geom.rope_theta)
        self.eps = float(geom.rms_eps)
        self.L = n_layers
        self.W = {k: bf16_bits_to_f64(_bits(v)) for k, v in weights.items()}
        self.E = bf16_bits_to_f64(_bits(embed_table))
        self.vt = self.E.shape[0]
        self.reset()

    def reset(self) -> None:
        self.K: List[List[np.ndarray]] = [[] for _ in range(self.L)]
        self.V: List[List[np.ndarray]] = [[] for _ in range(self.L)]

    @property
    def length(self) -> int:
        return len(self.K[0])

    def rollback(self, length: int) -> None:
        assert 0 <= length <= self.length
        for l in range(self.L):
            del self.K[l][length:]
            del self.V[l][length:]

    def step(self, tok: int) -> Tuple[np.ndarray, List[np.ndarray]]:
        """Feed one token at position `length`; returns (logits, taps)."""
        pos = self.length
        x = self.E[int(tok)].copy()
        resid = [x.copy()]                  # residual entering layer l, then the output
        for l in range(self.L):
            W = lambda k: self.W[f"layers.{l}.{k}"]
            a = rms_norm(x, W("attn_norm"), self.eps)
            q = (W("wq") @ a).reshape(self.nh, self.hd)
            k = (W("wk") @ a).reshape(self.nkv, self.hd)
            v = (W("wv") @ a).reshape(self.nkv, self.hd)
            q = rope_neox_partial(q, pos, self.hd, self.theta)
            k = rope_neox_partial(k, pos, self.hd, self.theta)
            self.K[l].append(k)
            self.V[l].append(v)
            o = attention_decode(q, np.stack(self.K[l]), np.stack(self.V[l]))
            h = x + W("wo") @ o.reshape(-1)
            z = rms_norm(h, W("mlp_norm"), self.eps)
            x = h + W("w_down") @ (silu(W("w_gate") @ z) * (W("w_up") @ z))
            resid.append(x.copy())
        logits = self.W["lm_head"] @ rms_norm(x, self.W["final_norm"], self.eps)
        taps = [resid[0], resid[self.L // 2], resid[self.L]]
        return logits, taps

    def greedy_token(self, logits: np.ndarray) -> int:
        return argmax_first(logits)
