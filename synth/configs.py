"""Drafter geometries and workload shapes used by tests and the benchmark.

Pure data: no arithmetic of the method lives here.  The five workloads are the
EAGLE-3 drafter shapes the speculative-decoding pages discuss (the memra_engine
`eagle.rs` listing prints the tensor shapes of one real drafter in its module
doc) plus smaller and larger members of the same family.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class DrafterConfig:
    name: str
    cfg_id: int              # seeds the synthetic tensors of this workload
    n_embd: int
    n_head: int
    n_head_kv: int
    head_dim: int
    n_ff: int
    draft_vocab: int
    target_vocab: int
    rope_dim: int            # rotated dims per head (NeoX halves), rest pass through
    rope_theta: float
    rms_eps: float = 1e-6
    n_aux: int = 3
    # workload
    context: int = 64        # committed draft-KV rows before the timed rounds
    gamma: int = 3
    max_ctx: int = 0         # admission bound; 0 -> context + 64
    max_seqs: int = 1
    prefill_chunk: int = 0   # 0 -> one shot
    trunk_layers: int = 0    # >0: a random-init target trunk of the same width exists

    @property
    def q_dim(self) -> int:
        return self.n_head * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_head_kv * self.head_dim

    @property
    def max_ctx_eff(self) -> int:
        return self.max_ctx if self.max_ctx > 0 else self.context + 64

    def step_weight_params(self) -> int:
        """Weight elements streamed by one draft step (fc excluded)."""
        n = self.n_embd
        return ((self.q_dim + 2 * self.kv_dim) * 2 * n + n * self.q_dim
                + 3 * self.n_ff * n + self.draft_vocab * n)

    def total_params(self) -> int:
        n = self.n_embd
        return self.step_weight_params() + 3 * n * n + 4 * n

    def with_(self, **kw) -> "DrafterConfig":
        return replace(self, **kw)


# Tiny drafter with a 2-layer trunk of the same width (greedy-equivalence loop).
TINY = DrafterConfig(
    name="tiny", cfg_id=1, n_embd=256, n_head=4, n_head_kv=2, head_dim=64,
    n_ff=768, draft_vocab=1024, target_vocab=4096, rope_dim=64, rope_theta=1e4,
    context=63, gamma=3, max_ctx=400, trunk_layers=2)

# Qwen3-8B-shaped drafter, batch 1, 1024 committed rows, gamma 3.
QWEN3_8B = DrafterConfig(
    name="qwen3-8b", cfg_id=2, n_embd=4096, n_head=32, n_head_kv=8, head_dim=128,
    n_ff=12288, draft_vocab=32000, target_vocab=151936, rope_dim=128,
    rope_theta=1e6, context=1024, gamma=3, max_ctx=1024 + 64)

# The geometry printed in the memra_engine eagle.rs module doc: 16/4 heads x 256,
# partial rope 64 of 256 at theta 1e7, 4096 committed rows.
PAGE4 = DrafterConfig(
    name="page4", cfg_id=3, n_embd=4096, n_head=16, n_head_kv=4, head_dim=256,
    n_ff=12288, draft_vocab=32000, target_vocab=248320, rope_dim=64,
    rope_theta=1e7, context=4096, gamma=3, max_ctx=4096 + 64)

# Batched drafting at the Qwen3-8B shape: 32 ragged sequences, gamma 4.
BATCHED = QWEN3_8B.with_(name="batched32", cfg_id=4, gamma=4, max_seqs=32,
                         context=8192, max_ctx=8192 + 4)

# Long context: a 32767-row prefill in one call (the engine appends it in passes of
# up to 4096 rows), gamma 3.
LONG = DrafterConfig(
    name="long32k", cfg_id=5, n_embd=5120, n_head=40, n_head_kv=8, head_dim=128,
    n_ff=17408, draft_vocab=32000, target_vocab=262144, rope_dim=128,
    rope_theta=1e6, context=32767, gamma=3, max_ctx=32768 + 64)

ALL = {c.name: c for c in (TINY, QWEN3_8B, PAGE4, BATCHED, LONG)}


def small_variant(name: str = "small-ragged", **kw) -> DrafterConfig:
    """A shape that spans several GEMV tiles and attention splits with ragged
    tails everywhere (odd vocab, rows not multiple of any tile, partial rope)."""
    base = DrafterConfig(
        name=name, cfg_id=11, n_embd=384, n_head=6, n_head_kv=2, head_dim=64,
        n_ff=1000, draft_vocab=1000, target_vocab=3001, rope_dim=32,
        rope_theta=1e4, context=300, gamma=4, max_ctx=700)
    return base.with_(**kw) if kw else base
