"""CPU oracle of the EAGLE-3 drafter round — TEST INFRASTRUCTURE ONLY.

A plain, slow numpy implementation (fp64 unless a caller asks otherwise) of what
the drafter hot path computes.  It exists to prove the GPU library right and is
never part of the product path: only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import it.  It shares no code with the GPU
library (no kernels, headers, helpers or constant tables); the only module both
sides use is `synth`, the seeded input generator, which holds none of the
method's arithmetic.

Sources (page titles as published):
  [memra]  memra_engine 0.121.0, `eagle.rs` source listing on docs.rs
           (module doc "Op-sequence"; `encode`; `draft_token`; `attn`;
           `d2t_map`; `Eagle3Scratch`; `generate_spec_eagle`; `EagleConfig`;
           `draft_rope_width_tests`)
  [pr707]  pegainfer PR #707 "feat(eagle3): Qwen3 EAGLE-3 drafter forward pass
           (single-step + chain rollout)" (PR description; review comments)
  [et153]  ExecuTorch PR #20153 "Add the Eagle3Speculator module for speculative
           decoding" (description)
  [et156]  ExecuTorch PR #20156 "Add the EAGLE-3 speculative-decoding runner
           (CUDA)" (description)

Parity pins: every function is pinned by a `-m "not gpu"` test against closed
forms, library routines, invariants the pages state, or brute force.  The layer's
structure (concat order, which norm sits where, the pre-norm residual, the MLP's
gate/up roles, rotary placement) is pinned by exact consequences of the memra
module doc's op sequence, each shown to fail under a planted mistake
(tests/test_oracle_structure.py).  One reading has no numerical pin ("parity
unpinned"): the token/feature pairing of committed rows (taps of position r with
the token at r + 1), taken from the ExecuTorch PR #20153 description and fixed by
the entry points' semantics rather than by a value any test can derive.
"""
from .numerics import (argmax_first, attention_causal, attention_decode, attention_verify,
                       bf16_bits_to_f64, rms_norm, rope_neox_partial, round_bf16, round_f16,
                       silu)
from .drafter import DrafterOracle, StatelessChain
from .ledger import Ledger, LedgerError
from .rope_width import resolve_rope_dim
from .trunk import TrunkOracle
from . import int4, kvquant
from .loop import greedy_plain, greedy_speculative

__all__ = [
    "argmax_first", "attention_causal", "attention_decode", "attention_verify", "bf16_bits_to_f64",
    "rms_norm", "rope_neox_partial", "round_bf16", "round_f16", "silu", "DrafterOracle", "StatelessChain",
    "Ledger", "LedgerError", "resolve_rope_dim", "TrunkOracle", "greedy_plain",
    "greedy_speculative", "int4", "kvquant",
]
