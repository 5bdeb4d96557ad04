"""Greedy decoding of the trunk, plain and speculative (test infrastructure).

The speculative loop follows the shifted scheme (ExecuTorch PR #20153 and
#20156 descriptions; memra_engine `generate_spec_eagle`):
  * the trunk primes on the prompt x_0..x_{P-1}; taps a_0..a_{P-1}; x_P is its
    greedy token and is emitted first;
  * the drafter is prefilled with rows (a_r, x_{r+1}) for r = 0..P-2 and the
    boundary is (a_{P-1}, x_P);
  * a round drafts d_1..d_g from the boundary, the trunk verifies
    [x_n, d_1..d_g] at positions n..n+g in one pass, the longest prefix with
    d_{i+1} == verify_ids[i] is accepted, verify_ids[a] is the bonus;
  * d_1..d_a and the bonus are emitted (truncated at max_new), the trunk rolls
    back to n + a + 1 entries, the drafter commits the a + 1 rows
    (a_{n-1}, x_n), (a_n, d_1), ..., (a_{n+a-1}, d_a) and the next boundary is
    (a_{n+a}, bonus).
The drafter is any object with `prefill(seq, aux, toks)`,
`draft_chain_ids(seq, boundary_aux, boundary_tok, gamma) -> list[int]` and
`rebuild_after_verify(seq, a, aux, toks)`; both the oracle drafter and the GPU
library's binding fit.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

from .numerics import argmax_first


def greedy_plain(trunk, prompt, max_new: int) -> List[int]:
    trunk.reset()
    logits = None
    for tok in prompt:
        logits, _ = trunk.step(int(tok))
    out = [argmax_first(logits)]
    while len(out) < max_new:
        logits, _ = trunk.step(out[-1])
        out.append(argmax_first(logits))
    return out[:max_new]


class OracleChainAdapter:
    """Exposes DrafterOracle through the loop's drafter interface."""

    def __init__(self, drafter):
        self.d = drafter

    def prefill(self, s, aux, toks):
        self.d.prefill(s, aux, toks)

    def draft_chain_ids(self, s, boundary_aux, boundary_tok, gamma):
        return [r.target_id for r in self.d.draft_chain(s, boundary_aux, boundary_tok, gamma)]

    def rebuild_after_verify(self, s, a, aux, toks):
        self.d.rebuild_after_verify(s, a, aux, toks)


def greedy_speculative(trunk, drafter, prompt, max_new: int, gamma: int,
                       seq: int = 0) -> Tuple[List[int], int, int]:
    """Returns (tokens, total_drafted, total_accepted)."""
    prompt = [int(t) for t in prompt]
    assert prompt, "prompt must be non-empty"
    trunk.reset()
    taps = []
    logits = None
    for tok in prompt:
        logits, tp = trunk.step(tok)
        taps.append(tp)
    P = len(prompt)
    x = argmax_first(logits)
    out = [x]
    if P >= 2:
        aux = [np.stack([taps[r][j] for r in range(P - 1)]) for j in range(3)]
        drafter.prefill(seq, aux, np.asarray(prompt[1:], dtype=np.int32))
    b_aux, b_tok, n = taps[P - 1], x, P
    drafted = accepted = 0
    while len(out) < max_new:
        drafts = [int(t) for t in drafter.draft_chain_ids(seq, b_aux, b_tok, gamma)]
        verify_ids, vtaps = [], []
        for tok in [b_tok] + drafts:
            lg, tp = trunk.step(tok)
            verify_ids.append(argmax_first(lg))
            vtaps.append(tp)
        a = 0
        while a < len(drafts) and drafts[a] == verify_ids[a]:
            a += 1
        bonus = verify_ids[a]
        drafted += len(drafts)
        accepted += a
        for j in range(a):
            if len(out) < max_new:
                out.append(drafts[j])
        if len(out) < max_new:
            out.append(bonus)
        trunk.rollback(n + a + 1)
        rows = [b_aux] + vtaps[:a]
        aux = [np.stack([r[j] for r in rows]) for j in range(3)]
        drafter.rebuild_after_verify(seq, a, aux,
                                     np.asarray([b_tok] + drafts[:a], dtype=np.int32))
        b_aux, b_tok, n = vtaps[a], bonus, n + a + 1
    return out[:max_new], drafted, accepted
