"""Parity at full drafter sizes: the Qwen3-8B-shaped drafter with 1024 committed
rows, the 16/4 x 256 partial-rope geometry with 4096 committed rows (gamma 3, 5
and 8) and the 5120-wide long-context drafter with a 32767-row prefill, in the
launch configuration the benchmark times.  The oracle recomputes every committed
K/V row from the same seeded inputs, then each chain round is compared step by
step (ids on pinned steps, logits and hidden states on those and the first
unpinned step), with rebuilds after full and partial acceptance in between.

Every engine variant is held to the same bar.  The default engine (fp32 KV,
fp16 teacher-forced activations) and the split-activation engine are compared
with exact rows; the other variants with the oracle mode that computes their
formats: bf16 KV against rows rounded to bf16, single-term fp16 / bf16
activations against rows from fp16- / bf16-rounded taps and projection inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from synth import LONG, PAGE4, QWEN3_8B, gen
from tests.common import make_oracle
from tests.gpu_harness import (check_round, compare_round, compared_steps, say)

pytestmark = pytest.mark.gpu


def _variants(names):
    from eagle_draft_head_amd import binding as B
    # name: (KV format, teacher-forced activations, oracle KV format, oracle append)
    table = {
        # the default path (fp16 appends) against exact rows: the parity bar itself
        "f32": (B.KV_F32, B.APPEND_DEFAULT, "exact", "exact"),
        "f32-split": (B.KV_F32, B.APPEND_SPLIT, "exact", "exact"),
        "f32-f16": (B.KV_F32, B.APPEND_F16, "exact", "f16"),
        "f32-act16": (B.KV_F32, B.APPEND_BF16, "exact", "bf16"),
        "bf16": (B.KV_BF16, B.APPEND_DEFAULT, "bf16", "f16"),
        "q8q5": (B.KV_Q8Q5, B.APPEND_DEFAULT, "q8q5", "f16"),
    }
    return [(n,) + table[n] for n in names]


ALL_VARIANTS = ["f32", "f32-split", "f32-f16", "f32-act16", "bf16"]


class _Pair:
    def __init__(self, name, dr, orc):
        self.name, self.dr, self.orc = name, dr, orc
        self.steps = self.pinned = self.compared = 0
        self.max_err = 0.0


def _setup(cfg, L, max_ctx, variants):
    """One GPU drafter per variant on the same weights and committed rows, each
    with an oracle in the matching KV format (oracles shared per format)."""
    from eagle_draft_head_amd.drafter import Drafter
    say(f"[fullsize] {cfg.name}: generating weights on the GPU")
    wd = gen.drafter_weights(cfg, device="cuda")
    wh = {k: v.cpu() for k, v in wd.items() if k != "embed"}
    aux = gen.aux_taps(cfg, 0, L, device="cuda")
    tok = gen.tokens(cfg, 0, L, device="cuda")
    aux_h = [a.double().cpu().numpy() for a in aux]
    tok_h = tok.cpu().numpy()
    pairs = []
    for name, kv, act, fmt, oact in _variants(variants):
        dr = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=max_ctx, kv_dtype=kv, append_act=act)
        dr.prefill(0, tok, aux)
        say(f"[fullsize] {cfg.name} {name}: oracle prefill of {L} rows ({fmt} KV, {oact} appends)")
        orc = make_oracle(cfg, wh, max_ctx=max_ctx, lazy_embed=True, kv_format=fmt, append_act=oact)
        orc.prefill(0, aux_h, tok_h)
        pairs.append(_Pair(name, dr, orc))
    del wd
    torch.cuda.empty_cache()
    return pairs


def _rounds(cfg, pairs, gammas, rebuild_pattern, stored=False):
    """Drive every (drafter, oracle) pair through the same rounds.  stored: the
    benchmark's protocol; every round starts from the boundary feature stored by
    the previous rebuild (the first by a boundary-only prefill), and every rebuild
    (rebuild_pattern then has no None) also takes the next round's taps."""
    b_auxs = [gen.aux_taps(cfg, 101 + i, 1, device="cuda") for i in range(len(gammas) + 1)]
    if stored:
        assert None not in rebuild_pattern
        for p in pairs:
            p.dr.prefill(0, gen.tokens(cfg, 0, 0, device="cuda"), [], next_aux=b_auxs[0])
    for gi, gamma in enumerate(gammas):
        b_aux = b_auxs[gi]
        b_tok = gen.tokens(cfg, 101 + gi, 1, device="cuda")
        a_pat = rebuild_pattern[gi % len(rebuild_pattern)]
        for p in pairs:
            recs = p.orc.draft_chain(0, [a[0].double().cpu().numpy() for a in b_aux], int(b_tok[0]),
                                     gamma)
            out, geff, logits, hidden = p.dr.draft_chain([0], b_tok, None if stored else b_aux, gamma,
                                                         debug=True)
            torch.cuda.synchronize()
            cmp = compare_round(recs, out, geff[0], logits, hidden)
            where = f"{cfg.name} {p.name} round {gi} gamma={gamma}"
            check_round(cmp, where)
            p.steps += len(cmp)
            p.pinned += sum(1 for c in cmp if c.pinned)
            nc = compared_steps(cmp)
            p.compared += nc
            p.max_err = max([p.max_err] + [c.logit_err for c in cmp[:nc]])
            say(f"[fullsize] {where}: ids {out[0].tolist()} oracle {[r.target_id for r in recs]} "
                f"margins {[round(r.margin, 3) for r in recs]} "
                f"logit err {[f'{c.logit_err:.1e}' for c in cmp[:nc]]}")
            if a_pat is not None:
                a = min(a_pat, geff[0])
                r_aux = gen.aux_taps(cfg, 300 + gi, a, device="cuda")
                rows_aux = [torch.cat([ba, ra]) for ba, ra in zip(b_aux, r_aux)]
                rows_tok = torch.tensor([int(b_tok[0])] + [r.target_id for r in recs[:a]],
                                        dtype=torch.int32, device="cuda")
                p.orc.rebuild_after_verify(0, a, [x.double().cpu().numpy() for x in rows_aux],
                                           rows_tok.cpu().numpy())
                p.dr.rebuild_after_verify([0], [a], rows_tok, rows_aux,
                                          next_aux=b_auxs[gi + 1] if stored else None)
                assert p.dr.kv_len(0) == (p.orc.ledger.committed(0), 0)
    for p in pairs:
        say(f"[fullsize] {cfg.name} {p.name}: {p.pinned}/{p.steps} steps pinned, {p.compared} "
            f"compared, max logit err {p.max_err:.2e}")


def _kv_check(p, rows=None):
    """Committed K/V rows (all, or the listed ones) within 1e-2 relative L2 per row."""
    L = p.orc.ledger.committed(0)
    k, v = p.dr.kv_read(0, 0, L)
    idx = list(range(L)) if rows is None else rows
    for gpu, ref in ((k, p.orc.K[0]), (v, p.orc.V[0])):
        g = gpu[idx].double().cpu().numpy()
        r = ref[idx]
        rel = np.linalg.norm((g - r).reshape(len(idx), -1), axis=1) / np.linalg.norm(
            r.reshape(len(idx), -1), axis=1)
        assert rel.max() < 1e-2, (p.name, rel.max())
    return k.dtype


def _close(pairs):
    for p in pairs:
        p.dr.close()


def test_qwen3_8b_shape_chain_parity():
    cfg = QWEN3_8B
    pairs = _setup(cfg, cfg.context, cfg.context + 64, ALL_VARIANTS)
    for p in pairs:
        _kv_check(p)
    _rounds(cfg, pairs, [3] * 8, [3, None, 0, 2])
    for p in pairs:
        assert p.pinned >= p.steps // 2, p.name
        dt = _kv_check(p)
        assert dt == (torch.bfloat16 if p.name == "bf16" else torch.float32)
    _close(pairs)


def test_qwen3_8b_shape_stored_boundary_rounds():
    """The benchmark's default protocol at full size: chains from the boundary
    feature the rebuild stored (its fc row rode on the rebuild's W_fc pass)."""
    cfg = QWEN3_8B
    pairs = _setup(cfg, cfg.context, cfg.context + 64, ALL_VARIANTS)
    _rounds(cfg, pairs, [3] * 8, [3, 0, 2, 1], stored=True)
    for p in pairs:
        assert p.pinned >= p.steps // 2, p.name
        _kv_check(p)
    _close(pairs)


def test_page4_geometry_chain_parity():
    cfg = PAGE4
    pairs = _setup(cfg, cfg.context, cfg.context + 64, ALL_VARIANTS)
    _rounds(cfg, pairs, [3, 5, 8, 8, 3, 5], [3, 5, None, 8, 1, 0])
    for p in pairs:
        assert p.pinned >= p.steps // 3, p.name
        _kv_check(p)
    _close(pairs)


def test_long_context_parity():
    """5120-wide drafter with a 32767-row prefill (4096-row passes) and chains
    whose attention splits across the whole cache: every row on both sides of
    each pass boundary is checked, then six rounds with rebuilds."""
    cfg = LONG
    L = cfg.context
    pairs = _setup(cfg, L, cfg.max_ctx, ALL_VARIANTS)
    rows = sorted({0, L - 1} | {r for k in range(1, (L + 4095) // 4096)
                                for r in (4096 * k - 1, 4096 * k, 4096 * k + 1) if r < L})
    assert len(rows) == 23
    for p in pairs:
        _kv_check(p, rows)
    _rounds(cfg, pairs, [3] * 6, [2, None, 3, 0, 1, 3])
    for p in pairs:
        assert p.pinned >= p.steps // 3, p.name
    _close(pairs)


def test_long_context_parity_q8q5():
    """The q8_0 / q5_1 draft KV at the 5120-wide drafter with a 32767-row prefill: the
    MFMA decode kernel streams the whole cache through its LDS ring in splits of an
    odd number of 64-row wave steps (576 rows here); rows on both sides of the first
    pass boundary and the last row, then four rounds with rebuilds, against the
    oracle's q8q5 mode."""
    cfg = LONG
    L = cfg.context
    pairs = _setup(cfg, L, cfg.max_ctx, ["q8q5"])
    for p in pairs:
        _kv_check(p, [0, 1, 4095, 4096, 4097, L - 1])
    _rounds(cfg, pairs, [3] * 4, [2, None, 3, 0])
    for p in pairs:
        assert p.pinned >= p.steps // 3, p.name
    _close(pairs)
