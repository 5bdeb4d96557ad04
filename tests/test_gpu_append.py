"""GPU parity of the teacher-forced append paths (prefill, rebuild_after_verify)
against the oracle: every multi-vector width of the small-row path, the MFMA
path, passes longer than the internal row budget, and packed multi-sequence
rebuilds."""
import numpy as np
import pytest
import torch

from synth import TINY, small_variant
from tests.common import aux_np, make_oracle, row_slice, toks_np
from tests.gpu_harness import gpu_drafter, say, to_dev_aux, weights_both

pytestmark = pytest.mark.gpu


def _tok(x):
    return torch.as_tensor(np.asarray(x), dtype=torch.int32).reshape(-1).cuda()


def _rel_rows(gpu, ref):
    g = gpu.double().cpu().numpy()
    num = np.linalg.norm((g - ref).reshape(len(ref), -1), axis=1)
    den = np.linalg.norm(ref.reshape(len(ref), -1), axis=1)
    return (num / den).max()


# teacher-forced activation forms: (engine append_act, oracle append_act)
ACTS = {"default": (0, "f16"), "split": (2, "exact"), "bf16": (1, "bf16"), "f16": (3, "f16")}
ROW_TOL = 2e-3   # relative L2 per K/V row against the oracle in the same form


def _drafter(cfg, wd, max_ctx, act, max_seqs=1):
    from eagle_draft_head_amd.drafter import Drafter
    return Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx, max_seqs=max_seqs, append_act=ACTS[act][0])


@pytest.mark.parametrize("act", sorted(ACTS))
@pytest.mark.parametrize("cfg", [TINY, small_variant()], ids=["tiny", "ragged"])
def test_prefill_pieces_of_every_width(cfg, act):
    say(f"[append] {cfg.name} {act}: pieces")
    wd, wh = weights_both(cfg)
    # 1..16 rows: the weight-streaming path at each width; 17, 24, 32: the 32-row
    # MFMA tile (partial and full); 40: the 128-row tile
    pieces = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 12, 13, 16, 17, 24, 32, 40]
    L = sum(pieces)
    dr = _drafter(cfg, wd, L + 8, act)
    orc = make_oracle(cfg, wh, max_ctx=L + 8, append_act=ACTS[act][1])
    aux, toks = aux_np(cfg, 7, L), toks_np(cfg, 7, L)
    r0 = 0
    for T in pieces:   # the oracle appends the same pieces (its rounding follows the piece size)
        orc.prefill(0, row_slice(aux, r0, r0 + T), toks[r0:r0 + T])
        dr.prefill(0, _tok(toks[r0:r0 + T]), to_dev_aux(row_slice(aux, r0, r0 + T)))
        r0 += T
    assert dr.kv_len(0) == (L, 0)
    k, v = dr.kv_read(0, 0, L)
    r0 = 0
    for T in pieces:
        ek = _rel_rows(k[r0:r0 + T], orc.K[0][r0:r0 + T])
        ev = _rel_rows(v[r0:r0 + T], orc.V[0][r0:r0 + T])
        assert ek < ROW_TOL and ev < ROW_TOL, (T, ek, ev)
        r0 += T
    assert dr.status() == 0


@pytest.mark.parametrize("act", ["split", "f16"])
def test_prefill_longer_than_one_pass(act):
    # the engine appends at most 4096 rows per pass; 4500 rows take two passes
    cfg = TINY
    wd, wh = weights_both(cfg)
    L = 4500
    dr = _drafter(cfg, wd, L + 8, act)
    aux, toks = aux_np(cfg, 8, L), toks_np(cfg, 8, L)
    dr.prefill(0, _tok(toks), to_dev_aux(aux))
    k, v = dr.kv_read(0, 0, L)
    orc = make_oracle(cfg, wh, max_ctx=L + 8, append_act=ACTS[act][1])
    orc.prefill(0, aux, toks)
    # rows on both sides of the pass boundary, and everything else in bulk
    for r in [0, 1, 2000, 4095, 4096, 4097, 4499]:
        assert _rel_rows(k[r:r + 1], orc.K[0][r:r + 1]) < ROW_TOL
        assert _rel_rows(v[r:r + 1], orc.V[0][r:r + 1]) < ROW_TOL
    assert _rel_rows(k, orc.K[0][:L]) < ROW_TOL and _rel_rows(v, orc.V[0][:L]) < ROW_TOL


def test_fp16_append_range_is_reported():
    """A tap outside the fp16 range is not rounded silently to infinity: the
    append raises EAGLE3_STATUS_APPEND_RANGE."""
    from eagle_draft_head_amd import binding as B
    cfg = TINY
    wd, _ = weights_both(cfg)
    dr = _drafter(cfg, wd, 100, "f16")
    aux, toks = aux_np(cfg, 8, 40), toks_np(cfg, 8, 40)
    aux[1][7, 3] = 1e6
    dr.prefill(0, _tok(toks), to_dev_aux(aux))
    assert dr.status() == B.STATUS_APPEND_RANGE
    dr.prefill(0, _tok(toks), to_dev_aux(aux_np(cfg, 9, 40)))
    assert dr.status() == 0
    dr.close()
    # a weight whose 2^8-scaled fp16 copy is not exact is reported after the load
    for bad in (300.0, 2.0 ** -27 * (1 + 2.0 ** -7)):   # beyond the fp16 range; a low bit below 2^-24
        w2 = dict(wd)
        w2["fc"] = wd["fc"].clone()
        w2["fc"][5, 9] = bad
        dr = _drafter(cfg, w2, 100, "default")
        assert dr.status() == B.STATUS_APPEND_RANGE, bad
        dr.close()
    w2 = dict(wd)
    w2["fc"] = wd["fc"].clone()
    w2["fc"][5, 9] = 2.0 ** -25           # the smallest exact magnitude
    dr = _drafter(cfg, w2, 100, "default")
    assert dr.status() == 0
    dr.close()


def test_packed_multi_sequence_rebuild():
    cfg = TINY
    wd, wh = weights_both(cfg)
    S, gamma = 4, 8
    dr = gpu_drafter(cfg, wd, max_ctx=120, max_seqs=S)
    orc = make_oracle(cfg, wh, max_ctx=120, max_seqs=S)
    lens = [5, 30, 0, 63]
    aux, toks = aux_np(cfg, 9, 400), toks_np(cfg, 9, 400)
    r0 = 0
    for s, L in enumerate(lens):
        if L:
            orc.prefill(s, row_slice(aux, r0, r0 + L), toks[r0:r0 + L])
            dr.prefill(s, _tok(toks[r0:r0 + L]), to_dev_aux(row_slice(aux, r0, r0 + L)))
        r0 += L
    # a chain round on every sequence (one call), then a packed rebuild
    baux = [a[r0:r0 + S] for a in aux]
    btok = toks[r0:r0 + S]
    r0 += S
    out, geff, _, _ = dr.draft_chain(list(range(S)), _tok(btok), to_dev_aux(baux), gamma)
    assert geff == [gamma] * S
    drafts = [[r.target_id for r in orc.draft_chain(s, [a[s] for a in baux], btok[s], gamma)]
              for s in range(S)]
    accepted = [8, 0, 3, 5]
    tok_rows, aux_rows = [], [[], [], []]
    for s, a in enumerate(accepted):
        # both sides commit the oracle's drafts as the verified tokens
        tok_rows += [int(btok[s])] + drafts[s][:a]
        for j in range(3):
            aux_rows[j].append(baux[j][s:s + 1])
            aux_rows[j].append(aux[j][r0:r0 + a])
        rows_s = [np.concatenate([baux[j][s:s + 1], aux[j][r0:r0 + a]]) for j in range(3)]
        orc.rebuild_after_verify(s, a, rows_s, np.array([btok[s]] + drafts[s][:a]))
        r0 += a
    aux_rows = [np.concatenate(x) for x in aux_rows]
    dr.rebuild_after_verify(list(range(S)), accepted, _tok(tok_rows), to_dev_aux(aux_rows))
    for s in range(S):
        c = orc.ledger.committed(s)
        assert dr.kv_len(s) == (c, 0)
        k, v = dr.kv_read(s, 0, c)
        assert _rel_rows(k, orc.K[s][:c]) < 1e-2 and _rel_rows(v, orc.V[s][:c]) < 1e-2
