"""GPU parity of the drafter engine against the oracle through the C ABI:
chain rounds (ids on pinned steps, logits, hidden), KV rows written by prefill
and by the chain, rewind bit-identity, determinism, the 97/3/100 capacity edge,
state errors, and the greedy speculative loop with a CPU trunk."""
import numpy as np
import pytest
import torch

from eagle_draft_head_amd import binding as B
from oracle import TrunkOracle, greedy_plain, greedy_speculative, round_f16
from synth import TINY, gen, small_variant
from tests.common import aux_np, make_oracle, row_slice, toks_np
from tests.gpu_harness import (GpuChainAdapter, check_round, compare_round, gpu_drafter, say,
                               to_dev_aux, weights_both)

pytestmark = pytest.mark.gpu


def _tok(x):
    return torch.as_tensor(np.asarray(x), dtype=torch.int32).reshape(-1).cuda()


def _run_rounds(cfg, rounds, L, gamma, rebuild_every=0, max_ctx=None, stored=False, kv_bf16=False,
                token_table=B.TABLE_DEFAULT):
    """stored: every round starts from the boundary feature stored by the prefill
    or the previous rebuild (given the round's boundary taps as next taps), and
    every round is followed by a rebuild.  kv_bf16: the bf16 draft-KV option,
    against the oracle storing bf16-rounded rows computed from the same fp16-rounded
    append inputs as the engine's default append form.  token_table: the chain
    step's QKV embedding half from the load-time table (the default with bf16
    weights) or streamed (TABLE_OFF)."""
    say(f"[parity] cfg={cfg.name} L={L} gamma={gamma} rounds={rounds} stored={stored} bf16={kv_bf16} "
        f"table={token_table}")
    if stored:
        rebuild_every = 1
    wd, wh = weights_both(cfg)
    max_ctx = max_ctx or (L + rounds * (gamma + 1) + gamma + 8)
    dr = gpu_drafter(cfg, wd, max_ctx=max_ctx, kv_dtype=B.KV_BF16 if kv_bf16 else B.KV_F32,
                     token_table=token_table)
    orc = make_oracle(cfg, wh, max_ctx=max_ctx, **(dict(kv_format="bf16", append_act="f16") if kv_bf16 else {}))
    aux = aux_np(cfg, 0, L)
    toks = toks_np(cfg, 0, L)
    baux = aux_np(cfg, 1, rounds + 1)
    btok = toks_np(cfg, 1, rounds)
    raux = aux_np(cfg, 2, rounds * (gamma + 1))
    orc.prefill(0, aux, toks)
    dr.prefill(0, _tok(toks), to_dev_aux(aux), next_aux=to_dev_aux(baux, slice(0, 1)) if stored else None)
    steps = pinned = 0
    worst_logit = worst_hidden = 0.0
    for r in range(rounds):
        b_aux = [a[r] for a in baux]
        recs = orc.draft_chain(0, b_aux, btok[r], gamma)
        out, geff, logits, hidden = dr.draft_chain([0], _tok([btok[r]]),
                                                   None if stored else to_dev_aux(baux, slice(r, r + 1)),
                                                   gamma, debug=True)
        torch.cuda.synchronize()
        # the encoded boundary feature; the prefill's pass carries the first
        # boundary row, so with more than 16 rows in that pass its taps take the
        # default fp16 form of an MFMA append
        f16_pass = stored and r == 0 and L + 1 > 16
        f_ref = orc.encode([round_f16(a) if f16_pass else a for a in b_aux])
        f_gpu = hidden[0, 0].double().cpu().numpy()
        assert np.linalg.norm(f_gpu - f_ref) / np.linalg.norm(f_ref) < 1e-5
        cmp = compare_round(recs, out, geff[0], logits, hidden)
        check_round(cmp, f"round {r}")
        steps += len(cmp)
        for c in cmp:
            if not c.pinned:
                break
            pinned += 1
            worst_logit = max(worst_logit, c.logit_err)
            worst_hidden = max(worst_hidden, c.hidden_rel)
        if geff[0] < gamma:
            assert out[0, geff[0]:].eq(-1).all()
        if rebuild_every and r % rebuild_every == rebuild_every - 1 and geff[0] > 0:
            a = r % (geff[0] + 1)
            rows = slice(r * (gamma + 1), r * (gamma + 1) + a)
            new_aux = [np.concatenate([ba[r:r + 1], ra[rows]]) for ba, ra in zip(baux, raux)]
            new_tok = np.array([btok[r]] + [x.target_id for x in recs[:a]], dtype=np.int32)
            orc.rebuild_after_verify(0, a, new_aux, new_tok)
            dr.rebuild_after_verify([0], [a], _tok(new_tok), to_dev_aux(new_aux),
                                    next_aux=to_dev_aux(baux, slice(r + 1, r + 2)) if stored else None)
        assert dr.kv_len(0) == (orc.ledger.committed(0), 0)
    say(f"[parity] {cfg.name}: {pinned}/{steps} steps pinned; worst logit {worst_logit:.2e}, "
        f"hidden {worst_hidden:.2e}")
    return pinned, steps


def test_tiny_chain_parity_many_rounds():
    pinned, steps = _run_rounds(TINY, rounds=200, L=63, gamma=3, rebuild_every=5)
    assert pinned >= 0.25 * steps


def test_ragged_shape_chain_parity():
    # rows, K and context all leave ragged tails over the kernels' tiles
    pinned, steps = _run_rounds(small_variant(), rounds=40, L=300, gamma=4, rebuild_every=3)
    assert pinned >= 0.25 * steps


@pytest.mark.parametrize("cfg,L,gamma,rounds", [(TINY, 63, 3, 40), (small_variant(), 300, 4, 16)],
                         ids=["tiny", "ragged"])
def test_streamed_embedding_half_chain_parity(cfg, L, gamma, rounds):
    """TABLE_OFF: both halves of W_qkv streamed every step; the same bar."""
    pinned, steps = _run_rounds(cfg, rounds=rounds, L=L, gamma=gamma, rebuild_every=3,
                                token_table=B.TABLE_OFF)
    assert pinned >= 0.25 * steps


def test_token_table_matches_streamed_half():
    """The table holds W_qkv[:, :n] . (input_layernorm * E[t]) for every target
    token (MFMA with (hi, lo) bf16 activations, relative error per product at most
    2^-18); a chain with it agrees with the streamed form to fp32 rounding:
    identical ids, logits and hidden within 1e-5 relative, over every step of
    several rounds whose boundary tokens cover the vocabulary's ends."""
    cfg = small_variant()
    wd, _ = weights_both(cfg)
    L, gamma = 40, 6
    drs = [gpu_drafter(cfg, wd, max_ctx=200, token_table=t) for t in (B.TABLE_ON, B.TABLE_OFF)]
    aux = aux_np(cfg, 0, L)
    toks = toks_np(cfg, 0, L)
    for dr in drs:
        dr.prefill(0, _tok(toks), to_dev_aux(aux))
    baux = aux_np(cfg, 1, 6)
    for r, t in enumerate([0, cfg.target_vocab - 1, 1, 17, cfg.target_vocab // 2, 5]):
        res = []
        for dr in drs:
            out, geff, logits, hidden = dr.draft_chain([0], _tok([t]), to_dev_aux(baux, slice(r, r + 1)), gamma,
                                                       debug=True)
            torch.cuda.synchronize()
            res.append((out.cpu(), int(geff[0]), logits.double().cpu(), hidden.double().cpu()))
            dr.rewind(0, L)
        (o1, g1, l1, h1), (o2, g2, l2, h2) = res
        assert g1 == g2 == gamma
        # the ids agree up to the first near-tie of the streamed form's logits
        top2 = torch.topk(l2[0, :g2], 2, dim=-1).values
        gap = (top2[:, 0] - top2[:, 1]).abs()
        ok = int(torch.nonzero(gap < 1e-4).min()) if bool((gap < 1e-4).any()) else g2
        assert torch.equal(o1[0, :ok], o2[0, :ok]), (r, o1, o2)
        # steps 0..ok read the same tokens: their logits and hidden states compare
        for j in range(min(ok + 1, g2)):
            assert (l1[0, j] - l2[0, j]).norm() / l2[0, j].norm() < 1e-5, (r, j)
        for j in range(min(ok + 2, g2 + 1)):
            assert (h1[0, j] - h2[0, j]).norm() / h2[0, j].norm() < 1e-5, (r, j)
    for dr in drs:
        dr.close()


@pytest.mark.parametrize("cfg,kv,weights", [(TINY, "f32", "bf16"), (TINY, "bf16", "bf16"),
                                             (small_variant(), "f32", "bf16"), (small_variant(), "bf16", "bf16"),
                                             (TINY, "f32", "int4")],
                         ids=["tiny-f32", "tiny-bf16", "ragged-f32", "ragged-bf16", "tiny-int4"])
def test_deferred_qkv_matches_the_fused_qkv_kernel(cfg, kv, weights, monkeypatch):
    """The default batch-1 step computes the hidden half of its QKV projection in the
    previous step's lm_head launch (alone for the first step) and finishes q and the
    new K/V row in the attention kernel, the new row merged from LDS by the block
    whose split holds it.  Against the fused QKV kernel (EAGLE3_DEFER_QKV=0): the same
    sums up to rounding order -- identical ids (up to near-ties), logits and hidden
    within 1e-5 relative, the chain's K/V rows within 1e-5 (bf16 K/V: the first step's
    row at most one bf16 step apart per element, everything else within 1e-3) -- from
    an empty cache (the
    new row alone in its split), a context whose new row opens a split (64 rows) and
    one of many splits, in the persistent and the round-local drafter; with int4
    weights the hidden half streams as int4 codes in the int4 lm_head launch (bar
    1e-4: the int4 GEMVs' fixed-point activations)."""
    from eagle_draft_head_amd.drafter import Drafter
    wd, _ = weights_both(cfg)
    gamma = 5
    kvd = B.KV_BF16 if kv == "bf16" else B.KV_F32
    wf = B.WEIGHTS_I4 if weights == "int4" else B.WEIGHTS_BF16

    def make():
        return Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=800, max_gamma=16, kv_dtype=kvd, weight_format=wf)

    monkeypatch.setenv("EAGLE3_DEFER_QKV", "0")
    ref = make()
    monkeypatch.delenv("EAGLE3_DEFER_QKV")
    dq = make()
    drs = [dq, ref]
    aux = aux_np(cfg, 0, 700)
    toks = toks_np(cfg, 0, 700)
    baux = aux_np(cfg, 1, 8)
    btok = toks_np(cfg, 1, 8)
    r = 0
    for L in (0, 64, 700):
        for dr in drs:
            dr.rewind(0, 0)
            if L:
                dr.prefill(0, _tok(toks[:L]), to_dev_aux([a[:L] for a in aux]))
        for local in (False, True):
            say(f"[deferred qkv] {cfg.name} kv={kv} weights={weights} L={L} round_local={local}")
            res = []
            for dr in drs:
                out, geff, logits, hidden = dr.draft_chain([0], _tok([btok[r]]), to_dev_aux(baux, slice(r, r + 1)),
                                                           gamma, debug=True, keep_spec=not local,
                                                           round_local=local)
                torch.cuda.synchronize()
                rows = None if local else [x.double().cpu() for x in dr.kv_read(0, L, gamma)]
                res.append((out.cpu(), int(geff[0]), logits.double().cpu(), hidden.double().cpu(), rows))
                if not local:
                    dr.rewind(0, L)
            (o1, g1, l1, h1, kv1), (o2, g2, l2, h2, kv2) = res
            assert g1 == g2 == gamma
            top2 = torch.topk(l2[0, :g2], 2, dim=-1).values
            gap = (top2[:, 0] - top2[:, 1]).abs()
            ok = int(torch.nonzero(gap < 1e-4).min()) if bool((gap < 1e-4).any()) else g2
            assert torch.equal(o1[0, :ok], o2[0, :ok]), (L, local, o1, o2)
            # bf16 K/V: a stored element may sit one bf16 step from the other path's, and
            # every later read sees it; int4: the GEMVs' per-group fixed-point activations
            # (steps of 2^-14 of a group's largest value) can take inputs a rounding
            # apart one step apart
            tol = 1e-3 if kv == "bf16" else (1e-4 if weights == "int4" else 1e-5)
            for j in range(min(ok + 1, g2)):
                assert (l1[0, j] - l2[0, j]).norm() / l2[0, j].norm() < tol, (L, local, j)
            for j in range(min(ok + 2, g2 + 1)):
                assert (h1[0, j] - h2[0, j]).norm() / h2[0, j].norm() < tol, (L, local, j)
            if kv1 is not None:
                for j in range(min(ok + 1, g2)):  # rows of steps that read the same tokens
                    for a1, a2 in zip(kv1, kv2):
                        if kv == "bf16":  # fp32 values a rounding apart may round to neighbouring bf16
                            if j == 0:  # the same inputs: at most one bf16 step apart
                                assert bool(((a1[j] - a2[j]).abs() <= 2.0 ** -7 * a2[j].abs()).all()), (L, j)
                            assert (a1[j] - a2[j]).norm() / a2[j].norm() < 1e-3, (L, j)
                        else:
                            assert (a1[j] - a2[j]).norm() / a2[j].norm() < tol, (L, j)
            r += 1
    for dr in drs:
        dr.close()


@pytest.mark.parametrize("hd,nh,nkv,kv", [(128, 4, 2, "f32"), (128, 4, 2, "bf16"), (256, 4, 1, "f32"),
                                          (256, 4, 1, "bf16")],
                         ids=["hd128-f32", "hd128-bf16-mfma", "hd256-f32", "hd256-bf16"])
def test_deferred_qkv_at_split_boundaries(hd, nh, nkv, kv, monkeypatch):
    """The deferred QKV's new row is taken into the softmax from LDS by the block whose
    split holds it; with 16-, 32- or 64-row splits (fp32 and bf16 on the VALU kernel,
    bf16 at head_dim 128 on the MFMA kernel) contexts of 0 to 2048 rows put the new row
    first, last and alone in its split.  Against the fused QKV kernel: ids equal up to
    near-ties, logits and hidden within 1e-5 (bf16 K/V: 1e-3), every chain K/V row
    within the same bars."""
    from eagle_draft_head_amd.drafter import Drafter
    cfg = small_variant(f"dq-hd{hd}", head_dim=hd, n_head=nh, n_head_kv=nkv, max_ctx=2200)
    wd, _ = weights_both(cfg)
    gamma = 4
    kvd = B.KV_BF16 if kv == "bf16" else B.KV_F32

    def make():
        return Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=2200, max_gamma=8, kv_dtype=kvd)

    monkeypatch.setenv("EAGLE3_DEFER_QKV", "0")
    ref = make()
    monkeypatch.delenv("EAGLE3_DEFER_QKV")
    dq = make()
    Lmax = 2048
    aux = aux_np(cfg, 0, Lmax)
    toks = toks_np(cfg, 0, Lmax)
    baux = aux_np(cfg, 1, 16)
    btok = toks_np(cfg, 1, 16)
    tol = 1e-3 if kv == "bf16" else 1e-5
    have = 0  # committed rows (rewind only shrinks: contexts grow by prefilled pieces)
    for r, L in enumerate([0, 1, 15, 16, 63, 64, 65, 127, 128, 511, 512, 1023, 2044, 2047]):
        say(f"[deferred qkv boundaries] hd={hd} kv={kv} L={L}")
        if L > have:
            for dr in (dq, ref):
                dr.prefill(0, _tok(toks[have:L]), to_dev_aux([a[have:L] for a in aux]))
            have = L
        res = []
        for dr in (dq, ref):
            out, geff, logits, hidden = dr.draft_chain([0], _tok([btok[r % 16]]), to_dev_aux(baux, slice(r % 16, r % 16 + 1)),
                                                       gamma, debug=True, keep_spec=True)
            torch.cuda.synchronize()
            rows = [x.double().cpu() for x in dr.kv_read(0, L, gamma)]
            res.append((out.cpu(), int(geff[0]), logits.double().cpu(), hidden.double().cpu(), rows))
            dr.rewind(0, L)
        (o1, g1, l1, h1, kv1), (o2, g2, l2, h2, kv2) = res
        assert g1 == g2 == gamma
        top2 = torch.topk(l2[0, :g2], 2, dim=-1).values
        gap = (top2[:, 0] - top2[:, 1]).abs()
        ok = int(torch.nonzero(gap < 1e-4).min()) if bool((gap < 1e-4).any()) else g2
        assert torch.equal(o1[0, :ok], o2[0, :ok]), (L, o1, o2)
        for j in range(min(ok + 1, g2)):
            assert (l1[0, j] - l2[0, j]).norm() / l2[0, j].norm() < tol, (L, j)
            for a1, a2 in zip(kv1, kv2):
                assert (a1[j] - a2[j]).norm() / a2[j].norm() < tol, (L, j)
        for j in range(min(ok + 2, g2 + 1)):
            assert (h1[0, j] - h2[0, j]).norm() / h2[0, j].norm() < tol, (L, j)
    for dr in (dq, ref):
        dr.close()


@pytest.mark.parametrize("cfg,weights", [(TINY, "bf16"), (small_variant(), "bf16"), (TINY, "int4")],
                         ids=["tiny", "ragged", "tiny-int4"])
def test_boundary_hidden_half_from_the_append(cfg, weights, monkeypatch):
    """With the deferred QKV, the append pass that stores a boundary feature (one
    boundary row with teacher-forced rows, multi-vector path) computes the feature's
    hidden-half QKV sums in its K/V launch, and the chain that starts from the stored
    feature runs no hidden-half launch of its own.  Against EAGLE3_BOUNDARY_QH=0 (that
    launch in every chain): ids equal up to near-ties, logits and hidden within 1e-5,
    over stored-boundary rounds on two sequence slots -- a prefill whose pass takes the
    boundary row past 16 rows (MFMA pass: no sums, the chain computes them), short
    prefills and single-sequence rebuilds (sums from the K/V launch), rebuilds of both
    sequences in one pass (two boundary rows: no sums) and a boundary-only prefill
    (no K/V launch: no sums); with int4 weights the sums stream the int4 codes of the
    hidden half in the int4 K/V launch."""
    from eagle_draft_head_amd.drafter import Drafter
    wd, _ = weights_both(cfg)
    gamma = 4
    wf = B.WEIGHTS_I4 if weights == "int4" else B.WEIGHTS_BF16
    nseq = 1 if weights == "int4" else 2  # int4 weights: batch-1 drafting only (one slot)

    def make():
        return Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=400, max_gamma=8, max_seqs=nseq, weight_format=wf)

    monkeypatch.setenv("EAGLE3_BOUNDARY_QH", "0")
    ref = make()
    monkeypatch.delenv("EAGLE3_BOUNDARY_QH")
    bq = make()
    drs = (bq, ref)
    aux = aux_np(cfg, 0, 300)
    toks = toks_np(cfg, 0, 300)
    baux = aux_np(cfg, 1, 64)
    btok = toks_np(cfg, 1, 64)
    raux = aux_np(cfg, 2, 64 * (gamma + 1))
    nb = 0  # next boundary row

    def nxt(k=1):
        nonlocal nb
        nb += k
        return slice(nb - k, nb)

    sl = nxt()
    for dr in drs:  # 40 rows + the boundary: one MFMA pass
        dr.prefill(0, _tok(toks[:40]), to_dev_aux([a[:40] for a in aux]), next_aux=to_dev_aux(baux, sl))
    sl = nxt()
    for dr in drs:  # 5 rows + the boundary: the multi-vector pass with the sums
        dr.prefill(nseq - 1, _tok(toks[40:45]), to_dev_aux([a[40:45] for a in aux]), next_aux=to_dev_aux(baux, sl))
    last_tok = {0: int(toks[39]) if nseq == 2 else int(toks[44]), nseq - 1: int(toks[44])}
    for r in range(12):
        for sq in range(nseq):
            say(f"[boundary qh] {cfg.name} {weights} round {r} seq {sq}")
            res = []
            for dr in drs:
                out, geff, logits, hidden = dr.draft_chain([sq], _tok([last_tok[sq]]), None, gamma, debug=True)
                torch.cuda.synchronize()
                res.append((out.cpu(), int(geff[0]), logits.double().cpu(), hidden.double().cpu()))
            (o1, g1, l1, h1), (o2, g2, l2, h2) = res
            assert g1 == g2 == gamma
            top2 = torch.topk(l2[0, :g2], 2, dim=-1).values
            gap = (top2[:, 0] - top2[:, 1]).abs()
            ok = int(torch.nonzero(gap < 1e-4).min()) if bool((gap < 1e-4).any()) else g2
            assert torch.equal(o1[0, :ok], o2[0, :ok]), (r, o1, o2)
            for j in range(min(ok + 1, g2)):
                assert (l1[0, j] - l2[0, j]).norm() / l2[0, j].norm() < 1e-5, (r, j)
            for j in range(min(ok + 2, g2 + 1)):
                assert (h1[0, j] - h2[0, j]).norm() / h2[0, j].norm() < 1e-5, (r, j)
        # the next boundary: rebuild one sequence, both in one pass, or (round 7)
        # a boundary-only prefill
        a = r % (gamma + 1)
        if r == 7:
            sl = nxt()
            for dr in drs:
                dr.prefill(nseq - 1, _tok([]), [None, None, None], next_aux=to_dev_aux(baux, sl))
            continue
        both = r % 4 == 3 and nseq == 2
        rs = [0, 1] if both else [r % nseq]
        rows = slice(r * (gamma + 1), r * (gamma + 1) + (a + 1) * len(rs))
        new_tok = toks_np(cfg, 3 + r, (a + 1) * len(rs))
        sl = nxt(len(rs))
        for dr in drs:
            dr.rebuild_after_verify(rs, [a] * len(rs), _tok(new_tok), to_dev_aux(raux, rows),
                                    next_aux=to_dev_aux(baux, sl))
        for i, sq in enumerate(rs):
            last_tok[sq] = int(new_tok[(i + 1) * (a + 1) - 1])
    for dr in drs:
        dr.close()


def test_chain_from_empty_cache():
    pinned, steps = _run_rounds(TINY, rounds=10, L=0, gamma=5)
    assert steps == 50


@pytest.mark.parametrize("cfg,L,gamma,rounds", [(TINY, 63, 3, 40), (small_variant(), 300, 4, 16),
                                                (TINY, 0, 5, 6), (TINY, 1500, 3, 8)],
                         ids=["tiny", "ragged", "empty", "long"])
def test_bf16_kv_chain_parity(cfg, L, gamma, rounds):
    """bf16 K/V: the decode attention runs on MFMA (head_dim 64 here) with ragged
    tiles, one split and many; held to the standard bar."""
    pinned, steps = _run_rounds(cfg, rounds=rounds, L=L, gamma=gamma, rebuild_every=3, kv_bf16=True)
    assert pinned >= 0.25 * steps


def test_stored_boundary_rounds_tiny():
    """Boundary features stored by prefill and by every rebuild (one fc pass over
    the accepted rows and the next boundary), chains starting from them."""
    pinned, steps = _run_rounds(TINY, rounds=60, L=63, gamma=3, stored=True)
    assert pinned >= 0.25 * steps


def test_stored_boundary_rounds_ragged_and_empty():
    pinned, steps = _run_rounds(small_variant(), rounds=12, L=300, gamma=4, stored=True)
    assert pinned >= 0.25 * steps
    _run_rounds(TINY, rounds=5, L=0, gamma=5, stored=True)  # boundary-only prefill


@pytest.mark.parametrize("cfg,L,gamma,rounds", [(TINY, 63, 3, 30), (TINY, 0, 8, 5),
                                                (small_variant(), 300, 5, 8)],
                         ids=["tiny", "empty", "ragged"])
def test_round_local_chain_parity(cfg, L, gamma, rounds):
    """The scratch-KV drafter: each round attends over its own rows only; the
    committed rows stay bit-identical and no length changes."""
    say(f"[parity] round-local cfg={cfg.name} L={L} gamma={gamma} rounds={rounds}")
    wd, wh = weights_both(cfg)
    dr = gpu_drafter(cfg, wd, max_ctx=L + 16, max_gamma=max(8, gamma))
    orc = make_oracle(cfg, wh, max_ctx=L + 16)
    aux, toks = aux_np(cfg, 0, L), toks_np(cfg, 0, L)
    orc.prefill(0, aux, toks)
    dr.prefill(0, _tok(toks), to_dev_aux(aux))
    if L:
        k0, v0 = (t.clone() for t in dr.kv_read(0, 0, L))
    baux, btok = aux_np(cfg, 1, rounds), toks_np(cfg, 1, rounds)
    steps = pinned = 0
    for r in range(rounds):
        recs = orc.draft_chain_round_local(0, [a[r] for a in baux], btok[r], gamma)
        out, geff, logits, hidden = dr.draft_chain([0], _tok([btok[r]]), to_dev_aux(baux, slice(r, r + 1)),
                                                   gamma, debug=True, round_local=True)
        torch.cuda.synchronize()
        assert geff == [gamma] and len(recs) == gamma
        cmp = compare_round(recs, out, geff[0], logits, hidden)
        check_round(cmp, f"round-local round {r}")
        steps += len(cmp)
        for c in cmp:
            if not c.pinned:
                break
            pinned += 1
        assert dr.kv_len(0) == (L, 0)
    if L:
        k1, v1 = dr.kv_read(0, 0, L)
        assert torch.equal(k0, k1) and torch.equal(v0, v1)
    say(f"[parity] round-local {cfg.name}: {pinned}/{steps} steps pinned")
    assert pinned >= max(1, rounds // 2)  # the comparison is not vacuous


def test_stored_boundary_state_errors(tiny):
    wd, _ = tiny
    dr = gpu_drafter(TINY, wd, max_ctx=200)
    aux, toks = aux_np(TINY, 0, 20), toks_np(TINY, 0, 20)
    dr.prefill(0, _tok(toks), to_dev_aux(aux))
    with pytest.raises(B.Eagle3Error) as e:
        dr.draft_chain([0], _tok([1]), None, 3)
    assert e.value.code == B.E_STATE
    assert dr.kv_len(0) == (20, 0)
    baux = to_dev_aux(aux_np(TINY, 1, 1))
    # taps together with the stored-boundary flag are rejected
    with pytest.raises(B.Eagle3Error) as e:
        B.eagle3_draft_chain(dr.ctx, [0], _tok([1]), baux[0], baux[1], baux[2], 3,
                             torch.empty((1, 3), dtype=torch.int32, device="cuda"),
                             flags=B.STORED_BOUNDARY)
    assert e.value.code == B.E_INVAL
    # only some of the three next-boundary streams
    with pytest.raises(B.Eagle3Error) as e:
        B.eagle3_prefill(dr.ctx, 0, 0, None, None, None, None, baux[0], None, baux[2])
    assert e.value.code == B.E_INVAL
    dr.prefill(0, _tok([]), [], next_aux=baux)  # boundary only
    out, geff, _, _ = dr.draft_chain([0], _tok([1]), None, 3)
    assert geff == [3] and dr.kv_len(0) == (20, 0)
    dr.rewind(0, 20)  # drops the stored feature
    with pytest.raises(B.Eagle3Error) as e:
        dr.draft_chain([0], _tok([1]), None, 3)
    assert e.value.code == B.E_STATE
    dr.close()


@pytest.fixture(scope="module")
def tiny():
    wd, wh = weights_both(TINY)
    return wd, wh


def test_prefill_kv_rows_match_oracle(tiny):
    wd, wh = tiny
    L = 63
    dr = gpu_drafter(TINY, wd, max_ctx=200)
    orc = make_oracle(TINY, wh, max_ctx=200)
    aux, toks = aux_np(TINY, 0, L), toks_np(TINY, 0, L)
    orc.prefill(0, aux, toks)
    dr.prefill(0, _tok(toks), to_dev_aux(aux))
    k, v = dr.kv_read(0, 0, L)
    for gpu, ref in ((k, orc.K[0][:L]), (v, orc.V[0][:L])):
        g = gpu.double().cpu().numpy()
        rel = np.linalg.norm(g - ref, axis=(1, 2)) / np.linalg.norm(ref, axis=(1, 2))
        assert rel.max() < 1e-2, rel.max()


def test_chain_kv_row_matches_step_and_rewinds_bit_identical(tiny):
    wd, wh = tiny
    L, gamma = 40, 4
    dr = gpu_drafter(TINY, wd, max_ctx=200)
    orc = make_oracle(TINY, wh, max_ctx=200)
    aux, toks = aux_np(TINY, 3, L + 1), toks_np(TINY, 3, L + 1)
    orc.prefill(0, row_slice(aux, 0, L), toks[:L])
    dr.prefill(0, _tok(toks[:L]), to_dev_aux(row_slice(aux, 0, L)))
    k0, v0 = dr.kv_read(0, 0, L)
    k0, v0 = k0.clone(), v0.clone()
    b_aux = [torch.as_tensor(a[L:L + 1], dtype=torch.float32).cuda() for a in aux]
    recs = orc.draft_chain(0, [a[L] for a in aux], toks[L], gamma)
    out, geff, _, _ = dr.draft_chain([0], _tok([toks[L]]), b_aux, gamma, keep_spec=True)
    assert dr.kv_len(0) == (L, gamma)
    k1, v1 = dr.kv_read(0, L, gamma)
    for j, r in enumerate(recs):
        if r.margin <= 0.05 or any(x.margin <= 0.05 for x in recs[:j]):
            break
        for gpu, ref in ((k1[j], r.k), (v1[j], r.v)):
            g = gpu.double().cpu().numpy()
            assert np.linalg.norm(g - ref) / np.linalg.norm(ref) < 1e-2
    with pytest.raises(B.Eagle3Error) as e:
        dr.draft_chain([0], _tok([toks[L]]), b_aux, gamma)
    assert e.value.code == B.E_STATE
    dr.rewind(0, L)
    assert dr.kv_len(0) == (L, 0)
    for _ in range(3):
        dr.draft_chain([0], _tok([toks[L]]), b_aux, gamma)
    k2, v2 = dr.kv_read(0, 0, L)
    assert torch.equal(k2.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(v2.view(torch.int16), v0.view(torch.int16))


def test_chain_is_deterministic(tiny):
    wd, _ = tiny
    dr = gpu_drafter(TINY, wd, max_ctx=200)
    aux, toks = aux_np(TINY, 4, 31), toks_np(TINY, 4, 31)
    dr.prefill(0, _tok(toks[:30]), to_dev_aux(row_slice(aux, 0, 30)))
    b_aux = [torch.as_tensor(a[30:31], dtype=torch.float32).cuda() for a in aux]
    o1, _, l1, h1 = dr.draft_chain([0], _tok([toks[30]]), b_aux, 6, debug=True)
    o2, _, l2, h2 = dr.draft_chain([0], _tok([toks[30]]), b_aux, 6, debug=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(h1, h2)


def test_capacity_edge_97_3_100(tiny):
    wd, wh = tiny
    dr = gpu_drafter(TINY, wd, max_ctx=100, max_seqs=2)
    aux, toks = aux_np(TINY, 5, 110), toks_np(TINY, 5, 110)
    dr.prefill(0, _tok(toks[:97]), to_dev_aux(row_slice(aux, 0, 97)))
    b_aux = [torch.as_tensor(a[97:98], dtype=torch.float32).cuda() for a in aux]
    out, geff, _, _ = dr.draft_chain([0], _tok([toks[97]]), b_aux, 3)
    assert geff == [3]
    orc = make_oracle(TINY, wh, max_ctx=100)
    orc.prefill(0, row_slice(aux, 0, 97), toks[:97])
    drafts = [r.target_id for r in orc.draft_chain(0, [a[97] for a in aux], toks[97], 3)]
    new_tok = np.array([toks[97]] + drafts, dtype=np.int32)     # full acceptance
    dr.rebuild_after_verify([0], [3], _tok(new_tok), to_dev_aux(row_slice(aux, 97, 101)))
    assert dr.kv_len(0) == (101, 0)
    # row 100 (the reserve) now holds the fourth committed row; the oracle agrees
    orc.rebuild_after_verify(0, 3, row_slice(aux, 97, 101), new_tok)
    k, v = dr.kv_read(0, 97, 4)
    rel = np.linalg.norm(k.double().cpu().numpy() - orc.K[0][97:101]) / np.linalg.norm(orc.K[0][97:101])
    assert rel < 1e-2
    # the next sequence's region (right after row 100) is untouched
    k1, v1 = dr.kv_read(1, 0, 101)
    assert not k1.view(torch.int16).any() and not v1.view(torch.int16).any()
    out, geff, _, _ = dr.draft_chain([0], _tok([toks[101]]), b_aux, 3)
    assert geff == [0] and out.eq(-1).all()
    with pytest.raises(B.Eagle3Error) as e:
        dr.rebuild_after_verify([0], [0], _tok(toks[101:102]), to_dev_aux(row_slice(aux, 101, 102)))
    assert e.value.code == B.E_CAPACITY
    assert dr.kv_len(0) == (101, 0)


def test_state_and_argument_errors(tiny):
    wd, _ = tiny
    dr = gpu_drafter(TINY, wd, max_ctx=50)
    aux, toks = aux_np(TINY, 6, 60), toks_np(TINY, 6, 60)
    with pytest.raises(B.Eagle3Error) as e:
        dr.prefill(0, _tok(toks[:51]), to_dev_aux(row_slice(aux, 0, 51)))
    assert e.value.code == B.E_CAPACITY
    with pytest.raises(B.Eagle3Error) as e:
        dr.rebuild_after_verify([0], [0], _tok(toks[:1]), to_dev_aux(row_slice(aux, 0, 1)))
    assert e.value.code == B.E_STATE
    with pytest.raises(B.Eagle3Error) as e:
        dr.draft_chain([1], _tok([1]), to_dev_aux(row_slice(aux, 0, 1)), 3)
    assert e.value.code == B.E_INVAL
    with pytest.raises(B.Eagle3Error) as e:
        dr.draft_chain([0], _tok([1]), to_dev_aux(row_slice(aux, 0, 1)), 17)
    assert e.value.code == B.E_INVAL
    out, geff, _, _ = dr.draft_chain([0], _tok([1]), to_dev_aux(row_slice(aux, 0, 1)), 2)
    with pytest.raises(B.Eagle3Error) as e:
        dr.rebuild_after_verify([0], [3], _tok(toks[:4]), to_dev_aux(row_slice(aux, 0, 4)))
    assert e.value.code == B.E_INVAL
    assert dr.kv_len(0) == (0, 0)
    with pytest.raises(B.Eagle3Error) as e:
        dr.rewind(0, 1)
    assert e.value.code == B.E_INVAL


@pytest.mark.parametrize("plen,gamma,max_new", [(1, 3, 16), (17, 3, 40), (64, 5, 40)])
def test_greedy_loop_with_gpu_drafter(tiny, plen, gamma, max_new):
    wd, wh = tiny
    tw = gen.trunk_weights(TINY)
    trunk = TrunkOracle(TINY, tw, wh["embed"], TINY.trunk_layers)
    prompt = gen.tokens(TINY, 50 + plen, plen).tolist()
    ref = greedy_plain(trunk, prompt, max_new)
    dr = gpu_drafter(TINY, wd, max_ctx=plen + max_new + gamma + 8)
    out, drafted, acc = greedy_speculative(trunk, GpuChainAdapter(dr), prompt, max_new, gamma)
    assert out == ref


@pytest.mark.parametrize("gamma", [1, 3, 5])
def test_greedy_loop_full_acceptance_on_gpu(tiny, gamma):
    from tests.test_oracle_loop import echo_weights
    wd, wh = tiny
    w_e, tw, image = echo_weights(wh, gen.trunk_weights(TINY))
    trunk = TrunkOracle(TINY, tw, w_e["embed"], TINY.trunk_layers)
    prompt = [int(image[7]), int(image[100]), int(image[33])]
    ref = greedy_plain(trunk, prompt, 30)
    dr = gpu_drafter(TINY, {k: v.cuda() for k, v in w_e.items()}, max_ctx=64)
    out, drafted, acc = greedy_speculative(trunk, GpuChainAdapter(dr), prompt, 30, gamma)
    assert out == ref
    assert acc == drafted > 0


class _RecordingOracleAdapter:
    """The oracle drafter through the loop's interface, keeping every round's
    records (ids and margins)."""

    def __init__(self, d):
        self.d = d
        self.rounds = []

    def prefill(self, s, aux, toks):
        self.d.prefill(s, aux, toks)

    def draft_chain_ids(self, s, boundary_aux, boundary_tok, gamma):
        recs = self.d.draft_chain(s, boundary_aux, boundary_tok, gamma)
        self.rounds.append(recs)
        return [r.target_id for r in recs]

    def rebuild_after_verify(self, s, a, aux, toks):
        self.d.rebuild_after_verify(s, a, aux, toks)
        self.rounds[-1] = (self.rounds[-1], a, self.d.ledger.committed(s))


class _RecordingGpuAdapter(GpuChainAdapter):
    def __init__(self, dr):
        super().__init__(dr)
        self.rounds = []

    def draft_chain_ids(self, s, boundary_aux, boundary_tok, gamma):
        ids = super().draft_chain_ids(s, boundary_aux, boundary_tok, gamma)
        self.rounds.append(ids)
        return ids

    def rebuild_after_verify(self, s, a, aux, toks):
        super().rebuild_after_verify(s, a, aux, toks)
        self.rounds[-1] = (self.rounds[-1], a, self.d.kv_len(s)[0])


@pytest.mark.parametrize("plen,gamma,max_new", [(17, 3, 60), (64, 5, 60)])
def test_greedy_loop_accept_counts_match_the_oracle_drafter(tiny, plen, gamma, max_new):
    """The same loop driven by the oracle drafter and by the GPU drafter.  While
    both drafters have seen identical inputs, the leading draft steps whose oracle
    margin exceeds the pinning bar must give the same ids; when the oracle's
    accept count falls inside that pinned prefix (or the whole round agrees), the
    accept counts and committed lengths must agree too and the next round starts
    from the same state."""
    from tests.gpu_harness import MARGIN
    wd, wh = tiny
    tw = gen.trunk_weights(TINY)
    prompt = gen.tokens(TINY, 50 + plen, plen).tolist()
    max_ctx = plen + max_new + gamma + 8
    t1 = TrunkOracle(TINY, tw, wh["embed"], TINY.trunk_layers)
    oa = _RecordingOracleAdapter(make_oracle(TINY, wh, max_ctx=max_ctx))
    out_o, drafted_o, acc_o = greedy_speculative(t1, oa, prompt, max_new, gamma)
    t2 = TrunkOracle(TINY, tw, wh["embed"], TINY.trunk_layers)
    ga = _RecordingGpuAdapter(gpu_drafter(TINY, wd, max_ctx=max_ctx))
    out_g, drafted_g, acc_g = greedy_speculative(t2, ga, prompt, max_new, gamma)
    assert out_o == out_g
    compared = 0
    for (recs, a_o, len_o), (ids, a_g, len_g) in zip(oa.rounds, ga.rounds):
        p = 0
        while p < len(recs) and recs[p].margin > MARGIN:
            p += 1
        assert ids[:p] == [r.target_id for r in recs[:p]]
        if a_o < p or ids == [r.target_id for r in recs]:
            assert a_g == a_o and len_g == len_o
            compared += 1
        else:
            break
    say(f"[loop] plen={plen} gamma={gamma}: {compared} of {len(oa.rounds)} rounds compared; "
        f"accepted {acc_g}/{drafted_g} (oracle drafter {acc_o}/{drafted_o})")
    assert compared >= 3
    if compared == len(oa.rounds):
        assert (drafted_g, acc_g) == (drafted_o, acc_o)


def _tied_weights(wh, row, lower, higher):
    """lm_head rows `lower` < `row` < `higher` set to copies of row `row`: those
    three logits are equal on both sides, so a step whose maximum is row `row` has
    a three-way tie that the lowest index must win."""
    w = dict(wh)
    lm = wh["lm_head"].clone()
    lm[lower] = lm[row]
    lm[higher] = lm[row]
    w["lm_head"] = lm
    return w


@pytest.mark.parametrize("batched", [False, True])
def test_argmax_tie_takes_the_lowest_draft_index(tiny, batched):
    wd, wh = tiny
    L, gamma = 40, 3
    aux, toks = aux_np(TINY, 9, L + 2), toks_np(TINY, 9, L + 2)
    orc = make_oracle(TINY, wh, max_ctx=96)
    orc.prefill(0, row_slice(aux, 0, L), toks[:L])
    b_aux = [a[L] for a in aux]
    top = orc.draft_chain(0, b_aux, toks[L], 1)[0].draft_id
    lower, higher = top // 2, (top + TINY.draft_vocab) // 2
    assert lower < top < higher
    wt = _tied_weights(wh, top, lower, higher)
    orc = make_oracle(TINY, wt, max_ctx=96, max_seqs=2)
    S = 2 if batched else 1
    dr = gpu_drafter(TINY, {k: v.cuda() for k, v in wt.items()}, max_ctx=96, max_seqs=S)
    for s in range(S):
        orc.prefill(s, row_slice(aux, 0, L), toks[:L])
        dr.prefill(s, _tok(toks[:L]), to_dev_aux(row_slice(aux, 0, L)))
    recs = orc.draft_chain(0, b_aux, toks[L], gamma)
    assert recs[0].draft_id == lower and recs[0].margin == 0.0
    assert recs[0].logits[lower] == recs[0].logits[top] == recs[0].logits[higher]
    baux_dev = to_dev_aux([np.stack([a[L]] * S) for a in aux])
    out, geff, logits, hidden = dr.draft_chain(list(range(S)), _tok([toks[L]] * S), baux_dev, gamma,
                                               debug=True)
    torch.cuda.synchronize()
    for s in range(S):
        lg = logits[s, 0]
        assert lg[lower] == lg[top] == lg[higher]            # an exact three-way tie on the GPU
        assert int(out[s, 0]) == recs[0].target_id == lower + int(wh["d2t"][lower])
        # the tied step's logits and hidden are within the bar; later steps see the
        # same token, so they compare as usual
        cmp = compare_round(recs, out, geff[s], logits, hidden, b=s)
        assert cmp[0].logit_err <= 2e-2 and cmp[0].hidden_rel <= 1e-2
        check_round(cmp[1:], f"after the tie, seq {s}")
    dr.close()


@pytest.mark.parametrize("seqs", [1, 2])
def test_status_reports_bad_tokens_and_nan_logits(tiny, seqs):
    """Bad device-side inputs are not corrected silently: an out-of-range token id
    (teacher-forced or boundary) raises EAGLE3_STATUS_BAD_TOKEN and taps that make
    every logit NaN raise EAGLE3_STATUS_NAN_LOGITS; eagle3_status returns the bits
    and clears them, and a clean round raises none."""
    wd, _ = tiny
    dr = gpu_drafter(TINY, wd, max_ctx=100, max_seqs=seqs)
    S = list(range(seqs))
    aux, toks = aux_np(TINY, 12, 40), toks_np(TINY, 12, 40)
    assert dr.status() == 0
    bad = toks[:10].copy()
    bad[4] = TINY.target_vocab + 5
    dr.prefill(0, _tok(bad), to_dev_aux(row_slice(aux, 0, 10)))
    assert dr.status() == B.STATUS_BAD_TOKEN
    assert dr.status() == 0
    for s in S[1:]:
        dr.prefill(s, _tok(toks[:10]), to_dev_aux(row_slice(aux, 0, 10)))
    b_aux = to_dev_aux([np.stack([a[20]] * seqs) for a in aux])
    dr.draft_chain(S, _tok([toks[20]] * seqs), b_aux, 3)
    assert dr.status() == 0
    dr.draft_chain(S, _tok([-3] * seqs), b_aux, 3)
    assert dr.status() == B.STATUS_BAD_TOKEN
    nan_aux = [a.clone() for a in b_aux]
    nan_aux[1][:, 7] = float("nan")
    dr.draft_chain(S, _tok([toks[20]] * seqs), nan_aux, 3)
    assert dr.status() == B.STATUS_NAN_LOGITS
    dr.draft_chain(S, _tok([toks[20]] * seqs), b_aux, 3)
    assert dr.status() == 0
    dr.close()
