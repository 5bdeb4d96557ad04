"""GPU parity of batched drafting: one draft_chain call over many sequences of
ragged committed lengths (every projection streams its weights once for all
sequences still drafting), against the oracle run sequence by sequence.

Covered: ragged lengths including an empty cache and sequences at the capacity
edge (admitted chains shorter than gamma, or zero), more sequences than one
pass holds, packed rebuilds between rounds, and the full-size batched workload
(32 Qwen3-8B-shaped sequences of 512..8192 committed rows) on sampled sequences."""
import numpy as np
import pytest
import torch

from synth import BATCHED, TINY, gen, small_variant
from tests.common import aux_np, make_oracle, row_slice, toks_np
from tests.gpu_harness import check_round, compare_round, gpu_drafter, say, to_dev_aux, weights_both

pytestmark = pytest.mark.gpu


def _tok(x):
    return torch.as_tensor(np.asarray(x), dtype=torch.int32).reshape(-1).cuda()


def _rounds(cfg, lens, gamma, rounds, max_ctx, seed, min_pinned=None, kv_bf16=False,
            stored=False):
    """stored: the boundary features come from the prefills and the packed rebuilds
    (given the next round's boundary taps) and every chain starts from them."""
    say(f"[batched] {cfg.name}: {len(lens)} sequences, gamma={gamma}, rounds={rounds}, "
        f"{'bf16' if kv_bf16 else 'fp32'} KV, stored={stored}")
    wd, wh = weights_both(cfg)
    S = len(lens)
    if kv_bf16:
        from eagle_draft_head_amd import binding as B
        from eagle_draft_head_amd.drafter import Drafter
        dr = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx, max_seqs=S, kv_dtype=B.KV_BF16)
    else:
        dr = gpu_drafter(cfg, wd, max_ctx=max_ctx, max_seqs=S)
    orc = make_oracle(cfg, wh, max_ctx=max_ctx, max_seqs=S, kv_format="bf16" if kv_bf16 else "exact")
    total = sum(lens)
    aux, toks = aux_np(cfg, 30, max(total, 1)), toks_np(cfg, 30, max(total, 1))
    r0 = 0
    b0 = aux_np(cfg, 40, S)
    for s, L in enumerate(lens):
        nxt = to_dev_aux(b0, slice(s, s + 1)) if stored else None
        if L:
            orc.prefill(s, row_slice(aux, r0, r0 + L), toks[r0:r0 + L])
            dr.prefill(s, _tok(toks[r0:r0 + L]), to_dev_aux(row_slice(aux, r0, r0 + L)), next_aux=nxt)
        elif stored:
            dr.prefill(s, _tok([]), [], next_aux=nxt)
        r0 += L
    rng = np.random.default_rng(seed)
    steps = pinned = 0
    for rd in range(rounds):
        baux, btok = aux_np(cfg, 40 + rd, S), toks_np(cfg, 40 + rd, S)
        out, geff, logits, hidden = dr.draft_chain(list(range(S)), _tok(btok),
                                                   None if stored else to_dev_aux(baux),
                                                   gamma, debug=True)
        torch.cuda.synchronize()
        drafts = []
        for s in range(S):
            recs = orc.draft_chain(s, [a[s] for a in baux], btok[s], gamma)
            assert geff[s] == len(recs), (s, geff[s], len(recs))
            assert out[s, len(recs):].tolist() == [-1] * (gamma - len(recs))
            cmp = compare_round(recs, out, geff[s], logits, hidden, b=s)
            # the bf16 draft-KV option is held to the same bar against the oracle's
            # bf16 KV storage
            check_round(cmp, f"{cfg.name} round {rd} seq {s} (L={orc.ledger.committed(s)})")
            steps += len(cmp)
            for c in cmp:
                if not c.pinned:
                    break
                pinned += 1
            drafts.append([r.target_id for r in recs])
        # packed rebuild of every sequence that drafted, the oracle's drafts as the
        # verified tokens
        live = [s for s in range(S) if geff[s] > 0]
        acc = [int(rng.integers(0, geff[s] + 1)) for s in live]
        raux = aux_np(cfg, 60 + rd, sum(acc) + len(live))
        tok_rows, aux_rows, q = [], [[], [], []], 0
        for s, a in zip(live, acc):
            rows_s = [np.concatenate([baux[j][s:s + 1], raux[j][q:q + a]]) for j in range(3)]
            toks_s = [int(btok[s])] + drafts[s][:a]
            orc.rebuild_after_verify(s, a, rows_s, np.array(toks_s))
            tok_rows += toks_s
            for j in range(3):
                aux_rows[j].append(rows_s[j])
            q += a
        if live:
            nxt = None
            if stored:  # the next round's boundary taps of the rebuilt sequences
                nb = aux_np(cfg, 40 + rd + 1, S)
                nxt = to_dev_aux([x[live] for x in nb])
            dr.rebuild_after_verify(live, acc, _tok(tok_rows),
                                    to_dev_aux([np.concatenate(x) for x in aux_rows]), next_aux=nxt)
        # (a sequence that drafted nothing is not rebuilt and keeps an older stored
        # feature; its committed length does not change, so it never drafts again)
        for s in range(S):
            assert dr.kv_len(s) == (orc.ledger.committed(s), 0)
    say(f"[batched] {cfg.name}: {pinned}/{steps} steps pinned")
    # enough steps have a clear top-1 to make the comparison meaningful
    assert pinned >= (steps // 3 if min_pinned is None else min_pinned)
    dr.close()


def test_batched_ragged_lengths_and_capacity_edge():
    cfg = small_variant()
    # an empty cache, ragged lengths, and sequences 3, 1 and 0 rows short of max_ctx
    _rounds(cfg, [0, 1, 37, 130, 300, 511, 640, 697, 699, 700], gamma=4, rounds=3, max_ctx=700,
            seed=5)


def test_batched_more_sequences_than_one_pass():
    _rounds(TINY, [int(x) for x in gen.lengths(TINY, 7, 35, 1, 120)], gamma=3, rounds=2,
            max_ctx=160, seed=6)


def test_batched_round_local():
    """Round-local batched chains (each sequence attends over its own round only):
    ragged committed lengths, sequences at the capacity edge draft the full gamma,
    and the committed rows and lengths are untouched."""
    cfg = small_variant()
    lens = [0, 1, 37, 300, 699, 700]
    S, gamma, max_ctx = len(lens), 5, 700
    wd, wh = weights_both(cfg)
    dr = gpu_drafter(cfg, wd, max_ctx=max_ctx, max_seqs=S)
    orc = make_oracle(cfg, wh, max_ctx=max_ctx, max_seqs=S)
    aux, toks = aux_np(cfg, 30, sum(lens)), toks_np(cfg, 30, sum(lens))
    r0 = 0
    for s, L in enumerate(lens):
        if L:
            orc.prefill(s, row_slice(aux, r0, r0 + L), toks[r0:r0 + L])
            dr.prefill(s, _tok(toks[r0:r0 + L]), to_dev_aux(row_slice(aux, r0, r0 + L)))
        r0 += L
    kv0 = {s: [t.clone() for t in dr.kv_read(s, 0, L)] for s, L in enumerate(lens) if L}
    for rd in range(3):
        baux, btok = aux_np(cfg, 40 + rd, S), toks_np(cfg, 40 + rd, S)
        out, geff, logits, hidden = dr.draft_chain(list(range(S)), _tok(btok), to_dev_aux(baux), gamma,
                                                   debug=True, round_local=True)
        torch.cuda.synchronize()
        assert geff == [gamma] * S
        for s in range(S):
            recs = orc.draft_chain_round_local(s, [a[s] for a in baux], btok[s], gamma)
            check_round(compare_round(recs, out, geff[s], logits, hidden, b=s),
                        f"round-local round {rd} seq {s}")
            assert dr.kv_len(s) == (lens[s], 0)
    for s, (k0, v0) in kv0.items():
        k1, v1 = dr.kv_read(s, 0, lens[s])
        assert torch.equal(k0, k1) and torch.equal(v0, v1)
    dr.close()


def test_batched_stored_boundaries():
    """Boundary features from prefill (one of them a boundary-only prefill of an
    empty cache) and from packed rebuilds: 35 sequences, so the rebuild's boundary
    rows span two passes of at most 32."""
    _rounds(TINY, [0] + [int(x) for x in gen.lengths(TINY, 8, 34, 1, 120)], gamma=3, rounds=3,
            max_ctx=160, seed=7, stored=True)
    _rounds(small_variant(), [0, 1, 37, 130, 300, 511], gamma=4, rounds=3, max_ctx=700, seed=8,
            stored=True)


def test_batched_wide_heads_partial_rope():
    """The page-4 head geometry at a small width: 256-wide heads, 64 of 256 dims
    rotated, four query heads per KV head."""
    cfg = small_variant("small-hd256", n_head=4, n_head_kv=1, head_dim=256, rope_dim=64)
    _rounds(cfg, [5, 77, 130, 281, 296], gamma=3, rounds=2, max_ctx=300, seed=8)


def test_batched_bf16_kv_option():
    _rounds(small_variant(), [12, 200, 333, 650], gamma=4, rounds=2, max_ctx=700, seed=9,
            kv_bf16=True)


def test_batched_two_sequences():
    _rounds(TINY, [50, 3], gamma=6, rounds=4, max_ctx=100, seed=7, min_pinned=4)


def test_batched_full_size_sampled():
    """32 sequences at the full drafter size with L_b in [512, 8192] and two at the
    capacity edge; the oracle follows eight of them, the rest are checked for
    valid ids and exact lengths (the edge pair, the shortest, the longest below the
    edge and four more are followed)."""
    cfg = BATCHED
    lens = gen.batch_lengths(cfg)
    S, gamma = len(lens), cfg.gamma
    sample = sorted({0, 1, int(np.argmin(lens)), int(np.argmax(lens[2:])) + 2, 5, 11, 19, 26})
    say(f"[batched-full] generating weights; lengths {lens}")
    wd = gen.drafter_weights(cfg, device="cuda")
    wh = {k: v.cpu() for k, v in wd.items() if k != "embed"}
    dr = gpu_drafter(cfg, wd, max_ctx=cfg.max_ctx, max_seqs=S)
    del wd
    torch.cuda.empty_cache()
    orc = make_oracle(cfg, wh, max_ctx=cfg.max_ctx, max_seqs=S, lazy_embed=True)
    for s, L in enumerate(lens):
        aux = gen.aux_taps(cfg, 100 + s, L, device="cuda")
        tok = gen.tokens(cfg, 100 + s, L, device="cuda")
        dr.prefill(s, tok, aux)
        if s in sample:
            say(f"[batched-full] oracle prefill of sequence {s} ({L} rows)")
            orc.prefill(s, [a.double().cpu().numpy() for a in aux], tok.cpu().numpy())
        else:
            orc.ledger.prefill(s, L)
        del aux, tok
    d2t = gen.d2t(cfg).numpy()
    image = set((np.arange(cfg.draft_vocab) + d2t).tolist())
    for rd, forced in enumerate([4, None]):
        b_aux = gen.aux_taps(cfg, 300 + rd, S, device="cuda")
        b_tok = gen.tokens(cfg, 300 + rd, S, device="cuda")
        out, geff, logits, hidden = dr.draft_chain(list(range(S)), b_tok, b_aux, gamma, debug=True)
        torch.cuda.synchronize()
        verified = {}  # tokens committed by the rebuild: the oracle's drafts, else seeded ids
        filler = gen.tokens(cfg, 500 + rd, S * gamma).view(S, gamma).tolist()
        for s in range(S):
            want = orc.ledger.chain(s, gamma) if s not in sample else None
            if s in sample:
                recs = orc.draft_chain(s, [a[s].double().cpu().numpy() for a in b_aux],
                                       int(b_tok[s]), gamma)
                cmp = compare_round(recs, out, geff[s], logits, hidden, b=s)
                check_round(cmp, f"batched32 round {rd} seq {s}")
                verified[s] = [r.target_id for r in recs]
                say(f"[batched-full] round {rd} seq {s}: ids {out[s].tolist()} oracle "
                    f"{[r.target_id for r in recs]} max logit err "
                    f"{max([c.logit_err for c in cmp] or [0]):.2e}")
            else:
                assert geff[s] == want
                ids = out[s].tolist()
                assert all(i in image for i in ids[:geff[s]]) and ids[geff[s]:] == [-1] * (gamma - geff[s])
                verified[s] = filler[s]
        # rebuild: sequences 0 and 1 accept everything in the first round (the edge:
        # their next admitted chain is empty), the others a seeded count
        rng = np.random.default_rng(11 + rd)
        live = [s for s in range(S) if geff[s] > 0]
        acc = [geff[s] if (forced is not None and s < 2) else int(rng.integers(0, geff[s] + 1))
               for s in live]
        r_aux = gen.aux_taps(cfg, 400 + rd, sum(acc), device="cuda")
        tok_rows, aux_rows, q = [], [[], [], []], 0
        for s, a in zip(live, acc):
            toks_s = [int(b_tok[s])] + verified[s][:a]
            rows_s = [torch.cat([b_aux[j][s:s + 1], r_aux[j][q:q + a]]) for j in range(3)]
            if s in sample:
                orc.rebuild_after_verify(s, a, [x.double().cpu().numpy() for x in rows_s],
                                         np.array(toks_s))
            else:
                orc.ledger.rebuild(s, a)
            tok_rows += toks_s
            for j in range(3):
                aux_rows[j].append(rows_s[j])
            q += a
        dr.rebuild_after_verify(live, acc, _tok(tok_rows), [torch.cat(x).contiguous() for x in aux_rows])
        for s in range(S):
            assert dr.kv_len(s) == (orc.ledger.committed(s), 0)
    # the edge sequences are full: no chain is admitted for them
    assert orc.ledger.committed(0) == cfg.max_ctx + 1 and geff[0] == 0 and geff[1] == 0
    dr.close()
