"""GPU parity of the int4 weight mode (EAGLE3_WEIGHTS_I4): the codes and scales the
library makes at load equal the oracle's bit for bit (integer work), and chain
rounds, prefill and rebuilds (passes of at most 16 rows) match the oracle built on
the same int4 weights, on the tiny shape and at the full Qwen3-8B shape."""
import numpy as np
import pytest
import torch

from eagle_draft_head_amd import binding as B
from eagle_draft_head_amd.drafter import Drafter
from oracle import int4
from synth import QWEN3_8B, TINY, gen
from tests.common import aux_np, make_oracle, row_slice, toks_np
from tests.gpu_harness import check_round, compare_round, say, to_dev_aux

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _read(dr, name, rows, K):
    codes = torch.empty(rows * K // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows * K // 32, dtype=torch.int16, device="cuda")
    B.eagle3_weights_i4_read(dr.ctx, name, codes, scales)
    torch.cuda.synchronize()
    return (codes.cpu().numpy().reshape(rows, K // 2),
            scales.cpu().numpy().view(np.uint16).reshape(rows, K // 32))


def _expect(bits):
    q, s = int4.quantize(bits)
    return int4.pack(q), s


def _rope_rows(heads, hd, rot):
    """Source row of each stored q/k row: rotary partners (i, i + rot / 2) adjacent."""
    src = []
    for h in range(heads):
        for p in range(hd):
            src.append(h * hd + (p if p >= rot else (p // 2 + (rot // 2 if p % 2 else 0))))
    return np.array(src)


def test_int4_codes_and_scales_bit_exact():
    cfg = TINY
    wd = gen.drafter_weights(cfg, device="cuda")
    dr = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=128, weight_format=B.WEIGHTS_I4)
    n, ff, qd, kvd = cfg.n_embd, cfg.n_ff, cfg.q_dim, cfg.kv_dim
    for name, key, rows, K in (("fc", "fc", n, 3 * n), ("o_proj", "o_proj", n, qd),
                               ("down_proj", "down_proj", n, ff), ("lm_head", "lm_head", cfg.draft_vocab, n)):
        got = _read(dr, name, rows, K)
        exp = _expect(_bits(wd[key]))
        assert np.array_equal(got[0], exp[0]) and np.array_equal(got[1], exp[1]), name
    gq, gs = _read(dr, "gate_up", 2 * ff, n)
    eg, es = _expect(_bits(wd["gate_proj"]))
    uq, us = _expect(_bits(wd["up_proj"]))
    assert np.array_equal(gq[0::2], eg) and np.array_equal(gq[1::2], uq)
    assert np.array_equal(gs[0::2], es) and np.array_equal(gs[1::2], us)
    qq, qs = _read(dr, "qkv", qd + 2 * kvd, 2 * n)
    for part, rows, key in ((slice(0, qd), _rope_rows(cfg.n_head, cfg.head_dim, cfg.rope_dim), "q_proj"),
                            (slice(qd, qd + kvd), _rope_rows(cfg.n_head_kv, cfg.head_dim, cfg.rope_dim), "k_proj"),
                            (slice(qd + kvd, qd + 2 * kvd), np.arange(kvd), "v_proj")):
        eq, es = _expect(_bits(wd[key])[rows])
        assert np.array_equal(qq[part], eq) and np.array_equal(qs[part], es), key
    dr.close()


@pytest.mark.parametrize("L,rounds,gamma,table", [(63, 40, 3, B.TABLE_DEFAULT), (0, 5, 5, B.TABLE_DEFAULT),
                                                  (63, 20, 3, B.TABLE_OFF)],
                         ids=["table", "empty-table", "streamed"])
def test_int4_chain_parity_tiny(L, rounds, gamma, table):
    """The default keeps the QKV embedding half in the token table (built from the
    int4 weights' exact values); TABLE_OFF streams both halves' codes."""
    cfg = TINY
    say(f"[int4] tiny L={L} rounds={rounds} gamma={gamma} table={table}")
    wd = gen.drafter_weights(cfg, device="cuda")
    wh = int4.int4_weights({k: v.cpu() for k, v in wd.items()})
    max_ctx = L + rounds * (gamma + 1) + 16
    dr = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=max_ctx, weight_format=B.WEIGHTS_I4, token_table=table)
    orc = make_oracle(cfg, wh, max_ctx=max_ctx)
    aux, toks = aux_np(cfg, 0, L), toks_np(cfg, 0, L)
    orc.prefill(0, aux, toks)
    baux, btok = aux_np(cfg, 1, rounds + 1), toks_np(cfg, 1, rounds)
    raux = aux_np(cfg, 2, rounds * (gamma + 1))
    dr.prefill(0, torch.as_tensor(toks, dtype=torch.int32).cuda(), to_dev_aux(aux),
               next_aux=to_dev_aux(baux, slice(0, 1)))
    steps = pinned = 0
    for r in range(rounds):
        recs = orc.draft_chain(0, [a[r] for a in baux], btok[r], gamma)
        out, geff, logits, hidden = dr.draft_chain([0], torch.tensor([int(btok[r])], dtype=torch.int32).cuda(),
                                                   None, gamma, debug=True)
        torch.cuda.synchronize()
        cmp = compare_round(recs, out, geff[0], logits, hidden)
        check_round(cmp, f"int4 round {r}")
        steps += len(cmp)
        for c in cmp:
            if not c.pinned:
                break
            pinned += 1
        a = r % (geff[0] + 1)
        rows = slice(r * (gamma + 1), r * (gamma + 1) + a)
        new_aux = [np.concatenate([ba[r:r + 1], ra[rows]]) for ba, ra in zip(baux, raux)]
        new_tok = np.array([btok[r]] + [x.target_id for x in recs[:a]], dtype=np.int32)
        orc.rebuild_after_verify(0, a, new_aux, new_tok)
        dr.rebuild_after_verify([0], [a], torch.as_tensor(new_tok).cuda(), to_dev_aux(new_aux),
                                next_aux=to_dev_aux(baux, slice(r + 1, r + 2)))
        assert dr.kv_len(0) == (orc.ledger.committed(0), 0)
    say(f"[int4] tiny: {pinned}/{steps} steps pinned")
    assert pinned >= max(1, rounds // 2)
    k, v = dr.kv_read(0, 0, orc.ledger.committed(0))
    for gpu, ref in ((k, orc.K[0]), (v, orc.V[0])):
        g = gpu.double().cpu().numpy()
        R = g.shape[0]
        rel = np.linalg.norm((g - ref[:R]).reshape(R, -1), axis=1) / np.linalg.norm(ref[:R].reshape(R, -1), axis=1)
        assert rel.max() < 1e-2, rel.max()
    dr.close()


def test_int4_qwen3_8b_shape():
    cfg = QWEN3_8B
    L = cfg.context
    say("[int4] qwen3-8b: weights and quantization")
    wd = gen.drafter_weights(cfg, device="cuda")
    wh = int4.int4_weights({k: v.cpu() for k, v in wd.items() if k != "embed"})
    dr = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=L + 64, weight_format=B.WEIGHTS_I4)
    del wd
    torch.cuda.empty_cache()
    orc = make_oracle(cfg, wh, max_ctx=L + 64, lazy_embed=True)
    aux = gen.aux_taps(cfg, 0, L, device="cuda")
    tok = gen.tokens(cfg, 0, L, device="cuda")
    dr.prefill(0, tok, aux)
    say("[int4] qwen3-8b: oracle prefill")
    orc.prefill(0, [a.double().cpu().numpy() for a in aux], tok.cpu().numpy())
    steps = pinned = 0
    for r in range(4):
        b_aux = gen.aux_taps(cfg, 101 + r, 1, device="cuda")
        b_tok = gen.tokens(cfg, 101 + r, 1, device="cuda")
        recs = orc.draft_chain(0, [a[0].double().cpu().numpy() for a in b_aux], int(b_tok[0]), 3)
        out, geff, logits, hidden = dr.draft_chain([0], b_tok, b_aux, 3, debug=True)
        torch.cuda.synchronize()
        cmp = compare_round(recs, out, geff[0], logits, hidden)
        check_round(cmp, f"int4 qwen3-8b round {r}")
        steps += len(cmp)
        for c in cmp:
            if not c.pinned:
                break
            pinned += 1
        say(f"[int4] qwen3-8b round {r}: ids {out[0].tolist()} margins {[round(x.margin, 3) for x in recs]}")
    assert pinned >= steps // 3
    dr.close()
