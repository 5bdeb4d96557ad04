"""GPU parity of the quantized draft KV (EAGLE3_KV_Q8Q5: q8_0 K rows, q5_1 V rows).

* The quantizers are integer work: fed the same fp32 rows, the library's codes
  equal the oracle's (oracle.kvquant) bit for bit.  Teacher-forced rows and a chain
  step's first row do not depend on the KV format, so a context with fp32 KV
  computes exactly the rows a quantized context quantizes: the quantized context's
  (dequantized) rows must equal oracle.kvquant applied to the fp32 context's rows.
  Covered: the teacher-forced store (passes of <= 16 rows and MFMA passes) and the
  attention block that quantizes a chain step's new row.
* Chain rounds, rebuilds and round-local chains match the oracle run with the same
  quantized KV to the usual bar (ids where the top-2 margin allows, logits,
  hidden states): head_dim 64 and 128 on the MFMA kernel (contexts of one split
  and of many), 256 on the VALU kernel.
"""
import numpy as np
import pytest
import torch

from eagle_draft_head_amd import binding as B
from eagle_draft_head_amd.drafter import Drafter
from oracle import int4, kvquant
from synth import TINY, gen, small_variant
from tests.common import aux_np, make_oracle, toks_np
from tests.gpu_harness import check_round, compare_round, say, to_dev_aux

pytestmark = pytest.mark.gpu

HD128 = small_variant(name="small-hd128", cfg_id=12, n_head=4, n_head_kv=2, head_dim=128, rope_dim=64)
# head_dim 256 attends on the VALU kernel (the MFMA one covers 64 and 128)
HD256 = small_variant(name="small-hd256", cfg_id=13, n_head=4, n_head_kv=2, head_dim=256, rope_dim=64)


def _pair(cfg, max_ctx):
    wd = gen.drafter_weights(cfg, device="cuda")
    f32 = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=max_ctx, kv_dtype=B.KV_F32)
    q = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=max_ctx, kv_dtype=B.KV_Q8Q5)
    return wd, f32, q


def _expect(k32, v32):
    return kvquant.k_stored(k32), kvquant.v_stored(v32)


@pytest.mark.parametrize("cfg", [TINY, HD128, HD256], ids=["hd64", "hd128", "hd256"])
def test_kvq_rows_bit_exact(cfg):
    L = 45  # an MFMA pass (> 16 rows) then a small pass (<= 16 rows)
    say(f"[kvq] {cfg.name}: append rows bit-exact")
    wd, f32, q = _pair(cfg, L + 32)
    aux, toks = aux_np(cfg, 0, L + 1), toks_np(cfg, 0, L + 1)
    for dr in (f32, q):
        dr.prefill(0, torch.as_tensor(toks[:37], dtype=torch.int32).cuda(), to_dev_aux(aux, slice(0, 37)))
        dr.prefill(0, torch.as_tensor(toks[37:L], dtype=torch.int32).cuda(), to_dev_aux(aux, slice(37, L)))
        # one chain step kept: its row L is quantized by the attention kernel
        dr.draft_chain([0], torch.tensor([int(toks[L])], dtype=torch.int32).cuda(),
                       to_dev_aux(aux, slice(L, L + 1)), 1, keep_spec=True)
    torch.cuda.synchronize()
    k32, v32 = f32.kv_read(0, 0, L + 1)
    kq, vq = q.kv_read(0, 0, L + 1)
    torch.cuda.synchronize()
    ek, ev = _expect(k32.cpu().numpy(), v32.cpu().numpy())
    gk, gv = kq.cpu().numpy().astype(np.float64), vq.cpu().numpy().astype(np.float64)
    # K: D * q is exact in fp32; V: fmaf(D, q, M) is D q + M rounded once to fp32
    assert np.array_equal(gk, ek), np.argwhere(gk != ek)[:5]
    assert np.array_equal(gv, ev.astype(np.float32).astype(np.float64)), np.argwhere(gv != ev)[:5]
    f32.close()
    q.close()


def _kv_close(dr, orc, R):
    """Dequantized rows vs the oracle's: equal but for codes decided one step apart
    (the oracle quantizes fp64-computed rows, the GPU rows from fp32-accumulated
    products of the same rounded activations, about 2^-16 relative apart; at 31 V
    levels over a block's span that flips of the order of 0.1-0.3 % of the codes)."""
    k, v = dr.kv_read(0, 0, R)
    torch.cuda.synchronize()
    for gpu, ref, levels in ((k, orc.K[0][:R], 127.0), (v, orc.V[0][:R], 31.0)):
        g = gpu.double().cpu().numpy().reshape(R, -1, 32)
        r = ref.reshape(R, -1, 32)
        span = np.abs(r).max(axis=2) if levels == 127.0 else r.max(axis=2) - r.min(axis=2)
        step = span / levels * (1 + 2.0 ** -9) + 1e-30
        d = np.abs(g - r)
        assert np.all(d <= step[..., None] * 1.01 + 1e-6 * np.abs(r)), d.max()
        off = d > 1e-6 * (np.abs(r) + 1e-6)
        assert off.mean() < 1e-2, off.mean()


@pytest.mark.parametrize("cfg,L,rounds,gamma,local,i4", [(TINY, 63, 24, 3, False, False),
                                                         (HD128, 200, 12, 4, False, False),
                                                         (HD128, 3001, 4, 4, False, False),
                                                         (TINY, 1537, 4, 3, False, False),
                                                         (HD256, 100, 8, 3, False, False),
                                                         (TINY, 63, 8, 4, True, False),
                                                         (TINY, 0, 4, 5, False, False),
                                                         (TINY, 63, 12, 3, False, True)],
                         ids=["tiny", "hd128", "hd128-long", "tiny-long", "hd256", "tiny-round-local", "empty",
                              "tiny-int4-weights"])
def test_kvq_chain_parity(cfg, L, rounds, gamma, local, i4):
    say(f"[kvq] {cfg.name} L={L} rounds={rounds} gamma={gamma} local={local} int4={i4}")
    wd = gen.drafter_weights(cfg, device="cuda")
    max_ctx = L + rounds * (gamma + 1) + 16
    dr = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=max_ctx, kv_dtype=B.KV_Q8Q5,
                 weight_format=B.WEIGHTS_I4 if i4 else B.WEIGHTS_BF16)
    wh = {k: v.cpu() for k, v in wd.items()}
    # the default teacher-forced form: fp16 appends with bf16 weights, split with int4
    orc = make_oracle(cfg, int4.int4_weights(wh) if i4 else wh, max_ctx=max_ctx, kv_format="q8q5",
                      append_act="exact" if i4 else "f16")
    aux, toks = aux_np(cfg, 0, L), toks_np(cfg, 0, L)
    orc.prefill(0, aux, toks)
    dr.prefill(0, torch.as_tensor(toks, dtype=torch.int32).cuda(), to_dev_aux(aux))
    baux, btok = aux_np(cfg, 1, rounds), toks_np(cfg, 1, rounds)
    raux = aux_np(cfg, 2, rounds * (gamma + 1))
    steps = pinned = 0
    for r in range(rounds):
        b_aux = [a[r] for a in baux]
        if local:
            recs = orc.draft_chain_round_local(0, b_aux, btok[r], gamma)
        else:
            recs = orc.draft_chain(0, b_aux, btok[r], gamma)
        out, geff, logits, hidden = dr.draft_chain([0], torch.tensor([int(btok[r])], dtype=torch.int32).cuda(),
                                                   to_dev_aux(baux, slice(r, r + 1)), gamma, debug=True,
                                                   round_local=local)
        torch.cuda.synchronize()
        cmp = compare_round(recs, out, geff[0], logits, hidden)
        check_round(cmp, f"kvq round {r}")
        steps += len(cmp)
        for c in cmp:
            if not c.pinned:
                break
            pinned += 1
        if local:
            continue
        a = r % (geff[0] + 1)
        rows = slice(r * (gamma + 1), r * (gamma + 1) + a)
        new_aux = [np.concatenate([ba[r:r + 1], ra[rows]]) for ba, ra in zip(baux, raux)]
        new_tok = np.array([btok[r]] + [x.target_id for x in recs[:a]], dtype=np.int32)
        orc.rebuild_after_verify(0, a, new_aux, new_tok)
        dr.rebuild_after_verify([0], [a], torch.as_tensor(new_tok).cuda(), to_dev_aux(new_aux))
        assert dr.kv_len(0) == (orc.ledger.committed(0), 0)
    say(f"[kvq] {cfg.name}: {pinned}/{steps} steps pinned")
    assert pinned >= max(1, rounds // 2)
    R = orc.ledger.committed(0)
    if R:
        _kv_close(dr, orc, R)
    dr.close()


@pytest.mark.parametrize("cfg,max_ctx", [(TINY, 95), (TINY, 90), (HD128, 127), (HD128, 121)],
                         ids=["hd64-cap96", "hd64-cap96-slack", "hd128-cap128", "hd128-cap128-slack"])
def test_kvq_chain_to_capacity(cfg, max_ctx):
    """The MFMA q8q5 attention reads whole 16-row tiles, past T up to the region's
    row count (max_ctx + 1 rounded up to 16, zeroed at load): chains and rebuilds
    that fill the cache to its last row (the tile past T then ends exactly at the
    region's end, or inside the rounding slack) match the oracle round by round,
    down to gamma_eff 0."""
    say(f"[kvq] {cfg.name} chains to capacity, max_ctx={max_ctx}")
    gamma = 4
    wd = gen.drafter_weights(cfg, device="cuda")
    dr = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=max_ctx, kv_dtype=B.KV_Q8Q5)
    wh = {k: v.cpu() for k, v in wd.items()}
    orc = make_oracle(cfg, wh, max_ctx=max_ctx, kv_format="q8q5", append_act="f16")
    L = max_ctx - 12
    aux, toks = aux_np(cfg, 0, L), toks_np(cfg, 0, L)
    orc.prefill(0, aux, toks)
    dr.prefill(0, torch.as_tensor(toks, dtype=torch.int32).cuda(), to_dev_aux(aux))
    rounds = 12
    baux, btok = aux_np(cfg, 1, rounds), toks_np(cfg, 1, rounds)
    raux = aux_np(cfg, 2, rounds * (gamma + 1))
    seen_full = False
    for r in range(rounds):
        b_aux = [a[r] for a in baux]
        recs = orc.draft_chain(0, b_aux, btok[r], gamma)
        out, geff, logits, hidden = dr.draft_chain([0], torch.tensor([int(btok[r])], dtype=torch.int32).cuda(),
                                                   to_dev_aux(baux, slice(r, r + 1)), gamma, debug=True)
        torch.cuda.synchronize()
        g = int(geff[0])
        assert g == len(recs), (g, len(recs))
        if g == 0:
            seen_full = True
            assert out[0].eq(-1).all()
            break
        check_round(compare_round(recs, out, g, logits, hidden), f"kvq capacity round {r}")
        committed = orc.ledger.committed(0)
        a = min(r % (g + 1), max_ctx - committed - 1)
        if a < 0:
            break
        rows = slice(r * (gamma + 1), r * (gamma + 1) + a)
        new_aux = [np.concatenate([ba[r:r + 1], ra[rows]]) for ba, ra in zip(baux, raux)]
        new_tok = np.array([btok[r]] + [x.target_id for x in recs[:a]], dtype=np.int32)
        orc.rebuild_after_verify(0, a, new_aux, new_tok)
        dr.rebuild_after_verify([0], [a], torch.as_tensor(new_tok).cuda(), to_dev_aux(new_aux))
        assert dr.kv_len(0) == (orc.ledger.committed(0), 0)
    assert seen_full or orc.ledger.committed(0) >= max_ctx - gamma
    _kv_close(dr, orc, orc.ledger.committed(0))
    dr.close()
