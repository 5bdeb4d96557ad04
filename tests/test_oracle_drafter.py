"""Pins of the oracle drafter: structure checks, cached-vs-stateless,
rewind bit-identity, prefill chunking, rebuild after match/mismatch, the
capacity edge and the shapes the pages print."""
import numpy as np
import pytest
import torch

from oracle import DrafterOracle, LedgerError, StatelessChain
from synth import PAGE4, QWEN3_8B, TINY, gen, small_variant
from tests.common import aux_np, make_oracle, row_slice, toks_np

TOL = dict(rtol=1e-10, atol=1e-12)


@pytest.fixture(scope="module")
def tiny_w():
    return gen.drafter_weights(TINY)


def test_encode_concat_order_and_orientation(tiny_w):
    d = make_oracle(TINY, tiny_w)
    n = TINY.n_embd
    a = np.random.default_rng(0).normal(size=n)
    z = np.zeros(n)
    fc = d.W["fc"]
    assert np.allclose(d.encode([a, z, z]), fc[:, :n] @ a, **TOL)
    assert np.allclose(d.encode([z, a, z]), fc[:, n:2 * n] @ a, **TOL)
    assert np.allclose(d.encode([z, z, a]), fc[:, 2 * n:] @ a, **TOL)


def test_d2t_is_a_delta_onto_the_seeded_subset(tiny_w):
    d = make_oracle(TINY, tiny_w)
    sub = gen.sorted_subset(TINY.cfg_id, gen.TID["d2t"], TINY.target_vocab, TINY.draft_vocab)
    image = [d.d2t_map(i) for i in range(TINY.draft_vocab)]
    assert image == sub.tolist()
    assert d.d2t_map(5) == 5 + int(tiny_w["d2t"][5])


def test_one_row_layer_equals_cached_step(tiny_w):
    d = make_oracle(TINY, tiny_w)
    g = np.random.default_rng(1).normal(size=TINY.n_embd)
    lg, gs = d.layer_full(g[None], [17])
    r = d.step(g, 17, 0, np.zeros((0, 2, 64)), np.zeros((0, 2, 64)))
    assert np.allclose(lg[0], r.logits, **TOL) and np.allclose(gs[0], r.gsum, **TOL)


def _zeroed(w, names):
    w = dict(w)
    for k in names:
        w[k] = torch.zeros_like(w[k])
    return w


def test_residual_is_the_prenorm_hidden(tiny_w):
    # With o_proj and down zeroed the layer adds nothing: g_next == g exactly.
    d = make_oracle(TINY, _zeroed(tiny_w, ["o_proj", "down_proj"]))
    g = np.random.default_rng(2).normal(size=TINY.n_embd) * 3.0
    r = d.step(g, 5, 0, np.zeros((0, 2, 64)), np.zeros((0, 2, 64)))
    assert np.array_equal(r.gsum, g)


def test_attention_feeds_o_proj_and_mlp_feeds_down(tiny_w):
    # zeroing v makes the attention contribution vanish: x1 = g, so the
    # result equals the one with o_proj zeroed
    d1 = make_oracle(TINY, _zeroed(tiny_w, ["v_proj"]))
    d2 = make_oracle(TINY, _zeroed(tiny_w, ["o_proj"]))
    g = np.random.default_rng(3).normal(size=TINY.n_embd)
    r1 = d1.step(g, 9, 0, np.zeros((0, 2, 64)), np.zeros((0, 2, 64)))
    r2 = d2.step(g, 9, 0, np.zeros((0, 2, 64)), np.zeros((0, 2, 64)))
    assert np.allclose(r1.gsum, r2.gsum, **TOL)
    # zeroing up kills the MLP: gsum = x1
    d3 = make_oracle(TINY, _zeroed(tiny_w, ["up_proj", "o_proj"]))
    r3 = d3.step(g, 9, 0, np.zeros((0, 2, 64)), np.zeros((0, 2, 64)))
    assert np.array_equal(r3.gsum, g)


@pytest.mark.parametrize("cfg,L,gamma,rounds", [(TINY, 63, 3, 6), (TINY, 1, 5, 2),
                                                (TINY, 0, 3, 1),
                                                (small_variant(), 40, 4, 2)])
def test_cached_chain_equals_stateless_recompute(cfg, L, gamma, rounds):
    d = make_oracle(cfg)
    aux = aux_np(cfg, 0, L + rounds)
    toks = toks_np(cfg, 0, L + rounds)
    d.prefill(0, row_slice(aux, 0, L), toks[:L])
    sc = StatelessChain(d)
    for r in range(rounds):
        b_aux = [a[L + r] for a in aux]
        recs = d.draft_chain(0, b_aux, toks[L + r], gamma)
        ref = sc.run(row_slice(aux, 0, L), toks[:L], b_aux, toks[L + r], gamma)
        assert [x.target_id for x in recs] == [x.target_id for x in ref]
        for a, b in zip(recs, ref):
            assert np.allclose(a.logits, b.logits, **TOL)
            assert np.allclose(a.gsum, b.gsum, **TOL)
            assert a.position == b.position


@pytest.mark.parametrize("cfg,L,gamma", [(TINY, 63, 3), (TINY, 0, 5), (small_variant(), 40, 4)])
def test_round_local_chain_equals_recompute_over_its_own_rows(cfg, L, gamma):
    """The scratch-KV drafter: each step is the full layer recomputed over the
    round's rows only, placed at positions L, L + 1, ..."""
    d = make_oracle(cfg)
    aux, toks = aux_np(cfg, 0, L + 1), toks_np(cfg, 0, L + 1)
    d.prefill(0, row_slice(aux, 0, L), toks[:L])
    K0, V0 = d.K[0][:L].copy(), d.V[0][:L].copy()
    b_aux = [a[L] for a in aux]
    recs = d.draft_chain_round_local(0, b_aux, toks[L], gamma)
    ref = StatelessChain(d).run(row_slice(aux, 0, 0), toks[:0], b_aux, toks[L], gamma, position0=L)
    assert len(recs) == gamma
    assert [x.target_id for x in recs] == [x.target_id for x in ref]
    for a, b in zip(recs, ref):
        assert np.allclose(a.logits, b.logits, **TOL)
        assert np.allclose(a.gsum, b.gsum, **TOL)
        assert a.position == b.position
    # the persistent rows and the lengths are untouched
    assert d.ledger.committed(0) == L and d.ledger.spec(0) == 0
    assert np.array_equal(d.K[0][:L], K0) and np.array_equal(d.V[0][:L], V0)


def test_round_local_chain_depends_on_relative_positions_only(tiny_w):
    """Rotary attention sees only position differences: the round-local chain at
    L equals the persistent chain of an empty cache (positions from 0)."""
    d = make_oracle(TINY, tiny_w, max_seqs=2)
    L = 50
    aux, toks = aux_np(TINY, 2, L + 1), toks_np(TINY, 2, L + 1)
    d.prefill(0, row_slice(aux, 0, L), toks[:L])
    b_aux = [a[L] for a in aux]
    loc = d.draft_chain_round_local(0, b_aux, toks[L], 4)
    emp = d.draft_chain(1, b_aux, toks[L], 4)
    assert [x.target_id for x in loc] == [x.target_id for x in emp]
    for a, b in zip(loc, emp):
        assert np.allclose(a.logits, b.logits, rtol=1e-9, atol=1e-11)
        assert a.position == b.position + L


def test_chain_round_leaves_kv_bit_identical(tiny_w):
    d = make_oracle(TINY, tiny_w)
    L = 63
    aux, toks = aux_np(TINY, 0, L + 1), toks_np(TINY, 0, L + 1)
    d.prefill(0, row_slice(aux, 0, L), toks[:L])
    K0, V0 = d.K[0][:L].copy(), d.V[0][:L].copy()
    recs = d.draft_chain(0, [a[L] for a in aux], toks[L], 3)
    assert len(recs) == 3
    assert d.ledger.committed(0) == L and d.ledger.spec(0) == 0
    assert np.array_equal(d.K[0][:L], K0) and np.array_equal(d.V[0][:L], V0)
    # and the round is repeatable: same drafts again
    recs2 = d.draft_chain(0, [a[L] for a in aux], toks[L], 3)
    assert [r.target_id for r in recs] == [r.target_id for r in recs2]


def test_prefill_chunked_equals_one_shot(tiny_w):
    L = 63
    aux, toks = aux_np(TINY, 0, L), toks_np(TINY, 0, L)
    d1 = make_oracle(TINY, tiny_w)
    d1.prefill(0, aux, toks)
    d2 = make_oracle(TINY, tiny_w)
    for c0 in range(0, L, 16):
        d2.prefill(0, row_slice(aux, c0, min(L, c0 + 16)), toks[c0:min(L, c0 + 16)])
    assert d1.ledger.committed(0) == d2.ledger.committed(0) == L
    assert np.allclose(d1.K[0][:L], d2.K[0][:L], rtol=1e-13, atol=1e-14)
    assert np.allclose(d1.V[0][:L], d2.V[0][:L], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("accept", [0, 1, 3])
def test_rebuild_after_verify_matches_stateless(tiny_w, accept):
    """Rebuild after a mismatch (a < gamma) and a full match (a = gamma): the
    next chain equals a from-scratch recompute over the extended rows."""
    d = make_oracle(TINY, tiny_w)
    L, gamma = 40, 3
    aux, toks = aux_np(TINY, 1, L + 10), toks_np(TINY, 1, L + 10)
    d.prefill(0, row_slice(aux, 0, L), toks[:L])
    b_aux, b_tok = [a[L] for a in aux], int(toks[L])
    recs = d.draft_chain(0, b_aux, b_tok, gamma)
    drafts = [r.target_id for r in recs]
    # committed rows: (boundary aux, boundary tok), (fresh aux, d_i) for i <= a
    new_aux = [np.concatenate([a[L:L + 1], a[L + 1:L + 1 + accept]]) for a in aux]
    new_tok = np.array([b_tok] + drafts[:accept], dtype=np.int64)
    d.rebuild_after_verify(0, accept, new_aux, new_tok)
    assert d.ledger.committed(0) == L + accept + 1
    all_aux = [np.concatenate([a[:L], na]) for a, na in zip(aux, new_aux)]
    all_tok = np.concatenate([toks[:L], new_tok])
    nb_aux, nb_tok = [a[L + 5] for a in aux], int(toks[L + 5])
    recs2 = d.draft_chain(0, nb_aux, nb_tok, gamma)
    ref = StatelessChain(d).run(all_aux, all_tok, nb_aux, nb_tok, gamma)
    assert [r.target_id for r in recs2] == [r.target_id for r in ref]
    for a, b in zip(recs2, ref):
        assert np.allclose(a.logits, b.logits, **TOL)


def test_capacity_edge_97_3_100(tiny_w):
    """PR #707 review: start=97, k=3, max=100 — full acceptance commits k+1 rows."""
    d = make_oracle(TINY, tiny_w, max_ctx=100)
    assert d.ledger.rows == 101
    aux, toks = aux_np(TINY, 2, 110), toks_np(TINY, 2, 110)
    d.prefill(0, row_slice(aux, 0, 97), toks[:97])
    sentinel = 1e300
    d.K[0][98:] = sentinel   # rows the chain may write: 97..99; row 100 = reserve
    recs = d.draft_chain(0, [a[97] for a in aux], toks[97], 3)
    assert len(recs) == 3
    assert np.all(d.K[0][100] == sentinel)          # the chain never touches the reserve
    drafts = [r.target_id for r in recs]
    d.rebuild_after_verify(0, 3, row_slice(aux, 97, 101),
                           np.array([toks[97]] + drafts))
    assert d.ledger.committed(0) == 101
    assert np.all(np.abs(d.K[0][97:101]) < 1e6)      # 4 rows written, 97..100
    assert d.ledger.admit_chain(0, 3) == 0           # next round cannot speculate
    assert d.draft_chain(0, [a[101] for a in aux], toks[101], 3) == []
    with pytest.raises(LedgerError):
        d.rebuild_after_verify(0, 0, row_slice(aux, 101, 102), toks[101:102])


def test_shape_asserts(tiny_w):
    bad = dict(tiny_w)
    bad["fc"] = tiny_w["fc"][:, :512]
    with pytest.raises(AssertionError):
        make_oracle(TINY, bad)
    bad = dict(tiny_w)
    bad["lm_head"] = tiny_w["lm_head"][:1000]
    with pytest.raises(AssertionError):
        make_oracle(TINY, bad)
    bad = dict(tiny_w)
    bad["d2t"] = tiny_w["d2t"].clone(); bad["d2t"][3] = 10 ** 6
    with pytest.raises(AssertionError):
        make_oracle(TINY, bad)


def test_page4_drafter_is_about_0p8_gb():
    # memra `Eagle3Draft` doc: the draft is ~0.8 GB (bf16 on disk)
    params = PAGE4.total_params()
    assert abs(params - 399.5e6) < 0.1e6
    assert 0.75e9 < 2 * params < 0.85e9
    # and its tensor shapes are the ones in the memra module doc
    s = gen.weight_shapes(PAGE4)
    assert s["fc"] == (4096, 12288) and s["q_proj"] == (4096, 8192)
    assert s["k_proj"] == (1024, 8192) and s["lm_head"] == (32000, 4096)
    assert s["gate_proj"] == (12288, 4096) and s["down_proj"] == (4096, 12288)


def test_bf16_kv_cache_holds_the_rounded_exact_rows(tiny_w):
    """kv_format="bf16": every stored K/V element is the exact row rounded to the
    nearest bfloat16, teacher-forced and chain rows alike, and the chain stays
    close to the exact-KV chain."""
    from oracle import round_bf16
    L = 40
    aux, toks = aux_np(TINY, 3, L + 1), toks_np(TINY, 3, L + 1)
    de = make_oracle(TINY, tiny_w)
    db = make_oracle(TINY, tiny_w, kv_format="bf16")
    for d in (de, db):
        d.prefill(0, row_slice(aux, 0, L), toks[:L])
    assert np.array_equal(db.K[0][:L], round_bf16(de.K[0][:L]))
    assert np.array_equal(db.V[0][:L], round_bf16(de.V[0][:L]))
    kb = torch.from_numpy(db.K[0][:L].copy()).to(torch.bfloat16).double().numpy()
    assert np.array_equal(kb, db.K[0][:L])          # representable in bf16
    b_aux = [a[L] for a in aux]
    re = de.draft_chain(0, b_aux, toks[L], 3, keep_spec=True)
    rb = db.draft_chain(0, b_aux, toks[L], 3, keep_spec=True)
    # the chain's first row: the rounded form of what the exact mode computed
    assert np.array_equal(db.K[0][L], round_bf16(re[0].k)) and np.array_equal(rb[0].k, db.K[0][L])
    assert not np.array_equal(rb[0].logits, re[0].logits)   # the rounding is seen
    assert np.abs(rb[0].logits - re[0].logits).max() < 5e-3


@pytest.mark.parametrize("cfg,L", [(TINY, 63), (small_variant(), 120)])
def test_fp32_timing_mode_tracks_the_fp64_oracle(cfg, L):
    """dtype=float32 runs the same operations on fp32 arrays (a CPU speed
    baseline only): its arrays stay fp32 and its chain stays within fp32
    rounding of the parity mode."""
    w = gen.drafter_weights(cfg)
    d64 = make_oracle(cfg, w)
    d32 = make_oracle(cfg, w, dtype=np.float32)
    aux, toks = aux_np(cfg, 4, L + 1), toks_np(cfg, 4, L + 1)
    for d in (d64, d32):
        d.prefill(0, row_slice(aux, 0, L), toks[:L])
    assert d32.K[0].dtype == np.float32 and d32.W["lm_head"].dtype == np.float32
    assert np.allclose(d32.K[0][:L], d64.K[0][:L], rtol=1e-4, atol=1e-5)
    b_aux = [a[L] for a in aux]
    r64 = d64.draft_chain(0, b_aux, toks[L], 3)
    r32 = d32.draft_chain(0, b_aux, toks[L], 3)
    for a, b in zip(r64, r32):
        assert b.logits.dtype == np.float32 and b.gsum.dtype == np.float32
        assert np.abs(a.logits - b.logits).max() < 1e-3
        if a.margin <= 0.05:
            break
        assert a.target_id == b.target_id


def test_bf16_append_activations_round_taps_and_projection_inputs(tiny_w):
    """append_act="bf16": a row of an append of more than 16 rows equals the exact
    row computed from bf16-rounded taps with its [eN ; gN] rounded before the K/V
    projection; appends of at most 16 rows are exact."""
    from oracle import round_bf16
    L = 30
    aux, toks = aux_np(TINY, 5, L + 1), toks_np(TINY, 5, L + 1)
    db = make_oracle(TINY, tiny_w, append_act="bf16")
    db.prefill(0, row_slice(aux, 0, L), toks[:L])
    de = make_oracle(TINY, tiny_w)
    f = de.encode([round_bf16(a[:L]) for a in aux])
    cat = round_bf16(de.input_cat(f, toks[:L]))
    _, k, v = de.qkv(cat, np.arange(L))
    assert np.array_equal(db.K[0][:L], k) and np.array_equal(db.V[0][:L], v)
    de.prefill(0, row_slice(aux, 0, L), toks[:L])
    assert not np.array_equal(db.K[0][:L], de.K[0][:L])
    # the fp16 form rounds the same inputs to IEEE half
    from oracle import round_f16
    dh = make_oracle(TINY, tiny_w, append_act="f16")
    dh.prefill(0, row_slice(aux, 0, L), toks[:L])
    f = de.encode([round_f16(a[:L]) for a in aux])
    _, k, v = de.qkv(round_f16(de.input_cat(f, toks[:L])), np.arange(L))
    assert np.array_equal(dh.K[0][:L], k) and np.array_equal(dh.V[0][:L], v)
    # a 16-row append is exact
    db2, de2 = make_oracle(TINY, tiny_w, append_act="bf16"), make_oracle(TINY, tiny_w)
    for d in (db2, de2):
        d.prefill(0, row_slice(aux, 0, 16), toks[:16])
    assert np.array_equal(db2.K[0][:16], de2.K[0][:16])
