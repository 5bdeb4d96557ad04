"""Structural pins of the oracle drafter layer, and proof that they bite.

The op sequence of one draft step is fixed by the memra_engine `eagle.rs` module
doc ("Op-sequence") and its `draft_token` method: the previous token's embedding
goes through input_layernorm and the recurrent hidden through hidden_norm, the two
are concatenated embedding first, the residual is the pre-norm hidden, the MLP
reads post_attention_layernorm(x1), the head reads norm(gsum), and the MLP is
down . (silu(gate . z) * (up . z)).  Nothing in this container holds golden
tensors for that sequence, so each choice is pinned by an exact consequence of
the text that a different choice would break:

  * input_layernorm = 0 makes the step independent of the token;
  * zeroing the first n input columns of q/k/v equals input_layernorm = 0 and
    zeroing the last n equals hidden_norm = 0 (the concat order);
  * hidden_norm = 0 makes the K/V row independent of g (g only in the residual);
  * post_attention_layernorm = 0 gives gsum = x1 (= gsum with down zeroed);
  * doubling `norm` doubles the logits and leaves gsum unchanged;
  * doubling up_proj doubles the MLP's contribution, doubling gate_proj does not;
  * with o_proj and down zeroed, g_next = g (pre-norm residual);
  * with eps = 0, scaling g or the embedding row leaves the K/V row unchanged;
  * attention equals torch's SDPA with contiguous GQA groups;
  * a chain's logits depend only on relative positions (q and k rotated, v not);
  * d2t is a delta; encode concatenates the taps in ascending order.

`test_every_planted_mistake_turns_a_pin_red` plants each plausible structural
mistake in a CPU subclass (or a patched helper) of the oracle and checks that at
least one pin fails on it.
"""
from __future__ import annotations

import contextlib

import numpy as np
import pytest
import torch

import oracle.drafter as odr
from oracle import DrafterOracle
from oracle.numerics import rms_norm, rope_neox_partial, silu
from synth import TINY, gen

CFG = TINY
N = CFG.n_embd
NKV, HD = CFG.n_head_kv, CFG.head_dim
BASE_W = gen.drafter_weights(CFG)


class _Factory:
    """Builds an oracle of class `cls` from the tiny weights with overrides."""

    def __init__(self, cls=DrafterOracle):
        self.cls = cls

    def __call__(self, cfg=CFG, **over):
        w = dict(BASE_W)
        w.update(over)
        return self.cls(cfg, w, w["embed"], w["d2t"], max_ctx=64)


def _ctx(seed, rows=5):
    r = np.random.default_rng(seed)
    return r.normal(0, 1, (rows, NKV, HD)), r.normal(0, 1, (rows, NKV, HD))


def _g(seed, scale=1.0):
    return np.random.default_rng(seed).normal(0, 1, N) * scale


def _step(d, g, tok, ctx=None):
    K, V = _ctx(7) if ctx is None else ctx
    return d.step(g, tok, K.shape[0], K, V)


def _zero(name):
    return torch.zeros_like(BASE_W[name])


def _times2(name):
    return (BASE_W[name].double() * 2).to(torch.bfloat16)   # exact in bf16


def _cols_zeroed(lo, hi):
    out = {}
    for k in ("q_proj", "k_proj", "v_proj"):
        w = BASE_W[k].clone()
        w[:, lo:hi] = 0
        out[k] = w
    return out


TOL = dict(rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- the pins
def pin_input_norm_zero_ignores_token(make):
    d = make(input_layernorm=_zero("input_layernorm"))
    g = _g(1)
    a, b = _step(d, g, 11), _step(d, g, 3001)
    assert np.array_equal(a.logits, b.logits) and np.array_equal(a.gsum, b.gsum)


def pin_embedding_is_the_first_half(make):
    g = _g(2)
    a = _step(make(**_cols_zeroed(0, N)), g, 17)
    b = _step(make(input_layernorm=_zero("input_layernorm")), g, 17)
    assert np.allclose(a.logits, b.logits, **TOL) and np.allclose(a.k, b.k, **TOL)


def pin_hidden_is_the_second_half(make):
    g = _g(3)
    a = _step(make(**_cols_zeroed(N, 2 * N)), g, 23)
    b = _step(make(hidden_norm=_zero("hidden_norm")), g, 23)
    assert np.allclose(a.logits, b.logits, **TOL) and np.allclose(a.v, b.v, **TOL)


def pin_hidden_norm_zero_keeps_g_out_of_kv(make):
    d = make(hidden_norm=_zero("hidden_norm"))
    a, b = _step(d, _g(4), 29), _step(d, _g(5), 29)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert not np.allclose(a.gsum, b.gsum)


def pin_post_norm_zero_gives_x1(make):
    g = _g(6)
    a = _step(make(post_attention_layernorm=_zero("post_attention_layernorm")), g, 31)
    b = _step(make(down_proj=_zero("down_proj")), g, 31)    # gsum = x1 by definition
    assert np.array_equal(a.gsum, b.gsum)


def pin_final_norm_scales_logits(make):
    g = _g(7)
    a = _step(make(), g, 37)
    b = _step(make(norm=_times2("norm")), g, 37)
    assert np.array_equal(a.gsum, b.gsum)
    assert np.allclose(b.logits, 2 * a.logits, rtol=1e-13, atol=1e-14)


def pin_head_normalises_gsum(make):
    # o_proj and down zeroed make gsum = g; with eps = 0 the head's RMSNorm makes
    # the logits invariant to scaling g
    d = make(CFG.with_(rms_eps=0.0), o_proj=_zero("o_proj"), down_proj=_zero("down_proj"))
    g = _g(15)
    a, b = _step(d, g, 59), _step(d, 4.0 * g, 59)
    assert np.allclose(a.logits, b.logits, rtol=1e-12, atol=1e-13)


def pin_up_is_linear_gate_is_silu(make):
    g = _g(8)
    x1 = _step(make(down_proj=_zero("down_proj")), g, 41).gsum
    base = _step(make(), g, 41).gsum - x1
    up2 = _step(make(up_proj=_times2("up_proj")), g, 41).gsum - x1
    gate2 = _step(make(gate_proj=_times2("gate_proj")), g, 41).gsum - x1
    assert np.allclose(up2, 2 * base, rtol=1e-9, atol=1e-12)
    assert not np.allclose(gate2, 2 * base, rtol=1e-3, atol=0)


def pin_residual_is_the_prenorm_hidden(make):
    d = make(o_proj=_zero("o_proj"), down_proj=_zero("down_proj"))
    g = _g(9, scale=3.0)
    assert np.array_equal(_step(d, g, 43).gsum, g)


def pin_norms_make_kv_scale_invariant(make):
    cfg0 = CFG.with_(rms_eps=0.0)
    d = make(cfg0)
    g = _g(10)
    a, b = _step(d, g, 47), _step(d, 4.0 * g, 47)
    assert np.allclose(a.k, b.k, **TOL) and np.allclose(a.v, b.v, **TOL)
    E4 = (BASE_W["embed"].double() * 4).to(torch.bfloat16)
    c = _step(make(cfg0, embed=E4), g, 47)
    assert np.allclose(a.k, c.k, **TOL) and np.allclose(a.v, c.v, **TOL)


def pin_attention_is_sdpa_with_contiguous_groups(make):
    # the attention the drafter module calls, against torch CPU SDPA (fp64) with
    # KV heads repeated per contiguous group
    r = np.random.default_rng(11)
    nh, nkv, hd, T = 6, 2, 16, 9
    q = r.normal(0, 1, (nh, hd))
    K, V = r.normal(0, 1, (T, nkv, hd)), r.normal(0, 1, (T, nkv, hd))
    o = odr.attention_decode(q, K, V)
    Kr = torch.from_numpy(np.repeat(K, nh // nkv, axis=1)).permute(1, 0, 2)
    Vr = torch.from_numpy(np.repeat(V, nh // nkv, axis=1)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[None]).permute(1, 0, 2), Kr, Vr).permute(1, 0, 2).numpy()[0]
    assert np.allclose(o, ref, rtol=1e-10, atol=1e-12)


def pin_chain_sees_relative_positions_only(make):
    # the same committed rows and chain placed at offsets 0 and 100: rotary q/k
    # scores see position differences only, and v carries no position
    d = make()
    r = np.random.default_rng(12)
    T = 6
    aux = [r.normal(0, 1, (T, N)) for _ in range(3)]
    toks = r.integers(0, CFG.target_vocab, T)
    f = d.encode(aux)
    cat = d.input_cat(f, toks)
    out = []
    for off in (0, 100):
        _, k, v = d.qkv(cat, off + np.arange(T))
        Kc = np.zeros((off + T, NKV, HD)); Vc = np.zeros_like(Kc)
        Kc[off:], Vc[off:] = k, v
        rec = d.step(_g(13), 53, off + T, Kc[off:], Vc[off:], nctx=T)
        out.append(rec)
    assert np.allclose(out[0].logits, out[1].logits, rtol=1e-9, atol=1e-11)
    assert np.array_equal(out[0].v, out[1].v)


def pin_d2t_is_a_delta(make):
    d = make()
    sub = gen.sorted_subset(CFG.cfg_id, gen.TID["d2t"], CFG.target_vocab, CFG.draft_vocab)
    assert [d.d2t_map(i) for i in range(CFG.draft_vocab)] == sub.tolist()


def pin_encode_taps_in_ascending_order(make):
    d = make()
    a, z = _g(14), np.zeros(N)
    fc = d.W["fc"]
    for j in range(3):
        taps = [z, z, z]
        taps[j] = a
        assert np.allclose(d.encode(taps), fc[:, j * N:(j + 1) * N] @ a, **TOL)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__[4:])
def test_pin_holds_for_the_oracle(pin):
    pin(_Factory())


# ------------------------------------------------- plausible planted mistakes
class _CatSwapped(DrafterOracle):
    def input_cat(self, g, toks):
        c = super().input_cat(g, toks)
        return np.concatenate([c[..., self.n:], c[..., :self.n]], axis=-1)


class _InHidSwapped(DrafterOracle):
    def input_cat(self, g, toks):
        e = self.embed(toks).reshape(np.shape(g))
        return np.concatenate([rms_norm(e, self.W["hidden_norm"], self.eps),
                               rms_norm(g, self.W["input_layernorm"], self.eps)], axis=-1)


class _NoEmbedNorm(DrafterOracle):
    def input_cat(self, g, toks):
        e = self.embed(toks).reshape(np.shape(g))
        return np.concatenate([e * self.W["input_layernorm"],
                               rms_norm(g, self.W["hidden_norm"], self.eps)], axis=-1)


class _NoHiddenNorm(DrafterOracle):
    def input_cat(self, g, toks):
        e = self.embed(toks).reshape(np.shape(g))
        return np.concatenate([rms_norm(e, self.W["input_layernorm"], self.eps),
                               g * self.W["hidden_norm"]], axis=-1)


def _after(self, o, g, post, mlp_in_norm=True, silu_on_up=False, resid_normed=False):
    r = rms_norm(g, self.W["hidden_norm"], self.eps) if resid_normed else g
    x1 = o @ self.W["o_proj"].T + r
    z = rms_norm(x1, self.W[post], self.eps) if mlp_in_norm else x1
    gt, up = z @ self.W["gate_proj"].T, z @ self.W["up_proj"].T
    act = gt * silu(up) if silu_on_up else silu(gt) * up
    return act @ self.W["down_proj"].T + x1


class _PostFinalSwapped(DrafterOracle):
    def after_attention(self, o, g):
        return _after(self, o, g, "norm")

    def head(self, gsum):
        return rms_norm(gsum, self.W["post_attention_layernorm"], self.eps) @ self.W["lm_head"].T


class _NoFinalNorm(DrafterOracle):
    def head(self, gsum):
        return (gsum * self.W["norm"]) @ self.W["lm_head"].T


class _NoPostNorm(DrafterOracle):
    def after_attention(self, o, g):
        return _after(self, o, g, "post_attention_layernorm", mlp_in_norm=False)


class _SiluOnUp(DrafterOracle):
    def after_attention(self, o, g):
        return _after(self, o, g, "post_attention_layernorm", silu_on_up=True)


class _ResidualNormed(DrafterOracle):
    def after_attention(self, o, g):
        return _after(self, o, g, "post_attention_layernorm", resid_normed=True)


def _qkv_variant(rope_q=True, rope_k=True, rope_v=False):
    class _Q(DrafterOracle):
        def qkv(self, cat, positions):
            lead = cat.shape[:-1]
            q = (cat @ self.W["q_proj"].T).reshape(*lead, self.nh, self.hd)
            k = (cat @ self.W["k_proj"].T).reshape(*lead, self.nkv, self.hd)
            v = (cat @ self.W["v_proj"].T).reshape(*lead, self.nkv, self.hd)
            rot = lambda x: rope_neox_partial(x, positions, self.rot, self.theta)
            return (rot(q) if rope_q else q), (rot(k) if rope_k else k), (rot(v) if rope_v else v)
    return _Q


class _D2tAbsolute(DrafterOracle):
    def d2t_map(self, draft_id):
        return int(self.d2t[draft_id]) % self.vt


class _EncodeReversed(DrafterOracle):
    def encode(self, aux):
        return super().encode(list(aux)[::-1])


def _attn_scaled_by_hd(q, K, V):
    n_head, hd = q.shape
    n_kv = K.shape[1]
    out = np.empty_like(q)
    for h in range(n_head):
        g = (h * n_kv) // n_head
        s = (K[:, g, :] @ q[h]) / hd
        p = np.exp(s - s.max())
        out[h] = (p / p.sum()) @ V[:, g, :]
    return out


def _attn_interleaved_groups(q, K, V):
    n_head, hd = q.shape
    n_kv = K.shape[1]
    out = np.empty_like(q)
    for h in range(n_head):
        g = h % n_kv
        s = (K[:, g, :] @ q[h]) / np.sqrt(hd)
        p = np.exp(s - s.max())
        out[h] = (p / p.sum()) @ V[:, g, :]
    return out


MUTANTS = {
    "concat [gN ; eN]": (_CatSwapped, None),
    "input_layernorm <-> hidden_norm": (_InHidSwapped, None),
    "no RMS over the embedding": (_NoEmbedNorm, None),
    "no RMS over g": (_NoHiddenNorm, None),
    "post_attention_layernorm <-> norm": (_PostFinalSwapped, None),
    "no final norm": (_NoFinalNorm, None),
    "MLP reads x1 unnormed": (_NoPostNorm, None),
    "silu on up instead of gate": (_SiluOnUp, None),
    "residual is the normed g": (_ResidualNormed, None),
    "q not rotated": (_qkv_variant(rope_q=False), None),
    "k not rotated": (_qkv_variant(rope_k=False), None),
    "v rotated too": (_qkv_variant(rope_v=True), None),
    "d2t read as absolute ids": (_D2tAbsolute, None),
    "taps concatenated in descending order": (_EncodeReversed, None),
    "attention scale 1/head_dim": (DrafterOracle, _attn_scaled_by_hd),
    "GQA groups interleaved": (DrafterOracle, _attn_interleaved_groups),
}


@contextlib.contextmanager
def _patched_attention(fn):
    if fn is None:
        yield
        return
    saved = odr.attention_decode
    odr.attention_decode = fn
    try:
        yield
    finally:
        odr.attention_decode = saved


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_turns_a_pin_red(name):
    cls, attn = MUTANTS[name]
    red = []
    with _patched_attention(attn):
        for pin in PINS:
            try:
                pin(_Factory(cls))
            except AssertionError:
                red.append(pin.__name__)
    assert red, f"no pin fails when the oracle has the mistake: {name}"
