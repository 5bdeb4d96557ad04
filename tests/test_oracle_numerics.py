"""Pins of the oracle's elementary ops against closed forms, invariants and
library routines (torch CPU SDPA, scipy expit)."""
import numpy as np
import pytest
import torch

from oracle import (argmax_first, attention_causal, attention_decode,
                    bf16_bits_to_f64, rms_norm, rope_neox_partial, silu)

rng = np.random.default_rng(1234)


def test_bf16_bits_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3E80, 0x0001, 0x7F7F], np.uint16)
    got = bf16_bits_to_f64(bits)
    want = [1.0, -2.0, 0.0, -0.0, 0.25, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127]
    assert np.array_equal(got, np.array(want))
    t = torch.randn(1000).to(torch.bfloat16)
    assert np.array_equal(bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16)),
                          t.double().numpy())


def test_rmsnorm_closed_forms():
    n = 64
    w = rng.normal(1, 0.1, n)
    # a constant vector normalises to the weight (sign kept), up to eps
    for c in (3.0, -0.5):
        y = rms_norm(np.full(n, c), w, 1e-12)
        assert np.allclose(y, np.sign(c) * w, rtol=1e-9)
    # scale invariance and unit mean-square output with unit weight
    x = rng.normal(0, 2, n)
    assert np.allclose(rms_norm(7 * x, w, 0.0), rms_norm(x, w, 0.0), rtol=1e-12)
    y = rms_norm(x, np.ones(n), 0.0)
    assert abs(np.mean(y * y) - 1) < 1e-12
    # eps enters under the root: x = [1, 0, 0, 0], eps = 0.75 -> 1/sqrt(0.25 + 0.75)
    y = rms_norm(np.array([1.0, 0, 0, 0]), np.ones(4), 0.75)
    assert np.allclose(y, [1.0, 0, 0, 0])
    # batched rows are normalised independently
    X = rng.normal(0, 1, (3, n))
    assert np.allclose(rms_norm(X, w, 1e-6)[1], rms_norm(X[1], w, 1e-6))


def test_silu_against_library():
    from scipy.special import expit
    x = np.linspace(-30, 30, 1001)
    assert np.allclose(silu(x), x * expit(x), rtol=1e-13, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0
    assert abs(silu(np.array([40.0]))[0] - 40.0) < 1e-12


@pytest.mark.parametrize("hd,rot", [(64, 64), (256, 64), (128, 32), (64, 2)])
def test_rope_invariants(hd, rot):
    theta = 1e4
    x = rng.normal(0, 1, (3, hd))
    # position 0 is the identity
    assert np.array_equal(rope_neox_partial(x, 0, rot, theta), x)
    y = rope_neox_partial(x, 37, rot, theta)
    # the pass-through band is bit-unchanged
    assert np.array_equal(y[:, rot:], x[:, rot:])
    # every rotated pair (i, i + rot/2) keeps its norm
    h = rot // 2
    assert np.allclose(y[:, :h] ** 2 + y[:, h:rot] ** 2, x[:, :h] ** 2 + x[:, h:rot] ** 2,
                       rtol=1e-12)
    # rotations compose: rope(rope(x, a), b) = rope(x, a + b)
    assert np.allclose(rope_neox_partial(rope_neox_partial(x, 5, rot, theta), 11, rot, theta),
                       rope_neox_partial(x, 16, rot, theta), atol=1e-12)
    # q.k depends only on the relative offset
    q, k = rng.normal(0, 1, hd), rng.normal(0, 1, hd)
    def score(pq, pk):
        return rope_neox_partial(q[None], pq, rot, theta)[0] @ rope_neox_partial(k[None], pk, rot, theta)[0]
    assert abs(score(100, 93) - score(7, 0)) < 1e-10
    assert abs(score(1000, 1000) - q @ k) < 1e-10


def test_rope_frequencies_use_rotated_width():
    # unit vector on dim i rotates into dim i + rot/2 by angle pos * theta^(-2i/rot)
    hd, rot, theta = 256, 64, 1e7
    h = rot // 2
    for i in (0, 1, h - 1):
        e = np.zeros((1, hd)); e[0, i] = 1.0
        y = rope_neox_partial(e, 1, rot, theta)[0]
        ang = np.arctan2(y[i + h], y[i])
        assert abs(ang - theta ** (-2.0 * i / rot)) < 1e-12
    # a full-width reading would give a different angle for i = h - 1
    assert abs(theta ** (-2.0 * (h - 1) / rot) - theta ** (-2.0 * (h - 1) / hd)) > 1e-3


def _sdpa_ref(q, K, V, causal):
    # torch CPU SDPA in float64 with KV heads repeated per contiguous group
    nh, nkv = q.shape[-2], K.shape[1]
    rep = nh // nkv
    Kr = torch.from_numpy(np.repeat(K, rep, axis=1)).permute(1, 0, 2)
    Vr = torch.from_numpy(np.repeat(V, rep, axis=1)).permute(1, 0, 2)
    Q = torch.from_numpy(q if q.ndim == 3 else q[None]).permute(1, 0, 2)
    O = torch.nn.functional.scaled_dot_product_attention(Q, Kr, Vr, is_causal=causal)
    return O.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("nh,nkv,hd,T", [(4, 2, 64, 1), (4, 2, 64, 37), (6, 2, 32, 130),
                                         (16, 4, 256, 9), (5, 1, 16, 50)])
def test_attention_against_torch_sdpa(nh, nkv, hd, T):
    q = rng.normal(0, 1, (nh, hd))
    K = rng.normal(0, 1, (T, nkv, hd))
    V = rng.normal(0, 1, (T, nkv, hd))
    o = attention_decode(q, K, V)
    ref = _sdpa_ref(q, K, V, False)[0]
    assert np.allclose(o, ref, rtol=1e-10, atol=1e-12)
    Q = rng.normal(0, 1, (T, nh, hd))
    O = attention_causal(Q, K, V)
    assert np.allclose(O, _sdpa_ref(Q, K, V, True), rtol=1e-10, atol=1e-12)


def test_attention_closed_forms():
    nh, nkv, hd = 4, 2, 8
    q = rng.normal(0, 1, (nh, hd))
    K = rng.normal(0, 1, (1, nkv, hd))
    V = rng.normal(0, 1, (1, nkv, hd))
    o = attention_decode(q, K, V)
    # one row: output is that row's value for every head of the group
    assert np.allclose(o[:2], V[0, 0]) and np.allclose(o[2:], V[0, 1])
    # identical keys: uniform weights, output is the mean value
    K = np.repeat(rng.normal(0, 1, (1, nkv, hd)), 5, axis=0)
    V = rng.normal(0, 1, (5, nkv, hd))
    o = attention_decode(q, K, V)
    assert np.allclose(o[0], V[:, 0].mean(0)) and np.allclose(o[3], V[:, 1].mean(0))


def test_argmax_lowest_index_on_ties():
    assert argmax_first(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert argmax_first(np.array([-1.0])) == 0


@pytest.mark.parametrize("nh,nkv,hd,ctx,M", [(4, 2, 64, 0, 4), (4, 2, 64, 37, 1), (8, 2, 32, 50, 5),
                                             (6, 3, 16, 9, 8)])
def test_verify_attention_against_torch_sdpa_with_a_window_mask(nh, nkv, hd, ctx, M):
    # the verify window: query row m sees rows 0..ctx+m (torch SDPA, explicit mask)
    from oracle import attention_verify
    T = ctx + M
    Q = rng.normal(0, 1, (M, nh, hd))
    K = rng.normal(0, 1, (T + 3, nkv, hd))  # rows past the window are never read
    V = rng.normal(0, 1, (T + 3, nkv, hd))
    O = attention_verify(Q, K, V, ctx)
    rep = nh // nkv
    Kr = torch.from_numpy(np.repeat(K[:T], rep, axis=1)).permute(1, 0, 2)
    Vr = torch.from_numpy(np.repeat(V[:T], rep, axis=1)).permute(1, 0, 2)
    mask = torch.from_numpy(np.arange(T)[None, :] <= ctx + np.arange(M)[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(Q).permute(1, 0, 2), Kr, Vr,
                                                           attn_mask=mask).permute(1, 0, 2).numpy()
    assert np.allclose(O, ref, rtol=1e-10, atol=1e-12)
    # and the window is the tail of causal self-attention over all T rows
    Qf = np.concatenate([rng.normal(0, 1, (ctx, nh, hd)), Q])
    assert np.allclose(attention_causal(Qf, K[:T], V[:T])[ctx:], O, rtol=1e-12, atol=1e-14)


def test_round_bf16_against_torch_and_ties():
    from oracle import round_bf16
    # fp32 inputs: torch's float32 -> bfloat16 conversion rounds to nearest even
    x = torch.randn(20000, dtype=torch.float32) * torch.exp(torch.randn(20000) * 4)
    want = x.to(torch.bfloat16).double().numpy()
    assert np.array_equal(round_bf16(x.double().numpy()), want)
    # hand-made ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> 1 (even);
    # 1 + 3 * 2^-8 between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> 1 + 2^-6
    assert round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert round_bf16(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == -(1 + 2.0 ** -6)
    # just past a tie rounds up; representable values and zero are unchanged
    assert round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7
    v = np.array([0.0, -0.0, 1.5, -3.0 * 2.0 ** -20, 2.0 ** 100])
    assert np.array_equal(round_bf16(v), v)
    # error at most half an ulp: 2^(e-8) <= |y| 2^-8 for y in [2^e, 2^(e+1))
    y = rng.normal(0, 1, 1000)
    assert np.all(np.abs(round_bf16(y) - y) <= np.abs(y) * 2.0 ** -8)


def test_round_f16_against_torch_and_ties():
    from oracle import round_f16
    x = torch.randn(20000, dtype=torch.float32) * torch.exp(torch.randn(20000) * 2)
    want = x.to(torch.float16).double().numpy()
    assert np.array_equal(round_f16(x.double().numpy()), want)
    # 1 + 2^-11 lies halfway between 1 and 1 + 2^-10 -> 1 (even); 1 + 3 * 2^-11 -> 1 + 2^-9
    assert round_f16(np.array([1 + 2.0 ** -11]))[0] == 1.0
    assert round_f16(np.array([1 + 3 * 2.0 ** -11]))[0] == 1 + 2.0 ** -9
    # a bf16 value times 2^8 is exact in fp16 (8 significant bits fit in 11)
    w = torch.randn(5000).mul(0.02).to(torch.bfloat16).double().numpy() * 256
    assert np.array_equal(round_f16(w), w)
