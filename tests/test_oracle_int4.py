"""Pins of the oracle's group-wise int4 weights (oracle/int4.py): exact round trip
of values on the quantization grid, the half-step error bound, zero groups, sign
symmetry, a hand-computed group, the nibble packing, and the cached chain with
int4 weights equal to the stateless recompute."""
import numpy as np
import pytest

from oracle import StatelessChain, bf16_bits_to_f64, int4
from synth import TINY, gen
from tests.common import aux_np, make_oracle, row_slice, toks_np


def test_values_on_the_grid_round_trip_exactly():
    rng = np.random.default_rng(1)
    # scale 2^-7 (exact in bf16); each group holds a +-7 so its max is 7 scales
    s = np.float32(2.0 ** -7)
    q = rng.integers(-7, 8, size=(3, 64)).astype(np.int8)
    q[:, 5] = 7
    q[:, 40] = -7
    w = q.astype(np.float32) * s
    codes, s_bits = int4.quantize(int4.f32_to_bf16_bits(w))
    assert np.array_equal(codes, q)
    assert np.all(bf16_bits_to_f64(s_bits) == float(s))
    assert np.array_equal(int4.dequantize(codes, s_bits), w.astype(np.float64))


def test_error_is_at_most_half_a_step():
    w = int4.f32_to_bf16_bits((np.random.default_rng(2).normal(size=(16, 256)) * 0.02).astype(np.float32))
    codes, s_bits = int4.quantize(w)
    err = np.abs(bf16_bits_to_f64(w) - int4.dequantize(codes, s_bits)).reshape(16, 8, 32)
    s = bf16_bits_to_f64(s_bits)
    assert np.all(err <= s[..., None] / 2 * (1 + 1e-6))
    assert codes.min() >= -7 and codes.max() <= 7
    # the largest magnitude of each group lands on +-7 (or +-6 when bf16 rounded
    # the scale up by more than 1/14 of a step, which it cannot)
    gmax = np.abs(codes.reshape(16, 8, 32)).max(axis=2)
    assert np.all(gmax == 7)


def test_zero_group_and_sign_symmetry():
    w = np.zeros((2, 64), dtype=np.float32)
    w[1, 32:] = np.linspace(-0.05, 0.04, 32, dtype=np.float32)
    b = int4.f32_to_bf16_bits(w)
    codes, s_bits = int4.quantize(b)
    assert np.all(codes[0] == 0) and np.all(s_bits[0] == 0) and np.all(codes[1, :32] == 0)
    codes_n, s_bits_n = int4.quantize(int4.f32_to_bf16_bits(-w))
    assert np.array_equal(codes_n, -codes) and np.array_equal(s_bits_n, s_bits)


def test_hand_computed_group():
    # the weights are bf16 first: 0.69921875, -0.349609375, 0.10009765625, 0, 0.25;
    # max / 7 = 0.09989 -> scale bf16 0x3DCD = 0.10009765625; codes 6.985 -> 7,
    # -3.493 -> -3, 1.0 -> 1, 0, 2.4976 -> 2
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, :5] = [0.7, -0.35, 0.1, 0.0, 0.25]
    codes, s_bits = int4.quantize(int4.f32_to_bf16_bits(w))
    assert s_bits[0, 0] == 0x3DCD
    assert codes[0, :5].tolist() == [7, -3, 1, 0, 2]


def test_nibble_packing():
    codes = np.array([[1, -2, -7, 7]], dtype=np.int8)
    p = int4.pack(codes)
    assert p.tolist() == [[(1 + 8) | ((-2 + 8) << 4), (-7 + 8) | ((7 + 8) << 4)]]
    assert np.array_equal(int4.unpack(p), codes)


def test_int4_chain_equals_stateless_recompute():
    w = int4.int4_weights(gen.drafter_weights(TINY))
    d = make_oracle(TINY, w)
    L = 40
    aux, toks = aux_np(TINY, 0, L + 1), toks_np(TINY, 0, L + 1)
    d.prefill(0, row_slice(aux, 0, L), toks[:L])
    b_aux = [a[L] for a in aux]
    recs = d.draft_chain(0, b_aux, toks[L], 3)
    ref = StatelessChain(d).run(row_slice(aux, 0, L), toks[:L], b_aux, toks[L], 3)
    assert [r.target_id for r in recs] == [r.target_id for r in ref]
    for a, b in zip(recs, ref):
        assert np.allclose(a.logits, b.logits, rtol=1e-10, atol=1e-12)
    # and the weights really are the int4 values: every fc group has at most 15 levels
    fc = w["fc"].reshape(TINY.n_embd, -1, 32)
    assert max(len(np.unique(g)) for g in fc.reshape(-1, 32)[:64]) <= 15
