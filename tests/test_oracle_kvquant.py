"""Pins of the quantized-KV oracle (oracle.kvquant): q8_0 K rows and q5_1 V rows.

memra_engine `eagle.rs` (`Eagle3Scratch` doc, `attn`): q8_0 K / q5_1 V by
default, 34 and 24 bytes per block of 32 values.
"""
import numpy as np
import pytest

from oracle import kvquant
from synth import TINY, gen
from tests.common import aux_np, make_oracle, row_slice, toks_np


def test_block_bytes_match_the_pages():
    # the pages' default KV formats: 34-byte K blocks and 24-byte V blocks of 32 values
    assert kvquant.block_bytes() == (34, 24)


def test_q8_0_hand_example():
    x = np.zeros(32, dtype=np.float32)
    x[:6] = [127.0, -63.5, 1.0, 2.5, -0.49, 126.6]
    q, D = kvquant.q8_0(x)
    assert D.shape == (1,) and float(D[0]) == 1.0          # 127 / 127, exact in fp16
    # rint ties to even: -63.5 -> -64, 2.5 -> 2; -0.49 -> -0; 126.6 -> 127
    assert q[:6].tolist() == [127, -64, 1, 2, 0, 127]
    assert np.all(q[6:] == 0)
    v = kvquant.q8_0_values(q, D)
    assert v[:6].tolist() == [127.0, -64.0, 1.0, 2.0, 0.0, 127.0]


def test_q5_1_hand_example():
    x = np.full(32, 3.0, dtype=np.float32)
    x[0], x[1], x[2], x[3] = -1.0, 30.0, 0.5, 14.5
    q, D, M = kvquant.q5_1(x)
    assert float(D[0]) == 1.0 and float(M[0]) == -1.0     # (30 - (-1)) / 31, min -1
    # x - M = 0, 31, 1.5, 15.5, 4: ties to even give 2 and 16
    assert q[:5].tolist() == [0, 31, 2, 16, 4]
    v = kvquant.q5_1_values(q, D, M)
    assert v[:5].tolist() == [-1.0, 30.0, 1.0, 15.0, 3.0]


def test_zero_and_constant_blocks():
    z = np.zeros(64, dtype=np.float32)
    q, D = kvquant.q8_0(z)
    assert np.all(q == 0) and np.all(D == 0)
    assert np.all(kvquant.q8_0_values(q, D) == 0)
    c = np.full(32, 0.75, dtype=np.float32)                # fp16-exact constant
    q5, D5, M5 = kvquant.q5_1(c)
    assert float(D5[0]) == 0.0 and float(M5[0]) == 0.75 and np.all(q5 == 0)
    assert np.all(kvquant.q5_1_values(q5, D5, M5) == 0.75)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_round_trip_error_bounds(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((8, 128)) * 10.0 ** rng.uniform(-3, 3, (8, 1))).astype(np.float32)
    b = x.reshape(8, 4, 32).astype(np.float64)
    # q8_0: half a step, plus what the clamp costs when D rounded below max|x| / 127
    q, D = kvquant.q8_0(x)
    d = np.abs(b).max(axis=2) / 127.0
    Dd = D.astype(np.float64)
    err = np.abs(kvquant.q8_0_values(q, D).reshape(8, 4, 32) - b).max(axis=2)
    assert np.all(err <= 0.5 * Dd + 127 * np.abs(d - Dd) + 1e-12 * np.abs(b).max(axis=2))
    # q5_1: half a step, plus the stored minimum's and scale's fp16 rounding
    q5, D5, M5 = kvquant.q5_1(x)
    d5 = (b.max(axis=2) - b.min(axis=2)) / 31.0
    D5d, M5d = D5.astype(np.float64), M5.astype(np.float64)
    err5 = np.abs(kvquant.q5_1_values(q5, D5, M5).reshape(8, 4, 32) - b).max(axis=2)
    bound = 0.5 * D5d + 31 * np.abs(d5 - D5d) + np.abs(b.min(axis=2) - M5d)
    assert np.all(err5 <= bound * (1 + 1e-6))


def test_codes_are_the_nearest_levels_brute_force():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(32 * 16).astype(np.float32)
    q, D = kvquant.q8_0(x)
    levels = np.arange(-127, 128, dtype=np.float64)
    for blk in range(16):
        Dv = float(D[blk])
        for i in range(32):
            xi = float(x[blk * 32 + i])
            t = xi / Dv
            if abs(abs(t - np.floor(t)) - 0.5) < 1e-3:
                continue  # near a tie: the fp32 division decides
            best = levels[np.argmin(np.abs(xi - Dv * levels))]
            assert q[blk * 32 + i] == best
    q5, D5, M5 = kvquant.q5_1(x)
    lv5 = np.arange(0, 32, dtype=np.float64)
    for blk in range(16):
        Dv, Mv = float(D5[blk]), float(M5[blk])
        for i in range(32):
            xi = float(x[blk * 32 + i])
            t = (xi - Mv) / Dv
            if abs(abs(t - np.floor(t)) - 0.5) < 1e-3:
                continue
            best = lv5[np.argmin(np.abs(xi - (Dv * lv5 + Mv)))]
            assert q5[blk * 32 + i] == best


def test_drafter_stores_quantized_rows():
    w = gen.drafter_weights(TINY)
    ex = make_oracle(TINY, w)
    qz = make_oracle(TINY, w, kv_format="q8q5")
    L = 24
    aux, toks = aux_np(TINY, 0, L + 1), toks_np(TINY, 0, L + 1)
    ex.prefill(0, row_slice(aux, 0, L), toks[:L])
    qz.prefill(0, row_slice(aux, 0, L), toks[:L])
    # the cache holds the quantized form of the exact rows
    assert np.array_equal(qz.K[0][:L], kvquant.k_stored(ex.K[0][:L]))
    assert np.array_equal(qz.V[0][:L], kvquant.v_stored(ex.V[0][:L]))
    assert not np.array_equal(qz.K[0][:L], ex.K[0][:L])
    # a chain over the quantized cache writes quantized rows and stays close
    b_aux = [a[L] for a in aux]
    r_ex = ex.draft_chain(0, b_aux, toks[L], 3, keep_spec=True)
    r_qz = qz.draft_chain(0, b_aux, toks[L], 3, keep_spec=True)
    assert np.array_equal(qz.K[0][L], kvquant.k_stored(r_ex[0].k))
    for a, b in zip(r_ex, r_qz):
        assert np.abs(a.logits - b.logits).max() < 0.05 * np.abs(a.logits).max() + 1e-3
