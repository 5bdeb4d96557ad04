"""The benchmark's algorithmic byte counts (the roofline's numerator), checked
against the matrix shapes of the Qwen3-8B-shaped drafter worked out by hand."""
import bench
from synth import QWEN3_8B as C


def test_lm_head_launch_bytes():
    n, dv = C.n_embd, C.draft_vocab
    weights = dv * n * 2                      # 32000 x 4096 bf16 = 262,144,000 B
    assert weights == 262_144_000
    # plus the staged activation (h * w_norm, fp32), its partial sums and the
    # per-block candidates: small next to the weights
    got = bench.kernel_bytes(C, "lm_head", 1024)
    assert 0 < got - weights < 64 * 1024
    assert got == 262_176_768


def test_step_weight_bytes_match_the_shapes():
    n, qd, kvd, ff, dv = C.n_embd, C.n_head * C.head_dim, C.n_head_kv * C.head_dim, C.n_ff, C.draft_vocab
    per_step = 2 * ((qd + 2 * kvd) * 2 * n + n * qd + 2 * ff * n + n * ff + dv * n)
    assert per_step == 698_351_616            # 698.35 MB of bf16 weights per draft step
    # the step adds its KV rows (fp32, 1024 rows and the new one, K and V) and
    # vectors; bf16 KV halves the KV share
    f32 = bench.kernel_bytes_step(C, 1024, 3, 4)
    bf16 = bench.kernel_bytes_step(C, 1024, 3, 2)
    kv_f32 = f32 - per_step
    assert 2 * 4 * kvd * 1024 <= kv_f32 < 2 * 4 * kvd * 1024 + 256 * 1024
    rows = (f32 - bf16) / (2 * 2 * kvd)     # KV rows read over the step (2 bytes saved each)
    assert rows == int(rows) and 1024 <= rows <= 1024 + 16
    assert f32 == 706_805_760


def test_int4_and_quantized_kv_byte_factors():
    # int4: half a byte per code plus a 2-byte scale per 32 weights
    assert bench.WB_I4 == 0.5 + 2 / 32
    saved = bench.WB
    try:
        bench.WB = bench.WB_I4
        assert bench.kernel_bytes(C, "lm_head", 1024) == 73_760_768
    finally:
        bench.WB = saved
    # q8_0 K (34 bytes per 32 values) and q5_1 V (24 per 32), averaged per element
    assert bench.KV_BYTES["q8q5"] * 64 == 34 + 24
