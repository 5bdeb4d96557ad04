"""The allocation-free verify attention (eagle3_verify_attention_noalloc, for
callers that cannot allocate device memory) against eagle3_verify_attention with
a caller workspace: the same kernels on the same inputs, so the outputs must be
bit-identical, on two calls in a row (the second smaller, the library's static
scratch keeping the first call's contents) and on a call that needs one split
only.  A call whose split partials exceed the static scratch is rejected before
any device work."""
import numpy as np
import pytest
import torch

from eagle_draft_head_amd import binding as B
from synth import gen

pytestmark = pytest.mark.gpu


def _inputs(nh, nkv, hd, cap, M, kv, seed):
    q = gen.normal(70 + seed, 1, (M, nh, hd), 1.0, device="cuda")
    k = gen.normal(70 + seed, 2, (nkv, cap, hd), 1.0, device="cuda")
    v = gen.normal(70 + seed, 3, (nkv, cap, hd), 1.0, device="cuda")
    if kv == B.KV_BF16:
        k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    return q, k, v


def _both(nh, nkv, hd, ctx, M, kv, seed):
    cap = ctx + M + 3
    q, k, v = _inputs(nh, nkv, hd, cap, M, kv, seed)
    ws_bytes = B.eagle3_verify_attention_workspace(M, nh, nkv, hd, ctx, kv)
    assert ws_bytes <= B.VERIFY_SCRATCH_BYTES
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
    ref = torch.full((M, nh, hd), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full((M, nh, hd), float("nan"), dtype=torch.float32, device="cuda")
    B.eagle3_verify_attention(q, k, v, kv, cap, ctx, M, nh, nkv, hd, ref, ws, ws_bytes)
    B.eagle3_verify_attention_noalloc(q, k, v, kv, cap, ctx, M, nh, nkv, hd, got)
    torch.cuda.synchronize()
    return got, ref, ws_bytes


@pytest.mark.parametrize("kv", [B.KV_F32, B.KV_BF16], ids=["f32", "bf16"])
def test_noalloc_verify_attention_matches_the_workspace_entry_point(kv):
    # a long call (many splits: the static scratch is used), then a smaller one
    # that reuses the scratch the first call filled, then a one-split call
    for nh, nkv, hd, ctx, M, seed in [(40, 8, 128, 32764, 4, 1), (8, 2, 64, 3001, 3, 2),
                                      (4, 2, 64, 20, 2, 3)]:
        got, ref, ws_bytes = _both(nh, nkv, hd, ctx, M, kv, seed)
        assert not torch.isnan(ref).any()
        assert torch.equal(got, ref), (nh, ctx, M, float((got - ref).abs().max()))
        print(f"[noalloc] heads {nh}/{nkv}x{hd} ctx {ctx} M {M}: {ws_bytes} scratch bytes, identical",
              flush=True)


def test_noalloc_verify_attention_rejects_oversized_partials():
    # partials beyond the static scratch: rejected on the host, nothing launched
    M, nh, nkv, hd, ctx = 64, 64, 8, 256, 1 << 20
    need = B.eagle3_verify_attention_workspace(M, nh, nkv, hd, ctx, B.KV_F32)
    assert need > B.VERIFY_SCRATCH_BYTES
    with pytest.raises(B.Eagle3Error) as e:
        B.eagle3_verify_attention_noalloc(1, 1, 1, B.KV_F32, ctx + M, ctx, M, nh, nkv, hd, 1)
    assert e.value.code == B.E_CAPACITY
    assert "static scratch" in B.eagle3_last_error(None)
