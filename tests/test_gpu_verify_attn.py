"""Verify-window attention (`eagle3_verify_attention`) against the oracle's
`attention_verify`: M query rows per head over a cache whose rows ctx..ctx+M-1 are
the window's own K/V, query row m seeing rows 0..ctx+m.  Small and ragged shapes
(one split and many, every head grouping, fp32 and bf16 K/V, an empty context)
and the long-context shape (32764 context rows, a 5-row window, 32/8 x 128 heads).
The argument checks run on the host, before any device work, and are covered
without a GPU."""
import numpy as np
import pytest
import torch

from eagle_draft_head_amd import binding as B
from oracle import attention_verify
from synth import gen


def _inputs(nh, nkv, hd, cap, M, kv, seed):
    q = gen.normal(90 + seed, 1, (M, nh, hd), 1.0)
    k = gen.normal(90 + seed, 2, (nkv, cap, hd), 1.0)
    v = gen.normal(90 + seed, 3, (nkv, cap, hd), 1.0)
    if kv == B.KV_BF16:
        k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    return q, k, v


def _run(q, k, v, kv, cap, ctx, M, nh, nkv, hd):
    ws_bytes = B.eagle3_verify_attention_workspace(M, nh, nkv, hd, ctx, kv)
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, nh, hd), dtype=torch.float32, device="cuda")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    B.eagle3_verify_attention(qd, kd, vd, kv, cap, ctx, M, nh, nkv, hd, out, ws, ws_bytes)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _oracle(q, k, v, ctx, M):
    K = k.double().permute(1, 0, 2).numpy()  # [rows][nkv][hd]
    V = v.double().permute(1, 0, 2).numpy()
    return attention_verify(q.double().numpy(), K, V, ctx)


@pytest.mark.gpu
@pytest.mark.parametrize("nh,nkv,hd,ctx,M,kv", [
    (4, 2, 64, 0, 4, B.KV_F32),        # empty context: the window alone
    (4, 2, 64, 37, 1, B.KV_F32),       # one query row (decode)
    (4, 2, 64, 513, 3, B.KV_BF16),     # head_dim 64 bf16: 8-byte V operand loads
    (8, 2, 128, 300, 5, B.KV_BF16),    # 4 heads per KV head, 20 query vectors
    (16, 4, 256, 50, 8, B.KV_F32),
    (6, 2, 64, 1000, 4, B.KV_F32),     # 3 heads per KV head: ragged query groups
    (5, 5, 128, 2999, 3, B.KV_BF16),   # no grouping, many splits with a tail
    (32, 8, 128, 4000, 4, B.KV_F32),
])
def test_verify_attention_parity(nh, nkv, hd, ctx, M, kv):
    cap = ctx + M + 7  # rows past the window are never read
    q, k, v = _inputs(nh, nkv, hd, cap, M, kv, seed=hd + M)
    got = _run(q, k, v, kv, cap, ctx, M, nh, nkv, hd)
    ref = _oracle(q, k, v, ctx, M)
    assert np.allclose(got, ref, rtol=1e-4, atol=2e-5), np.abs(got - ref).max()


@pytest.mark.gpu
@pytest.mark.parametrize("kv", [B.KV_F32, B.KV_BF16], ids=["f32", "bf16"])
def test_verify_attention_long_context(kv):
    nh, nkv, hd, M = 32, 8, 128, 5
    ctx = 32764
    cap = ctx + M
    q, k, v = _inputs(nh, nkv, hd, cap, M, kv, seed=7)
    got = _run(q, k, v, kv, cap, ctx, M, nh, nkv, hd)
    ref = _oracle(q, k, v, ctx, M)
    assert np.allclose(got, ref, rtol=1e-4, atol=2e-5), np.abs(got - ref).max()


def _call(**kw):
    a = dict(q=1, k=1, v=1, kv_dtype=B.KV_F32, cap=100, ctx_rows=10, M=4, n_head=8, n_head_kv=2,
             head_dim=128, out=1, workspace=None, workspace_bytes=0, stream=0)
    a.update(kw)
    with pytest.raises(B.Eagle3Error) as e:
        B.eagle3_verify_attention(**a)
    return e.value.code


def test_verify_attention_argument_checks():
    # rejected on the host before any device work (the pointers are never touched)
    assert _call(head_dim=96) == B.E_UNSUPPORTED
    assert _call(kv_dtype=B.KV_Q8Q5) == B.E_UNSUPPORTED
    assert _call(n_head=6, n_head_kv=4) == B.E_SHAPE
    assert _call(M=0) == B.E_INVAL
    assert _call(ctx_rows=97) == B.E_INVAL          # ctx + M > cap
    assert _call(q=None) == B.E_INVAL
    # a context long enough to split needs the workspace
    need = B.eagle3_verify_attention_workspace(4, 8, 2, 128, 5000, B.KV_F32)
    assert need > 0
    assert _call(cap=6000, ctx_rows=5000, workspace=1, workspace_bytes=need - 4) == B.E_INVAL
