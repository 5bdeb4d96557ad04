"""A chain round is capturable as a HIP graph: the round's launches read every
buffer through stable device pointers and make no host synchronisation, so a
round at a fixed position (boundary taps, rewound afterwards) replays exactly.
Each replay is checked against the eager round, with eager rounds and
synchronisations between the replays, for the persistent and the stored-boundary
protocol (ExecuTorch PR #20156 description: the verify and draft steps run on
stable buffers and can be graph-captured)."""
import pytest
import torch

from synth import TINY, gen, small_variant
from tests.common import aux_np, toks_np
from tests.gpu_harness import gpu_drafter, say, to_dev_aux

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("stored", [False, True], ids=["taps", "stored"])
@pytest.mark.parametrize("cfg,L,gamma", [(TINY, 63, 3), (small_variant(), 300, 5)], ids=["tiny", "ragged"])
def test_graph_replay_equals_eager_round(cfg, L, gamma, stored):
    say(f"[graph] {cfg.name} L={L} gamma={gamma} stored={stored}")
    wd = gen.drafter_weights(cfg, device="cuda")
    dr = gpu_drafter(cfg, wd, max_ctx=L + gamma + 16)
    aux, toks = aux_np(cfg, 0, L), toks_np(cfg, 0, L)
    baux = to_dev_aux(aux_np(cfg, 1, 1), slice(0, 1))
    btok = torch.as_tensor(toks_np(cfg, 1, 1), dtype=torch.int32).cuda()
    dr.prefill(0, torch.as_tensor(toks, dtype=torch.int32).cuda(), to_dev_aux(aux),
               next_aux=baux if stored else None)
    out = torch.empty((1, gamma), dtype=torch.int32, device="cuda")
    other = torch.empty_like(out)
    side = torch.cuda.Stream()

    def chain(o):
        dr.draft_chain([0], btok, None if stored else [a.contiguous() for a in baux], gamma, out=o,
                       stream=torch.cuda.current_stream())

    with torch.cuda.stream(side):
        chain(out)
    torch.cuda.synchronize()
    ref = out.clone()
    k0, v0 = dr.kv_read(0, 0, L + gamma)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(out)
    torch.cuda.synchronize()
    assert dr.kv_len(0) == (L, 0)          # the capture ran the round's bookkeeping once
    for _ in range(4):
        out.fill_(-7)
        with torch.cuda.stream(side):
            chain(other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(other, ref)
        k, v = dr.kv_read(0, 0, L + gamma)   # the same rows, the round's own included
        assert torch.equal(k, k0) and torch.equal(v, v0)
    assert dr.status() == 0
    del g
    dr.close()
