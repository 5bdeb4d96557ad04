"""The verify side on the GPU: the synthetic target trunk (eagle3_trunk_*) against
the oracle trunk, and the whole greedy speculative loop on the device
(eagle3_generate: the GPU drafter drafts, the GPU trunk verifies the window in one
forward, the accept walk runs on the device) against plain greedy decoding.

The greedy loop must reproduce greedy decoding token for token (ExecuTorch PR
#20156 description: greedy verification keeps the output identical; memra_engine
`generate_spec_eagle`).  Checked against the oracle's plain greedy decoding of
the same trunk (fp64, one token at a time) and against the GPU trunk decoding one
token at a time, for chain lengths 1, 3 and 5, prompts of 1, 17 and 64 tokens, and
with the structured "echo" weights under which every draft is accepted."""
import numpy as np
import pytest
import torch

from eagle_draft_head_amd import binding as B
from oracle import TrunkOracle, greedy_plain, greedy_speculative
from oracle.loop import OracleChainAdapter
from synth import TINY, gen
from tests.common import make_oracle
from tests.gpu_harness import gpu_drafter, say

pytestmark = pytest.mark.gpu

MAX_CTX = 400
MAX_TOKENS = 80


@pytest.fixture(scope="module")
def tiny():
    w = gen.drafter_weights(TINY)
    tw = gen.trunk_weights(TINY)
    return w, tw


class GpuTrunk:
    def __init__(self, tw, embed, max_ctx=MAX_CTX, max_tokens=MAX_TOKENS):
        self.dev = {k: v.cuda() for k, v in tw.items()}
        self.embed = embed.cuda()
        cfg = B.make_trunk_config(TINY, TINY.trunk_layers, max_ctx, max_tokens)
        self.h = B.eagle3_trunk_load(cfg, B.make_trunk_weights(self.dev, self.embed, TINY.trunk_layers))
        self.n = TINY.n_embd

    def forward(self, toks):
        T = len(toks)
        tok = torch.tensor(toks, dtype=torch.int32, device="cuda")
        ids = torch.empty(T, dtype=torch.int32, device="cuda")
        taps = [torch.empty((T, self.n), dtype=torch.float32, device="cuda") for _ in range(3)]
        B.eagle3_trunk_forward(self.h, T, tok, ids, *taps)
        torch.cuda.synchronize()
        return ids.tolist(), [t.cpu() for t in taps]

    def close(self):
        B.eagle3_trunk_free(self.h)


def _oracle_trunk(tw, embed):
    return TrunkOracle(TINY, tw, embed, TINY.trunk_layers)


def _top2(logits):
    p = np.partition(logits, -2)[-2:]
    return float(p[1] - p[0])


def test_trunk_forward_matches_the_oracle_trunk(tiny):
    w, tw = tiny
    prompt = gen.tokens(TINY, 77, 40).tolist()
    gt = GpuTrunk(tw, w["embed"])
    ids, taps = gt.forward(prompt)
    ot = _oracle_trunk(tw, w["embed"])
    for t, tok in enumerate(prompt):
        lg, tp = ot.step(tok)
        for j in range(3):
            ref = tp[j]
            got = taps[j][t].double().numpy()
            assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-5, (t, j)
        if _top2(lg) > 1e-4:
            assert ids[t] == int(np.argmax(lg)), t
    gt.close()


def test_trunk_window_equals_one_token_at_a_time(tiny):
    """A window of T tokens computes each row bit for bit as T forwards of one
    token do; rollback truncates the cache so a forward can be redone."""
    w, tw = tiny
    prompt = gen.tokens(TINY, 78, 23).tolist()
    win = gen.tokens(TINY, 79, 6).tolist()
    a = GpuTrunk(tw, w["embed"])
    a.forward(prompt)
    ids_w, taps_w = a.forward(win)
    b = GpuTrunk(tw, w["embed"])
    b.forward(prompt)
    for t, tok in enumerate(win):
        ids_1, taps_1 = b.forward([tok])
        assert ids_1[0] == ids_w[t]
        for j in range(3):
            assert torch.equal(taps_1[j][0], taps_w[j][t]), (t, j)
    assert B.eagle3_trunk_len(a.h) == len(prompt) + len(win)
    B.eagle3_trunk_rollback(a.h, len(prompt) + 2)
    ids_r, taps_r = a.forward(win[2:])
    assert ids_r == ids_w[2:] and all(torch.equal(taps_r[j], taps_w[j][2:]) for j in range(3))
    a.close()
    b.close()


def _gpu_greedy(gt, prompt, max_new):
    B.eagle3_trunk_rollback(gt.h, 0)
    ids, _ = gt.forward(prompt)
    out = [ids[-1]]
    while len(out) < max_new:
        ids, _ = gt.forward([out[-1]])
        out.append(ids[0])
    return out


@pytest.mark.parametrize("act", ["split", "default"])
@pytest.mark.parametrize("plen,gamma", [(1, 3), (17, 1), (17, 3), (64, 5)])
def test_device_loop_equals_greedy_decoding(tiny, plen, gamma, act):
    """Both append forms reproduce greedy decoding.  With split (fp32-grade)
    appends the drafter also drafts and accepts exactly as the oracle drafter does;
    the default's fp16 prompt rows may move a near-tied draft, which changes the
    counts but never the output."""
    w, tw = tiny
    max_new = 60
    prompt = gen.tokens(TINY, 50 + plen, plen).tolist()
    ref = greedy_plain(_oracle_trunk(tw, w["embed"]), prompt, max_new)
    gt = GpuTrunk(tw, w["embed"])
    assert _gpu_greedy(gt, prompt, max_new) == ref
    dr = gpu_drafter(TINY, {k: v.cuda() for k, v in w.items()}, max_ctx=MAX_CTX,
                     append_act=B.APPEND_SPLIT if act == "split" else B.APPEND_DEFAULT)
    out, drafted, accepted = B.eagle3_generate(dr.ctx, 0, gt.h, prompt, max_new, gamma)
    assert out == ref
    # the same loop with the oracle trunk and drafter drafts and accepts alike
    orc = make_oracle(TINY, w, max_ctx=MAX_CTX)
    o_out, o_dr, o_ac = greedy_speculative(_oracle_trunk(tw, w["embed"]), OracleChainAdapter(orc), prompt,
                                           max_new, gamma)
    assert o_out == ref
    say(f"[device loop] {act} plen={plen} gamma={gamma}: drafted {drafted} accepted {accepted} "
        f"(oracle loop {o_dr}/{o_ac})")
    if act == "split":
        assert (drafted, accepted) == (o_dr, o_ac)
    else:
        assert 0 <= accepted <= drafted and drafted > 0
    assert dr.kv_len(0)[1] == 0                       # no speculative rows are left
    dr.close()
    gt.close()


@pytest.mark.parametrize("gamma", [1, 3, 5])
def test_device_loop_full_acceptance(tiny, gamma):
    from tests.test_oracle_loop import echo_weights
    w, tw = tiny
    w_e, tw_e, image = echo_weights(w, tw)
    prompt = [int(image[7]), int(image[100]), int(image[33])]
    max_new = 40
    ref = greedy_plain(_oracle_trunk(tw_e, w_e["embed"]), prompt, max_new)
    assert len(set(ref)) == 1
    gt = GpuTrunk(tw_e, w_e["embed"])
    dr = gpu_drafter(TINY, {k: v.cuda() for k, v in w_e.items()}, max_ctx=MAX_CTX)
    out, drafted, accepted = B.eagle3_generate(dr.ctx, 0, gt.h, prompt, max_new, gamma)
    assert out == ref
    assert accepted == drafted > 0
    # every round accepts gamma drafts and adds the bonus: (max_new - 1) / (gamma + 1) rounds
    rounds = -(-(max_new - 1) // (gamma + 1))
    assert drafted == rounds * gamma
    dr.close()
    gt.close()


def test_trunk_errors_and_status(tiny):
    w, tw = tiny
    gt = GpuTrunk(tw, w["embed"], max_ctx=40, max_tokens=16)
    with pytest.raises(B.Eagle3Error) as e:
        gt.forward(list(range(17)))                    # window above max_tokens
    assert e.value.code == B.E_INVAL
    gt.forward(list(range(16)))
    gt.forward(list(range(16)))
    with pytest.raises(B.Eagle3Error) as e:
        gt.forward(list(range(9)))                     # 32 + 9 > 40 rows
    assert e.value.code == B.E_CAPACITY
    assert B.eagle3_trunk_len(gt.h) == 32
    with pytest.raises(B.Eagle3Error) as e:
        B.eagle3_trunk_rollback(gt.h, 33)
    assert e.value.code == B.E_INVAL
    assert B.eagle3_trunk_status(gt.h) == 0
    gt.forward([5, TINY.target_vocab + 3])            # an id outside the vocabulary
    assert B.eagle3_trunk_status(gt.h) == B.TRUNK_BAD_TOKEN
    assert B.eagle3_trunk_status(gt.h) == 0           # read and cleared
    dr = gpu_drafter(TINY, {k: v.cuda() for k, v in w.items()}, max_ctx=MAX_CTX)
    with pytest.raises(B.Eagle3Error) as e:            # window gamma + 1 above max_tokens
        B.eagle3_generate(dr.ctx, 0, gt.h, [1, 2], 10, 16)
    assert e.value.code == B.E_INVAL
    with pytest.raises(B.Eagle3Error) as e:            # prompt + max_new + gamma above max_ctx
        B.eagle3_generate(dr.ctx, 0, gt.h, [1, 2], 40, 3)
    assert e.value.code == B.E_CAPACITY
    dr.close()
    gt.close()


@pytest.mark.parametrize("gamma", [2, 3, 5])
def test_device_loop_partial_acceptance(tiny, gamma):
    """The alternating trunk: every round accepts the first draft and rejects the
    second, so the accept walk, the rollback and the rebuild of a + 1 = 2 rows run
    with 0 < a < gamma every round."""
    from tests.test_oracle_loop import alternating_weights
    w, tw = tiny
    w_a, tw_a, prompt = alternating_weights(w, tw)
    max_new = 41
    ref = greedy_plain(_oracle_trunk(tw_a, w_a["embed"]), prompt, max_new)
    gt = GpuTrunk(tw_a, w_a["embed"])
    dr = gpu_drafter(TINY, {k: v.cuda() for k, v in w_a.items()}, max_ctx=MAX_CTX)
    out, drafted, accepted = B.eagle3_generate(dr.ctx, 0, gt.h, prompt, max_new, gamma)
    assert out == ref
    assert drafted % gamma == 0 and accepted == drafted // gamma > 0
    orc = make_oracle(TINY, w_a, max_ctx=MAX_CTX)
    o_out, o_dr, o_ac = greedy_speculative(_oracle_trunk(tw_a, w_a["embed"]), OracleChainAdapter(orc),
                                           prompt, max_new, gamma)
    assert (o_out, o_dr, o_ac) == (ref, drafted, accepted)
    # committed rows = position of the pending boundary token - 1
    committed = len(prompt) - 1 + (drafted // gamma) * 2
    assert dr.kv_len(0) == (committed, 0)
    dr.close()
    gt.close()
