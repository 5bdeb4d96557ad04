"""The greedy speculative loop with the oracle drafter reproduces plain greedy
decoding of the tiny trunk token for token (memra `generate_spec_eagle` doc;
ExecuTorch PR #20153/#20156 descriptions)."""
import numpy as np
import pytest
import torch

from oracle import TrunkOracle, greedy_plain, greedy_speculative
from oracle.loop import OracleChainAdapter
from synth import TINY, gen
from tests.common import make_oracle


@pytest.fixture(scope="module")
def tiny():
    w = gen.drafter_weights(TINY)
    tw = gen.trunk_weights(TINY)
    return w, tw


def _trunk(tw, embed):
    return TrunkOracle(TINY, tw, embed, TINY.trunk_layers)


@pytest.mark.parametrize("plen,gamma,max_new", [(1, 3, 12), (2, 1, 10), (17, 3, 24),
                                                (64, 5, 30)])
def test_speculative_equals_greedy(tiny, plen, gamma, max_new):
    w, tw = tiny
    trunk = _trunk(tw, w["embed"])
    prompt = gen.tokens(TINY, 50 + plen, plen).tolist()
    ref = greedy_plain(trunk, prompt, max_new)
    d = make_oracle(TINY, w, max_ctx=plen + max_new + gamma + 4)
    out, drafted, acc = greedy_speculative(trunk, OracleChainAdapter(d), prompt,
                                           max_new, gamma)
    assert out == ref
    assert drafted > 0 and 0 <= acc <= drafted
    # committed rows = position of the boundary token - 1 (here: all emitted
    # tokens except the pending bonus are committed)
    assert d.ledger.committed(0) >= plen - 1


def echo_weights(w, tw):
    """Structured weights under which the trunk repeats its last token and the
    drafter predicts that repetition: full acceptance every round."""
    n = TINY.n_embd
    w = dict(w)
    tw = dict(tw)
    for k in list(tw):
        if k.startswith("layers.") and not k.endswith("norm"):
            tw[k] = torch.zeros_like(tw[k])
    tw["lm_head"] = w["embed"].clone()                 # tied: predicts "same token"
    fc = torch.zeros(n, 3 * n, dtype=torch.bfloat16)
    fc[:, :n] = torch.eye(n, dtype=torch.bfloat16)     # g = tap 0 = embedding
    w["fc"] = fc
    w["o_proj"] = torch.zeros_like(w["o_proj"])
    w["down_proj"] = torch.zeros_like(w["down_proj"])
    image = torch.arange(TINY.draft_vocab) + w["d2t"]
    w["lm_head"] = w["embed"][image].clone()           # draft row i ~ target row d2t(i)
    return w, tw, image


@pytest.mark.parametrize("gamma", [1, 3, 4])
def test_full_acceptance_path(tiny, gamma):
    w, tw, image = echo_weights(*tiny)
    trunk = _trunk(tw, w["embed"])
    prompt = [int(image[7]), int(image[100]), int(image[33])]
    ref = greedy_plain(trunk, prompt, 25)
    assert len(set(ref)) == 1                          # the trunk repeats
    d = make_oracle(TINY, w, max_ctx=64)
    out, drafted, acc = greedy_speculative(trunk, OracleChainAdapter(d), prompt, 25, gamma)
    assert out == ref
    assert acc == drafted > 0                          # every draft accepted


def alternating_weights(w, tw):
    """The echo weights with the trunk's lm_head rows swapped in pairs (2i <-> 2i+1):
    the trunk then alternates a, b, a, b, ... (b the pair partner of a), while the
    drafter still predicts the token before its input one.  The first draft of a
    round (x_{n-1} = x_{n+1}) is accepted and the second (x_{n-1} != x_{n+2}) is not,
    so every round of gamma >= 2 accepts exactly one draft.  Returns the weights and
    a prompt [a, b] whose pair lies in the drafter's vocabulary image."""
    w, tw, image = echo_weights(w, tw)
    E = w["embed"]
    perm = torch.arange(E.shape[0]) ^ 1
    tw["lm_head"] = E[perm].clone()
    img = set(image.tolist())
    a = next(int(t) for t in image.tolist() if t % 2 == 0 and t + 1 in img)
    return w, tw, [a, a + 1]


@pytest.mark.parametrize("gamma", [2, 3, 5])
def test_partial_acceptance_path(tiny, gamma):
    w, tw, prompt = alternating_weights(*tiny)
    trunk = _trunk(tw, w["embed"])
    ref = greedy_plain(trunk, prompt, 31)
    assert ref[:4] == [prompt[0], prompt[1], prompt[0], prompt[1]]   # the trunk alternates
    d = make_oracle(TINY, w, max_ctx=64)
    out, drafted, acc = greedy_speculative(trunk, OracleChainAdapter(d), prompt, 31, gamma)
    assert out == ref
    rounds = drafted // gamma
    assert acc == rounds                    # exactly one draft accepted per round
