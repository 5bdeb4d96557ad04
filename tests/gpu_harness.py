"""Helpers shared by the GPU tests: build the engine and the oracle on the same
seeded inputs, and compare a chain round step by step."""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import List

import numpy as np
import torch

from synth import gen
from synth.configs import DrafterConfig

MARGIN = 0.05        # a step is pinned iff the oracle's top-1 - top-2 margin exceeds this
LOGIT_TOL = 2e-2     # max-abs on pinned steps
HIDDEN_TOL = 1e-2    # relative L2 on pinned steps


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_drafter(cfg: DrafterConfig, weights_dev, max_ctx=None, max_gamma=16, max_seqs=1, append_act=0,
                kv_dtype=0, token_table=0):
    from eagle_draft_head_amd.drafter import Drafter
    return Drafter(cfg, weights_dev, weights_dev["d2t"].cpu(), max_ctx or cfg.max_ctx_eff,
                   max_gamma=max_gamma, max_seqs=max_seqs, append_act=append_act, kv_dtype=kv_dtype,
                   token_table=token_table)


def weights_both(cfg: DrafterConfig, lazy_embed_host=False):
    """(device weights, host weights) with identical bits; generated on the GPU."""
    wd = gen.drafter_weights(cfg, device="cuda")
    wh = {k: v.cpu() for k, v in wd.items() if not (lazy_embed_host and k == "embed")}
    return wd, wh


@dataclass
class StepCompare:
    pinned: bool
    id_gpu: int
    id_ref: int
    logit_err: float
    hidden_rel: float
    margin: float


def compare_round(recs, out_ids, geff, logits, hidden, b=0) -> List[StepCompare]:
    """Compare one sequence's chain round (GPU outputs) with oracle records."""
    assert geff == len(recs)
    res = []
    pinned = True
    ids = out_ids[b].tolist()
    for j, r in enumerate(recs):
        pinned = pinned and r.margin > MARGIN
        lg = logits[b, j].double().cpu().numpy()
        hg = hidden[b, j + 1].double().cpu().numpy()
        herr = float(np.linalg.norm(hg - r.gsum) / max(np.linalg.norm(r.gsum), 1e-30))
        res.append(StepCompare(pinned, int(ids[j]), int(r.target_id),
                               float(np.abs(lg - r.logits).max()), herr, r.margin))
    return res


def check_round(cmp: List[StepCompare], where=""):
    """Pinned steps: ids, logits and hidden.  The first unpinned step still has the
    oracle's inputs (every earlier id matched), so its logits and hidden are held
    to the same bar; only its id may differ.  Later steps are not compared."""
    for j, c in enumerate(cmp):
        assert c.logit_err <= LOGIT_TOL, f"{where} step {j}: logits max-abs {c.logit_err:.3e}"
        assert c.hidden_rel <= HIDDEN_TOL, f"{where} step {j}: hidden rel-L2 {c.hidden_rel:.3e}"
        if not c.pinned:
            break
        assert c.id_gpu == c.id_ref, f"{where} step {j}: id {c.id_gpu} != {c.id_ref} (margin {c.margin:.3f})"


def compared_steps(cmp: List[StepCompare]) -> int:
    """Steps whose logits and hidden check_round compares."""
    n = 0
    for c in cmp:
        n += 1
        if not c.pinned:
            break
    return n


def to_dev_aux(aux_np_list, rows=None):
    out = []
    for a in aux_np_list:
        t = torch.as_tensor(np.ascontiguousarray(a if rows is None else a[rows]), dtype=torch.float32)
        out.append(t.cuda().contiguous())
    return out


class GpuChainAdapter:
    """Exposes the GPU drafter through the greedy loop's drafter interface."""

    def __init__(self, drafter):
        self.d = drafter

    def prefill(self, s, aux, toks):
        self.d.prefill(s, torch.as_tensor(np.asarray(toks), dtype=torch.int32).cuda(),
                       to_dev_aux(aux))

    def draft_chain_ids(self, s, boundary_aux, boundary_tok, gamma):
        tok = torch.tensor([int(boundary_tok)], dtype=torch.int32, device="cuda")
        aux = [torch.as_tensor(np.asarray(a), dtype=torch.float32).reshape(1, -1).cuda()
               for a in boundary_aux]
        out, geff, _, _ = self.d.draft_chain([s], tok, aux, gamma)
        return out[0, :geff[0]].tolist()

    def rebuild_after_verify(self, s, a, aux, toks):
        self.d.rebuild_after_verify([s], [a], torch.as_tensor(np.asarray(toks), dtype=torch.int32).cuda(),
                                    to_dev_aux(aux))
