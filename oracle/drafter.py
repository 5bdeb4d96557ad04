"""fp64 EAGLE-3 drafter: encode, one decoder layer, draft head, d2t, with a
persistent draft KV (cached mode) and a from-scratch recompute (stateless mode).
Test infrastructure; see the package docstring.

Op sequence (memra_engine `eagle.rs`, module doc "Op-sequence", and the
`encode` / `draft_token` / `attn` methods):
  ENCODE, once per round:  g = fc . concat(aux_0, aux_1, aux_2)  (ascending tap order)
  DRAFT step, one token:
    e    = E[prev_tok]                      (an embedding row indexed by target id)
    cat  = [RMSNorm(e, input_layernorm) ; RMSNorm(g, hidden_norm)]    (2 n_embd)
    q,k,v= {q,k,v}_proj . cat; partial NeoX rope on q and k; append (k, v)
    attn = o_proj . SDPA(q, K, V)           (plain Llama attention, GQA)
    x1   = attn + g                         (the residual is the pre-norm g)
    z    = RMSNorm(x1, post_attention_layernorm)
    gsum = down . (silu(gate . z) * (up . z)) + x1
    logits = lm_head . RMSNorm(gsum, norm)  (draft vocabulary)
    g_next = gsum                           (the EAGLE recurrence)
  d2t (memra `d2t_map`): target_id = draft_id + d2t[draft_id].

Pairing and state (ExecuTorch PR #20153 description; pegainfer PR #707
description): a committed draft-KV row r pairs the target's tap features of
position r with the token at position r + 1; teacher-forced rows ("prefill",
"rebuild_after_verify") only need that row's K and V; a chain step j
(1-based) of a round over `committed` rows sits at position committed + j - 1,
and the round is rewound afterwards.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Union

import numpy as np

from . import kvquant
from .ledger import Ledger
from .numerics import (argmax_first, attention_causal, attention_decode,
                       bf16_bits_to_f64, rms_norm, rope_neox_partial, round_bf16, round_f16,
                       silu)

WEIGHT_NAMES = ("fc", "input_layernorm", "hidden_norm", "q_proj", "k_proj",
                "v_proj", "o_proj", "post_attention_layernorm", "gate_proj",
                "up_proj", "down_proj", "norm", "lm_head")


def _bits(t) -> np.ndarray:
    """uint16 bit patterns from a bf16 torch tensor or a uint16 array."""
    if isinstance(t, np.ndarray):
        assert t.dtype == np.uint16
        return t
    import torch
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass
class StepRecord:
    """What one draft step produced."""
    position: int
    g_in: np.ndarray            # recurrent hidden fed to the step
    tok_in: int                 # target id fed to the step
    logits: np.ndarray          # draft-vocabulary logits
    gsum: np.ndarray            # g_next
    draft_id: int
    target_id: int
    margin: float               # top-1 minus top-2 logit
    k: Optional[np.ndarray] = None   # KV row written ([n_kv, hd], roped k)
    v: Optional[np.ndarray] = None


def top2_margin(logits: np.ndarray) -> float:
    if logits.size < 2:
        return float("inf")
    part = np.partition(logits, -2)[-2:]
    return float(part[1] - part[0])


class DrafterOracle:
    """The drafter in fp64 with a persistent per-sequence draft KV."""

    def __init__(self, geom, weights: Dict[str, object],
                 embed: Union[np.ndarray, Callable[[np.ndarray], np.ndarray], object],
                 d2t, max_ctx: int = 0, max_seqs: int = 1, max_gamma: int = 16,
                 kv_format: str = "exact", dtype=np.float64, append_act: str = "exact"):
        """kv_format: "exact" keeps K/V rows as computed; "bf16" stores every
        element of a row rounded to the nearest bfloat16 (ties to even); "q8q5"
        stores each row in its quantized form (oracle.kvquant: q8_0 K, q5_1 V).
        With "bf16" and "q8q5" every read of the cache, the new row's own
        attention included, sees the stored values.
        dtype: float64 (the parity mode) or float32 (a timing mode: the same
        operations on fp32 arrays, used only as a CPU speed baseline).
        append_act: "exact", "bf16" or "f16": the rows of a teacher-forced append
        of more than 16 rows take their taps and their K/V-projection input
        [eN ; gN] rounded to the nearest bfloat16 / IEEE half (the engine's
        documented single-term activation formats for such appends; shorter
        appends are exact)."""
        assert append_act in ("exact", "bf16", "f16"), append_act
        self.append_round = {"exact": None, "bf16": round_bf16, "f16": round_f16}[append_act]
        assert dtype in (np.float64, np.float32), dtype
        self.dt = dtype
        assert kv_format in ("exact", "bf16", "q8q5"), kv_format
        self.kv_format = kv_format
        self.kv_q = kv_format == "q8q5"
        self.n = geom.n_embd
        self.nh = geom.n_head
        self.nkv = geom.n_head_kv
        self.hd = geom.head_dim
        self.ff = geom.n_ff
        self.dv = geom.draft_vocab
        self.vt = geom.target_vocab
        self.rot = geom.rope_dim
        self.theta = float(geom.rope_theta)
        self.eps = float(geom.rms_eps)
        # bf16 weights (bit patterns or tensors), or fp64 arrays used as given (the
        # int4 weights' exact values, oracle.int4)
        W = {k: (weights[k] if isinstance(weights[k], np.ndarray) and weights[k].dtype == np.float64
                 else bf16_bits_to_f64(_bits(weights[k]))).astype(dtype, copy=False)
             for k in WEIGHT_NAMES}
        self.W = W
        assert W["fc"].shape == (self.n, 3 * self.n), "fc in != 3 n_embd"
        assert W["q_proj"].shape == (self.nh * self.hd, 2 * self.n), "q_proj shape"
        assert W["k_proj"].shape == (self.nkv * self.hd, 2 * self.n), "k_proj shape"
        assert W["lm_head"].shape == (self.dv, self.n), "lm_head out != draft_vocab"
        d = np.asarray(d2t.cpu().numpy() if hasattr(d2t, "cpu") else d2t, dtype=np.int64)
        assert d.shape == (self.dv,)
        tgt = np.arange(self.dv, dtype=np.int64) + d
        assert tgt.min() >= 0 and tgt.max() < self.vt, "d2t maps outside the target vocab"
        self.d2t = d
        if callable(embed):
            self._embed_fn = embed
        else:
            tab = _bits(embed)
            assert tab.shape == (self.vt, self.n)
            self._embed_fn = lambda toks: tab[np.asarray(toks, dtype=np.int64)]
        self.ledger: Optional[Ledger] = None
        if max_ctx > 0:
            self.ledger = Ledger(max_ctx, max_seqs, max_gamma)
            rows = self.ledger.rows
            self.K = [np.zeros((rows, self.nkv, self.hd), dtype) for _ in range(max_seqs)]
            self.V = [np.zeros((rows, self.nkv, self.hd), dtype) for _ in range(max_seqs)]

    # ------------------------------------------------------------------
    # pieces of the op sequence
    # ------------------------------------------------------------------
    def embed(self, toks) -> np.ndarray:
        toks = np.asarray(toks, dtype=np.int64).reshape(-1)
        assert toks.min() >= 0 and toks.max() < self.vt
        return bf16_bits_to_f64(_bits(self._embed_fn(toks))).astype(self.dt, copy=False)

    def encode(self, aux: Sequence[np.ndarray]) -> np.ndarray:
        """g = fc . concat(aux_0, aux_1, aux_2) (memra `encode`); rows or one vector."""
        assert len(aux) == 3
        cat = np.concatenate([np.asarray(a, dtype=self.dt) for a in aux], axis=-1)
        return cat @ self.W["fc"].T

    def input_cat(self, g: np.ndarray, toks) -> np.ndarray:
        """[RMSNorm(E[tok], input_layernorm) ; RMSNorm(g, hidden_norm)] per row."""
        e = self.embed(toks).reshape(np.shape(g))
        eN = rms_norm(e, self.W["input_layernorm"], self.eps)
        gN = rms_norm(g, self.W["hidden_norm"], self.eps)
        return np.concatenate([eN, gN], axis=-1)

    def qkv(self, cat: np.ndarray, positions):
        """Roped q [.., nh, hd], roped k [.., nkv, hd] and v [.., nkv, hd]."""
        lead = cat.shape[:-1]
        q = (cat @ self.W["q_proj"].T).reshape(*lead, self.nh, self.hd)
        k = (cat @ self.W["k_proj"].T).reshape(*lead, self.nkv, self.hd)
        v = (cat @ self.W["v_proj"].T).reshape(*lead, self.nkv, self.hd)
        q = rope_neox_partial(q, positions, self.rot, self.theta)
        k = rope_neox_partial(k, positions, self.rot, self.theta)
        return q, k, v

    def after_attention(self, o: np.ndarray, g: np.ndarray):
        """o_proj + residual, post-attention norm, SwiGLU MLP + residual."""
        x1 = o @ self.W["o_proj"].T + g
        z = rms_norm(x1, self.W["post_attention_layernorm"], self.eps)
        act = silu(z @ self.W["gate_proj"].T) * (z @ self.W["up_proj"].T)
        return act @ self.W["down_proj"].T + x1

    def head(self, gsum: np.ndarray) -> np.ndarray:
        """Draft-vocabulary logits: lm_head . RMSNorm(gsum, norm)."""
        return rms_norm(gsum, self.W["norm"], self.eps) @ self.W["lm_head"].T

    def d2t_map(self, draft_id: int) -> int:
        """memra `d2t_map`: target = draft + d2t[draft] (d2t is a delta)."""
        return int(draft_id + self.d2t[draft_id])

    def pick(self, logits: np.ndarray):
        i = argmax_first(logits)
        return i, self.d2t_map(i)

    # ------------------------------------------------------------------
    # full layer over T rows from scratch (the plain definition)
    # ------------------------------------------------------------------
    def layer_full(self, G: np.ndarray, toks, positions=None):
        """Run the decoder layer over rows (G[t], toks[t]) at positions 0..T-1
        with causal attention; returns (logits [T, dv], gsum [T, n])."""
        T = G.shape[0]
        pos = np.arange(T) if positions is None else np.asarray(positions)
        cat = self.input_cat(G, toks)
        q, k, v = self.qkv(cat, pos)
        o = attention_causal(q, k, v).reshape(T, self.nh * self.hd)
        gsum = self.after_attention(o, G)
        return self.head(gsum), gsum

    # ------------------------------------------------------------------
    # one cached step: row at `pos` over K/V rows [0, pos)
    # ------------------------------------------------------------------
    def step(self, g: np.ndarray, tok: int, pos: int, Kctx: np.ndarray,
             Vctx: np.ndarray, nctx: int = None) -> StepRecord:
        """nctx: context rows Kctx[:nctx] attended before the new row (default pos,
        the persistent KV; a round-local scratch passes the round's own rows)."""
        nctx = pos if nctx is None else nctx
        cat = self.input_cat(g[None, :], [tok])[0]
        q, k, v = self.qkv(cat, pos)
        k, v = self._kv_rows(k, v)
        K = np.concatenate([Kctx[:nctx], k[None]], axis=0)
        V = np.concatenate([Vctx[:nctx], v[None]], axis=0)
        o = attention_decode(q, K, V).reshape(-1)
        gsum = self.after_attention(o, g)
        logits = self.head(gsum)
        i, t = self.pick(logits)
        return StepRecord(pos, g.copy(), int(tok), logits, gsum, i, t,
                          top2_margin(logits), k, v)

    # ------------------------------------------------------------------
    # stateful entry points (pegainfer PR #707 description)
    # ------------------------------------------------------------------
    def _kv_rows(self, k, v):
        """The K/V rows as the cache stores them."""
        if self.kv_format == "bf16":
            return round_bf16(k), round_bf16(v)
        if not self.kv_q:
            return k, v
        return kvquant.k_stored(k), kvquant.v_stored(v)

    def _append(self, s: int, start: int, aux, toks) -> None:
        toks = np.asarray(toks, dtype=np.int64).reshape(-1)
        T = toks.shape[0]
        if T == 0:
            return
        taps = [np.asarray(a).reshape(T, self.n) for a in aux]
        rnd = self.append_round if T > 16 else None
        if rnd:
            taps = [rnd(a).astype(self.dt) for a in taps]
        f = self.encode(taps)
        cat = self.input_cat(f, toks)
        if rnd:
            cat = rnd(cat).astype(self.dt)
        _, k, v = self.qkv(cat, start + np.arange(T))
        k, v = self._kv_rows(k, v)
        self.K[s][start:start + T] = k
        self.V[s][start:start + T] = v

    def prefill(self, s: int, aux, toks) -> None:
        """Teacher-forced rows (aux of position r, token of position r + 1)."""
        T = int(np.asarray(toks).size)
        start = self.ledger.prefill(s, T)
        self._append(s, start, aux, toks)

    def rebuild_after_verify(self, s: int, n_accepted: int, aux, toks) -> None:
        """Commit the a + 1 rows (boundary aux, boundary token),
        (aux of d_i's predecessor, d_i) for i <= a."""
        assert int(np.asarray(toks).size) == n_accepted + 1
        start = self.ledger.rebuild(s, n_accepted)
        self._append(s, start, aux, toks)

    def rewind(self, s: int, new_len: int) -> None:
        self.ledger.rewind(s, new_len)

    def draft_chain(self, s: int, boundary_aux, boundary_tok: int, gamma: int,
                    keep_spec: bool = False) -> List[StepRecord]:
        """One chain round: encode the boundary taps, gamma_eff greedy steps
        over the persistent KV, then rewind (unless keep_spec)."""
        L = self.ledger.committed(s)
        g_eff = self.ledger.chain(s, gamma, keep_spec=keep_spec)
        g = self.encode([np.asarray(a).reshape(self.n) for a in boundary_aux])
        tok = int(boundary_tok)
        recs: List[StepRecord] = []
        for j in range(g_eff):
            pos = L + j
            r = self.step(g, tok, pos, self.K[s], self.V[s])
            self.K[s][pos] = r.k
            self.V[s][pos] = r.v
            recs.append(r)
            g, tok = r.gsum, r.target_id
        return recs

    def draft_chain_round_local(self, s: int, boundary_aux, boundary_tok: int,
                                gamma: int) -> List[StepRecord]:
        """The scratch-KV drafter (memra_engine `eagle.rs`, `Eagle3Scratch`: a small
        draft KV emptied at the start of every round): step j attends over the
        round's own rows 0..j only; rope positions still continue from the
        committed length; the persistent KV and the ledger lengths are untouched."""
        L = self.ledger.committed(s)
        g_eff = self.ledger.chain(s, gamma, round_local=True)
        g = self.encode([np.asarray(a).reshape(self.n) for a in boundary_aux])
        tok = int(boundary_tok)
        Ks = np.zeros((max(g_eff, 1), self.nkv, self.hd), self.dt)
        Vs = np.zeros((max(g_eff, 1), self.nkv, self.hd), self.dt)
        recs: List[StepRecord] = []
        for j in range(g_eff):
            r = self.step(g, tok, L + j, Ks, Vs, nctx=j)
            Ks[j], Vs[j] = r.k, r.v
            recs.append(r)
            g, tok = r.gsum, r.target_id
        return recs


class StatelessChain:
    """The same chain computed from scratch at every step: all committed rows
    and all chain rows so far are run through the full layer with causal
    attention and the last row is read (ExecuTorch PR #20153 description: the
    cached chain must equal this recompute)."""

    def __init__(self, drafter: DrafterOracle):
        self.d = drafter

    def run(self, committed_aux, committed_toks, boundary_aux, boundary_tok,
            gamma: int, position0: int = 0) -> List[StepRecord]:
        """position0: position of the first row (the committed rows, else the first
        chain row); a round-local chain is the recompute over its own rows only,
        placed at the committed length."""
        d = self.d
        toks_c = np.asarray(committed_toks, dtype=np.int64).reshape(-1)
        L = toks_c.shape[0]
        if L:
            G_c = d.encode([np.asarray(a).reshape(L, d.n) for a in committed_aux])
        else:
            G_c = np.zeros((0, d.n), d.dt)
        g = d.encode([np.asarray(a).reshape(d.n) for a in boundary_aux])
        chain_G: List[np.ndarray] = []
        chain_T: List[int] = []
        tok = int(boundary_tok)
        recs: List[StepRecord] = []
        for j in range(gamma):
            chain_G.append(g)
            chain_T.append(tok)
            G = np.concatenate([G_c, np.stack(chain_G)], axis=0)
            T = np.concatenate([toks_c, np.asarray(chain_T, dtype=np.int64)])
            logits, gsum = d.layer_full(G, T, position0 + np.arange(G.shape[0]))
            lg, gs = logits[-1], gsum[-1]
            i, t = d.pick(lg)
            recs.append(StepRecord(position0 + L + j, g.copy(), tok, lg, gs, i, t,
                                   top2_margin(lg)))
            g, tok = gs, t
        return recs
