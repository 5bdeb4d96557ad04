"""A small object wrapper over the C entry points (argument marshalling only).

Device memory for inputs and outputs comes from torch tensors on the current
GPU; every computation runs inside libeagle3.so.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import torch

from . import binding as B


class Drafter:
    def __init__(self, geom, weights: Dict[str, torch.Tensor], d2t, max_ctx: int,
                 max_gamma: int = 16, max_seqs: int = 1, kv_dtype: int = B.KV_F32, stream=None,
                 weight_format: int = B.WEIGHTS_BF16, append_act: int = B.APPEND_DEFAULT,
                 token_table: int = B.TABLE_DEFAULT):
        if not torch.cuda.is_available():
            raise RuntimeError("the eagle3 engine needs a GPU")
        self.geom = geom
        self.n = geom.n_embd
        self.dv = geom.draft_vocab
        self.max_gamma = max_gamma
        self.kv_dtype = kv_dtype
        self.cfg = B.make_config(geom, max_ctx, max_gamma, max_seqs, kv_dtype, weight_format,
                                 append_act, token_table)
        self._w = B.make_weights(weights, d2t)
        self.ctx = B.eagle3_load(self.cfg, self._w, stream)

    def close(self):
        if self.ctx:
            B.eagle3_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- entry points ---------------------------------------------------------
    def prefill(self, seq: int, tok: torch.Tensor, aux: Sequence[torch.Tensor],
                next_aux: Optional[Sequence[torch.Tensor]] = None, stream=None):
        """Append the teacher-forced rows; with next_aux (three [n] fp32 taps) also
        store the boundary feature a chain with aux=None starts from."""
        T = int(tok.numel())
        a = aux if T > 0 else (None, None, None)
        na = next_aux if next_aux is not None else (None, None, None)
        B.eagle3_prefill(self.ctx, seq, T, tok if T > 0 else None, a[0], a[1], a[2], na[0], na[1],
                         na[2], stream)

    def draft_chain(self, seq_ids: Sequence[int], boundary_tok: torch.Tensor,
                    aux: Optional[Sequence[torch.Tensor]], gamma: int,
                    out: Optional[torch.Tensor] = None, keep_spec: bool = False,
                    debug: bool = False, stream=None, round_local: bool = False):
        """One chain round per sequence; aux=None starts from the stored boundary
        features (set by prefill / rebuild_after_verify with next_aux); round_local
        attends over the round's own rows only (a scratch KV emptied every round)."""
        n_seq = len(seq_ids)
        dev = boundary_tok.device
        if out is None:
            out = torch.empty((n_seq, max(gamma, 1)), dtype=torch.int32, device=dev)
        logits = hidden = None
        if debug:
            logits = torch.zeros((n_seq, max(gamma, 1), self.dv), dtype=torch.float32, device=dev)
            hidden = torch.zeros((n_seq, gamma + 1, self.n), dtype=torch.float32, device=dev)
        flags = ((B.KEEP_SPEC if keep_spec else 0) | (B.STORED_BOUNDARY if aux is None else 0)
                 | (B.ROUND_LOCAL if round_local else 0))
        a = aux if aux is not None else (None, None, None)
        geff = B.eagle3_draft_chain(self.ctx, list(seq_ids), boundary_tok, a[0], a[1], a[2],
                                    gamma, out, flags, logits, hidden, stream)
        return out, geff, logits, hidden

    def rebuild_after_verify(self, seq_ids: Sequence[int], n_accepted: Sequence[int],
                             tok: torch.Tensor, aux: Sequence[torch.Tensor],
                             next_aux: Optional[Sequence[torch.Tensor]] = None, stream=None):
        """Commit the accepted rows; with next_aux (three [n_seq, n] fp32 taps) also
        store each sequence's next boundary feature."""
        na = next_aux if next_aux is not None else (None, None, None)
        B.eagle3_rebuild_after_verify(self.ctx, list(seq_ids), list(n_accepted), tok, aux[0],
                                      aux[1], aux[2], na[0], na[1], na[2], stream)

    def rewind(self, seq: int, new_len: int):
        B.eagle3_rewind(self.ctx, seq, new_len)

    def status(self) -> int:
        """Device-side input problems since the last call (EAGLE3_STATUS_* bits)."""
        return B.eagle3_status(self.ctx)

    def kv_len(self, seq: int):
        return B.eagle3_kv_len(self.ctx, seq)

    def kv_read(self, seq: int, row0: int, nrows: int):
        g = self.geom
        dt = torch.bfloat16 if self.kv_dtype == B.KV_BF16 else torch.float32
        k = torch.empty((nrows, g.n_head_kv, g.head_dim), dtype=dt, device="cuda")
        v = torch.empty_like(k)
        B.eagle3_kv_read(self.ctx, seq, row0, nrows, k, v)
        return k, v
