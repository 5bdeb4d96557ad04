"""Draft-KV length bookkeeping (test infrastructure).

Per sequence the draft KV holds `committed` teacher-forced rows; a chain round
writes speculative rows after them and rewinds, so a round leaves nothing behind
but the drafted ids (pegainfer PR #707, PR description, `chain_round`).

Capacity (PR #707, review of the capacity check: a fully accepted chain of k
drafts commits k + 1 rows, so the extra row must be reserved or k shrunk at the
edge; the review's example is start 97, k 3, max 100):
  * `max_ctx` is the admission bound; the store holds max_ctx + 1 rows, the
    extra row being the reserve for the (k+1)-th commit of a fully accepted
    chain;
  * a chain is admitted with gamma_eff = clamp(max_ctx - committed, 0, gamma);
  * a rebuild of a accepted drafts commits a + 1 rows and needs
    a <= gamma_eff of the chain it follows and committed + a + 1 <= max_ctx + 1;
  * prefill needs committed + T <= max_ctx.
At start=97, k=3, max=100 the chain drafts 3, full acceptance commits 4 rows
(97..100), committed becomes 101 and the next chain is admitted with
gamma_eff = 0 (k shrunk, as seen from the next round).

Boundary feature (PR #707, PR description: prefill also builds the boundary
target feature, and rebuild_after_verify sets the one for the next round): a
prefill or rebuild that is given the next boundary's taps leaves a stored
feature, one without them drops it, and a rewind drops it; a chain may start
from the stored feature only while one is held.  A prefill of zero rows without
taps changes nothing (our reading; the pages are silent).

Round-local chains (the scratch-KV drafter of memra_engine `eagle.rs`, whose draft
KV is emptied every round) attend only over their own rows, so no capacity rule
applies: gamma_eff = gamma, and they change no length, no speculative count and
enable no rebuild.
"""
from __future__ import annotations

from dataclasses import dataclass

OK = 0
E_INVAL = -1
E_SHAPE = -2
E_UNSUPPORTED = -3
E_CAPACITY = -4
E_STATE = -5


class LedgerError(Exception):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


@dataclass
class _Seq:
    committed: int = 0
    spec: int = 0
    last_gamma: int = -1      # gamma_eff of the chain since the last commit; -1 none
    boundary: bool = False    # a stored boundary feature for the current length


class Ledger:
    def __init__(self, max_ctx: int, max_seqs: int = 1, max_gamma: int = 16):
        if max_ctx < 1 or max_seqs < 1 or max_gamma < 1:
            raise LedgerError(E_INVAL, "bad ledger geometry")
        self.max_ctx = max_ctx
        self.max_gamma = max_gamma
        self.rows = max_ctx + 1
        self.seqs = [_Seq() for _ in range(max_seqs)]

    def _seq(self, s: int) -> _Seq:
        if not (0 <= s < len(self.seqs)):
            raise LedgerError(E_INVAL, f"bad sequence id {s}")
        return self.seqs[s]

    def committed(self, s: int) -> int:
        return self._seq(s).committed

    def spec(self, s: int) -> int:
        return self._seq(s).spec

    # -- checks (no mutation) --------------------------------------------
    def check_prefill(self, s: int, T: int) -> None:
        q = self._seq(s)
        if T < 0:
            raise LedgerError(E_INVAL, "negative row count")
        if q.spec:
            raise LedgerError(E_STATE, "speculative rows are live")
        if q.committed + T > self.max_ctx:
            raise LedgerError(E_CAPACITY, "prefill past max_ctx")

    def admit_chain(self, s: int, gamma: int, stored_boundary: bool = False,
                    round_local: bool = False) -> int:
        q = self._seq(s)
        if gamma < 0 or gamma > self.max_gamma:
            raise LedgerError(E_INVAL, "gamma out of range")
        if q.spec:
            raise LedgerError(E_STATE, "speculative rows are live")
        if stored_boundary and not q.boundary:
            raise LedgerError(E_STATE, "no stored boundary feature")
        if round_local:
            return gamma
        return max(0, min(gamma, self.max_ctx - q.committed))

    def check_rebuild(self, s: int, a: int) -> None:
        q = self._seq(s)
        if q.spec:
            raise LedgerError(E_STATE, "speculative rows are live")
        if q.last_gamma < 0:
            raise LedgerError(E_STATE, "rebuild without a preceding chain")
        if a < 0 or a > q.last_gamma:
            raise LedgerError(E_INVAL, "accepted count exceeds the chain's gamma_eff")
        if q.committed + a + 1 > self.rows:
            raise LedgerError(E_CAPACITY, "rebuild past the reserved row")

    # -- transitions -------------------------------------------------------
    def prefill(self, s: int, T: int, boundary: bool = False) -> int:
        self.check_prefill(s, T)
        q = self.seqs[s]
        start = q.committed
        if T == 0 and not boundary:
            return start
        q.committed += T
        q.last_gamma = -1
        q.boundary = boundary
        return start

    def chain(self, s: int, gamma: int, keep_spec: bool = False,
              stored_boundary: bool = False, round_local: bool = False) -> int:
        if round_local and keep_spec:
            raise LedgerError(E_INVAL, "a round-local chain keeps no speculative rows")
        g = self.admit_chain(s, gamma, stored_boundary, round_local)
        if round_local:
            return g
        q = self.seqs[s]
        q.spec = g if keep_spec else 0
        q.last_gamma = g
        return g

    def rebuild(self, s: int, a: int, boundary: bool = False) -> int:
        self.check_rebuild(s, a)
        q = self.seqs[s]
        start = q.committed
        q.committed += a + 1
        q.last_gamma = -1
        q.boundary = boundary
        return start

    def rewind(self, s: int, new_len: int) -> None:
        q = self._seq(s)
        if new_len < 0 or new_len > q.committed:
            raise LedgerError(E_INVAL, "rewind target outside [0, committed]")
        q.committed = new_len
        q.spec = 0
        q.last_gamma = -1
        q.boundary = False
