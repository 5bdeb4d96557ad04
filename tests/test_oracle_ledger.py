"""The oracle's capacity rules (pegainfer PR #707 review: reserve k+1)."""
import pytest

from oracle.ledger import (E_CAPACITY, E_INVAL, E_STATE, Ledger, LedgerError)


def _code(fn, *a, **k):
    with pytest.raises(LedgerError) as e:
        fn(*a, **k)
    return e.value.code


def test_admission_and_reserve():
    L = Ledger(max_ctx=100)
    assert L.rows == 101
    L.prefill(0, 97)
    assert L.chain(0, 3) == 3
    L.rebuild(0, 3)
    assert L.committed(0) == 101
    assert L.chain(0, 3) == 0
    assert _code(L.rebuild, 0, 0) == E_CAPACITY
    L.rewind(0, 99)
    assert L.chain(0, 3) == 1                   # shrink near the edge
    assert _code(L.rebuild, 0, 2) == E_INVAL    # more than gamma_eff accepted
    L.rebuild(0, 1)
    assert L.committed(0) == 101


def test_state_errors_leave_state_unchanged():
    L = Ledger(max_ctx=50, max_seqs=2)
    assert _code(L.rebuild, 0, 0) == E_STATE    # no chain yet
    L.prefill(0, 10)
    assert L.chain(0, 4, keep_spec=True) == 4
    assert L.spec(0) == 4
    before = (L.committed(0), L.spec(0))
    assert _code(L.chain, 0, 2) == E_STATE
    assert _code(L.prefill, 0, 1) == E_STATE
    assert _code(L.rebuild, 0, 1) == E_STATE
    assert (L.committed(0), L.spec(0)) == before
    L.rewind(0, 10)
    assert L.spec(0) == 0
    assert _code(L.rewind, 0, 11) == E_INVAL
    assert _code(L.prefill, 0, 41) == E_CAPACITY
    assert L.committed(0) == 10
    assert _code(L.prefill, 2, 1) == E_INVAL
    assert _code(L.chain, 1, 17) == E_INVAL     # beyond max_gamma
    assert L.committed(1) == 0


def test_prefill_resets_the_drafted_state():
    L = Ledger(max_ctx=50)
    L.chain(0, 3)
    L.prefill(0, 5)
    assert _code(L.rebuild, 0, 0) == E_STATE
