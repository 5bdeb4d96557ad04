"""Host-side checks of the C ABI that need no GPU: the library loads and exports
every declared entry point, the rope-width resolver and the KV ledger agree
with the oracle, and eagle3_load rejects bad geometry before touching a device."""
import ctypes
import os
import random
import re

import numpy as np
import pytest

from eagle_draft_head_amd import binding as B
from oracle.ledger import Ledger, LedgerError
from oracle.rope_width import resolve_rope_dim
from synth import TINY, gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header):
    txt = open(os.path.join(ROOT, "include", header)).read()
    return sorted(set(re.findall(r"\b(eagle3_[a-z_]+)\s*\(", txt)))


@pytest.mark.parametrize("header,least", [("eagle3.h", 7), ("eagle3_ledger.h", 7), ("eagle3_trunk.h", 7),
                                          ("eagle3_testing.h", 2)])
def test_library_exports_every_declared_symbol(header, least):
    lib = B.library()
    names = _declared(header)
    assert len(names) >= least
    for n in names:
        assert hasattr(lib, n), f"{n} declared in {header} but not exported"


def test_rope_width_matches_oracle():
    cases = [(None, 0.25, 256), (None, None, 256), (32, 0.25, 256), (None, 2.0, 256),
             (None, 0.0, 256), (None, 0.5, 128), (None, 1.0, 64), (64, None, 64)]
    for rd, pf, hd in cases:
        assert B.eagle3_resolve_rope_dim(rd, pf, hd) == resolve_rope_dim(rd, pf, hd)
    for rd, pf, hd in [(3, None, 256), (0, None, 256), (258, None, 256), (None, 0.3, 256)]:
        with pytest.raises(B.Eagle3Error):
            B.eagle3_resolve_rope_dim(rd, pf, hd)
        with pytest.raises(ValueError):
            resolve_rope_dim(rd, pf, hd)


def _oracle_rc(fn, *a):
    try:
        r = fn(*a)
        return 0, r
    except LedgerError as e:
        return e.code, None


@pytest.mark.parametrize("seed", range(6))
def test_ledger_matches_oracle_on_random_histories(seed):
    rnd = random.Random(seed)
    max_ctx, seqs, mg = rnd.choice([(20, 2, 4), (100, 3, 8), (7, 1, 3)])
    ours, ref = B.HostLedger(max_ctx, seqs, mg), Ledger(max_ctx, seqs, mg)
    for _ in range(400):
        op = rnd.randrange(5)
        s = rnd.randrange(-1, seqs + 1)
        bnd = rnd.random() < 0.5
        if op == 0:
            T = rnd.randrange(-1, 8)
            rc = ours.prefill(s, T, bnd)
            rrc, _ = _oracle_rc(ref.prefill, s, T, bnd)
        elif op == 1:
            g = rnd.randrange(-1, mg + 2)
            keep = rnd.random() < 0.2
            loc = rnd.random() < 0.25
            rc, ge = ours.chain(s, g, keep, bnd, loc)
            rrc, rge = _oracle_rc(lambda: ref.chain(s, g, keep_spec=keep, stored_boundary=bnd,
                                                    round_local=loc))
            if rc == 0:
                assert ge == rge
        elif op == 2:
            a = rnd.randrange(-1, mg + 2)
            rc = ours.rebuild(s, a, bnd)
            rrc, _ = _oracle_rc(ref.rebuild, s, a, bnd)
        elif op == 3:
            nl = rnd.randrange(-1, max_ctx + 3)
            rc = ours.rewind(s, nl)
            rrc, _ = _oracle_rc(ref.rewind, s, nl)
        else:
            continue
        assert rc == rrc, (op, s)
        for q in range(seqs):
            _, c, sp = ours.length(q)
            assert (c, sp) == (ref.committed(q), ref.spec(q))


def test_ledger_stored_boundary_rules():
    L = B.HostLedger(100, 2, 8)
    assert L.chain(0, 3, stored_boundary=True) == (B.E_STATE, -1)
    assert L.prefill(0, 10) == 0
    assert L.chain(0, 3, stored_boundary=True)[0] == B.E_STATE   # prefill without taps
    assert L.prefill(0, 0, boundary=True) == 0                    # boundary only
    assert L.length(0) == (0, 10, 0)
    assert L.chain(0, 3, stored_boundary=True) == (0, 3)
    assert L.chain(0, 3, stored_boundary=True) == (0, 3)          # a round leaves it
    assert L.chain(1, 3, stored_boundary=True)[0] == B.E_STATE    # per sequence
    assert L.rebuild(0, 2, boundary=True) == 0
    assert L.chain(0, 3, stored_boundary=True) == (0, 3)
    assert L.rebuild(0, 1) == 0                                   # rebuild without taps
    assert L.chain(0, 3, stored_boundary=True)[0] == B.E_STATE
    assert L.prefill(0, 1, boundary=True) == 0
    assert L.rewind(0, 14) == 0                                   # rewind drops it
    assert L.chain(0, 3, stored_boundary=True)[0] == B.E_STATE


def test_ledger_round_local_rules():
    L = B.HostLedger(100, 1, 8)
    assert L.prefill(0, 98) == 0
    assert L.chain(0, 8, round_local=True) == (0, 8)       # no capacity clamp
    assert L.length(0) == (0, 98, 0)
    assert L.rebuild(0, 0) == B.E_STATE                     # no persistent round since the commit
    assert L.chain(0, 9, round_local=True)[0] == B.E_INVAL  # gamma range still applies
    assert L.chain(0, 3, keep_spec=True, round_local=True)[0] == B.E_INVAL
    assert L.chain(0, 3, keep_spec=True) == (0, 2)          # persistent: clamped, spec kept
    assert L.chain(0, 3, round_local=True)[0] == B.E_STATE  # speculative rows are live


def test_ledger_capacity_edge_97_3_100():
    L = B.HostLedger(100, 1, 8)
    assert L.prefill(0, 97) == 0
    assert L.chain(0, 3) == (0, 3)
    assert L.rebuild(0, 3) == 0
    assert L.length(0) == (0, 101, 0)
    assert L.chain(0, 3) == (0, 0)
    assert L.rebuild(0, 0) == B.E_CAPACITY


# ---- eagle3_load validation (fails before any device call) ----------------------

FAKE = 0x1000  # never dereferenced: every case below fails validation first


def _fake_weights(cfg, d2t, drop=None, reshape=None):
    n, q, kv = cfg.n_embd, cfg.q_dim, cfg.kv_dim
    shapes = {k: (v if len(v) == 2 else (v[0], 1)) for k, v in gen.weight_shapes(cfg).items()}
    w = B.eagle3_weights()
    for i, f in enumerate(B.WEIGHT_FIELDS):
        setattr(w, f, None if f == drop else FAKE)
        sh = shapes[f] if not (reshape and f in reshape) else reshape[f]
        w.shape[i][0], w.shape[i][1] = sh
    d = np.ascontiguousarray(d2t, dtype=np.int64)
    w._keep = d
    w.d2t_host = d.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    w.d2t_len = d.size
    return w


def _load_rc(cfg_struct, w):
    lib = B.library()
    out = ctypes.c_void_p(None)
    rc = lib.eagle3_load(ctypes.byref(cfg_struct), ctypes.byref(w), None, ctypes.byref(out))
    assert out.value is None
    return rc, B.eagle3_last_error(None)


@pytest.fixture(scope="module")
def d2t_tiny():
    return gen.d2t(TINY).numpy()


@pytest.mark.parametrize("field,shape", [("fc", (256, 512)), ("q_proj", (256, 256)),
                                         ("lm_head", (1000, 256)), ("embed", (4096, 128)),
                                         ("k_proj", (64, 512))])
def test_load_rejects_inconsistent_shapes(d2t_tiny, field, shape):
    rc, msg = _load_rc(B.make_config(TINY, 100), _fake_weights(TINY, d2t_tiny, reshape={field: shape}))
    assert rc == B.E_SHAPE and field in msg


def test_load_rejects_missing_embedding(d2t_tiny):
    rc, msg = _load_rc(B.make_config(TINY, 100), _fake_weights(TINY, d2t_tiny, drop="embed"))
    assert rc == B.E_INVAL and "embed" in msg


def test_load_rejects_d2t_problems(d2t_tiny):
    bad = d2t_tiny.copy()
    bad[5] = TINY.target_vocab
    rc, _ = _load_rc(B.make_config(TINY, 100), _fake_weights(TINY, bad))
    assert rc == B.E_INVAL
    rc, _ = _load_rc(B.make_config(TINY, 100), _fake_weights(TINY, d2t_tiny[:-1]))
    assert rc == B.E_SHAPE


@pytest.mark.parametrize("change,code", [(dict(head_dim=96), B.E_UNSUPPORTED),
                                         (dict(rope_dim=63), B.E_UNSUPPORTED),
                                         (dict(rope_dim=128), B.E_UNSUPPORTED),
                                         (dict(n_head_kv=3), B.E_SHAPE),
                                         (dict(n_aux=2), B.E_UNSUPPORTED),
                                         (dict(n_embd=200), B.E_UNSUPPORTED),
                                         (dict(max_ctx=0), B.E_INVAL),
                                         (dict(weight_format=7), B.E_INVAL),
                                         (dict(weight_format=B.WEIGHTS_I4, max_seqs=2), B.E_UNSUPPORTED),
                                         (dict(weight_format=B.WEIGHTS_I4, n_ff=776), B.E_UNSUPPORTED),
                                         (dict(kv_dtype=3), B.E_INVAL),
                                         (dict(kv_dtype=B.KV_Q8Q5, max_seqs=2), B.E_UNSUPPORTED)])
def test_load_rejects_unsupported_geometry(d2t_tiny, change, code):
    cfg = B.make_config(TINY, 100)
    for k, v in change.items():
        setattr(cfg, k, v)
    rc, _ = _load_rc(cfg, _fake_weights(TINY, d2t_tiny))
    assert rc == code
