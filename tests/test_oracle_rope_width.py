"""The five rope-width cases of the memra_engine eagle.rs rope-width tests,
on the oracle's resolver and on a config fixture (tests/golden)."""
import json
import os

import pytest

from oracle.rope_width import resolve_rope_dim, rope_facts_from_config_text

GOLD = os.path.join(os.path.dirname(__file__), "golden", "draft_config_partial_rope.json")


def _text(mutate=None):
    cfg = json.load(open(GOLD))
    cfg.pop("_source")
    if mutate:
        mutate(cfg)
    return json.dumps(cfg)


def _width(text):
    rd, pf, hd = rope_facts_from_config_text(text)
    return resolve_rope_dim(rd, pf, hd)


def test_declared_quarter_factor_gives_64_of_256():
    rd, pf, hd = rope_facts_from_config_text(_text())
    assert (rd, pf, hd) == (None, 0.25, 256)
    assert _width(_text()) == 64


def test_nested_only_factor_is_still_partial():
    assert _width(_text(lambda c: c.pop("partial_rotary_factor"))) == 64


def test_no_declaration_is_full_width():
    def drop(c):
        c.pop("partial_rotary_factor")
        c["rope_parameters"].pop("partial_rotary_factor")
    t = _text(drop)
    assert "partial_rotary_factor" not in t
    assert _width(t) == 256


def test_explicit_rotary_dim_wins():
    assert _width(_text(lambda c: c.__setitem__("rotary_dim", 32))) == 32


@pytest.mark.parametrize("f", [2.0, 0.0, -0.5, float("nan")])
def test_malformed_factor_takes_full_width(f):
    def bad(c):
        c["partial_rotary_factor"] = f
        c["rope_parameters"]["partial_rotary_factor"] = f
    assert resolve_rope_dim(None, f, 256) == 256
    if f == f:  # json cannot hold nan
        assert _width(_text(bad)) == 256


def test_rejections():
    for rd in (0, 3, 258, -2):
        with pytest.raises(ValueError):
            resolve_rope_dim(rd, None, 256)
    with pytest.raises(ValueError):
        resolve_rope_dim(None, 0.3, 256)      # 76.8 dims
