"""Rotary width of the draft attention (test infrastructure).

memra_engine `eagle.rs`, `EagleConfig::rope_dim_count` and the
`draft_rope_width_tests` module: an explicit rotated-dims count takes
precedence over a fractional declaration, which takes precedence over the full
head width; a malformed fraction (not in (0, 1]) takes the full width rather
than a rotation wider than the head or a vanishing one.  The tests on that page
fix five cases: factor 0.25 of 256 -> 64; the factor given only under the
nested rope-parameters object -> 64; no declaration -> 256; an explicit 32
together with factor 0.25 -> 32; factors 2.0 and 0.0 -> 256.

Our reading where the page is silent: an explicit count must be even and in
(0, head_dim]; a fraction must give an even whole number of dims.  Anything
else is rejected (ValueError) rather than rounded.
"""
from __future__ import annotations

import json
import math
from typing import Optional, Tuple


def resolve_rope_dim(rotary_dim: Optional[int], partial_factor: Optional[float],
                     head_dim: int) -> int:
    if head_dim <= 0 or head_dim % 2:
        raise ValueError("head_dim must be positive and even")
    if rotary_dim is not None:
        if rotary_dim <= 0 or rotary_dim > head_dim or rotary_dim % 2:
            raise ValueError("explicit rotary_dim must be even and in (0, head_dim]")
        return int(rotary_dim)
    if partial_factor is not None:
        f = float(partial_factor)
        if not (math.isfinite(f) and 0.0 < f <= 1.0):
            return head_dim                     # malformed -> full width
        dims = f * head_dim
        r = int(round(dims))
        if abs(dims - r) > 1e-9 or r % 2 or r == 0:
            raise ValueError("factor does not give an even whole number of dims")
        return r
    return head_dim


def rope_facts_from_config_text(text: str) -> Tuple[Optional[int], Optional[float], int]:
    """(rotary_dim, partial_rotary_factor, head_dim) declared by a draft
    config.json: the factor may sit at top level or under "rope_parameters"
    (the nested-only spelling the memra tests pin)."""
    cfg = json.loads(text)
    rd = cfg.get("rotary_dim")
    pf = cfg.get("partial_rotary_factor")
    if pf is None and isinstance(cfg.get("rope_parameters"), dict):
        pf = cfg["rope_parameters"].get("partial_rotary_factor")
    return (None if rd is None else int(rd),
            None if pf is None else float(pf),
            int(cfg["head_dim"]))
