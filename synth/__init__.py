"""Seeded synthetic workloads (shapes + inputs) shared by oracle, tests and bench."""
from .configs import (ALL, BATCHED, LONG, PAGE4, QWEN3_8B, TINY, DrafterConfig,
                      small_variant)
from . import gen

__all__ = ["ALL", "BATCHED", "LONG", "PAGE4", "QWEN3_8B", "TINY", "DrafterConfig",
           "small_variant", "gen"]
