"""MI355X (gfx950) EAGLE-3 drafter engine: HIP kernels behind a C ABI
(include/eagle3.h), with a thin Python binding of the same entry points."""
from . import binding
from .binding import (Eagle3Error, HostLedger, eagle3_draft_chain, eagle3_free, eagle3_kv_len,
                      eagle3_kv_read, eagle3_last_error, eagle3_load, eagle3_prefill,
                      eagle3_rebuild_after_verify, eagle3_resolve_rope_dim, eagle3_rewind)

__all__ = ["binding", "Eagle3Error", "HostLedger", "eagle3_draft_chain", "eagle3_free",
           "eagle3_kv_len", "eagle3_kv_read", "eagle3_last_error", "eagle3_load",
           "eagle3_prefill", "eagle3_rebuild_after_verify", "eagle3_resolve_rope_dim",
           "eagle3_rewind"]


def __getattr__(name):
    if name == "Drafter":
        from .drafter import Drafter
        return Drafter
    raise AttributeError(name)
