"""ctypes binding of libeagle3.so (include/eagle3.h, include/eagle3_ledger.h).

Argument marshalling only: every step of the drafter runs in the library's HIP
kernels.  Functions carry the C names; tensors are torch tensors on the GPU
(device pointers) unless a name says host.  A missing library is an error —
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_double, c_float, c_int32, c_int64, c_uint32, c_void_p
from typing import Dict, Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libeagle3.so")

OK, E_INVAL, E_SHAPE, E_UNSUPPORTED, E_CAPACITY, E_STATE, E_HIP, E_OOM = 0, -1, -2, -3, -4, -5, -6, -7
KEEP_SPEC = 1
STORED_BOUNDARY = 2
ROUND_LOCAL = 4
KV_F32, KV_BF16, KV_Q8Q5 = 0, 1, 2
APPEND_DEFAULT, APPEND_BF16, APPEND_SPLIT, APPEND_F16 = 0, 1, 2, 3
TABLE_DEFAULT, TABLE_OFF, TABLE_ON = 0, 1, 2
WEIGHTS_BF16, WEIGHTS_I4 = 0, 1

ERR_NAMES = {OK: "OK", E_INVAL: "E_INVAL", E_SHAPE: "E_SHAPE", E_UNSUPPORTED: "E_UNSUPPORTED",
             E_CAPACITY: "E_CAPACITY", E_STATE: "E_STATE", E_HIP: "E_HIP", E_OOM: "E_OOM"}

WEIGHT_FIELDS = ("fc", "input_layernorm", "hidden_norm", "q_proj", "k_proj", "v_proj", "o_proj",
                 "post_attention_layernorm", "gate_proj", "up_proj", "down_proj", "norm",
                 "lm_head", "embed")

PROFILE_KERNELS = {"lm_head": 0, "gate_up": 1, "qkv": 2, "down": 3, "o_proj": 4, "attention": 5,
                   "encode": 6, "prefill_fc_gemm": 7, "prefill_kv_gemm": 8, "lm_head_qkv": 9}


class Eagle3Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


class eagle3_config(ctypes.Structure):
    _fields_ = [("n_embd", c_int32), ("n_head", c_int32), ("n_head_kv", c_int32),
                ("head_dim", c_int32), ("n_ff", c_int32), ("draft_vocab", c_int32),
                ("target_vocab", c_int32), ("n_aux", c_int32), ("rope_dim", c_int32),
                ("rope_theta", c_float), ("rms_eps", c_float), ("max_ctx", c_int32),
                ("max_gamma", c_int32), ("max_seqs", c_int32), ("kv_dtype", c_int32),
                ("weight_format", c_int32), ("append_act", c_int32),
                ("token_table", c_int32)]


class eagle3_weights(ctypes.Structure):
    _fields_ = [(f, c_void_p) for f in WEIGHT_FIELDS] + [
        ("d2t_host", POINTER(c_int64)), ("d2t_len", c_int64), ("shape", (c_int64 * 2) * 14)]


class eagle3_trunk_config(ctypes.Structure):
    _fields_ = [("n_embd", c_int32), ("n_head", c_int32), ("n_head_kv", c_int32),
                ("head_dim", c_int32), ("n_ff", c_int32), ("vocab", c_int32), ("n_layers", c_int32),
                ("rope_theta", c_float), ("rms_eps", c_float), ("max_ctx", c_int32),
                ("max_tokens", c_int32)]


class eagle3_trunk_weights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("final_norm", c_void_p), ("lm_head", c_void_p),
                ("layers", POINTER(c_void_p)), ("shapes", POINTER(c_int64))]


TRUNK_LAYER_FIELDS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")
TRUNK_BAD_TOKEN, TRUNK_NAN_LOGITS = 1, 2


class eagle3_debug(ctypes.Structure):
    _fields_ = [("logits", c_void_p), ("hidden", c_void_p)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libeagle3.so (built in-tree by eagle_draft_head_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run eagle_draft_head_amd.build.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    sig = {
        "eagle3_resolve_rope_dim": ([c_int32, c_float, c_int32, POINTER(c_int32)], ctypes.c_int),
        "eagle3_load": ([POINTER(eagle3_config), POINTER(eagle3_weights), P, POINTER(P)], ctypes.c_int),
        "eagle3_free": ([P], ctypes.c_int),
        "eagle3_prefill": ([P, c_int32, c_int32, P, P, P, P, P, P, P, P], ctypes.c_int),
        "eagle3_draft_chain": ([P, c_int32, POINTER(c_int32), P, P, P, P, c_int32, c_uint32, P,
                                POINTER(c_int32), POINTER(eagle3_debug), P], ctypes.c_int),
        "eagle3_rebuild_after_verify": ([P, c_int32, POINTER(c_int32), POINTER(c_int32), P, P, P,
                                         P, P, P, P, P], ctypes.c_int),
        "eagle3_rewind": ([P, c_int32, c_int32], ctypes.c_int),
        "eagle3_kv_len": ([P, c_int32, POINTER(c_int32), POINTER(c_int32)], ctypes.c_int),
        "eagle3_status": ([P, POINTER(c_uint32)], ctypes.c_int),
        "eagle3_kv_read": ([P, c_int32, c_int32, c_int32, P, P, P], ctypes.c_int),
        "eagle3_weights_i4_read": ([P, c_int32, P, P, P], ctypes.c_int),
        "eagle3_verify_attention_workspace": ([c_int32, c_int32, c_int32, c_int32, c_int32, c_int32],
                                              ctypes.c_size_t),
        "eagle3_verify_attention": ([P, P, P, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                     c_int32, P, P, ctypes.c_size_t, P], ctypes.c_int),
        "eagle3_verify_attention_noalloc": ([P, P, P, c_int32, c_int32, c_int32, c_int32, c_int32,
                                             c_int32, c_int32, P, P], ctypes.c_int),
        "eagle3_last_error": ([P], c_char_p),
        "eagle3_profile_enable": ([P, c_int32, c_int32], ctypes.c_int),
        "eagle3_profile_read": ([P, POINTER(c_double), POINTER(c_int64)], ctypes.c_int),
        "eagle3_trunk_load": ([POINTER(eagle3_trunk_config), POINTER(eagle3_trunk_weights), P, POINTER(P)],
                              ctypes.c_int),
        "eagle3_trunk_free": ([P], ctypes.c_int),
        "eagle3_trunk_forward": ([P, c_int32, P, P, P, P, P, P], ctypes.c_int),
        "eagle3_trunk_rollback": ([P, c_int32], ctypes.c_int),
        "eagle3_trunk_len": ([P, POINTER(c_int32)], ctypes.c_int),
        "eagle3_trunk_status": ([P, POINTER(c_uint32)], ctypes.c_int),
        "eagle3_trunk_last_error": ([P], c_char_p),
        "eagle3_generate": ([P, c_int32, P, POINTER(c_int32), c_int32, c_int32, c_int32, POINTER(c_int32),
                             POINTER(c_int64), POINTER(c_int64), P], ctypes.c_int),
        "eagle3_calibrate_mfma": ([c_int32, c_int32, P, POINTER(c_double), P], ctypes.c_int),
        "eagle3_calibrate_stream": ([P, ctypes.c_size_t, P, ctypes.c_size_t, c_int32, P, POINTER(c_double), P],
                                    ctypes.c_int),
        "eagle3_ledger_create": ([c_int32, c_int32, c_int32, POINTER(P)], ctypes.c_int),
        "eagle3_ledger_destroy": ([P], None),
        "eagle3_ledger_prefill": ([P, c_int32, c_int32, c_int32], ctypes.c_int),
        "eagle3_ledger_chain": ([P, c_int32, c_int32, c_uint32, POINTER(c_int32)], ctypes.c_int),
        "eagle3_ledger_rebuild": ([P, c_int32, c_int32, c_int32], ctypes.c_int),
        "eagle3_ledger_rewind": ([P, c_int32, c_int32], ctypes.c_int),
        "eagle3_ledger_len": ([P, c_int32, POINTER(c_int32), POINTER(c_int32)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def exported_symbols() -> Sequence[str]:
    return [n for n in dir(library()) if n.startswith("eagle3_")]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(ctx, rc: int):
    if rc != OK:
        msg = library().eagle3_last_error(ctx)
        raise Eagle3Error(rc, (msg or b"").decode())


# ---------------------------------------------------------------------------
# the C entry points, same names
# ---------------------------------------------------------------------------

def eagle3_resolve_rope_dim(rotary_dim: Optional[int], partial_factor: Optional[float],
                            head_dim: int) -> int:
    out = c_int32(0)
    rc = library().eagle3_resolve_rope_dim(-1 if rotary_dim is None else int(rotary_dim),
                                           -1.0 if partial_factor is None else float(partial_factor),
                                           int(head_dim), byref(out))
    if rc != OK:
        raise Eagle3Error(rc, "rope width")
    return out.value


def make_config(geom, max_ctx: int, max_gamma: int = 16, max_seqs: int = 1,
                kv_dtype: int = KV_F32, weight_format: int = WEIGHTS_BF16,
                append_act: int = APPEND_DEFAULT, token_table: int = TABLE_DEFAULT) -> eagle3_config:
    return eagle3_config(
        n_embd=geom.n_embd, n_head=geom.n_head, n_head_kv=geom.n_head_kv, head_dim=geom.head_dim,
        n_ff=geom.n_ff, draft_vocab=geom.draft_vocab, target_vocab=geom.target_vocab,
        n_aux=getattr(geom, "n_aux", 3), rope_dim=geom.rope_dim, rope_theta=float(geom.rope_theta),
        rms_eps=float(geom.rms_eps), max_ctx=int(max_ctx), max_gamma=int(max_gamma),
        max_seqs=int(max_seqs), kv_dtype=int(kv_dtype), weight_format=int(weight_format),
        append_act=int(append_act), token_table=int(token_table))


def make_weights(tensors: Dict[str, object], d2t_host) -> eagle3_weights:
    """tensors: name -> bf16 device tensor ([out, in]; norms 1-D); d2t_host: int64
    CPU tensor.  The returned struct keeps a reference to the d2t buffer."""
    import torch
    w = eagle3_weights()
    for i, f in enumerate(WEIGHT_FIELDS):
        t = tensors.get(f)
        setattr(w, f, None if t is None else t.data_ptr())
        if t is not None:
            shp = tuple(t.shape) if t.dim() == 2 else (int(t.shape[0]), 1)
            w.shape[i][0], w.shape[i][1] = shp
    d = torch.as_tensor(d2t_host, dtype=torch.int64).contiguous().cpu()
    w._d2t_keep = d
    w.d2t_host = ctypes.cast(d.data_ptr(), POINTER(c_int64))
    w.d2t_len = d.numel()
    return w


def eagle3_load(cfg: eagle3_config, weights: eagle3_weights, stream=None) -> int:
    out = c_void_p(None)
    rc = library().eagle3_load(byref(cfg), byref(weights), _stream(stream), byref(out))
    _check(None, rc)
    return out.value


def eagle3_free(ctx: int) -> None:
    library().eagle3_free(ctx)


def eagle3_prefill(ctx, seq: int, T: int, tok, aux0, aux1, aux2, next_aux0=None, next_aux1=None,
                   next_aux2=None, stream=None) -> None:
    _check(ctx, library().eagle3_prefill(ctx, seq, T, _ptr(tok), _ptr(aux0), _ptr(aux1),
                                         _ptr(aux2), _ptr(next_aux0), _ptr(next_aux1),
                                         _ptr(next_aux2), _stream(stream)))


def eagle3_draft_chain(ctx, seq_ids: Sequence[int], boundary_tok, aux0, aux1, aux2, gamma: int,
                       out_ids, flags: int = 0, debug_logits=None, debug_hidden=None,
                       stream=None):
    """Returns the list of gamma_eff per sequence (filled before launch)."""
    n = len(seq_ids)
    ids = (c_int32 * n)(*seq_ids)
    geff = (c_int32 * n)()
    dbg = None
    if debug_logits is not None or debug_hidden is not None:
        dbg = eagle3_debug(_ptr(debug_logits), _ptr(debug_hidden))
    rc = library().eagle3_draft_chain(ctx, n, ids, _ptr(boundary_tok), _ptr(aux0), _ptr(aux1),
                                      _ptr(aux2), int(gamma), int(flags), _ptr(out_ids), geff,
                                      byref(dbg) if dbg is not None else None, _stream(stream))
    _check(ctx, rc)
    return list(geff)


def eagle3_rebuild_after_verify(ctx, seq_ids: Sequence[int], n_accepted: Sequence[int], tok, aux0,
                                aux1, aux2, next_aux0=None, next_aux1=None, next_aux2=None,
                                stream=None) -> None:
    n = len(seq_ids)
    ids = (c_int32 * n)(*seq_ids)
    acc = (c_int32 * n)(*n_accepted)
    _check(ctx, library().eagle3_rebuild_after_verify(ctx, n, ids, acc, _ptr(tok), _ptr(aux0),
                                                      _ptr(aux1), _ptr(aux2), _ptr(next_aux0),
                                                      _ptr(next_aux1), _ptr(next_aux2),
                                                      _stream(stream)))


def eagle3_rewind(ctx, seq: int, new_len: int) -> None:
    _check(ctx, library().eagle3_rewind(ctx, seq, new_len))


STATUS_BAD_TOKEN, STATUS_NAN_LOGITS, STATUS_APPEND_RANGE = 1, 2, 4


def eagle3_status(ctx) -> int:
    v = c_uint32(0)
    _check(ctx, library().eagle3_status(ctx, byref(v)))
    return v.value


def eagle3_kv_len(ctx, seq: int):
    c, s = c_int32(0), c_int32(0)
    _check(ctx, library().eagle3_kv_len(ctx, seq, byref(c), byref(s)))
    return c.value, s.value


def eagle3_kv_read(ctx, seq: int, row0: int, nrows: int, k_out, v_out, stream=None) -> None:
    _check(ctx, library().eagle3_kv_read(ctx, seq, row0, nrows, _ptr(k_out), _ptr(v_out),
                                         _stream(stream)))


I4_MATRICES = {"fc": 0, "qkv": 1, "o_proj": 2, "gate_up": 3, "down_proj": 4, "lm_head": 5}


def eagle3_weights_i4_read(ctx, matrix: str, codes, scales, stream=None) -> None:
    _check(ctx, library().eagle3_weights_i4_read(ctx, I4_MATRICES[matrix], _ptr(codes),
                                                 _ptr(scales), _stream(stream)))


def eagle3_verify_attention_workspace(M: int, n_head: int, n_head_kv: int, head_dim: int,
                                      ctx_rows: int, kv_dtype: int = KV_F32) -> int:
    return int(library().eagle3_verify_attention_workspace(M, n_head, n_head_kv, head_dim,
                                                           ctx_rows, kv_dtype))


def eagle3_verify_attention(q, k, v, kv_dtype: int, cap: int, ctx_rows: int, M: int, n_head: int,
                            n_head_kv: int, head_dim: int, out, workspace=None,
                            workspace_bytes: int = 0, stream=None) -> None:
    rc = library().eagle3_verify_attention(_ptr(q), _ptr(k), _ptr(v), kv_dtype, cap, ctx_rows, M,
                                           n_head, n_head_kv, head_dim, _ptr(out), _ptr(workspace),
                                           workspace_bytes, _stream(stream))
    if rc != OK:
        raise Eagle3Error(rc, "eagle3_verify_attention")


VERIFY_SCRATCH_BYTES = 16 << 20


def eagle3_verify_attention_noalloc(q, k, v, kv_dtype: int, cap: int, ctx_rows: int, M: int,
                                    n_head: int, n_head_kv: int, head_dim: int, out,
                                    stream=None) -> None:
    rc = library().eagle3_verify_attention_noalloc(_ptr(q), _ptr(k), _ptr(v), kv_dtype, cap, ctx_rows,
                                                   M, n_head, n_head_kv, head_dim, _ptr(out),
                                                   _stream(stream))
    _check(None, rc)


def eagle3_last_error(ctx) -> str:
    return (library().eagle3_last_error(ctx) or b"").decode()


def eagle3_profile_enable(ctx, kernel: str, enable: bool = True) -> None:
    _check(ctx, library().eagle3_profile_enable(ctx, PROFILE_KERNELS[kernel], int(enable)))


def eagle3_profile_read(ctx):
    ms, n = c_double(0), c_int64(0)
    _check(ctx, library().eagle3_profile_read(ctx, byref(ms), byref(n)))
    return ms.value, n.value


# ---- the synthetic target trunk and the speculative runner (eagle3_trunk.h) ----

def _check_trunk(t, rc: int):
    if rc != OK:
        msg = library().eagle3_trunk_last_error(t)
        raise Eagle3Error(rc, (msg or b"").decode())


def make_trunk_config(geom, n_layers: int, max_ctx: int, max_tokens: int) -> eagle3_trunk_config:
    return eagle3_trunk_config(
        n_embd=geom.n_embd, n_head=geom.n_head, n_head_kv=geom.n_head_kv, head_dim=geom.head_dim,
        n_ff=geom.n_ff, vocab=geom.target_vocab, n_layers=int(n_layers),
        rope_theta=float(geom.rope_theta), rms_eps=float(geom.rms_eps), max_ctx=int(max_ctx),
        max_tokens=int(max_tokens))


def make_trunk_weights(tensors: Dict[str, object], embed, n_layers: int) -> eagle3_trunk_weights:
    """tensors: "layers.{l}.{name}", "final_norm", "lm_head" -> bf16 device tensors;
    embed: the bf16 token embedding.  The struct keeps its pointer arrays alive."""
    order = [embed, tensors["final_norm"], tensors["lm_head"]]
    for l in range(n_layers):
        order += [tensors[f"layers.{l}.{f}"] for f in TRUNK_LAYER_FIELDS]
    shapes = []
    for t in order:
        shapes += list(t.shape) if t.dim() == 2 else [int(t.shape[0]), 1]
    layers = (c_void_p * (9 * n_layers))(*[t.data_ptr() for t in order[3:]])
    shp = (c_int64 * len(shapes))(*shapes)
    w = eagle3_trunk_weights(order[0].data_ptr(), order[1].data_ptr(), order[2].data_ptr(),
                             ctypes.cast(layers, POINTER(c_void_p)), ctypes.cast(shp, POINTER(c_int64)))
    w._keep = (layers, shp)
    return w


def eagle3_trunk_load(cfg: eagle3_trunk_config, weights: eagle3_trunk_weights, stream=None) -> int:
    out = c_void_p(None)
    _check_trunk(None, library().eagle3_trunk_load(byref(cfg), byref(weights), _stream(stream), byref(out)))
    return out.value


def eagle3_trunk_free(t) -> None:
    library().eagle3_trunk_free(t)


def eagle3_trunk_forward(t, T: int, tok, ids, tap0=None, tap1=None, tap2=None, stream=None) -> None:
    _check_trunk(t, library().eagle3_trunk_forward(t, int(T), _ptr(tok), _ptr(ids), _ptr(tap0), _ptr(tap1),
                                                   _ptr(tap2), _stream(stream)))


def eagle3_trunk_rollback(t, new_len: int) -> None:
    _check_trunk(t, library().eagle3_trunk_rollback(t, int(new_len)))


def eagle3_trunk_len(t) -> int:
    v = c_int32(0)
    _check_trunk(t, library().eagle3_trunk_len(t, byref(v)))
    return v.value


def eagle3_trunk_status(t) -> int:
    v = c_uint32(0)
    _check_trunk(t, library().eagle3_trunk_status(t, byref(v)))
    return v.value


def eagle3_generate(ctx, seq: int, trunk, prompt: Sequence[int], max_new: int, gamma: int, stream=None):
    """Returns (tokens, drafted, accepted)."""
    p = (c_int32 * len(prompt))(*[int(x) for x in prompt])
    out = (c_int32 * max_new)()
    dr, ac = c_int64(0), c_int64(0)
    rc = library().eagle3_generate(ctx, int(seq), trunk, p, len(prompt), int(max_new), int(gamma), out,
                                   byref(dr), byref(ac), _stream(stream))
    _check_trunk(trunk, rc)
    return list(out), dr.value, ac.value


# ---- calibration -----------------------------------------------------------------
CALIB_SINK_BYTES = 2 << 20


def eagle3_calibrate_mfma(iters: int, reps: int, sink, stream=None) -> float:
    v = c_double(0)
    rc = library().eagle3_calibrate_mfma(int(iters), int(reps), _ptr(sink), byref(v), _stream(stream))
    if rc != OK:
        raise Eagle3Error(rc, "eagle3_calibrate_mfma")
    return v.value


def eagle3_calibrate_stream(buf, nbytes: int, flush, flush_bytes: int, reps: int, sink, stream=None) -> float:
    v = c_double(0)
    rc = library().eagle3_calibrate_stream(_ptr(buf), int(nbytes), _ptr(flush), int(flush_bytes), int(reps),
                                           _ptr(sink), byref(v), _stream(stream))
    if rc != OK:
        raise Eagle3Error(rc, "eagle3_calibrate_stream")
    return v.value


# ---- the ledger on its own (host only) ---------------------------------------

class HostLedger:
    """The engine's draft-KV bookkeeping, driven without a device."""

    def __init__(self, max_ctx: int, max_seqs: int = 1, max_gamma: int = 16):
        out = c_void_p(None)
        rc = library().eagle3_ledger_create(max_ctx, max_seqs, max_gamma, byref(out))
        if rc != OK:
            raise Eagle3Error(rc, "ledger create")
        self._h = out.value

    def __del__(self):
        if getattr(self, "_h", None):
            library().eagle3_ledger_destroy(self._h)
            self._h = None

    def prefill(self, seq, T, boundary=False) -> int:
        return library().eagle3_ledger_prefill(self._h, seq, T, int(boundary))

    def chain(self, seq, gamma, keep_spec=False, stored_boundary=False, round_local=False):
        g = c_int32(-1)
        flags = ((KEEP_SPEC if keep_spec else 0) | (STORED_BOUNDARY if stored_boundary else 0)
                 | (ROUND_LOCAL if round_local else 0))
        rc = library().eagle3_ledger_chain(self._h, seq, gamma, flags, byref(g))
        return rc, g.value

    def rebuild(self, seq, a, boundary=False) -> int:
        return library().eagle3_ledger_rebuild(self._h, seq, a, int(boundary))

    def rewind(self, seq, new_len) -> int:
        return library().eagle3_ledger_rewind(self._h, seq, new_len)

    def length(self, seq):
        c, s = c_int32(0), c_int32(0)
        rc = library().eagle3_ledger_len(self._h, seq, byref(c), byref(s))
        return rc, c.value, s.value
