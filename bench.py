"""Benchmark of the drafter hot path on one GPU.

A step is one speculative round of the drafter at batch 1 on the Qwen3-8B-shaped
workload (n_embd 4096, 32/8 heads x 128, n_ff 12288, draft vocab 32000,
target vocab 151936, 1024 committed KV rows):
  draft_chain (gamma = 3 greedy draft steps from the boundary feature, then the
  rewind of its speculative rows) followed by rebuild_after_verify of a + 1
  teacher-forced rows (a cycles 0..3) that also encodes the next round's
  boundary taps in the same pass over W_fc.  The committed context grows by
  a + 1 rows a step, starting where its mean over the timed steps is 1024.
  --boundary taps: the chain encodes the boundary taps itself and each step ends
  with a rewind to exactly 1024 rows (the default for page4, whose rounds are
  rewound).
Inputs are seeded synthetic tensors already resident in HBM.  `value` is draft
tokens per second over the timed steps.  The dominant kernel (the lm_head GEMV
with fused final norm and argmax) is timed with HIP events on the launching
stream in a pass over the same steps; its algorithmic bytes per launch over its
average duration give `roofline.achieved`.  The CPU oracle is timed on a bounded
sample of the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--boundary stored|taps] [--drafter persistent|round-local] [--kv f32|bf16|q8q5]
       [--no-cpu] [--kernel lm_head|gate_up|qkv|down|o_proj|attention|encode]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CALIB_BYTES = 512 << 20
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "lm_head_qwen3-8b_hbm_traffic.md")


def kernel_source_digest() -> str:
    """Digest of the sources the measured kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in ("gemv.hip", "common.hpp", "gemv_cfg.hpp", "kernels.hpp"):
        with open(os.path.join(ROOT, "eagle_draft_head_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when the
    summary is missing, is for another kernel, or the kernel source changed."""
    try:
        txt = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    for line in txt.splitlines():
        if not line.startswith("traffic:"):
            continue
        vals = dict(kv.split("=") for kv in line[len("traffic:"):].split())
        if vals.get("kernel") == kernel and vals.get("source") == kernel_source_digest():
            return float(vals["bytes_per_launch"])
    return None


# HBM bytes per projection weight: bf16, or int4 codes plus one bf16 scale per 32
WB_BF16, WB_I4 = 2.0, 0.5 + 2.0 / 32
# KV bytes per element, K and V averaged: q8_0 K is 34 bytes per 32 values, q5_1 V 24
KV_BYTES = {"f32": 4.0, "bf16": 2.0, "q8q5": (34.0 + 24.0) / 64}
WB = WB_BF16
# the chain step's QKV embedding half read from the load-time token table (one
# fp32 row of the table and a sum of squares instead of W_qkv[:, :n], the
# embedding row and input_layernorm)
TABLE = False


BF16_MFMA_PEAK_TFLOPS = 2500.0


def calibrate(B, torch, stream_bytes: int = 262_144_000):
    """The ceilings on this GPU: the sustained bf16 MFMA rate (a pure MFMA loop)
    and the streaming HBM read rate of a buffer of stream_bytes (the lm_head
    matrix's size) read right after a 2 GiB flush read."""
    sink = torch.empty(B.CALIB_SINK_BYTES, dtype=torch.uint8, device="cuda")
    buf = torch.empty(stream_bytes, dtype=torch.uint8, device="cuda").fill_(1)
    flush = torch.empty(2 << 30, dtype=torch.uint8, device="cuda").fill_(2)
    torch.cuda.synchronize()
    tflops = B.eagle3_calibrate_mfma(10000, 3, sink)
    gbs = B.eagle3_calibrate_stream(buf, stream_bytes, flush, flush.numel(), 5, sink)
    del sink, buf, flush
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(tflops, 1), "hbm_stream_read_gbs": round(gbs, 1),
            "stream_bytes": stream_bytes,
            "how": "eagle3_calibrate_mfma (4 independent v_mfma_f32_32x32x16_bf16 chains per wave, "
                   "register operands, 2048x256 threads, best of 3) and eagle3_calibrate_stream "
                   "(coalesced 16-byte reads after a 2 GiB flush read, best of 5)"}


def kernel_bytes(cfg, kernel: str, L: int, kv_bytes: int = 4) -> float:
    """Algorithmic HBM bytes of one launch of a kernel family (K/V elements of
    kv_bytes bytes)."""
    n, qd, kvd, ff, dv = cfg.n_embd, cfg.q_dim, cfg.kv_dim, cfg.n_ff, cfg.draft_vocab
    if kernel == "lm_head":
        return WB * dv * n + 4 * n + 4 * n
    if kernel == "lm_head_qkv":
        # lm_head and the next step's hidden-half QKV rows (deferred QKV): both weight
        # streams, both staged vectors, the hidden-half sums written
        N = qd + 2 * kvd
        return WB * dv * n + 4 * n + 4 * n + WB * N * n + 4 * n + 4 * N
    if kernel == "gate_up":
        return WB * 2 * ff * n + 4 * n + 4 * n + 4 * ff
    if kernel == "qkv":
        if TABLE:
            return WB * (qd + 2 * kvd) * n + 4 * (qd + 2 * kvd) + 4 + 8 * n + 4 * qd + 2 * 2 * kvd
        return WB * (qd + 2 * kvd) * 2 * n + 2 * n + 4 * n + 8 * n + 4 * qd + 2 * 2 * kvd
    if kernel == "down":
        return WB * n * ff + 4 * ff + 4 * n + 4 * n
    if kernel == "o_proj":
        return WB * n * qd + 4 * qd + 4 * n + 4 * n
    if kernel == "encode":
        return WB * 3 * n * n + 12 * n + 4 * n
    if kernel == "attention":
        return 2.0 * kv_bytes * kvd * (L + 1) + 8 * qd
    raise KeyError(kernel)


def kernel_bytes_step(cfg, L: int, gamma: int, kv_bytes: int = 4) -> float:
    """Algorithmic HBM bytes of an average draft step of a round over L committed
    rows: the step's weights, norms, the embedding row, the K/V rows it reads
    (L + j + 1 at step j) and the row it writes."""
    n, qd, kvd, ff, dv = cfg.n_embd, cfg.q_dim, cfg.kv_dim, cfg.n_ff, cfg.draft_vocab
    rows = L + 1 + (gamma - 1) / 2 + 1
    return WB * p_step_weights(cfg) + 8 * n + tok_bytes(cfg) + rows * 2 * kv_bytes * kvd


def p_step_weights(cfg) -> float:
    """Weight elements one draft step streams."""
    n, qd, kvd, ff, dv = cfg.n_embd, cfg.q_dim, cfg.kv_dim, cfg.n_ff, cfg.draft_vocab
    return (qd + 2 * kvd) * (1 if TABLE else 2) * n + n * qd + 3 * ff * n + dv * n


def tok_bytes(cfg) -> float:
    """What a draft step reads for its token: the embedding row, or the token
    table's row and sum of squares."""
    return 4.0 * (cfg.q_dim + 2 * cfg.kv_dim) + 4 if TABLE else 2.0 * cfg.n_embd


def step_bytes(cfg, L: int, gamma: int, accepted: int, kv_bytes: int = 4,
               stored: bool = False, rebuild: bool = True) -> float:
    """Algorithmic HBM bytes of one round: encode, gamma draft steps, rebuild (K/V
    elements of kv_bytes bytes).  stored: the encode is the rebuild's extra row (the
    next boundary: its taps in, the feature and its weighted copy out) on the
    rebuild's one pass over W_fc."""
    n, qd, kvd, ff, dv = cfg.n_embd, cfg.q_dim, cfg.kv_dim, cfg.n_ff, cfg.draft_vocab
    p_step = p_step_weights(cfg)
    tot = 12.0 * n + 8 * n + 4 if stored else WB * 3 * n * n + 12 * n   # encode: W_fc + aux
    for j in range(gamma):
        rows = L + j                                      # rows attended before the new one
        tot += WB * p_step + 8 * n + tok_bytes(cfg) + (rows + 1) * 2 * kv_bytes * kvd
    if rebuild:
        T = accepted + 1                                  # rebuild rows
        tot += WB * 3 * n * n + WB * 2 * kvd * 2 * n + T * (12 * n + 4 + 2 * n + 2 * kv_bytes * kvd)
    return tot


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3-8b")
    ap.add_argument("--gamma", type=int, default=0, help="override the workload's chain length")
    ap.add_argument("--kernel", default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-rounds", type=int, default=5)
    ap.add_argument("--kv", choices=["f32", "bf16", "q8q5"], default="f32",
                    help="draft-KV element type")
    ap.add_argument("--token-table", choices=["default", "on", "off"], default="default",
                    help="the chain step's QKV embedding half from the load-time token table (default: on with "
                         "bf16 weights) or streamed (off)")
    ap.add_argument("--append", choices=["default", "split", "bf16", "f16"], default="default",
                    help="teacher-forced activation form of the prefill and rebuild GEMMs (default: fp16 with "
                         "bf16 weights, split with int4 weights)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration runs)")
    ap.add_argument("--weights", choices=["bf16", "int4"], default="bf16",
                    help="int4: projection weights quantized at load (groups of 32, bf16 scales)")
    ap.add_argument("--drafter", choices=["persistent", "round-local"], default="persistent",
                    help="round-local: the scratch-KV drafter (each round attends over its own rows "
                         "only; a step is one chain round from encoded taps, no rebuild)")
    ap.add_argument("--boundary", choices=["stored", "taps"], default=None,
                    help="stored: each rebuild also encodes the next round's boundary taps (one "
                         "W_fc pass) and the chain starts from that feature, the context growing "
                         "by a+1 rows per round around a mean of the workload's length; taps: the "
                         "chain encodes the boundary taps itself and every round is rewound to "
                         "the workload's length (the default for page4, whose rounds are rewound; "
                         "stored elsewhere)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="reference only: the vendor GEMM (torch.mm, fp16 and bf16, contiguous operands) at "
                         "the workload's prefill GEMM shapes (one append pass of up to 4096 rows), next to "
                         "the MFMA calibration loop")
    ap.add_argument("--graph-ab", action="store_true",
                    help="launch-overhead A/B: one chain round (boundary taps, rewound, so every round "
                         "runs at the same position) issued eagerly vs replayed from a captured HIP "
                         "graph of 1 and of 10 rounds; also the host time to issue one round")
    ap.add_argument("--stream-sizes", action="store_true",
                    help="the streaming read rate (the calibration kernel: the weight stream's access "
                         "pattern) against the size of the buffer read, 16 MB to 1 GiB")
    ap.add_argument("--verify-attn", action="store_true",
                    help="time eagle3_verify_attention alone: the workload's KV heads over its "
                         "context plus a gamma+1-row window, against gamma+1 single-row calls")
    args = ap.parse_args()
    args.kernel_set = args.kernel is not None
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU (--gpus 1); "
                                   "the engine has no multi-GPU sharding"}))
        sys.exit(2)

    import numpy as np
    import torch

    from eagle_draft_head_amd import binding as B
    from eagle_draft_head_amd.drafter import Drafter
    from synth import ALL, gen

    cfg = ALL[args.workload]
    if args.stream_sizes:
        return run_stream_sizes(args)
    if args.verify_attn:
        return run_verify_attn(args, cfg)
    if args.graph_ab:
        return run_graph_ab(args, cfg)
    if args.vendor_gemm:
        return run_vendor_gemm(args, cfg)
    if cfg.max_seqs > 1:
        return run_batched(args, cfg)
    gamma = args.gamma or cfg.gamma
    L = cfg.context
    dev = "cuda"
    torch.cuda.set_device(0)
    t0 = time.time()
    wd = gen.drafter_weights(cfg, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] weights generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    nsteps = args.steps + args.warmup
    local = args.drafter == "round-local"
    if args.boundary is None:
        args.boundary = "taps" if args.workload == "page4" else "stored"
    stored = args.boundary == "stored" and not local
    accepted = [i % (gamma + 1) for i in range(nsteps)]
    if stored:
        # committed rows before step i; the start is chosen so that the mean over
        # the timed steps is L
        grow = np.cumsum([0] + [a + 1 for a in accepted])
        L0 = L - int(round(float(grow[args.warmup:nsteps].mean())))
        L_at = [L0 + int(g) for g in grow[:nsteps]]
    else:
        L_at = [L] * nsteps
    max_ctx = max(L, max(L_at)) + gamma + 64
    kv_dtype = {"bf16": B.KV_BF16, "q8q5": B.KV_Q8Q5}.get(args.kv, B.KV_F32)
    i4 = args.weights == "int4"
    global WB, TABLE
    WB = WB_I4 if i4 else WB_BF16
    TABLE = args.token_table != "off"
    # with the token table (bf16 weights, not q8q5 K/V) the engine runs lm_head together
    # with the next step's hidden-half QKV (deferred QKV) in every step but a chain's
    # last; with stored boundaries the first step's hidden half is computed by the
    # append that stores the boundary (in its K/V launch), so a chain streams it gamma-1
    # times, not gamma
    deferred = (TABLE and not i4 and args.kv != "q8q5" and os.environ.get("EAGLE3_DEFER_QKV", "1") != "0")
    first_in_append = deferred and stored and os.environ.get("EAGLE3_BOUNDARY_QH", "1") != "0"
    if args.kernel is None:
        args.kernel = "lm_head_qkv" if deferred and gamma > 1 else "lm_head"
    dr = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=max_ctx, max_gamma=max(8, gamma), kv_dtype=kv_dtype,
                 weight_format=B.WEIGHTS_I4 if i4 else B.WEIGHTS_BF16,
                 append_act={"default": B.APPEND_DEFAULT, "split": B.APPEND_SPLIT, "bf16": B.APPEND_BF16,
                             "f16": B.APPEND_F16}[args.append],
                 token_table={"default": B.TABLE_DEFAULT, "on": B.TABLE_ON, "off": B.TABLE_OFF}[args.token_table])
    stream = torch.cuda.current_stream()

    # committed context
    aux_c = gen.aux_taps(cfg, 0, L, device=dev)
    tok_c = gen.tokens(cfg, 0, L, device=dev)
    torch.cuda.synchronize()
    tp = time.time()
    dr.prefill(0, tok_c, aux_c)
    torch.cuda.synchronize()
    prefill_s = time.time() - tp
    print(f"[bench] prefill {L} rows: {prefill_s * 1e3:.2f} ms (first call)", file=sys.stderr, flush=True)
    # a timed prefill of the same rows (rewind first)
    dr.rewind(0, 0)
    torch.cuda.synchronize()
    tp = time.time()
    dr.prefill(0, tok_c, aux_c)
    torch.cuda.synchronize()
    prefill_s = time.time() - tp
    n = cfg.n_embd
    prefill_flop = 2.0 * L * 3 * n * n + 2.0 * L * 2 * n * 2 * cfg.kv_dim

    b_aux = gen.aux_taps(cfg, 1, nsteps + 1, device=dev)
    b_tok = gen.tokens(cfg, 1, nsteps, device=dev)
    r_aux = gen.aux_taps(cfg, 2, nsteps * (gamma + 1), device=dev)
    r_tok = gen.tokens(cfg, 2, nsteps * (gamma + 1), device=dev)
    # a rebuild's first row is the round's boundary (taps, token)
    for i in range(nsteps):
        for x, b in zip(r_aux, b_aux):
            x[i * (gamma + 1)].copy_(b[i])
        r_tok[i * (gamma + 1)] = b_tok[i]
    out = torch.empty((1, gamma), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def reset(i):
        """The state before step i: L_at[i] committed rows and (stored) the boundary
        feature of step i (a boundary-only prefill).  Untimed."""
        dr.rewind(0, L_at[i])
        if stored:
            dr.prefill(0, r_tok[:0], [], next_aux=[a[i:i + 1] for a in b_aux])

    def chain(i):
        dr.draft_chain([0], b_tok[i:i + 1], None if stored else [a[i:i + 1] for a in b_aux], gamma,
                       out=out, round_local=local)

    def rebuild(i):
        if local:
            return
        a = accepted[i]
        r0 = i * (gamma + 1)
        dr.rebuild_after_verify([0], [a], r_tok[r0:r0 + a + 1], [x[r0:r0 + a + 1] for x in r_aux],
                                next_aux=[x[i + 1:i + 2] for x in b_aux] if stored else None)
        if not stored:
            dr.rewind(0, L)

    def step(i):
        chain(i)
        rebuild(i)

    if args.calib_copy:
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    reset(0)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.warmup, nsteps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    # the same steps again with HIP events around every launch of the measured
    # kernel on its stream (events add gaps, so this pass is not the one timed above)
    reset(args.warmup)
    torch.cuda.synchronize()
    B.eagle3_profile_enable(dr.ctx, args.kernel, True)
    for i in range(args.warmup, nsteps):
        step(i)
    torch.cuda.synchronize()
    k_ms, k_launches = B.eagle3_profile_read(dr.ctx)
    B.eagle3_profile_enable(dr.ctx, args.kernel, False)

    # round-time distribution and the chain alone (events around every step and
    # every draft_chain call, in a pass of its own), then the encode kernel's time
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    reset(args.warmup)
    for k, i in enumerate(range(args.warmup, nsteps)):
        e0, e1, e2 = ev[k]
        e0.record(stream)
        chain(i)
        e1.record(stream)
        rebuild(i)
        e2.record(stream)
    torch.cuda.synchronize()
    round_ms = sorted(e0.elapsed_time(e2) for e0, _, e2 in ev)
    chain_ms = sorted(e0.elapsed_time(e1) for e0, e1, _ in ev)
    pct = lambda v, q: v[min(len(v) - 1, int(q * len(v)))]
    reset(args.warmup)
    torch.cuda.synchronize()
    B.eagle3_profile_enable(dr.ctx, "encode", True)
    for i in range(args.warmup, nsteps):
        step(i)
    torch.cuda.synchronize()
    enc_ms, enc_n = B.eagle3_profile_read(dr.ctx)
    B.eagle3_profile_enable(dr.ctx, "encode", False)
    encode_us = enc_ms * 1e3 / max(enc_n, 1)
    per_step_us = (pct(chain_ms, 0.5) * 1e3 - encode_us) / gamma

    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = gamma * args.steps / elapsed
    k_avg_s = (k_ms / 1e3) / max(k_launches, 1)
    kvb = KV_BYTES[args.kv]
    k_bytes = kernel_bytes(cfg, args.kernel, 0 if local else L, kvb)
    achieved = k_bytes / k_avg_s / 1e9
    if local:
        sb = [step_bytes(cfg, 0, gamma, 0, kvb, rebuild=False) for i in range(args.warmup, nsteps)]
    else:
        sb = [step_bytes(cfg, L_at[i], gamma, accepted[i], kvb, stored) for i in range(args.warmup, nsteps)]
    step_gbs = (sum(sb) / args.steps) / (elapsed / args.steps) / 1e9

    # a draft step's bytes as the chain streams them (the first step's hidden half
    # comes from the append when first_in_append)
    chain_b = kernel_bytes_step(cfg, 0 if local else L, gamma, kvb)
    if first_in_append:
        chain_b -= WB * cfg.n_embd * (cfg.q_dim + 2 * cfg.kv_dim) / gamma
    cal = calibrate(B, torch)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, wd, aux_c, tok_c, b_aux, b_tok, gamma, args.cpu_rounds, int4_weights=i4)

    line = {
        "metric": "draft tokens/sec (gamma=3 chain, batch 1) and achieved HBM GB/s per draft step",
        "value": round(tokens_per_s, 2),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"int4 weights (groups of 32, bf16 scales)" if i4 else "bf16 weights")
                 + f", fp32 accumulate, {args.kv} draft KV",
        "data": "synthetic (seeded; random-init weights of the drafter architecture)",
        "config": {"workload": f"{cfg.name} drafter: n_embd {cfg.n_embd}, {cfg.n_head}/{cfg.n_head_kv} "
                               f"heads x {cfg.head_dim}, n_ff {cfg.n_ff}, draft vocab {cfg.draft_vocab}, "
                               f"target vocab {cfg.target_vocab}, {L} committed KV rows"
                               + (" (not attended: round-local drafter)" if local else "")
                               + (f" (mean over the timed rounds; {L_at[args.warmup]}.."
                                  f"{L_at[-1]})" if stored else ""),
                   "batch": 1, "gamma": gamma, "token_table": TABLE,
                   "step": ("draft_chain from the stored boundary feature + rebuild_after_verify("
                            f"a+1 rows, a cycling 0..{gamma}, with the next boundary's taps)")
                   if stored else
                   "round-local draft_chain (boundary taps; attention over the round's own rows; "
                   "no rebuild)" if local else
                   f"draft_chain(boundary taps) + rebuild_after_verify(a+1 rows, a cycling 0..{gamma}) "
                   "+ rewind"},
        "roofline": {"bound": "hbm", "kernel": args.kernel, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if i4 else committed_traffic(args.kernel),
                     "avg_launch_us": round(k_avg_s * 1e6, 3),
                     "launches": k_launches, "bytes_per_launch": k_bytes,
                     "calibrated_peak": cal["hbm_stream_read_gbs"],
                     "frac_calibrated": round(achieved / cal["hbm_stream_read_gbs"], 4)},
        "calibrated": cal,
        "step_hbm_gbs": round(step_gbs, 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "round_ms": {"p10": round(pct(round_ms, 0.1), 4), "p50": round(pct(round_ms, 0.5), 4),
                     "p90": round(pct(round_ms, 0.9), 4)},
        "chain_ms_p50": round(pct(chain_ms, 0.5), 4),
        "encode_us": round(encode_us, 2),
        "draft_step_us": round(per_step_us, 2),
        "draft_step_bytes": round(chain_b),
        "draft_step_hbm_frac": round(chain_b / (per_step_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "draft_step_hbm_frac_calibrated": round(chain_b / (per_step_us * 1e-6) / 1e9
                                                / cal["hbm_stream_read_gbs"], 4),
        "first_hidden_half_in_append": first_in_append,
        "prefill": {"rows": L, "ms": round(prefill_s * 1e3, 3), "append_act": args.append,
                    "tflops": round(prefill_flop / prefill_s / 1e12, 2),
                    "frac_bf16_peak": round(prefill_flop / prefill_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                    "frac_calibrated": round(prefill_flop / prefill_s / 1e12 / cal["mfma_bf16_tflops"], 4),
                    "note": "algorithmic flops (fc and K|V projections) over the wall time of the whole "
                            "prefill call"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    dr.close()


def batched_kernel_bytes(cfg, kernel: str, lens, gamma: int, kv_bytes: int = 4) -> float:
    """Algorithmic HBM bytes per launch of a batched-step kernel, averaged over the
    steps of a round (`lens`: committed rows per sequence; K/V elements of
    kv_bytes bytes)."""
    n, qd, kvd, ff, dv = cfg.n_embd, cfg.q_dim, cfg.kv_dim, cfg.n_ff, cfg.draft_vocab
    m = len(lens)
    if kernel == "attention":
        rows = sum(L + j + 1 for L in lens for j in range(gamma)) / gamma
        return 2.0 * kv_bytes * kvd * rows + m * (4 * qd + 4 * qd)
    act = {"lm_head": (dv, n), "gate_up": (2 * ff, n), "qkv": (qd + 2 * kvd, 2 * n),
           "down": (n, ff), "o_proj": (n, qd)}[kernel]
    return 2.0 * act[0] * act[1] + m * 4 * act[1]


def run_vendor_gemm(args, cfg):
    """What the vendor GEMM reaches at the prefill shapes: C = A . W^T for the fc
    ([rows, 3n] x [3n, n]) and the K|V projection ([rows, 2n] x [2n, 2 kv_dim]) of
    one append pass (rows = min(context, 4096)).  torch.mm dispatches to hipBLASLt;
    the engine never calls it.  HIP events around `steps` calls after `warmup`."""
    import torch

    from eagle_draft_head_amd import binding as B

    torch.cuda.set_device(0)
    cal = calibrate(B, torch)
    rows = min(cfg.context, 4096)
    n, kvd = cfg.n_embd, cfg.kv_dim
    shapes = {"fc": (rows, n, 3 * n), "kv": (rows, 2 * kvd, 2 * n)}
    res = {}
    for dt, tag in ((torch.float16, "fp16"), (torch.bfloat16, "bf16")):
        for name, (M, N, K) in shapes.items():
            a = torch.randn(M, K, device="cuda", dtype=dt)
            bt = torch.randn(K, N, device="cuda", dtype=dt).contiguous()
            for _ in range(args.warmup):
                c = torch.mm(a, bt)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                c = torch.mm(a, bt)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.steps
            res[f"{name}_{tag}"] = {"M": M, "N": N, "K": K, "us": round(us, 2),
                                    "tflops": round(2.0 * M * N * K / us / 1e6, 1)}
            del a, bt, c
    print(json.dumps({"metric": "vendor GEMM TFLOP/s at the prefill shapes (reference)", "unit": "TFLOP/s",
                      "value": res["fc_fp16"]["tflops"], "higher_is_better": True, "n_gpus": 1,
                      "steps": args.steps, "warmup": args.warmup, "gemms": res, "calibrated": cal,
                      "config": {"workload": f"{cfg.name}: one append pass of {rows} rows"}}), flush=True)


def run_graph_ab(args, cfg):
    """Eager launches vs HIP graph replay of one chain round.  The round starts from
    the boundary taps at the workload's committed length and is rewound afterwards,
    so every round writes the same KV rows and a replay of its captured kernels
    repeats it exactly.  Every replay is checked against the eager ids, with eager
    rounds and synchronisations between replays."""
    import torch

    from eagle_draft_head_amd.drafter import Drafter
    from synth import gen

    gamma = args.gamma or cfg.gamma
    L = cfg.context
    torch.cuda.set_device(0)
    wd = gen.drafter_weights(cfg, device="cuda")
    dr = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=L + gamma + 64, max_gamma=max(8, gamma))
    dr.prefill(0, gen.tokens(cfg, 0, L, device="cuda"), gen.aux_taps(cfg, 0, L, device="cuda"))
    b_aux = [a.contiguous() for a in gen.aux_taps(cfg, 1, 1, device="cuda")]
    b_tok = gen.tokens(cfg, 1, 1, device="cuda")
    out = torch.empty((1, gamma), dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    N = max(args.steps, 10) // 10 * 10

    def chain(o=out):
        dr.draft_chain([0], b_tok, b_aux, gamma, out=o, stream=torch.cuda.current_stream())

    def events(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    with torch.cuda.stream(side):
        for _ in range(args.warmup):
            chain()
        torch.cuda.synchronize()
        ref = out.clone()
        eager_us = events(chain, N) / N
        t0 = time.perf_counter()
        for _ in range(N):
            chain()
        issue_us = (time.perf_counter() - t0) * 1e6 / N
        torch.cuda.synchronize()
    res = {"eager_us": round(eager_us, 2), "host_issue_us": round(issue_us, 2)}
    other = torch.empty_like(out)
    ok = True
    for per in (1, 10):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per):
                chain()
        torch.cuda.synchronize()
        for _ in range(3):
            out.fill_(-7)
            with torch.cuda.stream(side):
                chain(other)                      # eager work between the replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ok = ok and torch.equal(out, ref) and torch.equal(other, ref)
        res[f"graph{per}_us"] = round(events(g.replay, N // per) / N, 2)
        del g
    dr.close()
    print(json.dumps({
        "metric": "chain round time: eager launches vs HIP graph replay", "unit": "us per round",
        "value": res["graph1_us"], "higher_is_better": False, "n_gpus": 1, "steps": N,
        "warmup": args.warmup, "replays_equal_eager": bool(ok), **res,
        "config": {"workload": f"{cfg.name}: one gamma={gamma} chain round from boundary taps over {L} "
                               f"committed rows, rewound (every round at the same position)"}}),
        flush=True)


def run_stream_sizes(args):
    """Streaming read rate against buffer size: each read of a buffer follows an
    untimed 2 GiB flush read (best of 5).  A launch pays a fixed ramp and drain, so
    smaller reads see a lower rate."""
    import torch
    from eagle_draft_head_amd import binding as B
    torch.cuda.set_device(0)
    sink = torch.empty(B.CALIB_SINK_BYTES, dtype=torch.uint8, device="cuda")
    flush = torch.empty(2 << 30, dtype=torch.uint8, device="cuda").fill_(2)
    rates = []
    for mb in (16, 32, 64, 128, 262.144, 512, 1024):
        nbytes = int(mb * 1e6) // 16 * 16 if mb != 1024 else 1 << 30
        buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        torch.cuda.synchronize()
        gbs = B.eagle3_calibrate_stream(buf, nbytes, flush, flush.numel(), 5, sink)
        rates.append({"bytes": nbytes, "gbs": round(gbs, 1), "us": round(nbytes / gbs / 1e3, 2)})
        print(f"[bench] {nbytes / 1e6:8.1f} MB: {gbs:7.1f} GB/s ({nbytes / gbs / 1e3:.1f} us)", file=sys.stderr,
              flush=True)
        del buf
    print(json.dumps({"metric": "streaming read rate by buffer size (HBM, after a 2 GiB flush read)",
                      "unit": "GB/s", "peak": HBM_PEAK_GBS, "rates": rates,
                      "how": "eagle3_calibrate_stream: each wave reads contiguous 16 KB runs with "
                             "non-temporal 16-byte loads, four in flight per lane; best of 5"}), flush=True)


def run_verify_attn(args, cfg):
    """The verify-window attention alone: the workload's heads (the drafter's, as a
    stand-in for a target of that shape) over its context plus a window of gamma + 1
    rows, fp32 or bf16 K/V resident in HBM.  One step = one eagle3_verify_attention
    call; bytes = the K/V rows read once + q + out.  Also times the same window as
    gamma + 1 single-row calls (row m over ctx + m + 1 rows), which read the rows
    gamma + 1 times."""
    import numpy as np
    import torch

    from eagle_draft_head_amd import binding as B
    from synth import gen

    gamma = args.gamma or cfg.gamma
    M = gamma + 1
    ctx = cfg.context
    nh, nkv, hd = cfg.n_head, cfg.n_head_kv, cfg.head_dim
    kv = B.KV_BF16 if args.kv == "bf16" else B.KV_F32
    if args.kv == "q8q5":
        print(json.dumps({"error": "verify attention takes fp32 or bf16 K/V"}))
        sys.exit(2)
    esz = 2 if kv == B.KV_BF16 else 4
    cap = ctx + M
    dt = torch.bfloat16 if kv == B.KV_BF16 else torch.float32
    q = gen.normal(98, 1, (M, nh, hd), 1.0, device="cuda")
    k = gen.normal(98, 2, (nkv, cap, hd), 1.0, device="cuda").to(dt)
    v = gen.normal(98, 3, (nkv, cap, hd), 1.0, device="cuda").to(dt)
    out = torch.empty((M, nh, hd), dtype=torch.float32, device="cuda")
    ws_bytes = max(B.eagle3_verify_attention_workspace(M, nh, nkv, hd, ctx + M - 1, kv), 4)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def window():
        B.eagle3_verify_attention(q, k, v, kv, cap, ctx, M, nh, nkv, hd, out, ws, ws_bytes, stream)

    def singles():
        for m in range(M):
            B.eagle3_verify_attention(q[m:m + 1], k, v, kv, cap, ctx + m, 1, nh, nkv, hd, out[m:m + 1],
                                      ws, ws_bytes, stream)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps * 1e3  # us per call

    us = timed(window)
    us_single = timed(singles)
    bytes_w = 2.0 * esz * nkv * hd * (ctx + M) + 4.0 * 2 * M * nh * hd
    gbs = bytes_w / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "verify-window attention GB/s (K/V rows read once)", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "us_per_call": round(us, 3), "us_per_window_as_single_rows": round(us_single, 3),
        "higher_is_better": True, "dtype": f"{args.kv} K/V, fp32 q and accumulate",
        "data": "synthetic (seeded)",
        "config": {"workload": f"{cfg.name} heads {nh}/{nkv} x {hd}, {ctx} context rows + a "
                               f"{M}-row window"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000.0, 4), "bytes_per_call": bytes_w},
    }))


def run_batched(args, cfg):
    """Batched drafting: one draft_chain over all sequences per step, then a packed
    rebuild of a_b + 1 rows per sequence (a_b seeded on [0, gamma]) and a rewind of
    every sequence to its seeded length."""
    if args.weights != "bf16" or args.kv == "q8q5":
        print(json.dumps({"error": "int4 weights and q8q5 KV are batch-1 modes"}))
        sys.exit(2)
    import numpy as np
    import torch

    from eagle_draft_head_amd import binding as B
    from eagle_draft_head_amd.drafter import Drafter
    from synth import gen

    gamma = args.gamma or cfg.gamma
    kernel = args.kernel if args.kernel_set else "attention"
    dev = "cuda"
    torch.cuda.set_device(0)
    lens = gen.batch_lengths(cfg)
    S = len(lens)
    wd = gen.drafter_weights(cfg, device=dev)
    kv_dtype = B.KV_BF16 if args.kv == "bf16" else B.KV_F32
    dr = Drafter(cfg, wd, wd["d2t"].cpu(), max_ctx=cfg.max_ctx, max_gamma=max(8, gamma), max_seqs=S,
                 kv_dtype=kv_dtype)
    t0 = time.time()
    for s, L in enumerate(lens):
        aux = gen.aux_taps(cfg, 100 + s, L, device=dev)
        tok = gen.tokens(cfg, 100 + s, L, device=dev)
        dr.prefill(s, tok, aux)
        del aux, tok
    torch.cuda.synchronize()
    print(f"[bench] prefill of {S} sequences ({sum(lens)} rows) in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)
    nsteps = args.steps + args.warmup
    b_aux = gen.aux_taps(cfg, 1, nsteps * S, device=dev)
    b_tok = gen.tokens(cfg, 1, nsteps * S, device=dev)
    r_aux = gen.aux_taps(cfg, 2, S * (gamma + 1), device=dev)
    r_tok = gen.tokens(cfg, 2, S * (gamma + 1), device=dev)
    acc_all = gen.uniform_int(cfg.cfg_id, 40_000, nsteps * S, gamma + 1).view(nsteps, S).tolist()
    out = torch.empty((S, gamma), dtype=torch.int32, device=dev)
    seqs = list(range(S))
    drafted = []

    def step(i):
        geff = dr.draft_chain(seqs, b_tok[i * S:(i + 1) * S],
                              [a[i * S:(i + 1) * S] for a in b_aux], gamma, out=out)[1]
        acc = [min(acc_all[i][s], geff[s]) for s in seqs]
        live = [s for s in seqs if geff[s] > 0]
        rows = sum(acc[s] + 1 for s in live)
        dr.rebuild_after_verify(live, [acc[s] for s in live], r_tok[:rows], [x[:rows] for x in r_aux])
        for s in seqs:
            dr.rewind(s, lens[s])
        drafted.append(sum(geff))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    drafted.clear()
    t_start = time.perf_counter()
    for i in range(args.warmup, nsteps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    tokens = sum(drafted)
    B.eagle3_profile_enable(dr.ctx, kernel, True)
    for i in range(args.warmup, nsteps):
        step(i)
    torch.cuda.synchronize()
    k_ms, k_launches = B.eagle3_profile_read(dr.ctx)
    B.eagle3_profile_enable(dr.ctx, kernel, False)
    k_avg_s = (k_ms / 1e3) / max(k_launches, 1)
    kvb = 2 if args.kv == "bf16" else 4
    k_bytes = batched_kernel_bytes(cfg, kernel, lens, gamma, kvb)
    achieved = k_bytes / k_avg_s / 1e9

    n, qd, kvd, ff, dv = cfg.n_embd, cfg.q_dim, cfg.kv_dim, cfg.n_ff, cfg.draft_vocab
    p_step = (qd + 2 * kvd) * 2 * n + n * qd + 3 * ff * n + dv * n
    kv_bytes = sum(2.0 * kvb * kvd * (L + j + 1) for L in lens for j in range(gamma))
    round_bytes = 6.0 * n * n + gamma * (2.0 * p_step) + kv_bytes
    step_gbs = round_bytes / (elapsed / args.steps) / 1e9

    cal = calibrate(B, torch)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline_batched(cfg, wd, lens, b_aux, b_tok, gamma)
    line = {
        "metric": f"draft tokens/sec (gamma={gamma} chain, batch {S}) and achieved HBM GB/s per draft step",
        "value": round(tokens / elapsed, 2),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"bf16 weights, fp32 accumulate, {args.kv} draft KV",
        "data": "synthetic (seeded; random-init weights of the drafter architecture)",
        "config": {"workload": f"{cfg.name}: {S} sequences of the {cfg.n_embd}-wide drafter with "
                               f"{min(lens)}..{max(lens)} committed rows (sum {sum(lens)})",
                   "batch": S, "gamma": gamma,
                   "step": "batched draft_chain + packed rebuild_after_verify + rewind to the seeded lengths"},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_us": round(k_avg_s * 1e6, 3),
                     "launches": k_launches, "bytes_per_launch": k_bytes,
                     "calibrated_peak": cal["hbm_stream_read_gbs"],
                     "frac_calibrated": round(achieved / cal["hbm_stream_read_gbs"], 4)},
        "calibrated": cal,
        "round_hbm_gbs": round(step_gbs, 1),
        "round_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    dr.close()


def _blas_threads_and_vendor():
    """(threads the BLAS may use = the CPUs this process is allowed on, vendor)."""
    cores = len(os.sched_getaffinity(0))
    vendor = "unknown"
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            vendor = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
    except Exception:
        pass
    return cores, vendor


def _timed_rounds(fn, rounds, threads):
    """Median seconds of `rounds` calls of fn(r) with the BLAS limited to `threads`."""
    from contextlib import nullcontext
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=threads, user_api="blas")
    except Exception:
        ctx = nullcontext()
    times = []
    with ctx:
        for r in range(rounds):
            t1 = time.perf_counter()
            fn(r)
            times.append(time.perf_counter() - t1)
    return sorted(times)[len(times) // 2]


def cpu_baseline_batched(cfg, wd, lens, b_aux, b_tok, gamma, rounds=5):
    """The oracle's fp32 timing mode on a sample of the batched workload: chain
    rounds of the shortest sequence (its prefill is untimed setup); a batched round
    on the host is the sequences' rounds one after another, so tokens/s is the
    per-sequence rate."""
    import numpy as np
    from synth import gen
    from tests.common import make_oracle
    cores, vendor = _blas_threads_and_vendor()
    wh = {k: v.cpu() for k, v in wd.items() if k != "embed"}
    s = int(np.argmin(lens))
    orc = make_oracle(cfg, wh, max_ctx=cfg.max_ctx, max_seqs=len(lens), lazy_embed=True,
                      dtype=np.float32)
    aux = gen.aux_taps(cfg, 100 + s, lens[s])
    tok = gen.tokens(cfg, 100 + s, lens[s])
    orc.prefill(s, [a.numpy() for a in aux], tok.numpy())
    S = len(lens)

    def one(r):
        orc.draft_chain(s, [a[r * S + s].cpu().numpy() for a in b_aux], int(b_tok[r * S + s]), gamma)

    med = _timed_rounds(one, rounds, cores)
    med1 = _timed_rounds(one, 3, 1)
    return {"value": round(gamma / med, 3), "unit": "draft tokens/s", "cores": cores,
            "kind": "oracle fp32", "blas": vendor, "value_1thread": round(gamma / med1, 3),
            "sample": f"the oracle's fp32 timing mode (numpy): median of {rounds} gamma={gamma} "
                      f"chain rounds of sequence {s} ({lens[s]} committed rows) with {cores} BLAS "
                      f"threads, and of 3 rounds with 1 thread; a batched round on the host runs "
                      f"the sequences one after another; prefill untimed"}


def cpu_baseline(cfg, wd, aux_c, tok_c, b_aux, b_tok, gamma, rounds, int4_weights=False):
    """The oracle's fp32 timing mode (numpy) on the host: prefill of the committed
    rows (untimed setup), then chain rounds of gamma steps, the median of `rounds`
    with the BLAS on every allowed CPU and of 3 rounds on one thread."""
    import numpy as np
    from tests.common import make_oracle
    cores, vendor = _blas_threads_and_vendor()
    wh = {k: v.cpu() for k, v in wd.items() if k != "embed"}
    if int4_weights:  # the same int4 weights the GPU streams (untimed setup)
        from oracle import int4
        wh = int4.int4_weights(wh)
    L = int(tok_c.numel())
    orc = make_oracle(cfg, wh, max_ctx=L + 64, lazy_embed=True, dtype=np.float32)
    t0 = time.perf_counter()
    orc.prefill(0, [a.cpu().numpy() for a in aux_c], tok_c.cpu().numpy())
    setup_s = time.perf_counter() - t0

    def one(r):
        orc.draft_chain(0, [a[r].cpu().numpy() for a in b_aux], int(b_tok[r]), gamma)

    med = _timed_rounds(one, rounds, cores)
    med1 = _timed_rounds(one, 3, 1)
    return {"value": round(gamma / med, 4), "unit": "draft tokens/s", "cores": cores,
            "kind": "oracle fp32", "blas": vendor, "value_1thread": round(gamma / med1, 4),
            "sample": f"the oracle's fp32 timing mode (numpy"
                      f"{', int4 weights' if int4_weights else ''}): median of {rounds} chain rounds "
                      f"of gamma={gamma} over {L} committed rows with {cores} BLAS threads "
                      f"({med:.3f} s a round), and of 3 rounds with 1 thread ({med1:.3f} s); "
                      f"untimed setup prefill {setup_s:.1f} s"}


if __name__ == "__main__":
    main()
