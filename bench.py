#!/usr/bin/env python3
"""Throughput of one approximate-attention prefill layer on one MI355X.

A step is one pass of the whole path on inputs already resident in HBM:
spava_score_topk -> spava_gather_passing -> spava_attn_fwd -> spava_lse_merge
(--order partials-first: the attention's LOCAL phase, scores from the query
partials, gather, the PASSING phase, merge; --selector context: the
context-driven selector in place of spava_score_topk).
Default workload: Qwen2.5-VL-7B-like attention at 256K tokens (28 query / 4
KV heads, d=128; anchor 4096; 32 virtual hosts x 8128 frame-structured
tokens; query 512; lp=4096), bf16 -- the largest single-GPU configuration.
--workload picks another (e.g. qwen2.5vl3b_32k).

Prints ONE JSON line.  Besides the throughput it reports the roofline of the
dominant call (the fused attention) from HIP events recorded on the stream
the library launches on, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "approx-attention prefill tokens/s per layer; TFLOP/s and % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X float32 vector ALUs (the float32 path does not use MFMA)
PEAK_HBM_GBS = 8000.0


def attn_pairs_per_head(w, lp=None) -> int:
    """Unmasked (query, key) pairs of one query head over the whole layer."""
    la, V, L, nq = w.n_anchor, w.n_hosts, w.host_len, w.n_query
    lp = w.lp if lp is None else lp
    anchor = la * (la + 1) // 2
    context = sum(L * (la + h * lp) + L * (L + 1) // 2 for h in range(V))
    query = nq * la + nq * (nq + 1) // 2 + V * nq * L
    return anchor + context + query


def attn_flops(w) -> float:
    return 4.0 * w.head_dim * w.n_q_heads * attn_pairs_per_head(w)


def score_flops(w, selector="query") -> float:
    """One Q K^T pass of the scoring rows over their keys (both score passes
    recompute it; only one is counted as algorithmic work): the query rows
    over every block, or (context selector) each block's tokens causally over
    the block's own keys."""
    if selector == "context":
        L = w.host_len
        return 2.0 * w.head_dim * w.n_q_heads * w.n_hosts * (L * (L + 1) // 2)
    return 2.0 * w.head_dim * (w.n_query * w.n_q_heads) * (w.n_hosts * w.host_len)


# Copy-calibrated FETCH_SIZE + WRITE_SIZE summaries of the attention kernel,
# one per workload: profiles/attn_fwd_<workload>_traffic.md.
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
# The attention kernel's sources: its file and the headers that define its
# unit order and copy helpers.
ATTN_SOURCES = [os.path.join(ROOT, "sequence_approximate_attention_amd", "csrc", f)
                for f in ("attn_bf16.hip", "spava_common.h", "lds_dma.h")]


def attn_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM-side bytes per attention launch from the committed counter summary
    of this workload (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when
    there is none or it was taken on a different kernel source than the one
    built here."""
    import glob
    for path in sorted(glob.glob(os.path.join(TRAFFIC_DIR, "attn_fwd_*_traffic.md"))):
        try:
            fields = {}
            for line in open(path):
                if " = " in line:
                    key, val = line.strip().split(" = ", 1)
                    fields[key] = val
            if fields.get("workload") != workload:
                continue
            if fields.get("kernel_source_sha256") != attn_source_sha256():
                return None
            return float(fields["traffic_bytes_per_launch"])
        except (OSError, KeyError, ValueError):
            continue
    return None


def host_cpu():
    """(logical CPUs this process may run on, CPU model name)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, model


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        return 1


def cpu_baseline(w, x, selector="query", attn_budget_s=10.0, row_stride=61):
    """The oracle as it stands, on a bounded sample of the same layer.

    Scoring, top-lp selection and the gather run in full (with the context
    selector, the scores of one of the V * Hkv lists are timed and
    extrapolated).  The attention then runs on a deterministic row sample:
    every ``row_stride``-th token of a host (a prime, so every tile residue
    is hit) with every query head, hosts taken in a spread order (0, V-1,
    V/2, V/4, 3V/4, then the rest) until about ``attn_budget_s`` seconds have
    been timed, plus every ``row_stride``-th query token (through its V+1
    partials and the merge).  The attention time is extrapolated to the
    whole layer by the ratio of visible (query, key) pairs: "sampled,
    flop-extrapolated"."""
    import oracle as O
    la, V, L, nq, lp = w.n_anchor, w.n_hosts, w.host_len, w.n_query, w.lp
    Hq = w.n_q_heads
    scale = 1.0 / math.sqrt(w.head_dim)
    G = w.group
    x32 = {n: x[n] for n in ("q", "k", "v")}
    t0 = time.perf_counter()
    t_extra = 0.0
    if selector == "context":
        sc = np.zeros((V, w.n_kv_heads, L))
        sc[0, 0] = O.context_block_scores(x32["q"][la:la + L, :G], x32["k"][la:la + L, :1], 0, 1, L, 0,
                                          scale)[0, 0]
        t_extra = (time.perf_counter() - t0) * (V * w.n_kv_heads - 1)
    else:
        sc = O.block_scores(x32["q"], x32["k"], la, V, L, nq)
    idx = O.select_passing(sc, lp)
    kp, vp = O.gather_passing(x32["k"], x32["v"], idx, la, L)
    t1 = time.perf_counter()
    threads = blas_threads()   # after the matrix products: the pool the oracle used

    hosts = []
    for h in [0, V - 1, V // 2, V // 4, 3 * V // 4] + list(range(V)):
        if h not in hosts:
            hosts.append(h)
    q0 = la + V * L
    qrows = [(t, a) for t in range(q0, q0 + nq, row_stride) for a in range(Hq)]
    sample_pairs = 0
    # Query tokens: anchor + causal query prefix, then every block in full.
    for t, _ in qrows:
        sample_pairs += la + (t - q0 + 1) + V * L
    O.sampled_rows(x32["q"], x32["k"], x32["v"], kp, vp, la, V, L, nq, qrows, scale)
    done = []
    for h in hosts:
        if done and time.perf_counter() - t1 >= attn_budget_s:
            break
        b0 = la + h * L
        rows = [(t, a) for t in range(b0, b0 + L, row_stride) for a in range(Hq)]
        O.sampled_rows(x32["q"], x32["k"], x32["v"], kp, vp, la, V, L, nq, rows, scale)
        sample_pairs += sum(la + h * lp + (t - b0) + 1 for t, _ in rows)
        done.append(h)
    t2 = time.perf_counter()
    total_pairs = attn_pairs_per_head(w) * Hq
    t_select = (t1 - t0) + t_extra
    t_layer = t_select + (t2 - t1) * total_pairs / sample_pairs
    nproc, model = host_cpu()
    return {
        "value": w.n_tokens / t_layer,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "nproc": nproc,
        "cpu_model": model,
        "sample": (f"sampled, flop-extrapolated. float64 numpy oracle on {threads} BLAS threads "
                   f"({nproc} logical CPUs available, {model}): {selector} scores + top-lp + gather of "
                   f"the full layer ({t_select:.1f} s"
                   + (", context scores of one of the V*Hkv lists timed and extrapolated"
                      if selector == "context" else "")
                   + f"); attention of every {row_stride}th token with all {Hq} query heads of hosts "
                   f"{', '.join(str(h) for h in done)} and every {row_stride}th query token "
                   f"({len(qrows)} query rows through their {V + 1} partials) "
                   f"({t2 - t1:.1f} s for {sample_pairs:.3g} of {total_pairs:.3g} visible pairs); "
                   f"attention extrapolated by pair count ({total_pairs / sample_pairs:.0f}x) "
                   f"to {t_layer:.1f} s per layer"),
    }


# Row-statistics work (scoring rows x keys, summed over blocks and KV heads)
# above which the Figure 5 order pays for its second attention launch: the
# pass it saves then outweighs the first launch's tail.  Measured: 256K
# frame shape (3.7e9) and 128K text layer (2.1e9) faster with partials-first,
# the 32K layers (6.3e7) faster in one pass.
PARTIALS_FIRST_MIN_WORK = 1e9


def pick_order(w, selector="query"):
    if selector != "query" or w.n_query == 0 or w.n_hosts < 2:
        return "one-pass"
    work = w.n_query * w.group * w.host_len * w.n_hosts * w.n_kv_heads
    return "partials-first" if work >= PARTIALS_FIRST_MIN_WORK else "one-pass"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="qwen2.5vl7b_256k_frames")
    ap.add_argument("--lp", type=int, default=None, help="override the workload's passing length")
    ap.add_argument("--dense", action="store_true",
                    help="time the library's dense causal plan over the workload's tokens and heads "
                         "(one host of N tokens, no anchor, query or passing blocks) instead")
    ap.add_argument("--order", choices=("auto", "one-pass", "partials-first"), default="auto",
                    help="one-pass: score, gather, one attention call; partials-first: the rows "
                         "that need no passing block first, scores from the query partials' LSEs, "
                         "then gather and the remaining rows (Figure 5 ordering); auto: "
                         "partials-first when the separate row-statistics pass it saves is long "
                         "(see pick_order)")
    ap.add_argument("--selector", choices=("query", "context"), default="query",
                    help="which rule scores the keys: the query block's attention (the pages' "
                         "method) or each block's own tokens (the referee's alternative)")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="after the timed loop, this many more steps each preceded (untimed) by a "
                         "512 MiB write that evicts the inputs from L2 and the Infinity Cache; "
                         "reported as cold_cache, not in value")
    ap.add_argument("--no-dense-context", action="store_true",
                    help="skip the six launches of the dense causal plan that are reported as "
                         "context (profiled runs use it so that every attention dispatch is the "
                         "workload's own)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a reference "
                         "kernel of known traffic for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the virtual hosts are batched on a single device).", file=sys.stderr)
        sys.exit(2)

    import torch
    import sequence_approximate_attention_amd as S
    import workloads as W

    wl = {w.name: w for w in W.WORKLOADS + W.PAGE_DEFAULT_WORKLOADS + [W.QWEN3B_32K_PAGE_DEFAULTS_Q128]}[args.workload]
    if args.lp is not None:
        wl = wl.with_(lp=args.lp)
    x = W.make_inputs(wl)   # the dense plan runs over the same tokens
    if args.dense:
        wl = wl.with_(name=wl.name + "_dense", n_anchor=0, n_hosts=1, host_len=wl.n_tokens, n_query=0, lp=0)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    plan = S.plan_for(wl)
    if wl.dtype == "bf16":
        to = lambda n: torch.from_numpy(x[n + "16"].view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        to = lambda n: torch.from_numpy(np.ascontiguousarray(x[n])).to(dev)
    q, k, v = to("q"), to("k"), to("v")
    bufs = S.alloc_buffers(plan, dev)
    if args.selector == "context":
        score_topk = S.spava_score_topk_context
        ws_score = torch.empty(max(256, S.spava_score_topk_context_ws_bytes(plan)), dtype=torch.uint8, device=dev)
    else:
        score_topk, ws_score = S.spava_score_topk, bufs.ws_score
    stream = torch.cuda.current_stream()
    q0 = wl.n_anchor + wl.n_hosts * wl.host_len

    if args.order == "auto":
        args.order = pick_order(wl, args.selector)
    if args.order == "partials-first" and args.selector == "context":
        print("--order partials-first scores from the query partials; it takes the query selector",
              file=sys.stderr)
        sys.exit(2)
    attn = lambda phase: S.spava_attn_fwd_phase(plan, phase, q, k, v, bufs.kp, bufs.vp, bufs.o, bufs.lse,
                                                bufs.o_part, bufs.lse_part, stream)
    rec = lambda ev, i: ev[i].record(stream) if ev is not None else None

    merge = lambda: S.spava_lse_merge(bufs.o_part, bufs.lse_part, bufs.o[q0:], plan.n_q_heads * plan.head_dim,
                                      bufs.lse[:, q0:], plan.n_tokens, stream)
    # Events around the calls of a step and the spans (pairs of events) that
    # make up each stage.  One pass: score | gather | attention | merge.
    # Figure 5 order: LOCAL phase | scores from the query partials | gather |
    # PASSING phase | merge.  (Merging right after the LOCAL phase, while its
    # partials are freshly written, measured slower: 59.7 against 56.1 us.)
    SPANS = {
        "one-pass": {"score_topk": [(0, 1)], "gather": [(1, 2)], "attn_fwd": [(2, 3)], "lse_merge": [(3, 4)],
                     "step": [(0, 4)]},
        "partials-first": {"attn_fwd": [(0, 1), (3, 4)], "score_topk": [(1, 2)], "gather": [(2, 3)],
                           "lse_merge": [(4, 5)], "step": [(0, 5)]},
    }[args.order]
    N_EV = 6
    span_ms = lambda ev, name: sum(ev[a].elapsed_time(ev[b]) for a, b in SPANS[name])

    def step(ev=None):
        if args.order == "partials-first":
            rec(ev, 0)
            attn(S.SPAVA_PHASE_LOCAL)
            rec(ev, 1)
            S.spava_score_topk_from_partials(plan, q, k, bufs.lse_part, bufs.scores, bufs.idx, stream)
            rec(ev, 2)
            S.spava_gather_passing(plan, k, v, bufs.idx, bufs.kp, bufs.vp, stream)
            rec(ev, 3)
            attn(S.SPAVA_PHASE_PASSING)
            rec(ev, 4)
            merge()
            rec(ev, 5)
        else:
            rec(ev, 0)
            score_topk(plan, q, k, bufs.scores, bufs.idx, ws_score, stream)
            rec(ev, 1)
            S.spava_gather_passing(plan, k, v, bufs.idx, bufs.kp, bufs.vp, stream)
            rec(ev, 2)
            attn(S.SPAVA_PHASE_ALL)
            rec(ev, 3)
            merge()
            rec(ev, 4)

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(N_EV)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Cold-cache steps: the 32K layer's inputs (~0.17 GB) fit in the 256 MB
    # Infinity Cache, so the loop above runs warm; a real model evicts them
    # between layers.  Per-step HIP-event time after a 512 MiB write.
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(N_EV)] for _ in range(args.cold_steps)]
        for i in range(args.cold_steps):
            flush.fill_(i & 255)
            step(cold_ev[i])
        torch.cuda.synchronize()
        step_ms = [span_ms(ev, "step") for ev in cold_ev]
        attn_cold = [span_ms(ev, "attn_fwd") for ev in cold_ev]
        cold = {"steps": args.cold_steps, "flush_mb": 512, "ms_per_step_median": float(np.median(step_ms)),
                "attn_ms_median": float(np.median(attn_cold))}
        del flush

    # Context: dense causal attention over the same tokens with the same
    # library (one host of N tokens), the one-GPU analogue of the pages'
    # speedups over FlashAttention.
    dense_ms = None
    if not args.dense and not args.no_dense_context:
        dplan = S.Plan(0, 1, wl.n_tokens, 0, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, 0, plan.dtype)
        db = S.alloc_buffers(dplan, dev)
        d_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        dts = []
        for i in range(6):
            d_ev[0].record(stream)
            S.spava_attn_fwd(dplan, q, k, v, db.kp, db.vp, db.o, db.lse, db.o_part, db.lse_part, stream)
            d_ev[1].record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                dts.append(d_ev[0].elapsed_time(d_ev[1]))
        dense_ms = float(np.median(dts))
        del db

    stage = {kk: [span_ms(ev, kk) for ev in events] for kk in ("score_topk", "gather", "attn_fwd", "lse_merge")}
    stage_ms = {kk: float(np.mean(vv)) for kk, vv in stage.items()}
    # Per-step GPU time from the events (the four calls back to back).
    step_ev = [sum(stage[kk][i] for kk in stage) for i in range(args.steps)]
    attn_ms = stage_ms["attn_fwd"]
    F_attn = attn_flops(wl)
    achieved = F_attn / (attn_ms * 1e-3) / 1e12
    tokens_per_s = wl.n_tokens / (ms_per_step * 1e-3)
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_VALU_TFLOPS

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.n_tokens, "q_heads": wl.n_q_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "anchor": wl.n_anchor,
                   "hosts": wl.n_hosts, "host_len": wl.host_len, "query": wl.n_query, "lp": wl.lp,
                   "selector": args.selector, "order": args.order},
        "roofline": {"bound": "mfma" if wl.dtype == "bf16" else "alu", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": measured_traffic(wl.name) if args.lp is None and not args.dense else None},
        "attn_tflop_per_launch": F_attn / 1e12,
        "step_tflops": (F_attn + score_flops(wl, args.selector)) / (ms_per_step * 1e-3) / 1e12,
        "score_tflops": score_flops(wl, args.selector) / (stage_ms["score_topk"] * 1e-3) / 1e12,
        "stage_ms": stage_ms,
        "step_event_ms": {"median": float(np.median(step_ev)), "min": float(np.min(step_ev))},
        # HBM-bound stages: algorithmic bytes / HIP-event time.  The scoring
        # call (MFMA- and exp-bound, listed for completeness) reads every
        # block's keys and the scoring rows' Q once and writes the scores and
        # the indices.
        "hbm_gbps": {
            "score_topk": (wl.n_hosts * wl.host_len * wl.n_kv_heads * wl.head_dim * 2
                           + (wl.n_query if args.selector == "query" else wl.n_hosts * wl.host_len)
                           * wl.n_q_heads * wl.head_dim * 2
                           + wl.n_hosts * wl.n_kv_heads * (wl.host_len + wl.lp) * 4)
                          / (stage_ms["score_topk"] * 1e-3) / 1e9,
            "gather": 4.0 * wl.n_hosts * wl.n_kv_heads * wl.lp * wl.head_dim * 2 / (stage_ms["gather"] * 1e-3) / 1e9,
            "lse_merge": ((wl.n_hosts + 1) * wl.n_query * wl.n_q_heads * (wl.head_dim + 1) * 4
                          + wl.n_query * wl.n_q_heads * (wl.head_dim * 2 + 4)) / (stage_ms["lse_merge"] * 1e-3) / 1e9,
        },
        "cold_cache": cold,
        "context": {
            "dense_causal_ms": dense_ms,
            "speedup_vs_dense_causal": (dense_ms / ms_per_step) if dense_ms else None,
            "pages_end_to_end": "12.72x vs FlashAttn, 1.70x vs ZigZagRing, 1.18x vs APB: whole long-video "
                                "LMM inference on 8 A800 GPUs, not comparable to this one-GPU layer",
        },
    }
    if not args.no_cpu_baseline and not args.dense:
        out["cpu_baseline"] = cpu_baseline(wl, x, args.selector)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
