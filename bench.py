#!/usr/bin/env python3
"""Throughput of the SemKV hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
rank the prompt's tokens (top-r), quantize + pack K and V of every layer and
KV head into the two precision pools, then run the workload's decode steps
(attention over the packed cache for all layers, fresh queries each step).
Inputs are generated on the device and resident in HBM before timing.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload llama8b_32k]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

METRIC = "KV quantize-pack GB/s + mixed-prec decode-attn tokens/s, % of HBM peak"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
ROOT = os.path.dirname(os.path.abspath(__file__))
DOMINANT = "decode_partials"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def cap16(x):
    return max(16, (int(x) + 15) // 16 * 16)


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_src):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    entry = t.get(DOMINANT)
    if not entry or entry.get("source_hash") != source_hash(kernel_src):
        return None
    return entry.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="decode steps per step (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--keynorm-score", action="store_true",
                    help="score the tokens in the step by key norm over the last 4 layers "
                         "(semkv_score_keynorm) instead of the workload's precomputed score; "
                         "a variant of the workload, not its headline")
    ap.add_argument("--event-every", type=int, default=8,
                    help="time every k-th decode partials launch with an event pair (the "
                         "roofline's average); the other launches carry no event packets")
    ap.add_argument("--rotate", action="store_true",
                    help="Hadamard-rotated cache (the optional quantizer rotation); a variant of "
                         "the workload, not its headline: no extra legs, no CPU baseline")
    ap.add_argument("--cpu-layers", type=int, default=16,
                    help="layers of the bounded oracle sample")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the generation, per-layer graph and copy legs")
    ap.add_argument("--no-cliff", action="store_true",
                    help="skip the cliff-grid sweep (20 level settings, batch 4 x 32,768)")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the mistral7b_128k (131,072-token) leg")
    ap.add_argument("--gen-steps", type=int, default=None,
                    help="generated tokens per sequence in the generation leg "
                         "(default: the gen_16x8k workload's)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a streaming copy of MIB MiB (read + write) three times, "
                         "the reference kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the hot path on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note, not a built path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        n_el = args.calibrate_copy * (1 << 20) // 4
        src = torch.arange(n_el, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)            # one 4-byte read + one 4-byte write per element
        torch.cuda.synchronize()
        assert int(dst[-1]) == -(n_el - 1)
        print(json.dumps({"copy_bytes_read": n_el * 4, "copy_bytes_written": n_el * 4,
                          "launches": 3}), flush=True)
        return

    import workloads as W
    from kv_cache_mixed_top_amd import semkv as sk

    w = W.WORKLOADS[args.workload]
    D = w.decode_steps if args.decode_steps is None else args.decode_steps
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)           # default priority
    B, n, layers, kv, Hq = w.batch, w.n, w.layers, w.kv_heads, w.q_heads
    k = sk.semkv_topr_count(n, w.r)

    t0 = time.time()
    with torch.cuda.stream(stream):
        K, V, _ = W.make_kv_torch(w, dev)
        if w.score == "attn_mass":
            scores = W.attention_mass_torch(K, w, dev)
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(3)
            scores = torch.rand((B, n), generator=g, device=dev)
        q = W.make_q_torch(w, D, dev)
        cache = sk.SemKVCache(B, layers, kv, Hq, w.L_high, w.L_low, cap16(k), cap16(n - k),
                              block=w.block, max_tokens=n, rotate=args.rotate)
        perm = torch.empty((B, n), dtype=torch.int32, device=dev)
        mask = torch.empty((B, (n + 31) // 32), dtype=torch.int32, device=dev)
        out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device=dev)
    stream.synchronize()
    log(f"inputs ready: {args.workload} K/V {2 * K.numel() * 2 / 1e9:.2f} GB in "
        f"{time.time() - t0:.1f}s; k={k} of n={n}, {D} decode steps per step")

    # algorithmic bytes (what the method must move; see the measurement section)
    Rh, Rl = sk.semkv_row_bytes(w.L_high), sk.semkv_row_bytes(w.L_low)
    planes = B * layers * kv * 2
    rank_bytes = B * n * (4 + 4) + B * ((n + 31) // 32) * 4
    quant_bytes = (planes * (k * (256 + Rh + 4) + (n - k) * (256 + Rl + 4))
                   + B * n * 4 + B * n * 4)                   # perm read, tok map write
    kv_packed = planes * (k * (Rh + 4) + (n - k) * (Rl + 4))
    q_bytes = B * layers * Hq * 128 * 2
    decode_bytes = kv_packed + q_bytes + B * layers * Hq * 128 * 4
    partial_bytes = kv_packed + q_bytes                       # per decode_partials launch
    kn_layer0 = max(0, layers - 4)
    score_bytes = (B * (layers - kn_layer0) * kv * n * 256 + B * n * 4) if args.keynorm_score else 0
    step_bytes = score_bytes + rank_bytes + quant_bytes + D * decode_bytes

    # HIP events on the work stream: quantize-pack and the decode loop of
    # every timed step, and every `every`-th decode_partials launch (their
    # mean is the roofline's launch time).  An event is a queue packet
    # between kernels that costs about 1.5 us of the step, so the other
    # launches carry none, the merge before each timed launch gets one
    # marker, and the decode time per step is the loop's.  (With no marker
    # between a merge and the next partials event, that event pair measured
    # the partials launch about 5 us longer than rocprofv3's kernel time.)
    Ev = lambda: torch.cuda.Event(enable_timing=True)
    ev_q = [(Ev(), Ev()) for _ in range(args.steps)]
    ev_l = [Ev() for _ in range(args.steps)]                 # decode loop end
    every = max(1, args.event_every)
    ev_p = [[(Ev(), Ev()) for _ in range(0, D, every)] for _ in range(args.steps)]
    ev_m = Ev()                                              # marker after a merge

    def step(i=None):
        cache.reset()
        if args.keynorm_score:
            sk.semkv_score_keynorm(K, scores, kn_layer0, layers - kn_layer0, stream=stream)
        sk.semkv_rank_topr(scores, k, perm, mask, stream=stream)
        if i is not None:
            ev_q[i][0].record(stream)
        sk.semkv_quantize_pack(cache, K, V, perm, k, stream=stream)
        if i is not None:
            ev_q[i][1].record(stream)
        for j in range(D):
            timed = i is not None and j % every == 0
            if timed:
                ev_p[i][j // every][0].record(stream)
            sk.semkv_decode_partials(cache, q[j], stream=stream)
            if timed:
                ev_p[i][j // every][1].record(stream)
            sk.semkv_decode_merge(cache, out, stream=stream)
            if i is not None and (j + 1) % every == 0:
                ev_m.record(stream)                          # before the next timed launch
        if i is not None:
            ev_l[i].record(stream)

    for _ in range(args.warmup):
        step()
    sk.semkv_sync_check(stream)
    log(f"warmup done ({args.warmup} steps)")

    start, end = Ev(), Ev()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    sk.semkv_sync_check(stream)
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    ms_quant = float(np.mean([a.elapsed_time(b) for a, b in ev_q]))
    ms_part = float(np.mean([a.elapsed_time(b) for row in ev_p for a, b in row])) if D else 0.0
    ms_dec = (float(np.mean([q1.elapsed_time(e) for (_, q1), e in zip(ev_q, ev_l)])) / D
              if D else 0.0)
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step; quantize {ms_quant:.3f} ms; "
        f"decode {ms_dec * 1e3:.1f} us/step (partials {ms_part * 1e3:.1f} us)")

    value = step_bytes / (ms_step * 1e-3) / 1e9
    quant_gbs = quant_bytes / (ms_quant * 1e-3) / 1e9
    dec_gbs = decode_bytes / (ms_dec * 1e-3) / 1e9 if D else 0.0
    part_gbs = partial_bytes / (ms_part * 1e-3) / 1e9 if D else 0.0
    kernel_src = ["kv_cache_mixed_top_amd/csrc/decode_mfma.hip",
                  "kv_cache_mixed_top_amd/csrc/decode_mfma_kernel.h",
                  "kv_cache_mixed_top_amd/csrc/semkv_internal.h",
                  "kv_cache_mixed_top_amd/csrc/semkv_common.h"]
    traffic = traffic_for(kernel_src)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "layers": layers, "kv_heads": kv,
                   "q_heads": Hq, "head_dim": 128, "tokens": n, "r": w.r,
                   "levels": [w.L_high, w.L_low], "decode_steps": D,
                   "v_dist": w.v_dist,
                   "score": "keynorm_last4" if args.keynorm_score else w.score,
                   "rotate": bool(args.rotate)},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "quantize_pack": {"ms": round(ms_quant, 4), "GB/s": round(quant_gbs, 1),
                          "pct_hbm_peak": round(100.0 * quant_gbs / HBM_PEAK_GBS, 2),
                          "algorithmic_bytes": quant_bytes},
        "decode_attn": {"us_per_step": round(ms_dec * 1e3, 2),
                        "tokens/s": round(B / (ms_dec * 1e-3), 1) if D else None,
                        "GB/s": round(dec_gbs, 1),
                        "pct_hbm_peak": round(100.0 * dec_gbs / HBM_PEAK_GBS, 2),
                        "algorithmic_bytes_per_step": decode_bytes},
        "roofline": {"kernel": DOMINANT, "bound": "hbm", "achieved": round(part_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(part_gbs / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(ms_part * 1e3, 2),
                     "launches_timed": args.steps * len(range(0, D, every)),
                     "algorithmic_bytes_per_launch": partial_bytes,
                     "traffic": traffic},
        "cpu_baseline": None,
    }

    if not args.no_extra and not args.rotate and not args.keynorm_score:
        result["decode_graph_per_layer"] = graph_leg(sk, torch, cache, q, D, layers, B, Hq,
                                                     decode_bytes, stream)
        log(f"per-layer graph: {result['decode_graph_per_layer']['us_per_step']} us/step")
        result["hbm_copy_context"] = copy_leg(torch, stream)
        log(f"copy context: {result['hbm_copy_context']['GB/s']} GB/s")
        result["score_keynorm"] = score_leg(sk, torch, K, stream)
        log(f"key-norm score: {result['score_keynorm']['us']} us, "
            f"{result['score_keynorm']['GB/s']} GB/s")
        del K, V
        torch.cuda.empty_cache()
        result["score_hidden_delta"] = delta_leg(sk, W, torch, w, dev, stream)
        log(f"delta-norm score: {result['score_hidden_delta']['us']} us, "
            f"{result['score_hidden_delta']['GB/s']} GB/s")
        torch.cuda.empty_cache()
        result["generation"] = gen_leg(sk, W, torch, dev, stream, args.gen_steps)
        g = result["generation"]
        log(f"generation: decode {g['decode_us_per_step']} us/step, "
            f"{g['decode_tokens/s']} tok/s; block quantize {g['block_quantize_us']} us")
        K = V = None
        torch.cuda.empty_cache()
        if not args.no_long:
            m = strip_private(workload_leg(sk, W, torch, dev, stream, "mistral7b_128k"))
            result["mistral7b_128k"] = m
            log(f"mistral7b_128k: quantize {m['quantize_ms']} ms ({m['quantize_pct_hbm_peak']}%), "
                f"decode partials {m['partials_us']} us ({m['partials_pct_hbm_peak']}%)")
            torch.cuda.empty_cache()
            torch.cuda.empty_cache()
        m = strip_private(workload_leg(sk, W, torch, dev, stream, "mix43_r075"))
        m.update(mix_accounting(sk, W.WORKLOADS["mix43_r075"]))
        result["mix43_r075"] = m
        log(f"mix43_r075: quantize {m['quantize_ms']} ms ({m['quantize_pct_hbm_peak']}%), "
            f"decode partials {m['partials_us']} us ({m['partials_pct_hbm_peak']}%)")
        torch.cuda.empty_cache()
        if not args.no_cliff:
            result["cliff_4x32k"] = cliff_leg(sk, W, torch, dev, stream)
            torch.cuda.empty_cache()

    if not args.no_cpu_baseline and not args.rotate and not args.keynorm_score:
        import cpu_baseline
        import oracle as O
        ls = max(1, min(args.cpu_layers, layers))
        if K is None:                      # freed by the extra legs: draw them again
            K, V, _ = W.make_kv_torch(w, dev)
        Ks = K[0, :ls].cpu().numpy()
        Vs = V[0, :ls].cpu().numpy()
        ps = perm[0].cpu().numpy()
        qs = q[0][0, :ls].cpu().numpy()
        sc = scores[0].cpu().numpy()
        t0 = time.perf_counter()
        O.rank_topr(sc, k)
        t_rank = time.perf_counter() - t0
        tq, td, workers = cpu_baseline.time_oracle(Ks, Vs, ps, k, w.L_high, w.L_low, qs,
                                                   w.sm_scale)
        cpu_step_s = B * (t_rank + (tq + D * td) * layers / ls)
        result["cpu_baseline"] = {
            "value": round(step_bytes / cpu_step_s / 1e9, 4),
            "unit": "GB/s", "cores": workers, "kind": "oracle",
            "cores_available": cpu_baseline.available_cores(),
            "cpu_model": cpu_baseline.cpu_model(),
            "sample": (f"oracle rank of 1 sequence, quantize+pack of {ls} of {layers} layers "
                       f"(sequence 0) and one decode step over those layers, in {workers} "
                       f"single-threaded worker processes ({cpu_baseline.available_cores()} cores "
                       f"available); measured rank {t_rank:.2f}s, quantize {tq:.2f}s, decode "
                       f"{td:.2f}s, scaled to {B} sequence(s) x {layers} layers x {D} decode "
                       f"steps = {cpu_step_s:.1f}s per step"),
        }
        log(f"cpu baseline: {cpu_step_s:.1f} s/step extrapolated ({workers} workers)")

    print(json.dumps(result), flush=True)


def graph_leg(sk, torch, cache, q, D, layers, B, Hq, decode_bytes, stream):
    """Decode as 32 per-layer launch pairs (partials + merge) captured once in
    a HIP graph and replayed per step; the output is checked against the
    one-launch form."""
    Ev = lambda: torch.cuda.Event(enable_timing=True)
    steps = min(D, 32)
    out_g = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device=q.device)
    out_e = torch.empty_like(out_g)
    qbuf = torch.empty_like(q[0])
    cap_stream = torch.cuda.Stream(device=q.device)   # default priority
    graph = torch.cuda.CUDAGraph()
    qbuf.copy_(q[0])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap_stream):
        for layer in range(layers):
            sk.semkv_decode_partials(cache, qbuf[:, layer:layer + 1], layer0=layer,
                                     stream=cap_stream)
            sk.semkv_decode_merge(cache, out_g[:, layer:layer + 1], stream=cap_stream)
    worst = 0.0
    for j in (0, steps - 1):                    # replays against the one-launch result
        with torch.cuda.stream(stream):
            qbuf.copy_(q[j])
        stream.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        sk.semkv_decode_attn(cache, q[j], out_e, stream=stream)
        stream.synchronize()
        rel = (out_g - out_e).abs() / out_e.abs().clamp(min=1.0)
        worst = max(worst, float(rel.max()))
    # per-layer launches split the rows into different chunks (each chunk has
    # its own fixed-point weight scale), so the two forms differ by their two
    # approximation errors, each within the 2e-3 parity bound of the exact
    # attention: at most twice that bound apart
    assert worst <= 4e-3, f"graph replay differs from the one-launch decode by {worst}"
    times = []
    for j in range(steps):
        with torch.cuda.stream(stream):
            qbuf.copy_(q[j])
        a, b = Ev(), Ev()
        torch.cuda.synchronize()
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    us = 1e3 * sum(times) / len(times)
    sk.semkv_sync_check(stream)
    return {"launches_per_step": 2 * layers, "steps": steps, "us_per_step": round(us, 2),
            "GB/s": round(decode_bytes / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100.0 * decode_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "max_rel_diff_vs_one_launch": worst}


def score_leg(sk, torch, K, stream, window=4, reps=10):
    """Key-norm scores of the workload's K over its last `window` layers
    (semkv_score_keynorm), mean of `reps` launches timed by HIP events on the
    launch stream.  Algorithmic bytes: the window's key rows read once plus
    the fp32 scores written."""
    import numpy as np
    Ev = lambda: torch.cuda.Event(enable_timing=True)
    B, layers, kv, n, D = K.shape
    layer0 = max(0, layers - window)
    nl = layers - layer0
    scores = torch.empty((B, n), dtype=torch.float32, device=K.device)
    sk.semkv_score_keynorm(K, scores, layer0, nl, stream=stream)
    stream.synchronize()
    ev = [(Ev(), Ev()) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        sk.semkv_score_keynorm(K, scores, layer0, nl, stream=stream)
        b.record(stream)
    stream.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    nbytes = B * nl * kv * n * D * 2 + B * n * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"layers": [layer0, layers], "algorithmic_bytes": nbytes, "us": round(ms * 1e3, 2),
            "GB/s": round(gbs, 1), "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2)}


def delta_leg(sk, W, torch, w, dev, stream, states=5, reps=10):
    """Hidden-state delta-norm scores (semkv_score_hidden_delta, the pages'
    default indicator over the last 4 layers) of synthetic hidden states at
    the workload's token count and the backbone's hidden size, mean of `reps`
    launches timed by HIP events; then the top-r rank of those scores.
    Algorithmic bytes: the states read once plus the fp32 scores written."""
    import numpy as np
    Ev = lambda: torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        H = W.make_hidden_states_torch(w, dev, states=states)
    stream.synchronize()
    B, S1, n, d = H.shape
    scores = torch.empty((B, n), dtype=torch.float32, device=dev)
    perm = torch.empty((B, n), dtype=torch.int32, device=dev)
    k = sk.semkv_topr_count(n, w.r)
    sk.semkv_score_hidden_delta(H, scores, stream=stream)
    stream.synchronize()
    ev = [(Ev(), Ev(), Ev()) for _ in range(reps)]
    for a, b, c in ev:
        a.record(stream)
        sk.semkv_score_hidden_delta(H, scores, stream=stream)
        b.record(stream)
        sk.semkv_rank_topr(scores, k, perm, stream=stream)
        c.record(stream)
    stream.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    rank_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
    nbytes = B * S1 * n * d * 2 + B * n * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    del H
    return {"states": S1, "hidden_size": d, "tokens": n, "batch": B, "algorithmic_bytes": nbytes,
            "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
            "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2), "rank_us": round(rank_ms * 1e3, 2),
            "inputs": "synthetic: h_0 ~ N(0,1), per-layer updates N(0,1) x U(0.05, 0.5) per token"}


def copy_leg(torch, stream, mib=2048):
    """Device-to-device copy of `mib` MiB (read + write), as the achievable
    HBM rate on this machine for context; not a roofline peak."""
    Ev = lambda: torch.cuda.Event(enable_timing=True)
    n = mib * (1 << 20) // 4
    with torch.cuda.stream(stream):
        src = torch.ones(n, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
    stream.synchronize()
    best = float("inf")
    for _ in range(5):
        a, b = Ev(), Ev()
        a.record(stream)
        with torch.cuda.stream(stream):
            dst.copy_(src)
        b.record(stream)
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    gbs = 2 * n * 4 / (best * 1e-3) / 1e9
    del src, dst
    return {"kind": "torch device copy, best of 5", "bytes_moved": 2 * n * 4,
            "ms": round(best, 4), "GB/s": round(gbs, 1),
            "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2)}


def workload_leg(sk, W, torch, dev, stream, name, levels=None, r=None, inputs=None,
                 quant_reps=5, every=8, rotate=False):
    """One prompt workload outside the headline step: rank + quantize-pack
    (median of `quant_reps` timed repetitions on the same cache), then the
    workload's decode steps (partials + merge over all layers, fresh queries
    each step), timed like the headline: every `every`-th partials launch and
    the whole loop.  `levels`/`r` override the workload's; `inputs` reuses
    (K, V, scores) already on the device; `rotate` builds a Hadamard-rotated
    cache."""
    import numpy as np
    w = W.WORKLOADS[name]
    Lh, Ll = levels if levels is not None else (w.L_high, w.L_low)
    r = w.r if r is None else r
    B, n, layers, kv, Hq, D = w.batch, w.n, w.layers, w.kv_heads, w.q_heads, w.decode_steps
    Ev = lambda: torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        if inputs is None:
            K, V, _ = W.make_kv_torch(w, dev)
            scores = W.attention_mass_torch(K, w, dev)
        else:
            K, V, scores = inputs
        q = W.make_q_torch(w, D, dev)
        k = sk.semkv_topr_count(n, r)
        cache = sk.SemKVCache(B, layers, kv, Hq, Lh, Ll, cap16(k), cap16(n - k), block=w.block,
                              max_tokens=n, rotate=rotate)
        perm = torch.empty((B, n), dtype=torch.int32, device=dev)
        out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device=dev)
    stream.synchronize()
    Rh, Rl = sk.semkv_row_bytes(Lh), sk.semkv_row_bytes(Ll)
    planes = B * layers * kv * 2
    quant_bytes = planes * (k * (256 + Rh + 4) + (n - k) * (Rl + 4 + 256)) + B * n * 8
    kv_packed = planes * (k * (Rh + 4) + (n - k) * (Rl + 4))
    partial_bytes = kv_packed + B * layers * Hq * 128 * 2
    decode_bytes = partial_bytes + B * layers * Hq * 128 * 4
    sk.semkv_rank_topr(scores, k, perm, stream=stream)
    qt = []
    for rep in range(quant_reps + 1):
        cache.reset()
        a, b = Ev(), Ev()
        a.record(stream)
        sk.semkv_quantize_pack(cache, K, V, perm, k, stream=stream)
        b.record(stream)
        qt.append((a, b))
    ev_p = [(Ev(), Ev()) for _ in range(0, D, every)]
    m_ev = Ev()
    start, end = Ev(), Ev()
    for j in range(min(D, 8)):                       # warm-up launches
        sk.semkv_decode_partials(cache, q[j], stream=stream)
    start.record(stream)
    for j in range(D):
        if j % every == 0:
            ev_p[j // every][0].record(stream)
        sk.semkv_decode_partials(cache, q[j], stream=stream)
        if j % every == 0:
            ev_p[j // every][1].record(stream)
        sk.semkv_decode_merge(cache, out, stream=stream)
        if (j + 1) % every == 0:
            m_ev.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    sk.semkv_sync_check(stream)
    ms_q = float(np.median([a.elapsed_time(b) for a, b in qt[1:]]))
    us_p = 1e3 * float(np.mean([a.elapsed_time(b) for a, b in ev_p]))
    us_step = 1e3 * start.elapsed_time(end) / D
    qg = quant_bytes / (ms_q * 1e-3) / 1e9
    pg = partial_bytes / (us_p * 1e-6) / 1e9
    dg = decode_bytes / (us_step * 1e-6) / 1e9
    res = {"workload": name, "batch": B, "tokens": n, "layers": layers, "r": r, "levels": [Lh, Ll],
           "v_dist": w.v_dist, "decode_steps": D,
           "quantize_ms": round(ms_q, 4), "quantize_GB/s": round(qg, 1),
           "quantize_pct_hbm_peak": round(100 * qg / HBM_PEAK_GBS, 2),
           "quantize_algorithmic_bytes": quant_bytes,
           "partials_us": round(us_p, 2), "partials_GB/s": round(pg, 1),
           "partials_pct_hbm_peak": round(100 * pg / HBM_PEAK_GBS, 2),
           "partials_algorithmic_bytes": partial_bytes,
           "decode_us_per_step": round(us_step, 2), "decode_tokens/s": round(B / (us_step * 1e-6), 1),
           "decode_GB/s": round(dg, 1), "decode_pct_hbm_peak": round(100 * dg / HBM_PEAK_GBS, 2)}
    res["_cache"] = cache
    res["_q"] = q
    res["_out"] = out
    res["_perm"] = perm
    return res


def mix_accounting(sk, w):
    """Storage accounting of a two-level mix: the nominal bits (log2 of the
    level counts), this format's stored bits (packed rows + 4 meta bytes per
    128 values), and the pages' accounting (SemKV Table 6: code bits of
    packing g codes in ceil(g log2 L) bits at the best g <= 5, plus the
    metadata per value: two fp16 scalars per row for the affine base, one
    for TurboQuant-MSE), each with its compression against fp16."""
    import math
    n, Lh, Ll = w.n, w.L_high, w.L_low
    k = sk.semkv_topr_count(n, w.r)
    nominal = (k * math.log2(Lh) + (n - k) * math.log2(Ll)) / n
    stored = (k * (sk.semkv_row_bytes(Lh) + 4) + (n - k) * (sk.semkv_row_bytes(Ll) + 4)) * 8 / (128 * n)
    page_code = lambda L: min(math.ceil(g * math.log2(L) - 1e-12) / g for g in range(1, 6))
    code = (k * page_code(Lh) + (n - k) * page_code(Ll)) / n
    return {"nominal_bits": round(nominal, 4), "stored_bits": round(stored, 4),
            "compression_vs_fp16": round(16 / stored, 3),
            "page_code_bits": round(code, 4),
            "page_eff_bits_affine": round(code + 0.25, 4),
            "page_compression_affine": round(16 / (code + 0.25), 3),
            "page_eff_bits_turboquant": round(code + 0.125, 4),
            "page_compression_turboquant": round(16 / (code + 0.125), 3)}


def cliff_leg(sk, W, torch, dev, stream):
    """Cliff-grid sweep (batch 4 x 32,768 tokens, 8B shape): uniform levels
    L in {4, 5, 6, 8, 16} (one pool) and the adjacent pairs (5,4), (6,5),
    (8,6) at r in {.1, .25, .5, .75, .9}.  Each setting: quantize-pack and 64
    decode steps (rates as in the headline), and the quality proxies:
    nominal and stored bits per value, reconstruction MSE of K and of V over
    layers 0 and 31 (rows reconstructed by semkv_dequantize_rows), and the
    largest |out - ref| / max(1, |ref|) of the last decode step against fp32
    attention over the fp16 cache (sequence 0, layers 0 and 31).  Three more
    settings repeat (4,4), (5,4) at r = .5 and (6,5) at r = .5 on a
    Hadamard-rotated cache (SemKV Table 2's quantizer with rotation), whose
    proxies show what the rotation does to the outlier channels of K."""
    import math
    w = W.WORKLOADS["cliff_4x32k"]
    B, n, layers, kv, Hq = w.batch, w.n, w.layers, w.kv_heads, w.q_heads
    with torch.cuda.stream(stream):
        K, V, _ = W.make_kv_torch(w, dev)
        scores = W.attention_mass_torch(K, w, dev)
    stream.synchronize()
    settings = [(L, L, 0.0, False) for L in W.CLIFF_UNIFORM]
    settings += [(Lh, Ll, r, False) for Lh, Ll in W.CLIFF_PAIRS for r in W.CLIFF_RS]
    settings += [(4, 4, 0.0, True), (5, 4, 0.5, True), (6, 5, 0.5, True)]
    sample_layers = (0, layers - 1)
    rows = []
    for Lh, Ll, r, rot in settings:
        leg = workload_leg(sk, W, torch, dev, stream, "cliff_4x32k", levels=(Lh, Ll), r=r,
                           inputs=(K, V, scores), quant_reps=3, rotate=rot)
        cache, q, out = leg["_cache"], leg["_q"], leg["_out"]
        k = sk.semkv_topr_count(n, r)
        Rh, Rl = sk.semkv_row_bytes(Lh), sk.semkv_row_bytes(Ll)
        nominal = (k * math.log2(Lh) + (n - k) * math.log2(Ll)) / n
        stored = (k * (Rh + 4) + (n - k) * (Rl + 4)) * 8.0 / (128 * n)
        se = {0: 0.0, 1: 0.0}
        cnt = 0
        with torch.cuda.stream(stream):
            for layer in sample_layers:
                for high, nrows in ((True, cache.n_high), (False, cache.n_low)):
                    if nrows == 0:
                        continue
                    xh = torch.empty((B, kv, 2, nrows, 128), dtype=torch.float32, device=dev)
                    sk.semkv_dequantize_rows(cache, high, layer, 0, nrows, xh, stream=stream)
                    tok = cache.tok_view(high)[:, :nrows].long()              # [B][nrows]
                    idx = tok[:, None, :, None].expand(B, kv, nrows, 128)
                    for sel, X in ((0, K), (1, V)):
                        x = torch.gather(X[:, layer].float(), 2, idx)
                        se[sel] += float(((xh[:, :, sel] - x) ** 2).sum())
                    cnt += B * kv * nrows * 128
            # fp32 attention over the fp16 cache for the last decode step
            worst = 0.0
            qd = q[w.decode_steps - 1]
            for layer in sample_layers:
                kk = K[0, layer].float()                                       # [kv][n][128]
                vv = V[0, layer].float()
                qq = qd[0, layer].float().view(kv, Hq // kv, 128)
                z = torch.bmm(qq, kk.transpose(1, 2).contiguous()) * w.sm_scale
                ref = torch.bmm(torch.softmax(z, dim=-1), vv).reshape(Hq, 128)
                err = (out[0, layer] - ref).abs() / ref.abs().clamp(min=1.0)
                worst = max(worst, float(err.max()))
        stream.synchronize()
        row = strip_private(leg)
        row.update({"rotate": rot,
                    "nominal_bits": round(nominal, 4), "stored_bits": round(stored, 4),
                    "compression_vs_fp16": round(16.0 / stored, 3),
                    "mse_K": se[0] / cnt, "mse_V": se[1] / cnt,
                    "attn_err_vs_fp16_cache": worst})
        for key in ("workload", "batch", "tokens", "layers", "v_dist", "decode_steps",
                    "quantize_algorithmic_bytes", "partials_algorithmic_bytes"):
            row.pop(key, None)
        rows.append(row)
        log(f"cliff ({Lh},{Ll}) r={r}{' rotated' if rot else ''}: quantize {row['quantize_pct_hbm_peak']}%, partials "
            f"{row['partials_pct_hbm_peak']}%, {row['stored_bits']} bits, attn err "
            f"{worst:.2e}")
        del cache, q, out, leg
        torch.cuda.empty_cache()
    return {"workload": "cliff_4x32k", "batch": B, "tokens": n, "layers": layers,
            "decode_steps": w.decode_steps, "quality_sample": "sequence 0 (attention), "
            "all sequences (MSE), layers 0 and 31", "settings": rows}


def strip_private(d):
    return {k: v for k, v in d.items() if not k.startswith("_")}


def gen_leg(sk, W, torch, dev, stream, gen_steps=None):
    """Generation workload (16 x 8,192-token prompts, r = 0.25): quantize the
    prompts, then per step append one token per sequence (a block of 128 is
    ranked, quantized and packed when the tail fills) and decode all layers
    over the pools plus the fp16 tail."""
    import numpy as np
    w = W.WORKLOADS["gen_16x8k"]
    T = w.gen_tokens if gen_steps is None else gen_steps
    B, n = w.batch, w.n
    k = sk.semkv_topr_count(n, w.r)
    kb = sk.semkv_topr_count(w.block, w.r)
    Ev = lambda: torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        K, V, chans = W.make_kv_torch(w, dev)
        scores = W.attention_mass_torch(K, w, dev)
        Kg, Vg, Sg = W.make_gen_tokens_torch(w, T, dev, chans=chans)
        Qg = W.make_q_torch(w, T, dev)
        cache = sk.SemKVCache(B, w.layers, w.kv_heads, w.q_heads, w.L_high, w.L_low,
                              cap16(k + (T // w.block + 1) * kb),
                              cap16(n - k + (T // w.block + 1) * (w.block - kb)),
                              block=w.block, max_tokens=n + T)
        perm = torch.empty((B, n), dtype=torch.int32, device=dev)
        out = torch.empty((B, w.layers, w.q_heads, 128), dtype=torch.float32, device=dev)
    stream.synchronize()
    Rh, Rl = sk.semkv_row_bytes(w.L_high), sk.semkv_row_bytes(w.L_low)
    planes = B * w.layers * w.kv_heads * 2
    # the prompt's rank + quantize-pack: the median of 3 passes over the same
    # cache after an untimed first one, as the other legs time their
    # quantize (each pass writes the same pools again)
    qev = []
    for rep in range(4):
        cache.reset()
        qa, qb = Ev(), Ev()
        qa.record(stream)
        sk.semkv_rank_topr(scores, k, perm, stream=stream)
        sk.semkv_quantize_pack(cache, K, V, perm, k, stream=stream)
        qb.record(stream)
        qev.append((qa, qb))
    del K, V
    ev_app = [(Ev(), Ev()) for _ in range(T)]
    ev_dec = [(Ev(), Ev()) for _ in range(T)]
    pool_rows = []
    start, end = Ev(), Ev()
    start.record(stream)
    for i in range(T):
        ev_app[i][0].record(stream)
        sk.semkv_append_block(cache, Kg[i].unsqueeze(3), Vg[i].unsqueeze(3), Sg[i].unsqueeze(1),
                              w.r, stream=stream)
        ev_app[i][1].record(stream)
        pool_rows.append((cache.n_high, cache.n_low, cache.n_tail))
        ev_dec[i][0].record(stream)
        sk.semkv_decode_attn(cache, Qg[i], out, sm_scale=w.sm_scale, stream=stream)
        ev_dec[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    sk.semkv_sync_check(stream)
    t_app = [a.elapsed_time(b) for a, b in ev_app]
    t_dec = [a.elapsed_time(b) for a, b in ev_dec]
    blocks = [i for i in range(T) if pool_rows[i][2] == 0]
    plain = [t_app[i] for i in range(T) if pool_rows[i][2] != 0]
    dec_bytes = []
    for nh, nl_, nt in pool_rows:
        dec_bytes.append(B * w.layers * w.kv_heads * 2 * (nh * (Rh + 4) + nl_ * (Rl + 4)
                                                            + nt * 256)
                         + B * w.layers * w.q_heads * 128 * (2 + 4))
    ms_dec = sum(t_dec) / T
    dec_gbs = sum(dec_bytes) / (sum(t_dec) * 1e-3) / 1e9
    blk_bytes = planes * (kb * (256 + Rh + 4) + (w.block - kb) * (256 + Rl + 4))
    ms_blk = sum(t_app[i] for i in blocks) / max(1, len(blocks))
    prompt_ms = float(np.median([x.elapsed_time(y) for x, y in qev[1:]]))
    prompt_bytes = planes * (k * (256 + Rh + 4) + (n - k) * (256 + Rl + 4))
    res = {"workload": "gen_16x8k", "batch": B, "prompt_tokens": n, "r": w.r,
           "generated_tokens": T,
           "prompt_rank_quantize_ms": round(prompt_ms, 3),
           "prompt_quantize_GB/s": round(prompt_bytes / (prompt_ms * 1e-3) / 1e9, 1),
           "append_us_per_step": round(1e3 * sum(plain) / max(1, len(plain)), 2),
           "blocks": len(blocks),
           "block_quantize_us": round(1e3 * ms_blk, 2),
           "block_GB/s": round(blk_bytes / (ms_blk * 1e-3) / 1e9, 1) if blocks else None,
           "decode_us_per_step": round(1e3 * ms_dec, 2),
           "decode_tokens/s": round(B / (ms_dec * 1e-3), 1),
           "decode_GB/s": round(dec_gbs, 1),
           "decode_pct_hbm_peak": round(100.0 * dec_gbs / HBM_PEAK_GBS, 2),
           "ms_total": round(start.elapsed_time(end), 2)}
    del cache, Kg, Vg, Qg
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
