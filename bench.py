"""Benchmark of the block-sparse decode hot path on one MI355X.

A step is one decode step of the Forecast-scored 128K workload (batch 8, 32
query heads, 8 KV heads, head_dim 128, bf16, top-k 64 + 1 initial + 2 local
blocks): append the compressed-key window completed by the newest token, score
and select blocks with the per-group Forecast vectors, and attend with the real
queries over the selected blocks (split-K, merged with log-sum-exp weights).
Inputs are seeded synthetic tensors resident in HBM before timing; R replicas
at distinct addresses are rotated so the 256 MB last-level cache cannot serve
one step's bytes from the previous step.

Prints one JSON line: throughput (tokens/s = batch / step time), the achieved
HBM bandwidth of the dominant kernel (decode attention) on its algorithmic
bytes against the 8 TB/s peak, and the CPU oracle timed on the same inputs.
Other workloads: --workload decode_gqa_bf16_32k | decode_tiny_f32_8k |
crosslayer_bf16_64k | lookahead_forecast_bf16_128k | tokenindex_forecast_bf16_128k |
decode_cobs_gqa_bf16_128k | prefill_chunk_bf16_128k.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, vendor figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_forecast_bf16_128k")
    ap.add_argument("--replicas", type=int, default=None,
                    help="input replicas rotated per step (default: 8 for the single-layer decode "
                         "workloads, whose per-step bytes are about the size of the 256 MB last-level "
                         "cache; 3 for the token-index workload; prefill takes at most 2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--n-split", type=int, default=0)
    ap.add_argument("--separate-calls", action="store_true",
                    help="time a decode step as three library calls (compress, select, decode) "
                         "instead of one sparse_attn_decode_step call")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step as a captured HIP graph (slower on this stack: a graph "
                         "launch costs more than the launch gaps it removes)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py runs on one GPU (the kernels work on a single device); run with --gpus 1"}))
        sys.exit(2)
    import torch
    import synth
    from block_sparse_attention_12_amd.pipeline import SparseDecoder

    if args.workload == "copy_calibration":
        return copy_calibration(args)
    if args.replicas is None:
        args.replicas = 3 if args.workload in synth.TOKEN_WORKLOADS else (2 if args.workload.startswith("prefill") else 8)
    if args.workload.startswith("prefill"):
        return bench_prefill(args)
    if args.workload in synth.TOKEN_WORKLOADS:
        return bench_token(args, synth.TOKEN_WORKLOADS[args.workload])
    w = synth.WORKLOADS[args.workload]
    if w.cobs:
        return bench_cobs(args, w)
    if w.lookahead:
        return bench_lookahead(args, w)
    if w.layers > 1:
        return bench_crosslayer(args, w)
    return bench_decode(args, w)


def recorded_traffic(name):
    """HBM bytes per launch recorded from profiler counters in profiles/<name>_traffic.md,
    or None when the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for src in fields["sources"].split(","):
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() != fields["source_sha256"]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def copy_calibration(args):
    """A plain device copy of known size (1 GiB read + 1 GiB written per launch),
    used to scale the HBM byte counters (FETCH_SIZE / WRITE_SIZE) of a profiler
    run: bytes per counter unit = 2^30 / counter value of this copy."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(max(1, args.steps)):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": a.numel() * 4,
                                           "bytes_written_per_launch": b.numel() * 4,
                                           "launches": max(1, args.steps)}}), flush=True)


def measured_stream_read_gbs(dev, gib=4, reps=5, launches=5):
    """HBM stream-read ceiling measured with the library's stream-read kernel
    (a whole-GPU grid reading a 4 GiB buffer once per launch, 5 launches back to
    back per timing): median GB/s."""
    import statistics
    import torch
    from block_sparse_attention_12_amd import stream_read
    buf = torch.ones((gib << 30) // 4, dtype=torch.int32, device=dev)
    out = stream_read(buf)
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        e0, e1 = _events(2)
        e0.record(stream)
        for _ in range(launches):
            stream_read(buf, out)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / launches)
    del buf
    return round((gib << 30) / 1e9 / (statistics.median(times) * 1e-3), 1)


def measured_matmul_tflops(dev, n=8192, reps=10):
    """bf16 dense GEMM ceiling measured with torch.matmul (the vendor library) on
    n x n x n: median TFLOP/s."""
    import statistics
    import torch
    a = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    c = torch.matmul(a, b)
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        e0, e1 = _events(2)
        e0.record(stream)
        torch.matmul(a, b, out=c)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return round(2.0 * n ** 3 / (statistics.median(times) * 1e-3) / 1e12, 1)


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def bench_decode(args, w):
    import torch
    import synth
    from block_sparse_attention_12_amd.pipeline import SparseDecoder
    from block_sparse_attention_12_amd import n_compressed, n_blocks

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_decode_inputs(w, device=dev)
    T = w.T
    lens_now = inp["seq_lens"]
    lens_prev = lens_now - 1
    dec = SparseDecoder(w.B, w.Hq, w.Hkv, T, w.top_k, w.n_init, w.n_local, w.selector,
                        w.score_mode, device=dev, n_split=args.n_split)
    sel_name = "F" if w.selector == "forecast" else "Q"
    reps = []
    for r in range(args.replicas):
        rep = {k: (inp[k] if r == 0 else inp[k].clone()) for k in ("Q", "K", "V", sel_name)}
        rep["Kc"] = dec.new_kc(inp["K"].dtype)
        dec.build(rep["K"], rep["Kc"], lens_prev)        # windows up to the previous token
        reps.append(rep)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def phases_of(rep):
        return {
            "append": lambda: dec.append(rep["K"], rep["Kc"], lens_prev, lens_now),
            "select": lambda: dec.select(rep[sel_name], rep["Kc"], lens_now),
            "attend": lambda: dec.attend(rep["Q"], rep["K"], rep["V"], lens_now),
        }

    def whole_step(rep):
        if args.separate_calls:
            for f in phases_of(rep).values():
                f()
        else:                                   # sparse_attn_decode_step: one call
            dec.fused_step(rep["Q"], rep[sel_name], rep["K"], rep["V"], rep["Kc"], lens_prev,
                           lens_now)

    if not args.graph:
        steps_fn = [lambda rep=rep: whole_step(rep) for rep in reps]
    else:
        graphs = [dec.capture(lambda rep=rep: whole_step(rep)) for rep in reps]
        steps_fn = [g.replay for g in graphs]
    for i in range(args.warmup):
        steps_fn[i % len(reps)]()
    torch.cuda.synchronize()
    ev0, ev1 = _events(2)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        steps_fn[i % len(reps)]()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    gpu_ms = ev0.elapsed_time(ev1) / args.steps

    # GPU time of each whole step call (events around every call)
    n_ph = max(10, min(args.steps, 100))
    evs = [_events(2) for _ in range(n_ph)]
    for i in range(n_ph):
        evs[i][0].record(stream)
        steps_fn[i % len(reps)]()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    step_call_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / n_ph

    # per-phase GPU time: each phase captured on its own, replays bracketed by events
    mean = {}
    for name in ("append", "select", "attend"):
        fns = [phases_of(rep)[name] for rep in reps]
        if args.graph:
            fns = [dec.capture(f).replay for f in fns]
        for i in range(3):
            fns[i % len(fns)]()
        evs = [_events(2) for _ in range(n_ph)]
        for i in range(n_ph):
            evs[i][0].record(stream)
            fns[i % len(fns)]()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        mean[name] = sum(e[0].elapsed_time(e[1]) for e in evs) / n_ph

    # algorithmic bytes, from the actual selections and lengths
    cnt = dec.cnt.cpu()
    idx = dec.idx.cpu()
    elem = inp["K"].element_size()
    lens = [int(x) for x in lens_now.cpu()]
    row = 128 * elem
    attn_bytes = 0
    for b in range(w.B):
        L = lens[b]
        for h in range(w.Hkv):
            for blk in idx[b, h, :int(cnt[b, h])].tolist():
                attn_bytes += 2 * row * max(0, min(64, L - 64 * blk))
    attn_bytes += w.B * w.Hq * 128 * elem + w.B * w.Hq * (128 * 4 + 4)   # Q in, O + LSE out
    sel_bytes = 0
    for b in range(w.B):
        L = lens[b]
        nb = n_blocks(L)
        n_cand = max(0, nb - w.n_local - min(w.n_init, nb))
        if w.score_mode == "raw_sum":
            sel_bytes += w.Hkv * 3 * n_cand * row
        else:
            sel_bytes += w.Hkv * n_compressed(L) * row
    sel_in = inp[sel_name]
    sel_bytes += sel_in.numel() * elem
    new_entries = sum(n_compressed(L) - n_compressed(L - 1) for L in lens) * w.Hkv
    append_bytes = new_entries * (32 * row + row)
    step_bytes = attn_bytes + sel_bytes + append_bytes
    attn_gbs = attn_bytes / (mean["attend"] * 1e-3) / 1e9
    step_gbs = step_bytes / (gpu_ms * 1e-3) / 1e9            # timed region, HIP events
    call_gbs = step_bytes / (step_call_ms * 1e-3) / 1e9

    out = {
        "metric": "sparse decode attn tokens/s and HBM GB/s (% of peak) at 128K ctx, 1 GPU",
        "value": round(w.B / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1), planted blocks)",
        "config": {"workload": w.name, "batch": w.B, "context": w.T, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.d, "top_k": w.top_k, "n_init": w.n_init,
                   "n_local": w.n_local, "selector": w.selector, "score_mode": w.score_mode,
                   "replicas": args.replicas, "n_split": args.n_split or "auto",
                   "launch": ("hip graph per step" if args.graph else "eager, one stream") + (
                       ", compress + select + decode calls" if args.separate_calls
                       else ", one sparse_attn_decode_step call"),
                   "parallelism": "none (1 GPU)"},
        "gpu_ms_per_step": round(gpu_ms, 5),
        "phase_ms": {k: round(v, 5) for k, v in mean.items()},
        "step_bytes": step_bytes,
        "step_hbm_gbs": round(step_bytes / (gpu_ms * 1e-3) / 1e9, 1),
        "step_call_ms": round(step_call_ms, 5),
    }
    separate = {"kernel": "sparse_attn_decode called alone (decode_kernel with the split merge)",
                "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(f"{w.name}_decode"), "bytes_per_launch": attn_bytes}
    if not args.separate_calls:
        # the timed step is one sparse_attn_decode_step call: its launches (the
        # scorer, then the attention with the top-k prologue and the in-kernel
        # split merge) timed together, as the average step time between HIP
        # events on the launch stream at both ends of the timed region, on the
        # step's algorithmic bytes; call_ms adds events around every call
        # (each pair costs ~2 us of its own)
        if w.score_mode == "softmax_sum":
            launches = ("score_softmax_kernel with the append; decode_kernel with the top-k and "
                        "the split merge")
        elif w.dtype == "bf16":
            launches = ("score_raw_kernel; decode_kernel with the top-k, the append and the split "
                        "merge")
        else:
            launches = "score_raw_kernel with the append; decode_kernel with the top-k and the split merge"
        out["roofline"] = {"bound": "hbm",
                           "kernel": f"sparse_attn_decode_step call ({launches})",
                           "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                           "traffic": recorded_traffic(f"{w.name}_step"),
                           "bytes_per_launch": step_bytes, "launch_ms": round(gpu_ms, 5),
                           "call_ms": round(step_call_ms, 5), "call_achieved": round(call_gbs, 1),
                           "separate_call_attention": separate}
    else:
        out["roofline"] = dict(bound="hbm", **separate)
        out["roofline"]["step_calls_ms"] = round(step_call_ms, 5)
    out["selection_quality"] = selection_quality(w, reps[0], dec, sel_name, lens_now)
    ceil = measured_stream_read_gbs(dev)
    out["roofline"]["measured_ceiling"] = {"what": "stream read (sparse_attn_stream_read, 4 GiB)",
                                           "GB/s": ceil,
                                           "frac": round(out["roofline"]["achieved"] / ceil, 4),
                                           "step_frac": round(out["step_hbm_gbs"] / ceil, 4)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w, inp, lens, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def selection_quality(w, rep, dec, sel_name, lens):
    """Recall of the dense attention mass by the selected blocks (exact block
    masses from sparse_attn_block_mass on the first replica, the selection made
    by that replica's step), next to the best recall any set of the same shape
    (init + local + k candidates) could reach: the k candidates of largest mass,
    taken on the host from the kernel's masses."""
    import numpy as np
    import torch
    from block_sparse_attention_12_amd import block_mass

    dec.select(rep[sel_name], rep["Kc"], lens)
    ev0, ev1 = _events(2)
    stream = torch.cuda.current_stream()
    ev0.record(stream)
    mass, rec = block_mass(rep["Q"], rep["K"], lens, 1.0, idx=dec.idx, cnt=dec.cnt)
    ev1.record(stream)
    torch.cuda.synchronize()
    M, R = mass.cpu().numpy().astype(np.float64), rec.cpu().numpy()
    best = []
    for b in range(w.B):
        nb = -(-int(lens[b]) // 64)
        cand = np.arange(w.n_init, nb - w.n_local)
        for hq in range(w.Hq):
            m = M[b, hq, :nb]
            top = np.sort(m[cand])[::-1][:w.top_k].sum() if len(cand) else 0.0
            best.append(m[:w.n_init].sum() + m[nb - w.n_local:].sum() + top)
    best = np.array(best)
    return {"recall_mean": round(float(R.mean()), 4), "recall_min": round(float(R.min()), 4),
            "mass_optimal_recall_mean": round(float(best.mean()), 4),
            "uniform_share": round((w.top_k + w.n_init + w.n_local) / (-(-w.T // 64)), 4),
            "block_mass_ms": round(ev0.elapsed_time(ev1), 4),
            "note": "dense attention mass of each query head captured by its KV head's selected "
                    "blocks (mean / min over heads); synthetic queries are independent of the "
                    "selector except along planted directions"}


def bench_lookahead(args, w):
    """A decode step through w.layers layers of the 128K Forecast workload, each
    layer appending, selecting with its own Forecast and attending. Measured
    in order on one stream and with layer l+1's selection on a second stream
    while layer l attends; both as eager launches and as one captured graph per
    step, and with one sparse_attn_decode_step call per layer (eager and as a
    graph). value = sequences / step time of the fastest of these schedules."""
    import torch
    import synth
    from block_sparse_attention_12_amd.pipeline import LookaheadDecoder
    from block_sparse_attention_12_amd import n_blocks

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    la = LookaheadDecoder(w.B, w.Hq, w.Hkv, w.T, w.top_k, w.n_init, w.n_local, device=dev,
                          n_split=args.n_split)
    layers = []
    for l in range(w.layers):
        inp = synth.make_decode_inputs(w, device=dev, layer=l)
        lens = inp["seq_lens"]
        Kc = la.new_kc(inp["K"].dtype)
        la.build(inp["K"], Kc, lens - 1)
        layers.append(dict(Q=inp["Q"], F=inp["F"], K=inp["K"], V=inp["V"], Kc=Kc))
        del inp
    lens_now = lens
    lens_prev = lens_now - 1
    outs = [(torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device=dev),
             torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)) for _ in range(w.layers)]
    stream = torch.cuda.current_stream()

    def run(fn, steps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = _events(2)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps

    def seq():
        la.step(layers, lens_prev, lens_now, outs, lookahead=False)

    def ahead():
        la.step(layers, lens_prev, lens_now, outs, lookahead=True)

    def one_call():
        la.step_one_call(layers, lens_prev, lens_now, outs)

    # the two-stream schedule last among the eager ones: measured after it,
    # the one-call schedule's eager launches ran 1.5x slower than before it
    res = {"eager_in_order": run(seq, args.steps), "eager_one_call": run(one_call, args.steps),
           "eager_lookahead": run(ahead, args.steps)}
    g_seq = la.dec[0].capture(seq)
    g_ahead = la.dec[0].capture(ahead)
    g_one = la.dec[0].capture(one_call)
    res["graph_in_order"] = run(g_seq.replay, args.steps)
    res["graph_lookahead"] = run(g_ahead.replay, args.steps)
    res["graph_one_call"] = run(g_one.replay, args.steps)
    best = min(res, key=lambda k: res[k][0])            # fastest schedule by wall time
    ms_step, gpu_ms = res[best]
    row = 128 * 2
    L = w.T
    seq()                                       # leaves the last layer's set in dec[(layers-1) % 2]
    torch.cuda.synchronize()
    idx = la.dec[(w.layers - 1) % 2].idx.cpu().numpy()
    cnt = la.dec[(w.layers - 1) % 2].cnt.cpu().numpy()
    per_layer_kv = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            for blk in idx[b, h, :int(cnt[b, h])].tolist():
                per_layer_kv += 2 * row * max(0, min(64, L - 64 * blk))
    nb = n_blocks(L)
    scan = w.B * w.Hkv * (nb - w.n_init - w.n_local) * 3 * row      # inside entries of candidates
    step_bytes = w.layers * (per_layer_kv + scan + w.B * w.Hq * (row + 128 * 4 + 4))
    out = {
        "metric": "decode tokens/s through 4 Forecast-selected layers at 128K (fastest of in-order, one-call and lookahead schedules), 1 GPU",
        "value": round(w.B / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), planted blocks)",
        "config": {"workload": w.name, "batch": w.B, "context": w.T, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.d, "layers": w.layers, "top_k": w.top_k,
                   "selector": "forecast", "schedule": best,
                   "parallelism": "none (1 GPU)"},
        "gpu_ms_per_step": round(gpu_ms, 5),
        "modes_ms_per_step": {k: {"wall": round(v[0], 5), "gpu": round(v[1], 5)} for k, v in res.items()},
        "hidden_selection_us_per_step": round((res["graph_in_order"][1] - res["graph_lookahead"][1]) * 1e3, 2),
        "per_layer_us": round(gpu_ms * 1e3 / w.layers, 2),
        "step_bytes": step_bytes, "step_hbm_gbs": round(step_bytes / (gpu_ms * 1e-3) / 1e9, 1),
    }
    ceil = measured_stream_read_gbs(dev)
    out["measured_ceiling"] = {"what": "stream read (sparse_attn_stream_read, 4 GiB)", "GB/s": ceil,
                               "step_frac": round(out["step_hbm_gbs"] / ceil, 4)}
    print(json.dumps(out), flush=True)


def cpu_baseline_decode(w, inp, lens, budget_s):
    """The CPU oracle, as it is, on the same inputs: whole decode steps until the budget."""
    import numpy as np
    import threadpoolctl
    import oracle

    sel_name = "F" if w.selector == "forecast" else "Q"
    Q = inp["Q"].float().cpu().numpy()
    S = inp[sel_name].float().cpu().numpy()
    p = oracle.SelectParams(w.top_k, w.n_init, w.n_local, w.score_mode)
    Gs = S.shape[1] // w.Hkv
    units = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    host = {}
    for (b, h) in units:                               # setup, not timed
        K = inp["K"][b, h].float().cpu().numpy()
        V = inp["V"][b, h].float().cpu().numpy()
        Kc = oracle.compressed_keys(K, lens[b] - 1, w.dtype)
        host[(b, h)] = (K, V, Kc)
    done, t_units = 0, 0.0
    n_threads = min(len(os.sched_getaffinity(0)), 16)
    with threadpoolctl.threadpool_limits(n_threads):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            for (b, h) in units:
                K, V, Kc = host[(b, h)]
                L = lens[b]
                Kc2 = oracle.append_compressed_keys(K, Kc, L - 1, L, w.dtype)
                oracle.decode_unit(Q[b, h * w.G:(h + 1) * w.G], S[b, h * Gs:(h + 1) * Gs], K, V,
                                   Kc2, L, p, 1.0)
            done += 1
        t_units = time.perf_counter() - t0
    sec_per_step = t_units / done
    return {"value": round(w.B / sec_per_step, 3), "unit": "tokens/s", "cores": n_threads,
            "kind": "oracle",
            "sample": f"{done} full decode steps of {w.name} (all {len(units)} units: append, "
                      f"select, attend), numpy fp64, BLAS threads = {n_threads} (CPU affinity, "
                      f"at most 16), {t_units:.1f} s"}


def bench_cobs(args, w):
    """One decode step selected by block statistics (second order): append the
    statistics of the block the newest token completes, score every complete
    block by its estimated attention mass (mean and per-channel variance) with
    the group's queries, top-k + union, attend. value = batch / step time.
    Also reports, on the first replica, the dense attention mass captured by
    the second-order selection, by the first-order one (block mean only) and
    by the compressed-key selection of the same queries."""
    import numpy as np
    import torch
    import synth
    from block_sparse_attention_12_amd.pipeline import CobsDecoder, SparseDecoder
    from block_sparse_attention_12_amd import block_mass, n_blocks

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_decode_inputs(w, device=dev)
    lens_now = inp["seq_lens"]
    lens_prev = lens_now - 1
    dec = CobsDecoder(w.B, w.Hq, w.Hkv, w.T, w.top_k, w.n_init, w.n_local, w.selector,
                      w.score_mode, device=dev, n_split=args.n_split, order=2)
    reps = []
    for r in range(args.replicas):
        rep = {k: (inp[k] if r == 0 else inp[k].clone()) for k in ("Q", "K", "V")}
        rep["S"] = dec.new_stats(inp["K"].dtype)
        dec.build(rep["K"], rep["S"], lens_prev)           # blocks complete before the new token
        reps.append(rep)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def phases_of(rep):
        return {
            "append": lambda: dec.append(rep["K"], rep["S"], lens_prev, lens_now),
            "select": lambda: dec.select(rep["Q"], rep["S"], lens_now),
            "attend": lambda: dec.attend(rep["Q"], rep["K"], rep["V"], lens_now),
        }

    def whole_step(rep):
        if args.separate_calls:
            for f in phases_of(rep).values():
                f()
        else:                                   # sparse_attn_cobs_decode_step: one call
            dec.fused_step(rep["Q"], rep["Q"], rep["K"], rep["V"], rep["S"], lens_prev, lens_now)

    steps_fn = [lambda rep=rep: whole_step(rep) for rep in reps]
    for i in range(args.warmup):
        steps_fn[i % len(reps)]()
    torch.cuda.synchronize()
    ev0, ev1 = _events(2)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        steps_fn[i % len(reps)]()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    mean = {}
    n_ph = max(10, min(args.steps, 100))
    for name in ("append", "select", "attend"):
        fns = [phases_of(rep)[name] for rep in reps]
        for i in range(3):
            fns[i % len(fns)]()
        evs = [_events(2) for _ in range(n_ph)]
        for i in range(n_ph):
            evs[i][0].record(stream)
            fns[i % len(fns)]()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        mean[name] = sum(e[0].elapsed_time(e[1]) for e in evs) / n_ph

    elem = inp["K"].element_size()
    lens = [int(x) for x in lens_now.cpu()]
    row = 128 * elem
    cnt, idx = dec.cnt.cpu(), dec.idx.cpu()
    attn_bytes = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            for blk in idx[b, h, :int(cnt[b, h])].tolist():
                attn_bytes += 2 * row * max(0, min(64, lens[b] - 64 * blk))
    attn_bytes += w.B * w.Hq * 128 * elem + w.B * w.Hq * (128 * 4 + 4)
    sel_bytes = sum(L // 64 for L in lens) * w.Hkv * 2 * row + inp["Q"].numel() * elem
    append_bytes = sum((L // 64) - ((L - 1) // 64) for L in lens) * w.Hkv * (64 * row + 2 * row)
    step_bytes = attn_bytes + sel_bytes + append_bytes
    attn_gbs = attn_bytes / (mean["attend"] * 1e-3) / 1e9
    sel_gbs = sel_bytes / (mean["select"] * 1e-3) / 1e9

    # selection quality on the first replica: second order, first order, compressed keys
    rep = reps[0]
    quality = {}
    sets = {}
    for order in (2, 1):
        dec.select(rep["Q"], rep["S"], lens_now, order=order)
        sets[f"order{order}"] = (dec.idx.clone(), dec.cnt.clone())
    kc_dec = SparseDecoder(w.B, w.Hq, w.Hkv, w.T, w.top_k, w.n_init, w.n_local, w.selector,
                           w.score_mode, device=dev)
    Kc = kc_dec.new_kc(inp["K"].dtype)
    kc_dec.build(rep["K"], Kc, lens_now)
    kc_dec.select(rep["Q"], Kc, lens_now)
    sets["compressed_keys"] = (kc_dec.idx, kc_dec.cnt)
    for name, (ix, cn) in sets.items():
        mass, rec = block_mass(rep["Q"], rep["K"], lens_now, 1.0, idx=ix, cnt=cn)
        R = rec.cpu().numpy()
        rows = ix.cpu().numpy()
        hit = tot = 0
        for b in range(w.B):
            for h in range(w.Hkv):
                got = set(rows[b, h].tolist())
                hit += sum(1 for x in inp["spread"][b][h] if x in got)
                tot += len(inp["spread"][b][h])
        quality[name] = {"recall_mean": round(float(R.mean()), 4),
                         "recall_min": round(float(R.min()), 4),
                         "spread_blocks_selected": round(hit / max(tot, 1), 4)}
    M = mass.cpu().numpy().astype(np.float64)
    best = []
    for b in range(w.B):
        nb = n_blocks(lens[b])
        cand = np.arange(w.n_init, nb - w.n_local)
        for hq in range(w.Hq):
            m = M[b, hq, :nb]
            best.append(m[:w.n_init].sum() + m[nb - w.n_local:].sum()
                        + np.sort(m[cand])[::-1][:w.top_k].sum())
    quality["mass_optimal_recall_mean"] = round(float(np.mean(best)), 4)
    ceil = measured_stream_read_gbs(dev)
    out = {
        "metric": "sparse decode tokens/s at 128K with second-order block-statistic selection, 1 GPU",
        "value": round(w.B / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), planted mean-shifted and high-variance blocks)",
        "config": {"workload": w.name, "batch": w.B, "context": w.T, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.d, "top_k": w.top_k, "n_init": w.n_init,
                   "n_local": w.n_local, "selector": w.selector, "score_mode": w.score_mode,
                   "statistic": "block mean + per-channel variance (second order)",
                   "replicas": args.replicas,
                   "launch": ("eager, one stream, three calls" if args.separate_calls else
                              "eager, one stream, one sparse_attn_cobs_decode_step call"),
                   "parallelism": "none (1 GPU)"},
        "gpu_ms_per_step": round(gpu_ms, 5),
        "phase_ms": {k: round(v, 5) for k, v in mean.items()},
        "step_bytes": step_bytes, "step_hbm_gbs": round(step_bytes / (gpu_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm",
                     "kernel": "sparse_attn_decode (decode_kernel with the split merge)",
                     "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(f"{w.name}_decode"),
                     "bytes_per_launch": attn_bytes,
                     "measured_ceiling": {"what": "stream read (sparse_attn_stream_read, 4 GiB)",
                                          "GB/s": ceil, "frac": round(attn_gbs / ceil, 4)}},
        "select": {"kernel": "sparse_attn_cobs_select (statistics scan, group softmax, top-k)",
                   "GB/s": round(sel_gbs, 1), "frac_of_ceiling": round(sel_gbs / ceil, 4),
                   "bytes": sel_bytes},
        "selection_quality": quality,
    }
    print(json.dumps(out), flush=True)


def bench_token(args, w):
    """One decode step of the token-index workload: the anchor's token index is
    computed once (scores of every visible token's index key, exact top-k, kept
    initial/local tokens) and w.layers layers attend over that token list.
    value = sequences / step time."""
    import numpy as np
    import torch
    import synth
    from block_sparse_attention_12_amd.pipeline import TokenIndexDecoder

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_token_inputs(w, device=dev)
    lens = inp["seq_lens"]
    dec = TokenIndexDecoder(w.B, w.Hq, w.Hkv, w.T, w.top_k, w.n_init, w.n_local, device=dev,
                            n_split=args.n_split)
    reps = [inp]
    for r in range(1, args.replicas):
        reps.append(dict(Ki=inp["Ki"].clone(), Fi=inp["Fi"].clone(),
                         layers=[{k: v.clone() for k, v in lay.items()} for lay in inp["layers"]]))
    outs = [(torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev),
             torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)) for _ in range(w.layers)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    steps_fn = [lambda rep=rep: dec.step(rep["Fi"], rep["Ki"], rep["layers"], lens, outs)
                for rep in reps]
    for i in range(args.warmup):
        steps_fn[i % len(reps)]()
    torch.cuda.synchronize()
    ev0, ev1 = _events(2)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        steps_fn[i % len(reps)]()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    gpu_ms = ev0.elapsed_time(ev1) / args.steps

    # per-phase GPU time (events on the launch stream around each call)
    n_ph = max(10, min(args.steps, 100))
    phases = {
        "select": [lambda rep=rep: dec.select(rep["Fi"], rep["Ki"], lens) for rep in reps],
        "attend_one_layer": [lambda rep=rep: dec.attend(rep["layers"][0]["Q"], rep["layers"][0]["K"],
                                                        rep["layers"][0]["V"], lens, *outs[0])
                             for rep in reps],
    }
    mean = {}
    for name, fns in phases.items():
        for i in range(3):
            fns[i % len(fns)]()
        evs = [_events(2) for _ in range(n_ph)]
        for i in range(n_ph):
            evs[i][0].record(stream)
            fns[i % len(fns)]()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        mean[name] = sum(e[0].elapsed_time(e[1]) for e in evs) / n_ph

    # algorithmic bytes: every visible token's index key (plus the selector),
    # and per layer the selected tokens' K and V rows, Q in, O + LSE out
    elem = inp["Ki"].element_size()
    L = [int(x) for x in lens.cpu()]
    sel_bytes = sum(L) * w.Hkv * w.d_i * elem + inp["Fi"].numel() * elem
    cnt = dec.cnt.cpu().numpy()
    attn_bytes = int(cnt.sum()) * 2 * w.d * elem + w.B * w.Hq * (w.d * elem + w.d * 4 + 4)
    step_bytes = sel_bytes + w.layers * attn_bytes
    sel_gbs = sel_bytes / (mean["select"] * 1e-3) / 1e9
    attn_gbs = attn_bytes / (mean["attend_one_layer"] * 1e-3) / 1e9
    # planted tokens recovered by the index (quality check of the synthetic setup)
    idx = dec.idx.cpu().numpy()
    hit = tot = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            got = set(idx[b, h, :int(cnt[b, h])].tolist())
            hit += sum(1 for t in inp["planted"][b][h] if t in got)
            tot += len(inp["planted"][b][h])
    ceil = measured_stream_read_gbs(dev)
    out = {
        "metric": "decode tokens/s through 4 layers sharing one token-level index at 128K, 1 GPU",
        "value": round(w.B / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), planted tokens)",
        "config": {"workload": w.name, "batch": w.B, "context": w.T, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.d, "index_dim": w.d_i, "layers": w.layers,
                   "top_k_tokens": w.top_k, "n_init_tokens": w.n_init,
                   "n_local_tokens": w.n_local, "replicas": args.replicas,
                   "launch": "eager, one stream", "parallelism": "none (1 GPU)"},
        "gpu_ms_per_step": round(gpu_ms, 5),
        "phase_ms": {k: round(v, 5) for k, v in mean.items()},
        "step_bytes": step_bytes, "step_hbm_gbs": round(step_bytes / (gpu_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm",
                     "kernel": "sparse_attn_token_select (index-key scan, 3 radix passes, count, "
                               "write)",
                     "achieved": round(sel_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(sel_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(f"{w.name}_score"),
                     "bytes_per_launch": sel_bytes,
                     "measured_ceiling": {"what": "stream read (sparse_attn_stream_read, 4 GiB)",
                                          "GB/s": ceil, "frac": round(sel_gbs / ceil, 4)}},
        "attend": {"kernel": "sparse_attn_token_decode (gathered rows, split merge in the kernel), one layer",
                   "GB/s": round(attn_gbs, 1), "frac_of_peak": round(attn_gbs / HBM_PEAK_GBS, 4),
                   "frac_of_ceiling": round(attn_gbs / ceil, 4), "bytes": attn_bytes},
        "planted_tokens_recovered": round(hit / max(tot, 1), 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_token(w, inp, L, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_token(w, inp, lens, budget_s):
    """The CPU oracle on the same inputs: whole units (select + every layer's
    attention) until the budget, scaled to a step of all B * Hkv units."""
    import numpy as np
    import threadpoolctl
    import oracle

    Fi = inp["Fi"].float().cpu().numpy()
    units = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    n_threads = min(len(os.sched_getaffinity(0)), 16)
    done, t_run = 0, 0.0
    with threadpoolctl.threadpool_limits(n_threads):
        while t_run < budget_s and done < len(units):
            b, h = units[done]
            Ki = inp["Ki"][b, h].float().cpu().numpy()          # host copies: not timed
            lay = [(l["Q"][b, h * w.G:(h + 1) * w.G].float().cpu().numpy(),
                    l["K"][b, h].float().cpu().numpy(), l["V"][b, h].float().cpu().numpy())
                   for l in inp["layers"]]
            t0 = time.perf_counter()
            toks = oracle.select_tokens(Fi[b, h:h + 1], Ki, lens[b], w.top_k, w.n_init, w.n_local)
            for q, K, V in lay:
                oracle.token_decode_unit(q, K, V, toks, 1.0)
            t_run += time.perf_counter() - t0
            done += 1
    sec_per_step = t_run / done * len(units)
    return {"value": round(w.B / sec_per_step, 3), "unit": "tokens/s", "cores": n_threads,
            "kind": "oracle",
            "sample": f"{done} of {len(units)} (sequence, KV head) units of {w.name} (token select "
                      f"+ {w.layers} layers' attention), numpy fp64, BLAS threads = {n_threads}, "
                      f"{t_run:.1f} s, scaled to a whole step"}


def bench_crosslayer(args, w):
    """One decode step of the cross-layer workload: layer 0 appends its compressed
    keys, selects and attends in one sparse_attn_decode_step call; the other
    layers attend over that selection. The 16 appended
    tokens' keys and values are in the cache from the start; a step advances
    the lengths by one, and the 16-step cycle repeats."""
    import torch
    import synth
    from block_sparse_attention_12_amd.pipeline import SparseDecoder
    from block_sparse_attention_12_amd import n_compressed

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T_cap = w.T + w.steps
    layers = []
    for l in range(w.layers):
        inp = synth.make_decode_inputs(w, device=dev, T_cap=T_cap, layer=l)
        qs = synth.make_decode_queries(w, w.steps, device=dev, seed_offset=100 + l)
        layers.append(dict(K=inp["K"], V=inp["V"], qs=qs))
        del inp
    dec = SparseDecoder(w.B, w.Hq, w.Hkv, T_cap, w.top_k, w.n_init, w.n_local, "query",
                        w.score_mode, device=dev, n_split=args.n_split)
    Kc = dec.new_kc(layers[0]["K"].dtype)
    lens = [torch.full((w.B,), w.T + s, dtype=torch.int32, device=dev) for s in range(w.steps + 1)]
    dec.build(layers[0]["K"], Kc, lens[0])
    outs = [(torch.empty_like(dec.O), torch.empty_like(dec.lse)) for _ in range(w.layers)]
    stream = torch.cuda.current_stream()

    def step(i):
        s = i % w.steps
        lay = [dict(Q=L["qs"][s], K=L["K"], V=L["V"]) for L in layers]
        dec.crosslayer_step(lay, Kc, lens[s], lens[s + 1], outs=outs)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = _events(2)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    # bytes of the last step (L = T + steps): anchor scan + 4 attentions
    cnt, idx = dec.cnt.cpu(), dec.idx.cpu()
    L = w.T + w.steps
    row = 128 * 2
    attn = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            for blk in idx[b, h, :int(cnt[b, h])].tolist():
                attn += 2 * row * max(0, min(64, L - 64 * blk))
    attn = attn * w.layers + w.layers * w.B * w.Hq * (128 * 2 + 128 * 4 + 4)
    scan = w.B * w.Hkv * n_compressed(L) * row + w.B * w.Hq * row
    step_bytes = attn + scan
    # dominant kernel: the attention of a follower layer over the shared sets
    # (one sparse_attn_decode call: decode_kernel with the split merge), timed with
    # events around each call on the launch stream, at the last step's lengths
    per_layer_attn = attn // w.layers
    n_ev = max(10, min(args.steps, 60))
    evs = [_events(2) for _ in range(n_ev)]
    for i in range(n_ev):
        lay = layers[1 + i % (w.layers - 1)]
        evs[i][0].record(stream)
        dec.attend(lay["qs"][w.steps - 1], lay["K"], lay["V"], lens[w.steps], O=outs[1][0],
                   lse=outs[1][1])
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    attn_call_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / n_ev
    attn_gbs = per_layer_attn / (attn_call_ms * 1e-3) / 1e9
    out = {
        "metric": "cross-layer sparse decode tokens/s (4 layers share one selection) and HBM GB/s",
        "value": round(w.B / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1))",
        "config": {"workload": w.name, "batch": w.B, "context": f"{w.T}..{w.T + w.steps}",
                   "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d, "layers": w.layers,
                   "top_k": w.top_k, "launch": "eager, one stream; anchor layer in one decode-step call",
                   "parallelism": "none (1 GPU)"},
        "gpu_ms_per_step": round(gpu_ms, 5), "step_bytes": step_bytes,
        "step_hbm_gbs": round(step_bytes / (gpu_ms * 1e-3) / 1e9, 1),
    }
    out["roofline"] = {"bound": "hbm",
                       "kernel": "sparse_attn_decode of a follower layer (decode_kernel with "
                                 "the split merge) over the anchor's block sets",
                       "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                       "traffic": recorded_traffic(f"{w.name}_decode"),
                       "bytes_per_launch": per_layer_attn, "launch_ms": round(attn_call_ms, 5)}
    ceil = measured_stream_read_gbs(dev)
    out["measured_ceiling"] = {"what": "stream read (sparse_attn_stream_read, 4 GiB)", "GB/s": ceil,
                               "step_frac": round(out["step_hbm_gbs"] / ceil, 4)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_crosslayer(w, layers, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_crosslayer(w, layers, budget_s):
    """The CPU oracle, as it is, on the cross-layer workload's first step
    (L = T -> T + 1): the anchor's append, selection and attention plus the
    other layers' attention over the shared sets, on a deterministic prefix
    of the (sequence, KV head) units (units are independent), scaled linearly
    to all units."""
    import numpy as np
    import threadpoolctl
    import oracle

    p = oracle.SelectParams(w.top_k, w.n_init, w.n_local, w.score_mode)
    L0, L1 = w.T, w.T + 1
    units = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    n_threads = min(len(os.sched_getaffinity(0)), 16)
    done, spent = 0, 0.0
    with threadpoolctl.threadpool_limits(n_threads):
        for (b, h) in units:
            lay = []
            for l, L in enumerate(layers):                  # setup, not timed
                lay.append(dict(Q=L["qs"][0][b:b + 1].float().cpu().numpy(),
                                K=L["K"][b:b + 1, h:h + 1, :L1].float().cpu().numpy(),
                                V=L["V"][b:b + 1, h:h + 1, :L1].float().cpu().numpy()))
            for d in lay:                                    # the unit's query heads only
                d["Q"] = d["Q"][:, h * w.G:(h + 1) * w.G]
            kc0 = oracle.compressed_keys(lay[0]["K"][0, 0], L0, w.dtype)
            Kc = np.zeros((1, 1, max(oracle.n_compressed(L1), 1), kc0.shape[1]), dtype=kc0.dtype)
            Kc[0, 0, :kc0.shape[0]] = kc0
            t0 = time.perf_counter()
            oracle.crosslayer_step(lay, Kc, np.array([L0]), np.array([L1]), p, 1.0, w.dtype)
            spent += time.perf_counter() - t0
            done += 1
            if spent >= budget_s:
                break
    sec_per_step = spent / done * len(units)
    return {"value": round(w.B / sec_per_step, 4), "unit": "tokens/s", "cores": n_threads,
            "kind": "oracle",
            "sample": f"first decode step of {w.name} on {done} of {len(units)} (sequence, KV head) "
                      f"units (4 layers each: anchor append + select + attend, 3 follower "
                      f"attentions), {spent:.1f} s, scaled linearly to all units; numpy fp64, "
                      f"BLAS threads = {n_threads}"}


def cpu_baseline_prefill(w, inp, Kc, budget_s):
    """The CPU oracle, as it is, on the prefill chunk: tile selection and causal
    attention of a deterministic prefix of the (64-query tile, KV head) units
    (units are independent), scaled linearly to the whole chunk."""
    import threadpoolctl
    import oracle

    p = oracle.SelectParams(w.top_k, w.n_init, w.n_local, "softmax_sum")
    n_tiles = (w.Tq + 63) // 64
    units = [(t, h) for t in range(n_tiles) for h in range(w.Hkv)]
    Q = inp["Q"].float().cpu().numpy()
    K = inp["K"][0].float().cpu().numpy()
    V = inp["V"][0].float().cpu().numpy()
    Kcn = Kc.float().cpu().numpy()
    n_threads = min(len(os.sched_getaffinity(0)), 16)
    done, spent = 0, 0.0
    with threadpoolctl.threadpool_limits(n_threads):
        for u in units:
            t0 = time.perf_counter()
            oracle.prefill_chunk(Q, K, V, Kcn, w.q_start, p, 1.0, tiles=[u])
            spent += time.perf_counter() - t0
            done += 1
            if spent >= budget_s:
                break
    sec_per_chunk = spent / done * len(units)
    return {"value": round(w.Tq / sec_per_chunk, 4), "unit": "tokens/s", "cores": n_threads,
            "kind": "oracle",
            "sample": f"{done} of {len(units)} (64-query tile, KV head) units of {w.name} "
                      f"(per-query selection, tile union, causal attention), {spent:.1f} s, "
                      f"scaled linearly to the whole {w.Tq}-query chunk; numpy fp64, BLAS "
                      f"threads = {n_threads}"}


def bench_prefill(args):
    """One chunk of sparse prefill: tile selection (scores on matrix cores, exact
    per-query top-k, tile unions) and causal attention over the unions."""
    import numpy as np
    import torch
    import synth
    from block_sparse_attention_12_amd.pipeline import SparsePrefill
    from block_sparse_attention_12_amd import compress, n_compressed

    w = synth.PREFILL_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_prefill_inputs(w, device=dev)
    lens = torch.tensor([w.T], dtype=torch.int32, device=dev)
    reps = []
    for r in range(max(1, min(args.replicas, 2))):
        K = inp["K"] if r == 0 else inp["K"].clone()
        V = inp["V"] if r == 0 else inp["V"].clone()
        Kc = torch.empty((1, w.Hkv, n_compressed(w.T), 128), dtype=torch.bfloat16, device=dev)
        compress(K, Kc, torch.zeros_like(lens), lens)
        reps.append(dict(Q=inp["Q"] if r == 0 else inp["Q"].clone(), K=K[0], V=V[0], Kc=Kc[0]))
    pf = SparsePrefill(w.Hq, w.Hkv, w.q_start, w.Tq, w.top_k, w.n_init, w.n_local, "softmax_sum",
                       device=dev)
    stream = torch.cuda.current_stream()

    def run(i):
        r = reps[i % len(reps)]
        pf.run(r["Q"], r["K"], r["V"], r["Kc"])

    def attend(i):
        r = reps[i % len(reps)]
        pf.attend(r["Q"], r["K"], r["V"])

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    ev0, ev1 = _events(2)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        run(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    evs = [_events(2) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        attend(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    attn_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps

    # algorithmic FLOPs from the tile sets: QK^T and PV over unmasked query-key pairs
    tidx, tcnt = pf.tile_idx.cpu().numpy(), pf.tile_cnt.cpu().numpy()
    pairs = 0
    n_tiles = (w.Tq + 63) // 64
    for t in range(n_tiles):
        nq = min(64, w.Tq - 64 * t)
        bt = w.q_start // 64 + t
        for h in range(w.Hkv):
            blocks = tidx[t, h, :tcnt[t, h]]
            full = int((blocks < bt).sum())
            pairs += full * 64 * nq + (nq * (nq + 1) // 2 if bt in blocks else 0)
    G = w.Hq // w.Hkv
    attn_flops = pairs * G * 128 * 4
    sel_flops = sum(n_compressed(w.q_start + i + 1) for i in range(w.Tq)) * w.Hq * 128 * 2 * 2
    attn_tf = attn_flops / (attn_ms * 1e-3) / 1e12
    out = {
        "metric": "sparse chunked-prefill tokens/s and MFMA TFLOP/s (% of bf16 peak), 1 GPU",
        "value": round(w.Tq / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1))",
        "config": {"workload": w.name, "context": w.T, "chunk": f"{w.q_start}..{w.T - 1}",
                   "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d, "top_k": w.top_k,
                   "n_init": w.n_init, "n_local": w.n_local, "parallelism": "none (1 GPU)"},
        "gpu_ms_per_step": round(gpu_ms, 5),
        "phase_ms": {"select": round(gpu_ms - attn_ms, 5), "attend": round(attn_ms, 5)},
        "mean_union_blocks": round(float(tcnt.mean()), 1), "max_union_blocks": int(tcnt.max()),
        "attn_tflop": round(attn_flops / 1e12, 4), "select_tflop": round(sel_flops / 1e12, 4),
        "roofline": {"bound": "mfma", "kernel": "prefill_attn_kernel (sparse_attn_prefill_attend)",
                     "achieved": round(attn_tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tf / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic(f"{w.name}_attn"), "flops_per_launch": attn_flops},
    }
    ceil = measured_matmul_tflops(dev)
    out["roofline"]["measured_ceiling"] = {"what": "bf16 GEMM 8192^3 (torch.matmul)",
                                           "TFLOP/s": ceil, "frac": round(attn_tf / ceil, 4)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_prefill(w, inp, reps[0]["Kc"], args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
