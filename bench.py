#!/usr/bin/env python3
"""Decode-step benchmark of the native-sparse-attention hot path on one MI355X.

Workload: the NOSA-1B-shaped batched decode (batch 8, contexts uniform in
[8192, 32768] packed by cu_seqlens, 16 query heads, 2 KV heads, head_dim 128,
bf16, compression 32/16, CIS pooled and fused into the block scores, top-64
blocks of 64 tokens with the init block and a 1024-token local window forced).

One step = one decode step of one attention layer over the whole batch: refresh
of the newest compressed window (keys and CIS), compressed scores, block scores
and top-k, selected-block attention.  Steps rotate over 28 distinct layer
buffers (the NOSA-1B layer count; ~4.7 GB of KV) so every step reads KV that is
not resident in the 256 MB last-level cache.  The timed steps are replayed from
one HIP graph.  value = decode tokens/s = batch / step time.

Printed: one JSON line (rank 0).  `roofline` is the selected-attention kernel:
algorithmic bytes per launch (selected K and V tokens, queries, outputs,
indices) over its mean duration, measured by HIP events recorded at the
kernel's own start and end.  `cpu_baseline` times the float64 oracle on the
host cores for layer 0 of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

METRIC = "decode tokens/s + achieved HBM GB/s, selected-block attn at 32K ctx, 1 GPU"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2800)
    ap.add_argument("--warmup", type=int, default=280)
    ap.add_argument("--layers", type=int, default=None,
                    help="distinct layer buffers the decode steps rotate over (default 28 for "
                         "decode, 12 for decode-long: enough that the selected K/V of the "
                         "rotation exceeds the 256 MB Infinity Cache)")
    ap.add_argument("--pinned-32k", action="store_true", help="all contexts 32768")
    ap.add_argument("--batch", type=int, default=8,
                    help="decode: sequences per step (the metric's configuration is 8; larger "
                         "batches show the kernels at larger launch sizes)")
    ap.add_argument("--kc-dtype", choices=["f32", "bf16"], default="f32")
    ap.add_argument("--n-cand", type=int, default=0,
                    help="decode: > 0 selects in two stages (the n_cand best blocks by the "
                         "compressed-attention score, re-ranked by the pooled CIS)")
    ap.add_argument("--profile-steps", type=int, default=280)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps one by one instead of from a HIP graph "
                         "(for counter-collection runs, which serialise dispatches)")
    ap.add_argument("--cis-weight", type=float, default=None,
                    help="decode: weight of the pooled CIS in the block score (default: the "
                         "workload's, 1.0)")
    ap.add_argument("--pool-slots", type=int, default=128,
                    help="decode-offload: device block slots per (sequence, KV head)")
    ap.add_argument("--queries", type=int, default=16,
                    help="decode-offload: distinct queries the steps cycle through (1: every "
                         "step repeats one selection, so the pool holds it after the first)")
    ap.add_argument("--seq", type=int, default=16384,
                    help="prefill-blockmask: tokens per sequence (the pages' table: 1024, 4096, 16384)")
    ap.add_argument("--causal", action="store_true", help="prefill-blockmask: lower triangle only")
    ap.add_argument("--selected-path", choices=["blocks", "rows"], default="blocks",
                    help="prefill workloads: selected attention key-block stationary (its "
                         "workspace given) or row by row")
    ap.add_argument("--workload", choices=["decode", "decode-long", "decode-tiny", "decode-offload",
                                           "prefill-selected", "prefill-nsa", "prefill-blockmask",
                                           "prefill-selected-bwd", "prefill-nsa-bwd"],
                    default="decode",
                    help="decode: the headline NOSA-1B-shaped decode (default); decode-long: "
                         "CIS-weighted decode of 4 x 131072 tokens; decode-tiny: the float32 "
                         "decode of one 4096-token sequence; prefill-selected: "
                         "selected-block attention prefill with given indices (batch 8 x 16384); "
                         "prefill-nsa: the three-branch prefill (65536 tokens, 64 heads); "
                         "prefill-selected-bwd: the gradient of the selected-block attention "
                         "for the prefill-selected batch; prefill-nsa-bwd: the gradient of the "
                         "three-branch prefill (65536 tokens, 64 heads)")
    ap.add_argument("--trace-stats", metavar="CSV", default=None,
                    help="print per-kernel duration statistics (count, mean, median, p10, p90, "
                         "min, max in microseconds) of a rocprofv3 kernel-trace CSV and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="finish with three streaming kernels (fp32 negation) that read and "
                         "write 256 MiB each, the reference dispatch that scales the HBM "
                         "byte counters")
    return ap.parse_args()


COPY_BYTES = 256 << 20
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
TRAFFIC_FILES = {  # counter summaries of the select-and-attend kernel, per decode workload
    "nosa1b_decode_b8_L8k-32k": os.path.join(PROFILES, "select_attn_decode_nosa1b_counters.md"),
    "cis_decode_b4_L131072": os.path.join(PROFILES, "select_attn_decode_cis_b4_L131072_counters.md"),
}
ATTN_SOURCES = ["sparse_attention_compress_amd/csrc/attn.hip",
                "sparse_attention_compress_amd/csrc/common.h",
                "sparse_attention_compress_amd/csrc/select_core.h"]
# counter summaries of the key-block selected attention (partial kernel), per
# prefill workload, and the sources they were taken with
BLOCK_TRAFFIC_FILES = {
    "selected_prefill_b8_T16384": os.path.join(PROFILES, "block_attn_selected_prefill_b8_T16384_counters.md"),
}
BLOCK_SOURCES = ["sparse_attention_compress_amd/csrc/attn_blocks.hip",
                 "sparse_attention_compress_amd/csrc/common.h"]


def attn_source_hash(sources=None) -> str:
    """sha256 (first 16 hex digits) of a kernel's sources (by default the
    select-and-attend kernel's) with comments and whitespace removed, so that
    only a change of code invalidates the stored counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in sources or ATTN_SOURCES:
        with open(os.path.join(root, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def counter_traffic(path, sources=None):
    """HBM bytes per launch of a kernel from a committed counter summary.

    The summary holds FETCH_SIZE and WRITE_SIZE of the kernel, each scaled by what
    the same counter reads for a plain copy of known size, and the hash of the
    kernel sources it was taken with.  None when it is missing or the sources
    have changed since."""
    if path is None:
        return None
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        line = line.strip().strip("`")
        if ":" in line and line.split(":", 1)[0].strip() in ("source_hash", "traffic_bytes_per_launch"):
            k_, v_ = line.split(":", 1)
            vals[k_.strip()] = v_.strip()
    if vals.get("source_hash") != attn_source_hash(sources) or "traffic_bytes_per_launch" not in vals:
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def copy_calibration(dev):
    """Three fp32 negations of COPY_BYTES: a plain elementwise kernel whose
    FETCH_SIZE and WRITE_SIZE scale the counters of the library's kernels (a
    device-to-device copy_ would be a DMA blit, not a kernel dispatch)."""
    import torch
    src = torch.zeros(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"[bench] calibration: 3 fp32 negations reading and writing {COPY_BYTES} bytes each",
          file=sys.stderr, flush=True)


def trace_stats(path):
    """Per-kernel duration statistics of a rocprofv3 kernel-trace CSV (the
    `*_kernel_trace.csv` that `rocprofv3 --kernel-trace` writes)."""
    import csv

    import numpy as np
    durs = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            durs.setdefault(name, []).append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    out = []
    for name, d in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        a = np.asarray(d)
        out.append({"kernel": name[:120], "count": int(a.size), "mean_us": round(float(a.mean()), 3),
                    "median_us": round(float(np.median(a)), 3),
                    "p10_us": round(float(np.percentile(a, 10)), 3),
                    "p90_us": round(float(np.percentile(a, 90)), 3),
                    "min_us": round(float(a.min()), 3), "max_us": round(float(a.max()), 3)})
    for r in out:
        print(json.dumps(r))


def host_cpu():
    """Host facts the CPU baseline is reported with: the CPU model, the logical
    CPUs of the machine and those this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def kernel_stats_us(pairs):
    """mean, median, p10 and p90 (microseconds) of a list of (start, stop) events."""
    import numpy as np
    a = np.asarray([s.elapsed_time(e) for s, e in pairs]) * 1e3
    return {"mean": round(float(a.mean()), 3), "median": round(float(np.median(a)), 3),
            "p10": round(float(np.percentile(a, 10)), 3), "p90": round(float(np.percentile(a, 90)), 3)}


def main():
    args = parse()
    if args.trace_stats:
        trace_stats(args.trace_stats)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but the library runs on one GPU only "
              "(no multi-GPU path exists; the decode would shard over (sequence, KV head) "
              "with no exchange between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_compress_amd as nsa
    from gen import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.workload == "decode-offload":
        offload_main(args, dev)
        return
    if args.workload == "prefill-blockmask":
        blockmask_main(args, dev)
        return
    if args.workload == "prefill-selected-bwd":
        selected_bwd_main(args, dev)
        return
    if args.workload == "prefill-nsa-bwd":
        nsa_bwd_main(args, dev)
        return
    if args.workload not in ("decode", "decode-long", "decode-tiny"):
        prefill_main(args, dev)
        return
    if args.workload == "decode-long":
        w = W.cis_decode()
        n_layers = args.layers or 12
    elif args.workload == "decode-tiny":
        w = W.tiny_decode()
        # 2.1 MB of selected fp32 K/V per step: 128 buffers exceed the Infinity Cache
        n_layers = args.layers or 128
    else:
        w = W.nosa1b_decode(pinned_32k=args.pinned_32k, batch=args.batch)
        # enough layer buffers that a rotation's selected K/V (4 MiB per sequence)
        # exceeds the 256 MB Infinity Cache: 28 (the model's layers) at batch 8
        n_layers = args.layers or max(2, -(-28 * 8 // args.batch))
    B, H, Hkv, D = w.batch, w.heads, w.kv_heads, w.head_dim
    lengths = list(w.lengths)
    nc = [nsa.window_count(L) for L in lengths]
    cu_k = nsa.cu_seqlens_of(lengths, dev)
    cu_c = nsa.cu_seqlens_of(nc, dev)
    max_len = max(lengths)
    kc_dt = torch.float32 if args.kc_dtype == "f32" else torch.bfloat16
    dt_name = "f32" if w.dtype == torch.float32 else "bf16"
    print(f"[bench] workload {w.name} lengths={lengths} layers={n_layers}", file=sys.stderr, flush=True)

    layers = []
    for li in range(n_layers):
        q = W.decode_query(w, dev, layer=li)
        k, v = W.keys_values(w, dev, layer=li)
        cis = W.cis_scores(w, dev, layer=li)
        kc = torch.empty((sum(nc), Hkv, D), dtype=kc_dt, device=dev)
        cp = torch.empty((sum(nc), Hkv), dtype=torch.float32, device=dev)
        nsa.nsa_compress_k(k, kc, cu_k, cu_c, max(nc))
        nsa.nsa_cis_mean_pool_varlen(cis, cp, cu_k, cu_c, max(nc))
        out = torch.empty((B, H, D), dtype=w.dtype, device=dev)
        idx = torch.empty((B, Hkv, w.topk), dtype=torch.int32, device=dev)
        p = nsa.decode_params(q, k, v, kc, cu_k, cu_c, max_len, out, topk=w.topk, n_init=w.n_init,
                              n_local=w.n_local, cis=cis, cis_pooled=cp if w.cis_select else None,
                              cis_weight=w.cis_weight, cis_values=w.cis_values, append_window=True,
                              indices=idx, n_cand=args.n_cand)
        layers.append(dict(q=q, k=k, v=v, cis=cis, kc=kc, cp=cp, out=out, idx=idx, p=p))
    torch.cuda.synchronize()
    ws = torch.zeros(nsa.decode_workspace_size(layers[0]["p"]), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    nl = len(layers)

    def step(i):
        nsa.nsa_decode_step(layers[i % nl]["p"], workspace=ws)

    with torch.cuda.stream(stream):
        for i in range(nl):
            step(i)
    torch.cuda.synchronize()
    print("[bench] eager steps done; capturing graphs", file=sys.stderr, flush=True)

    # the timed steps continue the warm-up's rotation over the layer buffers, so
    # the first timed step does not re-read what the last warm-up steps touched
    def capture(n, start):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(start, start + n):
                step(i)
        return g

    n_warm = max(1, args.warmup)
    if args.eager:
        def run(n, start):
            with torch.cuda.stream(stream):
                for i in range(start, start + n):
                    step(i)
    else:
        g_warm = capture(n_warm, 0)
        g_timed = capture(args.steps, n_warm)
        run = None
    torch.cuda.synchronize()
    if args.eager:
        run(n_warm, 0)
    else:
        g_warm.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if args.eager:
        run(args.steps, n_warm)
    else:
        with torch.cuda.stream(stream):
            g_timed.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_s = t1 - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall_s * 1e3 / args.steps
    tokens_per_s = B * args.steps / wall_s
    print(f"[bench] timed {args.steps} steps: wall {wall_s * 1e3:.2f} ms, events {gpu_ms:.2f} ms",
          file=sys.stderr, flush=True)

    # per-kernel durations, from events recorded at each kernel's own start and end
    # bf16 decode with up to 2048 blocks and 256 selected blocks per sequence runs the
    # selection inside the attention kernel (one launch per step fewer)
    fused = (w.dtype == torch.bfloat16 and -(-max_len // 64) <= 2048 and w.topk <= 256)
    if fused:
        kinds = {"logits_and_refresh": nsa.KERNEL_LOGITS,
                 "select_and_attn": nsa.KERNEL_SELECTED_ATTN, "combine": nsa.KERNEL_COMBINE}
        attn_key = "select_and_attn"
    else:
        kinds = {"logits_and_refresh": nsa.KERNEL_LOGITS, "block_scores_topk": nsa.KERNEL_BLOCK_SCORES,
                 "selected_attn": nsa.KERNEL_SELECTED_ATTN, "combine": nsa.KERNEL_COMBINE}
        attn_key = "selected_attn"
    n_prof = max(1, args.profile_steps)
    evs = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(n_prof)] for name in kinds}
    with torch.cuda.stream(stream):
        for name in kinds:
            for a, b in evs[name]:
                a.record(stream)
                b.record(stream)
        torch.cuda.synchronize()
        for i in range(n_prof):
            for name, kind in kinds.items():
                a, b = evs[name][i]
                nsa.nsa_profile_next_launch(kind, a, b)
            step(i)
    torch.cuda.synchronize()
    kern_us = {name: float(np.mean([a.elapsed_time(b) for a, b in evs[name]])) * 1e3 for name in kinds}
    kern_stats = {name: kernel_stats_us(evs[name]) for name in kinds}

    # algorithmic bytes of one selected-attention launch (identical for every layer)
    idx0 = layers[0]["idx"].cpu().numpy()
    sel_tokens = 0
    for b_, L in enumerate(lengths):
        for g in range(Hkv):
            for blk in idx0[b_, g]:
                if blk >= 0:
                    sel_tokens += min(64, L - 64 * int(blk))
    elt = 2 if w.dtype == torch.bfloat16 else 4
    G = H // Hkv
    if fused:
        # the selection's inputs: logits, chunk (max, sum) pairs, block CIS maxima
        sel_in = sum(Hkv * (G * c * 4 + -(-c // 64) * G * 8 + -(-L // 64) * 4)
                     for L, c in zip(lengths, nc))
    else:
        sel_in = B * Hkv * w.topk * 4                 # block ids
    cis_sel = sel_tokens * 4 if w.cis_values else 0  # CIS of the selected tokens
    attn_bytes = (sel_tokens * D * elt * 2            # selected K and V rows
                  + 2 * B * H * D * elt               # queries in, outputs out
                  + sel_in + cis_sel)
    kc_elt = 4 if kc_dt == torch.float32 else 2
    score_bytes = (sum(nc) * Hkv * D * kc_elt         # compressed keys
                   + sum(nc) * Hkv * 4                # pooled CIS
                   + B * H * D * elt)                 # queries
    refresh_bytes = B * (32 * Hkv * D * elt + 32 * Hkv * 4 + Hkv * D * kc_elt + Hkv * 4)
    step_bytes = attn_bytes + score_bytes + refresh_bytes
    attn_gbs = attn_bytes / (kern_us[attn_key] * 1e-6) / 1e9

    # The selected-block attention kernel alone (nsa_selected_attn_fwd over the ids
    # each layer's step chose), rotating over the layers like the step: the part of
    # the step that streams the selected K/V, without the selection's latency.
    sa_out = torch.empty_like(layers[0]["out"])
    sa_ws = torch.zeros(max(1, nsa.selected_attn_workspace_size(B, H, Hkv, D, w.topk, True)),
                        dtype=torch.uint8, device=dev)
    sa_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_prof)]

    def sa_call(i):
        L_ = layers[i % nl]
        nsa.nsa_selected_attn_fwd(L_["q"], L_["k"], L_["v"], L_["idx"], cu_k, max_len, sa_out,
                                  cis=L_["cis"] if w.cis_values else None, workspace=sa_ws)

    with torch.cuda.stream(stream):
        for i in range(nl):
            sa_call(i)
        for a, b in sa_evs:
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        for i in range(n_prof):
            nsa.nsa_profile_next_launch(nsa.KERNEL_SELECTED_ATTN, *sa_evs[i])
            sa_call(i)
    torch.cuda.synchronize()
    sa_us = float(np.mean([a.elapsed_time(b) for a, b in sa_evs])) * 1e3
    sa_bytes = sel_tokens * D * elt * 2 + 2 * B * H * D * elt + B * Hkv * w.topk * 4 + cis_sel

    # Practical ceiling at this launch size: a plain streaming kernel (fp32
    # negation, half the bytes read and half written) moving the fused kernel's
    # algorithmic bytes, timed the same way, over buffers rotated like the layers.
    n_el = attn_bytes // 8
    cp_src = [torch.zeros(n_el, dtype=torch.float32, device=dev) for _ in range(nl)]
    cp_dst = [torch.empty_like(x) for x in cp_src]
    torch.cuda.synchronize()
    cp_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_prof)]
    with torch.cuda.stream(stream):
        for i in range(nl):
            torch.neg(cp_src[i], out=cp_dst[i])
        for i in range(n_prof):
            a, b = cp_evs[i]
            a.record(stream)
            torch.neg(cp_src[i % nl], out=cp_dst[i % nl])
            b.record(stream)
    torch.cuda.synchronize()
    cp_us = float(np.median([a.elapsed_time(b) for a, b in cp_evs])) * 1e3
    cp_bytes = n_el * 8
    del cp_src, cp_dst

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic (seeded N(0,1) Q/K/V, sigmoid(N(0,1)) CIS; no dataset)",
        "config": {
            "workload": w.name,
            "batch": B, "context_lengths": lengths, "heads": H, "kv_heads": Hkv, "head_dim": D,
            "compress_kernel": w.kernel, "compress_stride": w.stride, "block": w.block,
            "topk": w.topk, "forced_init_blocks": w.n_init, "forced_local_blocks": w.n_local,
            "cis_fused": bool(w.cis_select), "cis_values": bool(w.cis_values),
            "compressed_key_dtype": args.kc_dtype,
            "selection": (f"two-stage, {args.n_cand} candidates" if args.n_cand > 0 else
                          "one fused score"),
            "layer_buffers_rotated": nl, "step": "one layer, whole batch, HIP-graph replay",
        },
        "roofline": {
            "kernel": ("select_attn_kernel (decode: block scores, top-k and attention over "
                       "the selected blocks, split over blocks)" if fused else
                       "selected_attn_valu_kernel (decode, float32, split over selected blocks)"
                       if w.dtype == torch.float32 else
                       "selected_attn_mfma_kernel (decode, split over selected blocks)"),
            "bound": "hbm",
            "achieved": round(attn_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
            # the stored counters belong to the fused kernel on the 8K-32K batch
            "traffic": (counter_traffic(TRAFFIC_FILES.get(w.name)) if fused and args.n_cand == 0
                        and args.kc_dtype == "f32" else None),
            "algorithmic_bytes_per_launch": attn_bytes,
            "mean_kernel_us": round(kern_us[attn_key], 3),
            "source_hash": attn_source_hash(),
        },
        "kernel_us": {k_: round(v_, 3) for k_, v_ in kern_us.items()},
        "kernel_us_stats": kern_stats,
        "selected_attn_alone": {
            "kernel": ("selected_attn_mfma_kernel" if w.dtype == torch.bfloat16 else
                       "selected_attn_valu_kernel") + " (nsa_selected_attn_fwd on the step's ids)",
            "mean_kernel_us": round(sa_us, 3), "algorithmic_bytes_per_launch": sa_bytes,
            "achieved": round(sa_bytes / (sa_us * 1e-6) / 1e9, 1), "unit": "GB/s",
            "frac": round(sa_bytes / (sa_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "copy_ceiling": {
            "kernel": "fp32 negation (torch.neg) of the same byte count, launch to launch events",
            "bytes": cp_bytes, "median_us": round(cp_us, 3),
            "achieved": round(cp_bytes / (cp_us * 1e-6) / 1e9, 1), "unit": "GB/s",
            "frac": round(cp_bytes / (cp_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_gbs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "tokens_per_s_28_layers": round(tokens_per_s / 28.0, 1),
        "timed_gpu_ms": round(gpu_ms, 3),
    }

    if args.calibrate_copy:
        copy_calibration(dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity_layer0"] = cpu_baseline(w, layers[0], lengths, args)
    print(json.dumps(result), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def _timed(fn, steps, warmup, stream):
    import torch
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps):
            fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, ev0.elapsed_time(ev1)


def _kernel_us(nsa, fn, kinds, reps, stream):
    """Mean duration of each armed kernel kind over `reps` eager calls of fn."""
    import numpy as np
    import torch
    evs = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)] for n in kinds}
    with torch.cuda.stream(stream):
        for n in kinds:
            for a, b in evs[n]:
                a.record(stream)
                b.record(stream)
        torch.cuda.synchronize()
        for i in range(reps):
            for n, kind in kinds.items():
                a, b = evs[n][i]
                nsa.nsa_profile_next_launch(kind, a, b)
            fn()
    torch.cuda.synchronize()
    return {n: float(np.mean([a.elapsed_time(b) for a, b in evs[n]])) * 1e3 for n in kinds}


HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def offload_main(args, dev):
    """The batched decode with its K/V cache in pinned host memory: every step
    scores and selects on the device and copies only the selected blocks that the
    device pool does not hold.  The steps cycle through `--queries` distinct query
    sets (fresh selections each step: the least reuse); the pool starts empty."""
    import numpy as np
    import torch

    import sparse_attention_compress_amd as nsa
    from gen import workloads as W

    w = W.nosa1b_decode()
    B, H, Hkv, D = w.batch, w.heads, w.kv_heads, w.head_dim
    lengths = list(w.lengths)
    nc = [nsa.window_count(L) for L in lengths]
    cu_k, cu_c = nsa.cu_seqlens_of(lengths, dev), nsa.cu_seqlens_of(nc, dev)
    max_len = max(lengths)
    nb_max = -(-max_len // 64)
    print(f"[bench] workload {w.name} (K/V in host memory) pool_slots={args.pool_slots} "
          f"queries={args.queries}", file=sys.stderr, flush=True)
    k, v = W.keys_values(w, dev)
    cis = W.cis_scores(w, dev)
    kc = torch.empty((sum(nc), Hkv, D), dtype=torch.float32, device=dev)
    cp = torch.empty((sum(nc), Hkv), dtype=torch.float32, device=dev)
    nsa.nsa_compress_k(k, kc, cu_k, cu_c, max(nc))
    nsa.nsa_cis_mean_pool_varlen(cis, cp, cu_k, cu_c, max(nc))
    k_host = torch.empty(k.shape, dtype=k.dtype, pin_memory=True)
    v_host = torch.empty(v.shape, dtype=v.dtype, pin_memory=True)
    k_host.copy_(k)
    v_host.copy_(v)
    torch.cuda.synchronize()
    del k, v
    torch.cuda.empty_cache()
    st, keep = nsa.offload_state(B, Hkv, args.pool_slots, nb_max, dev)
    out = torch.empty((B, H, D), dtype=w.dtype, device=dev)
    cis_w = w.cis_weight if args.cis_weight is None else args.cis_weight
    qs = [W.decode_query(w, dev, layer=i) for i in range(args.queries)]  # kept alive: params hold pointers
    ps = [nsa.decode_params(q_, k_host, v_host, kc, cu_k, cu_c, max_len, out, topk=w.topk,
                            n_init=w.n_init, n_local=w.n_local, cis=cis, cis_pooled=cp,
                            cis_weight=cis_w, append_window=True, n_cand=args.n_cand)
          for q_ in qs]
    ws = torch.zeros(nsa.decode_offload_workspace_size(ps[0], st), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    n_all = args.warmup + args.steps

    def step(i):
        nsa.nsa_decode_step_offload(ps[i % len(ps)], st, workspace=ws)

    # pass 1, eager: blocks fetched by every step of the sequence the timed run replays
    fetched = []
    with torch.cuda.stream(stream):
        nsa.nsa_offload_reset(st, B, Hkv)
        for i in range(n_all):
            step(i)
            torch.cuda.synchronize()
            fetched.append(int(keep["fetched"].sum().item()))
    f_timed = fetched[args.warmup:]
    blk_bytes = 64 * D * 2 * 2  # K and V rows of one block of one KV head
    # pass 2: the same sequence from an empty pool, warm-up then timed, from HIP graphs
    with torch.cuda.stream(stream):
        nsa.nsa_offload_reset(st, B, Hkv)
    torch.cuda.synchronize()

    def capture(lo, hi):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(lo, hi):
                step(i)
        return g

    g_warm, g_timed = capture(0, args.warmup), capture(args.warmup, n_all)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        nsa.nsa_offload_reset(st, B, Hkv)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        g_timed.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-kernel durations over a few more eager steps (continuing the sequence)
    kinds = {"logits_and_refresh": nsa.KERNEL_LOGITS, "select": nsa.KERNEL_BLOCK_SCORES,
             "fetch": nsa.KERNEL_FETCH, "pool_attn": nsa.KERNEL_SELECTED_ATTN,
             "combine": nsa.KERNEL_COMBINE}
    nxt = [n_all]

    def step_next():
        step(nxt[0])
        nxt[0] += 1
    kern = _kernel_us(nsa, step_next, kinds, min(56, max(8, args.profile_steps)), stream)
    mean_fetch = float(np.mean(f_timed)) if f_timed else 0.0
    fetch_gbs = mean_fetch * blk_bytes / (kern["fetch"] * 1e-6) / 1e9 if kern["fetch"] > 0 else 0.0
    result = {
        "metric": METRIC + " (KV offloaded to host memory)",
        "value": round(B * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, sigmoid(N(0,1)) CIS; no dataset)",
        "config": {"workload": w.name + "_kv_offload", "batch": B, "context_lengths": lengths,
                   "heads": H, "kv_heads": Hkv, "head_dim": D, "topk": w.topk,
                   "pool_slots": args.pool_slots, "distinct_queries": args.queries,
                   "cis_weight": cis_w,
                   "kv_location": "pinned host memory", "step": "one layer, whole batch, HIP-graph replay"},
        "roofline": {"kernel": "offload_fetch_kernel (selected blocks copied from host memory)",
                     "bound": "host-link", "achieved": round(fetch_gbs, 2), "peak": HOST_LINK_PEAK_GBS,
                     "unit": "GB/s", "frac": round(fetch_gbs / HOST_LINK_PEAK_GBS, 4), "traffic": None},
        "fetched_blocks_per_step": round(mean_fetch, 2),
        "fetched_bytes_per_step": round(mean_fetch * blk_bytes, 1),
        "selected_blocks_per_step": B * Hkv * w.topk,
        "kernel_us": {k_: round(v_, 3) for k_, v_ in kern.items()},
    }
    print(json.dumps(result), flush=True)


# The pages' TileLang block-sparse timings on H100-80GB (batch 8, 16 heads, dim
# 128, 50% of 64 x 64 blocks, fp16 storage): ms per call at 1024 / 4096 / 16384.
PAGES_BLOCKMASK_H100_MS = {1024: 3.2, 4096: 42.3, 16384: 318.6}


def blockmask_main(args, dev):
    """Block-mask attention at the pages' benchmark shape: one step = one call over
    the batch; value = query tokens/s; roofline = algorithmic bf16 MFMA flops
    (4 * 128 per (query, head, attended key))."""
    import numpy as np
    import torch

    import sparse_attention_compress_amd as nsa
    from gen import workloads as W

    w = W.blockmask_prefill(args.seq, args.causal)
    print(f"[bench] workload {w.name}", file=sys.stderr, flush=True)
    D, seq = w.head_dim, args.seq
    q = W.prefill_query(w, dev)
    k, v = W.keys_values(w, dev)
    mask = W.block_mask(w, dev)
    cu = nsa.cu_seqlens_of(w.lengths, dev)
    out = torch.empty_like(q)
    ws = torch.empty(nsa.blockmask_attn_workspace_size(w.batch, seq, w.heads), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.Stream(device=dev)

    def fn():
        nsa.nsa_blockmask_attn_fwd(q, k, v, mask, cu, seq, out, causal=args.causal, workspace=ws)
    steps = args.steps if args.steps != 2800 else (200 if seq <= 4096 else 10)
    warmup = args.warmup if args.warmup != 280 else 3
    wall_s, gpu_ms = _timed(fn, steps, warmup, stream)
    kern = _kernel_us(nsa, fn, {"blockmask_attn": nsa.KERNEL_BLOCKMASK_ATTN}, 3, stream)
    # attended (query, key) pairs per head, from the mask
    m = mask.cpu().numpy().astype(np.int64)        # [B, H, nb, nb]
    nb = m.shape[-1]
    full = 64 * 64
    if args.causal:
        tri = np.tril(np.ones((nb, nb), dtype=np.int64), -1)
        pairs = float((m * tri).sum() * full + np.trace(m, axis1=2, axis2=3).sum() * (64 * 65 // 2))
    else:
        pairs = float(m.sum() * full)
    flops = 4.0 * D * pairs
    tfl = flops / (kern["blockmask_attn"] * 1e-6) / 1e12
    ms = wall_s * 1e3 / steps
    value = w.total_tokens * steps / wall_s
    pages_ms = PAGES_BLOCKMASK_H100_MS.get(seq) if not args.causal else None
    result = {
        "metric": f"prefill tokens/s ({w.name})",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(pages_ms / ms, 3) if pages_ms else None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, seeded 50% block mask; no dataset)",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": seq, "heads": w.heads,
                   "head_dim": D, "block": 64, "density": 0.5, "causal": bool(args.causal),
                   "active_blocks": int(m.sum())},
        "roofline": {"kernel": "blockmask_attn_kernel", "bound": "mfma", "achieved": round(tfl, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops_per_launch": flops,
                     "mean_kernel_us": round(kern["blockmask_attn"], 1)},
        "pages_context": ({"h100_tilelang_ms": pages_ms, "note": "H100-80GB, fp16 storage; "
                           "vs_baseline = their ms / ours"} if pages_ms else None),
        "timed_gpu_ms": round(gpu_ms, 3),
    }
    if not args.no_cpu_baseline:
        import oracle
        qn = q.float().cpu().numpy().astype(np.float64)
        kn, vn = k.float().cpu().numpy().astype(np.float64), v.float().cpu().numpy().astype(np.float64)
        scale = 1.0 / math.sqrt(D)

        def rows_fn(rows):
            for r in rows:
                b_, t_ = divmod(r, seq)
                s0 = b_ * seq
                oracle.blockmask_attention_row(qn[r], kn[s0:s0 + seq], vn[s0:s0 + seq], m[b_], t_,
                                               64, scale, args.causal)
        result["cpu_baseline"] = sampled_oracle_baseline(rows_fn, w.total_tokens, w.total_tokens,
                                                         args.cpu_seconds, "query rows")
    print(json.dumps(result), flush=True)


def sampled_oracle_baseline(rows_fn, n_rows_total, tokens_total, seconds, what, chunk=1,
                            fixed_fn=None):
    """CPU baseline of a prefill workload: the float64 oracle on one host thread
    over evenly strided sample rows (calls of `chunk` rows) until `seconds` are
    spent, extrapolated to every row of the step.  `fixed_fn`, if given, is the
    per-call work done once for the whole step (pooling the sequence): it is timed
    once, taken out of every call and counted once."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    order = np.linspace(0, n_rows_total - 1, num=min(n_rows_total, 8192)).round().astype(np.int64)
    done, spent, calls, fixed = 0, 0.0, 0, 0.0
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        if ctx:
            ctx.__enter__()
        if fixed_fn is not None:
            t0 = time.perf_counter()
            fixed_fn()
            fixed = time.perf_counter() - t0
        for i in range(0, len(order), chunk):
            rows = [int(r) for r in order[i:i + chunk]]
            t0 = time.perf_counter()
            rows_fn(rows)
            spent += time.perf_counter() - t0
            done += len(rows)
            calls += 1
            if spent >= seconds:
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    per_row = max(spent - calls * fixed, 1e-9) / done
    step_s = fixed + per_row * n_rows_total
    return {"value": round(tokens_total / step_s, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {n_rows_total} {what} (evenly strided), {spent:.1f} s on one host "
                      f"thread, extrapolated to the whole step ({step_s:.4g} s)",
            **host_cpu()}


def prefill_main(args, dev):
    """Prefill workloads: one step = the whole batch's prefill; value = prefill
    tokens/s; roofline = the dominant kernel's algorithmic bf16 MFMA flops."""
    import numpy as np
    import torch

    import sparse_attention_compress_amd as nsa
    from gen import workloads as W

    stream = torch.cuda.Stream(device=dev)
    steps = args.steps if args.steps != 2800 else (20 if args.workload == "prefill-selected" else 5)
    warmup = args.warmup if args.warmup != 280 else 2
    D = 128
    if args.workload == "prefill-selected":
        w = W.selected_prefill()
        print(f"[bench] workload {w.name}", file=sys.stderr, flush=True)
        q = W.prefill_query(w, dev)
        k, v = W.keys_values(w, dev)
        idx = W.given_block_indices(w, dev)
        cu = nsa.cu_seqlens_of(w.lengths, dev)
        out = torch.empty_like(q)
        blocks = args.selected_path == "blocks"
        need = nsa.selected_attn_workspace_size(q.shape[0], w.heads, w.kv_heads, D, w.topk, False)
        sws = torch.empty(need if blocks else 0, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

        def fn():
            nsa.nsa_selected_attn_fwd(q, k, v, idx, cu, max(w.lengths), out, cu_seqlens_q=cu,
                                      workspace=sws)
        kinds = {"selected_attn": nsa.KERNEL_SELECTED_ATTN}
        if blocks:  # the partial states' merge
            kinds["merge"] = nsa.KERNEL_COMBINE
        # algorithmic work: every (row, head) attends to the tokens j <= t of its blocks
        ids = idx.cpu().numpy().astype(np.int64).reshape(-1, w.topk)
        pos = np.concatenate([np.arange(L) for L in w.lengths])
        t = np.repeat(pos, w.kv_heads).reshape(-1, 1)
        keys = np.where(ids >= 0, np.clip(t - 64 * ids + 1, 0, 64), 0).sum()
        G = w.heads // w.kv_heads
        flops = {"selected_attn": 4.0 * D * G * float(keys)}
        gathered = float(keys) * D * 2 * 2  # K and V rows of every (row, kv head)
        dominant = "selected_attn"
    else:
        w = W.nsa_prefill()
        print(f"[bench] workload {w.name}", file=sys.stderr, flush=True)
        q = W.prefill_query(w, dev)
        k, v = W.keys_values(w, dev)
        g = W.gates(w, dev)
        L = w.lengths[0]
        nc = nsa.window_count(L)
        cu = nsa.cu_seqlens_of(w.lengths, dev)
        cuc = nsa.cu_seqlens_of([nc], dev)
        kc = torch.empty((nc, w.kv_heads, D), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        out = torch.empty_like(q)
        idx = torch.empty((L, w.kv_heads, w.topk), dtype=torch.int32, device=dev)
        p = nsa.prefill_params(q, k, v, kc, vc, g, cu, cu, cuc, L, out, topk=w.topk,
                               window=w.window, indices=idx)
        ws_bytes = (nsa.prefill_workspace_size(p) if args.selected_path == "blocks"
                    else nsa.prefill_workspace_size_min(p))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

        def fn():
            nsa.nsa_prefill_step(p, workspace=ws)
        kinds = {"pool": nsa.KERNEL_POOL, "compressed_lse": nsa.KERNEL_COMPRESSED_LSE,
                 "compressed_attn": nsa.KERNEL_COMPRESSED_ATTN,
                 "select": nsa.KERNEL_BLOCK_SCORES, "selected_attn": nsa.KERNEL_SELECTED_ATTN,
                 "window_attn": nsa.KERNEL_WINDOW_ATTN}
        if args.selected_path == "blocks":  # the selected branch's partial-state merge
            kinds["selected_merge"] = nsa.KERNEL_COMBINE
        fn()
        torch.cuda.synchronize()
        t = np.arange(L, dtype=np.int64)
        nvis = np.where(t >= 31, np.minimum(nc, (t - 31) // 16 + 1), 0)
        win = np.minimum(t + 1, w.window)
        ids = idx.cpu().numpy().astype(np.int64)
        sel = np.where(ids >= 0, np.clip(t[:, None, None] - 64 * ids + 1, 0, 64), 0).sum()
        H = w.heads
        G = H // w.kv_heads
        flops = {"compressed_lse": 2.0 * D * H * float(nvis.sum()),
                 "compressed_attn": 4.0 * D * H * float(nvis.sum()),
                 "selected_attn": 4.0 * D * G * float(sel),
                 "window_attn": 4.0 * D * H * float(win.sum())}
        gathered = float(sel) * D * 2 * 2
        dominant = None
    wall_s, gpu_ms = _timed(fn, steps, warmup, stream)
    kern = _kernel_us(nsa, fn, kinds, 3, stream)
    if dominant is None:  # the longest of the kernels that carry the branches' flops
        dominant = max(flops, key=lambda n: kern[n])
    tokens = w.total_tokens
    ms_per_step = wall_s * 1e3 / steps
    tflops = {n: flops[n] / (kern[n] * 1e-6) / 1e12 for n in flops}
    algo_flops = sum(v for n, v in flops.items() if n != "compressed_lse")
    result = {
        "metric": f"prefill tokens/s ({w.name})",
        "value": round(tokens * steps / wall_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V" + (", sigmoid(N(0,1)) gates" if args.workload == "prefill-nsa" else ", uniform causal block indices") + "; no dataset)",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": max(w.lengths), "heads": w.heads,
                   "kv_heads": w.kv_heads, "head_dim": D, "topk": w.topk,
                   **({"window": w.window} if args.workload == "prefill-nsa" else {}),
                   "selected_path": args.selected_path},
        "roofline": {
            "kernel": dominant,
            "bound": "mfma",
            "achieved": round(tflops[dominant], 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops[dominant] / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": (counter_traffic(BLOCK_TRAFFIC_FILES.get(w.name), BLOCK_SOURCES)
                        if args.workload == "prefill-selected" and args.selected_path == "blocks"
                        else None),
            "algorithmic_flops_per_launch": flops[dominant],
            "mean_kernel_us": round(kern[dominant], 1),
        },
        "kernel_us": {n: round(x, 1) for n, x in kern.items()},
        "kernel_tflops": {n: round(x, 2) for n, x in tflops.items()},
        "step_algorithmic_tflops": round(algo_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "selected_gathered_gbs": round(gathered / (kern["selected_attn"] * 1e-6) / 1e9, 1),
        "timed_gpu_ms": round(gpu_ms, 3),
    }
    if args.workload == "prefill-selected" and args.selected_path == "blocks":
        # the key-block path moves partial states instead of gathering K/V rows:
        # 256 B of bf16 output + 8 B of (max, sum) per (row, head, valid place),
        # written by the partial kernel and read back by the merge
        pos_k = np.repeat(pos, w.kv_heads)
        valid = ((ids >= 0) & (64 * ids <= pos_k[:, None])).sum()
        pbytes = float(valid) * G * 264
        result["partial_state_bytes"] = pbytes
        result["partial_write_gbs"] = round(pbytes / (kern["selected_attn"] * 1e-6) / 1e9, 1)
        result["merge_read_gbs"] = round(pbytes / (kern["merge"] * 1e-6) / 1e9, 1)
        # the partial kernel's own ceiling is HBM: its counted bytes (partial states
        # written, query/index/K/V rows fetched) per launch over its duration
        tr = result["roofline"]["traffic"]
        if tr is not None:
            gbs = tr / (kern["selected_attn"] * 1e-6) / 1e9
            result["partial_kernel_hbm"] = {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if args.selected_path == "blocks":  # no per-row gather on the key-block path
        del result["selected_gathered_gbs"]
    if args.calibrate_copy:
        copy_calibration(dev)
    if not args.no_cpu_baseline:
        import oracle
        scale = 1.0 / math.sqrt(D)
        kn, vn = k.float().cpu().numpy().astype(np.float64), v.float().cpu().numpy().astype(np.float64)
        qn = q.float().cpu().numpy().astype(np.float64)
        if args.workload == "prefill-selected":
            idn = idx.cpu().numpy()
            L0 = w.lengths[0]

            def rows_fn(rows):  # rows of equal-length sequences, packed
                for r in rows:
                    b_, t_ = divmod(r, L0)
                    s0 = b_ * L0
                    oracle.selected_attention_row(qn[r], kn[s0:s0 + L0], vn[s0:s0 + L0], idn[r], t_,
                                                  64, scale)
            result["cpu_baseline"] = sampled_oracle_baseline(rows_fn, w.total_tokens, w.total_tokens,
                                                             args.cpu_seconds, "query rows")
        else:
            gn = g.float().cpu().numpy().astype(np.float64)
            one = np.array([0, w.lengths[0]])
            onec = np.array([0, nc])

            def pool():  # what every oracle call redoes once: K and V pooled
                oracle.mean_pool_varlen(kn, one, onec, 32, 16)
                oracle.mean_pool_varlen(vn, one, onec, 32, 16)

            def rows_fn(rows):
                oracle.nsa_prefill_rows(qn, kn, vn, gn, rows, topk=w.topk, window=w.window)
            result["cpu_baseline"] = sampled_oracle_baseline(rows_fn, w.total_tokens, w.total_tokens,
                                                             args.cpu_seconds, "query rows",
                                                             chunk=32, fixed_fn=pool)
    print(json.dumps(result), flush=True)


def selected_bwd_main(args, dev):
    """Backward of the selected attention over the prefill-selected batch: one
    step = the gradient (dq, dk, dv) of the whole batch from the forward's
    output, log-normaliser and a given upstream gradient; value = prefill tokens/s
    of the backward.  The dq and dk/dv contractions run on the bf16 matrix cores
    (fp32 accumulation), so the roofline is the algorithmic flops of the longer
    of the two kernels against the bf16 matrix-core peak."""
    import numpy as np
    import torch

    import sparse_attention_compress_amd as nsa
    from gen import workloads as W

    stream = torch.cuda.Stream(device=dev)
    steps = args.steps if args.steps != 2800 else 5
    warmup = args.warmup if args.warmup != 280 else 1
    D = 128
    w = W.selected_prefill()
    print(f"[bench] workload {w.name} (backward)", file=sys.stderr, flush=True)
    q = W.prefill_query(w, dev)
    k, v = W.keys_values(w, dev)
    idx = W.given_block_indices(w, dev)
    d_out = W.prefill_out_grad(w, dev)
    cu = nsa.cu_seqlens_of(w.lengths, dev)
    L_max = max(w.lengths)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    nsa.nsa_selected_attn_fwd(q, k, v, idx, cu, L_max, out, lse=lse, cu_seqlens_q=cu)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(nsa.selected_attn_bwd_workspace_size(w.batch, w.total_tokens, L_max, w.heads,
                                                          w.kv_heads, w.topk),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def fn():
        nsa.nsa_selected_attn_bwd(q, k, v, out, d_out, lse, idx, cu, cu, L_max, dq, dk, dv,
                                  workspace=ws)
    kinds = {"lists": nsa.KERNEL_SELECTED_BWD_LISTS, "dq": nsa.KERNEL_SELECTED_BWD_DQ,
             "dkdv": nsa.KERNEL_SELECTED_BWD_DKDV, "dq_sum": nsa.KERNEL_SELECTED_BWD_DQ_SUM}
    ids = idx.cpu().numpy().astype(np.int64).reshape(-1, w.topk)
    pos = np.concatenate([np.arange(L) for L in w.lengths])
    t = np.repeat(pos, w.kv_heads).reshape(-1, 1)
    keys = float(np.where(ids >= 0, np.clip(t - 64 * ids + 1, 0, 64), 0).sum())
    G = w.heads // w.kv_heads
    # per attended (row, head, key): q.k, dO.v and ds.k for dq (3 dot products of
    # D); q.k, dO.v and the dk, dv updates for dk/dv (4)
    flops = {"dq": 6.0 * D * G * keys, "dkdv": 8.0 * D * G * keys}
    wall_s, gpu_ms = _timed(fn, steps, warmup, stream)
    kern = _kernel_us(nsa, fn, kinds, 3, stream)
    dominant = max(flops, key=lambda n: kern[n])
    tflops = {n: flops[n] / (kern[n] * 1e-6) / 1e12 for n in flops}
    ms_per_step = wall_s * 1e3 / steps
    result = {
        "metric": f"prefill backward tokens/s ({w.name})",
        "value": round(w.total_tokens * steps / wall_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V and upstream gradient, uniform causal block "
                "indices; no dataset)",
        "config": {"workload": w.name + "_bwd", "batch": w.batch, "seq_len": L_max,
                   "heads": w.heads, "kv_heads": w.kv_heads, "head_dim": D, "topk": w.topk},
        "roofline": {
            "kernel": dominant,
            "bound": "mfma",
            "achieved": round(tflops[dominant], 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops[dominant] / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": flops[dominant],
            "mean_kernel_us": round(kern[dominant], 1),
        },
        "kernel_us": {n: round(x, 1) for n, x in kern.items()},
        "kernel_tflops": {n: round(x, 2) for n, x in tflops.items()},
        "timed_gpu_ms": round(gpu_ms, 3),
    }
    if not args.no_cpu_baseline:
        import oracle
        scale = 1.0 / math.sqrt(D)
        kn, vn = k.float().cpu().numpy().astype(np.float64), v.float().cpu().numpy().astype(np.float64)
        qn = q.float().cpu().numpy().astype(np.float64)
        don = d_out.float().cpu().numpy().astype(np.float64)
        idn = idx.cpu().numpy()
        L0 = w.lengths[0]
        dk_s = np.zeros((L0,) + kn.shape[1:])
        dv_s = np.zeros((L0,) + vn.shape[1:])

        def rows_fn(rows):  # rows of equal-length sequences, packed
            for r in rows:
                b_, t_ = divmod(r, L0)
                s0 = b_ * L0
                oracle.selected_attention_row_grad(qn[r], kn[s0:s0 + L0], vn[s0:s0 + L0], idn[r],
                                                   t_, 64, scale, don[r], dk_s, dv_s)
        result["cpu_baseline"] = sampled_oracle_baseline(rows_fn, w.total_tokens, w.total_tokens,
                                                         args.cpu_seconds, "query rows")
    print(json.dumps(result), flush=True)


def nsa_bwd_main(args, dev):
    """Backward of the three-branch prefill (65536 tokens, 64 query heads over 4
    KV heads, window 512, top-16): one step = the gate gradients and the
    per-branch output gradients, the selected, window and compressed branches'
    dq, dk, dv (sharing the output arrays) and the window-mean transpose of the
    compressed keys' and values' gradients, from the forward's branch outputs,
    normalisers and block choice (computed once before the timed region).  The
    contractions run on the bf16 matrix cores: roofline = algorithmic flops of
    the longest branch against the bf16 matrix-core peak."""
    import numpy as np
    import torch

    import sparse_attention_compress_amd as nsa
    from gen import workloads as W

    stream = torch.cuda.Stream(device=dev)
    steps = args.steps if args.steps != 2800 else 3
    warmup = args.warmup if args.warmup != 280 else 1
    D = 128
    w = W.nsa_prefill()
    print(f"[bench] workload {w.name} (backward)", file=sys.stderr, flush=True)
    L, H, Hkv = w.lengths[0], w.heads, w.kv_heads
    q = W.prefill_query(w, dev)
    k, v = W.keys_values(w, dev)
    g = W.gates(w, dev)
    d_out = W.prefill_out_grad(w, dev)
    nc = nsa.window_count(L)
    cu = nsa.cu_seqlens_of(w.lengths, dev)
    cuc = nsa.cu_seqlens_of([nc], dev)
    kc = torch.empty((nc, Hkv, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    nsa.nsa_compress_k(k, kc, cu, cuc, nc)
    nsa.nsa_compress_k(v, vc, cu, cuc, nc)
    nb = -(-L // 64)
    o_cmp, o_sel, o_win = (torch.empty_like(q) for _ in range(3))
    lse = [torch.empty((L, H), dtype=torch.float32, device=dev) for _ in range(3)]
    bs = torch.empty((L, Hkv, nb), dtype=torch.float32, device=dev)
    nsa.nsa_compressed_attn_fwd(q, kc, vc, cu, cu, cuc, L, o_cmp, lse=lse[0], block_scores=bs)
    idx = torch.empty((L, Hkv, w.topk), dtype=torch.int32, device=dev)
    nsa.nsa_select_topk(bs, idx, cu, L, w.topk, 0, 0, cu_seqlens_q=cu)
    nsa.nsa_selected_attn_fwd(q, k, v, idx, cu, L, o_sel, lse=lse[1], cu_seqlens_q=cu)
    nsa.nsa_window_attn_fwd(q, k, v, cu, cu, L, o_win, window=w.window, lse=lse[2])
    del bs
    do_b = [torch.empty_like(q) for _ in range(3)]
    d_gates = torch.empty((L, H, 3), dtype=torch.float32, device=dev)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    dkc = torch.empty(kc.shape, dtype=torch.float32, device=dev)
    dvc = torch.empty(vc.shape, dtype=torch.float32, device=dev)
    ws_sel = torch.empty(nsa.selected_attn_bwd_workspace_size(1, L, L, H, Hkv, w.topk),
                         dtype=torch.uint8, device=dev)
    ws_br = torch.empty(nsa.branch_attn_bwd_workspace_size(L, H), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    parts = {
        "gates": lambda: nsa.nsa_gates_bwd(d_out, o_cmp, o_sel, o_win, g, *do_b, d_gates),
        "selected": lambda: nsa.nsa_selected_attn_bwd(q, k, v, o_sel, do_b[1], lse[1], idx, cu, cu,
                                                      L, dq, dk, dv, workspace=ws_sel),
        "window": lambda: nsa.nsa_window_attn_bwd(q, k, v, o_win, do_b[2], lse[2], cu, cu, L, dq,
                                                  dk, dv, window=w.window, accumulate=3,
                                                  workspace=ws_br),
        "compressed": lambda: nsa.nsa_compressed_attn_bwd(q, kc, vc, o_cmp, do_b[0], lse[0], cu,
                                                          cu, cuc, L, dq, dkc, dvc, accumulate=1,
                                                          workspace=ws_br),
        "pool_transpose": lambda: (nsa.nsa_compress_bwd(dkc, dk, cu, cuc, L, accumulate=True),
                                   nsa.nsa_compress_bwd(dvc, dv, cu, cuc, L, accumulate=True)),
    }

    def fn():
        for f in parts.values():
            f()
    wall_s, gpu_ms = _timed(fn, steps, warmup, stream)
    # per-part durations: stream events around each part over one more step
    evs = {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for n in parts}
    with torch.cuda.stream(stream):
        for n, f in parts.items():
            evs[n][0].record(stream)
            f()
            evs[n][1].record(stream)
    torch.cuda.synchronize()
    part_ms = {n: a.elapsed_time(b) for n, (a, b) in evs.items()}
    t = np.arange(L, dtype=np.int64)
    nvis = np.where(t >= 31, np.minimum(nc, (t - 31) // 16 + 1), 0)
    win = np.minimum(t + 1, w.window)
    ids = idx.cpu().numpy().astype(np.int64)
    sel = np.where(ids >= 0, np.clip(t[:, None, None] - 64 * ids + 1, 0, 64), 0).sum()
    G = H // Hkv
    # per attended (row, head, key): 6 * 128 flops in dq and 8 * 128 in dk/dv
    per = 14.0 * D
    flops = {"selected": per * G * float(sel), "window": per * H * float(win.sum()),
             "compressed": per * H * float(nvis.sum())}
    tflops = {n: flops[n] / (part_ms[n] * 1e-3) / 1e12 for n in flops}
    dominant = max(flops, key=lambda n: part_ms[n])
    ms_per_step = wall_s * 1e3 / steps
    result = {
        "metric": f"prefill backward tokens/s ({w.name})",
        "value": round(L * steps / wall_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V and upstream gradient, sigmoid(N(0,1)) gates; "
                "no dataset)",
        "config": {"workload": w.name + "_bwd", "batch": 1, "seq_len": L, "heads": H,
                   "kv_heads": Hkv, "head_dim": D, "topk": w.topk, "window": w.window},
        "roofline": {
            "kernel": f"{dominant} branch (dq and dk/dv kernels)",
            "bound": "mfma",
            "achieved": round(tflops[dominant], 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops[dominant] / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": flops[dominant],
            "mean_kernel_us": round(part_ms[dominant] * 1e3, 1),
        },
        "part_ms": {n: round(x, 3) for n, x in part_ms.items()},
        "part_tflops": {n: round(x, 2) for n, x in tflops.items()},
        "timed_gpu_ms": round(gpu_ms, 3),
    }
    if not args.no_cpu_baseline:
        import oracle
        f64 = lambda x: x.float().cpu().numpy().astype(np.float64)  # noqa: E731
        qn, kn, vn, gn, don = f64(q), f64(k), f64(v), f64(g), f64(d_out)

        one, onec = np.array([0, L]), np.array([0, nc])

        def pool():  # what every oracle call redoes once: K and V pooled (twice) and transposed
            for x in (kn, vn, kn, vn):
                oracle.mean_pool_varlen(x, one, onec, 32, 16)
            z = np.zeros((nc,) + kn.shape[1:])
            oracle.mean_pool_varlen_bwd(z, one, onec, 32, 16, L)
            oracle.mean_pool_varlen_bwd(z, one, onec, 32, 16, L)

        def rows_fn(rows):
            oracle.nsa_prefill_rows_grad(qn, kn, vn, gn, don, rows, topk=w.topk, window=w.window)
        result["cpu_baseline"] = sampled_oracle_baseline(rows_fn, L, L, args.cpu_seconds,
                                                         "query rows", chunk=32, fixed_fn=pool)
    print(json.dumps(result), flush=True)


def cpu_baseline(w, layer, lengths, args):
    """Time the float64 oracle on one core for layer 0 and compare the GPU output."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None

    def f64(t):
        return t.detach().float().cpu().numpy().astype(np.float64)

    q, k, v, cis = f64(layer["q"]), f64(layer["k"]), f64(layer["v"]), f64(layer["cis"])
    cu = oracle.cu_from_lengths(lengths)
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    reps, t_total, res = 0, 0.0, None
    try:
        if ctx:
            ctx.__enter__()
        while reps == 0 or t_total < args.cpu_seconds:
            t0 = time.perf_counter()
            res = oracle.decode_step(q, k, v, cu, kernel=w.kernel, stride=w.stride, block=w.block,
                                     topk=w.topk, n_init=w.n_init, n_local=w.n_local, cis=cis,
                                     cis_select=w.cis_select, cis_values=w.cis_values,
                                     cis_weight=w.cis_weight, n_cand=args.n_cand)
            t_total += time.perf_counter() - t0
            reps += 1
            if reps >= 200:  # bounds the leg if the host is much faster than expected
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    base = {
        "value": round(w.batch * reps / t_total, 3),
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"layer 0 of the same workload, full batch of {w.batch} sequences, "
                  f"{reps} decode step(s), {t_total:.1f} s on one host thread; every oracle "
                  f"step pools the whole K (and CIS) cache into windows, where the GPU step "
                  f"refreshes only the newest window",
        **host_cpu(),
    }
    got_idx = layer["idx"].cpu().numpy()
    got = f64(layer["out"])
    same = 0
    err = 0.0
    G = w.heads // w.kv_heads
    for b in range(w.batch):
        for g in range(w.kv_heads):
            if got_idx[b, g].tolist() == res["indices"][b, g].tolist():
                same += 1
                err = max(err, float(np.abs(got[b, g * G:(g + 1) * G] - res["out"][b, g * G:(g + 1) * G]).max()))
    parity = {"index_sets_identical": f"{same}/{w.batch * w.kv_heads}",
              "max_abs_err_out_on_identical_sets": err}
    return base, parity


if __name__ == "__main__":
    main()
