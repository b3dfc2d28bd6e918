#!/usr/bin/env python3
"""Decode-attention bench on one MI355X.

One step = the whole hot path for one batch: mqa_append_kv then
mqa_decode_attn for every layer of the workload, inputs resident in HBM.
Default workload: gqa-70b (b=64, h=64, g=8, d=128, bf16 cache of capacity
4096, ragged lengths U[1024, 4096], seeded N(0,1) values).

Prints one JSON line:
  value        achieved HBM GB/s of the step (algorithmic bytes / step time)
  ms_per_step  step time (µs/step = 1000 * ms_per_step, also in "us_per_step"):
               the --steps timed steps back to back, / steps; "trials" cuts the
               same steps into --trials consecutive trials (events between them)
               and gives their median and spread
  roofline     for the dominant kernel launch (mqa_decode_attn), timed with
               HIP events on the stream the kernels run on (a second pass over
               the same steps, each behind a spin kernel so that the events
               time the kernels and not Python's issue of the calls)
  cpu_baseline the CPU oracle, timed on the host's cores on a bounded sample
               (and on one thread, for scale): as many threads as the host grants
               this process (OMP_NUM_THREADS if set, else every CPU of the
               affinity mask; --cpu-threads overrides), with the rule, nproc,
               the affinity count and the CPU model string recorded
  graph        the same steps captured once in a HIP graph and replayed: the
               step time without Python's issue of the calls (context; the
               small configurations are bound by that issue time when eager)
  hbm_copy_gbs a plain 1 GiB device-to-device copy (read + write bytes / time):
               what a simple streaming kernel attains on this part (context)
  launch_us    time per launch of a chain of 200 empty kernels on the stream,
               issued eagerly from Python and replayed from a HIP graph (the
               floors under any one-kernel call; context)

Algorithmic bytes per decode launch and layer: the K and V rows attended
(sum_i 2*g*L_i*d*B) + q (b*h*d*B) + out (b*h*d*4). The append adds
2*b*g*d*B read and the same written. Bytes the method avoids (the h/g times
larger MHA cache) are not counted.

With --page-size P the cache is paged (pages of P rows in a shuffled pool,
one int32 block table per batch): mqa_append_kv_paged + mqa_decode_attn_paged,
whose algorithmic bytes add the block-table entries read (sum_i ceil(L_i/P)*4,
and 4*b for the append).

With --tokens T each sequence brings T query tokens per step (a draft of T
tokens verified at once, causal mask): mqa_append_kv_multi + mqa_decode_attn_multi
(or their paged forms); q and out are T times larger, the K/V bytes the same.

With --kv-dtype fp8 the cache holds fp8 e4m3 codes with per-K/V-head scales
(mqa_append_kv_fp8 quantises the new rows, mqa_decode_attn_fp8 reads one byte
per element): the K/V bytes per position halve; q stays bf16. --kv-dtype int8
does the same with int8 codes (mqa_append_kv_int8, decode through
mqa_decode_attn_ex).

With --window W the decode is mqa_decode_attn_ex with a sliding window of W
positions: a query at position p reads only (p - W, p], so the K/V bytes count
the L - max(0, L - T + 1 - W) positions the step's tokens see.

With --rope the append is mqa_rope_q + mqa_append_kv_rope (query and new key
rows rotated at their positions from a cos/sin table built once by the caller,
contiguous bf16 cache); the rotation adds q read and written
(2*b*T*h*d*B) and the table rows read (2*b*T*(d/2)*8) to the step's bytes.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--page-size P]
                       [--tokens T] [--kv-dtype bf16|fp8|int8] [--window W] [--rope]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s
SRC = os.path.join(ROOT, "transformer_decode_attention_amd", "csrc", "mqa_decode.hip")
HEADER = os.path.join(ROOT, "include", "mqa_decode.h")  # included by SRC: its constants build into the kernels


def code_text(src: str) -> str:
    """C++ source without its comments: // and /* */ comments outside string
    and character literals removed, trailing blanks cut, empty lines dropped.
    What the compiler turns into code is left as it is, so editing, adding or
    removing a comment leaves this text unchanged and any other edit does not."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":  # a literal, up to its unescaped closing quote
            j = i + 1
            while j < n and src[j] != c and src[j] != "\n":
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def source_sha() -> str:
    """Hash of what the library is built from: the code of the kernel source
    and of the C header it includes (comments left out, since they build to
    nothing) and the compiler flags. A traffic record taken on another build
    is not reported."""
    from transformer_decode_attention_amd import build
    h = hashlib.sha256()
    for path in (SRC, HEADER):
        h.update(code_text(open(path, encoding="utf-8").read()).encode())
        h.update(b"\0")
    h.update(" ".join(build.FLAGS).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa-70b")
    ap.add_argument("--split-chunk", type=int, default=0)
    ap.add_argument("--kernel", choices=["auto", "valu", "mfma", "deterministic"], default="auto",
                    help="partition kernel (auto: mqa_decode_attn's own choice; deterministic: "
                         "matrix cores, bitwise-reproducible balanced schedule)")
    ap.add_argument("--trials", type=int, default=5,
                    help="the timed steps are cut into this many trials (median and spread reported)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the CPU-oracle baseline (0: the host's CPU share: "
                         "OMP_NUM_THREADS if set, else every core the process may run on)")
    ap.add_argument("--replicas", type=int, default=0,
                    help="distinct cache copies rotated across steps (0: enough for >= 2 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="wall-clock budget of the CPU-oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--page-size", type=int, default=0,
                    help="paged KV cache with pages of this many rows (0: contiguous cache)")
    ap.add_argument("--tokens", type=int, default=1,
                    help="query tokens per sequence per step (causal; 1: plain decode)")
    ap.add_argument("--kv-dtype", choices=["bf16", "fp8", "int8"], default="bf16",
                    help="cache element type (fp8: e4m3 codes with per-K/V-head scales)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window of this many positions (mqa_decode_attn_ex); 0: none")
    ap.add_argument("--rope", action="store_true",
                    help="rotate q and the new keys at their positions before the append")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay timing")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    return ap.parse_args()


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library runs on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import transformer_decode_attention_amd as mqa
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[args.workload]
    layers = w.layers
    cache_bytes = 2 * w.b * w.g * w.S * w.d * w.elem_bytes  # K + V capacity, one layer
    if layers > 1:
        reps = layers  # every layer has its own cache
    else:
        reps = args.replicas or max(2, math.ceil((2 << 30) / cache_bytes))
    print(f"[bench] workload {w.name}: b={w.b} h={w.h} g={w.g} d={w.d} S={w.S} layers={layers} "
          f"copies={reps} ({reps * cache_bytes / 2**30:.2f} GiB of cache)", file=sys.stderr, flush=True)

    P = args.page_size
    T = args.tokens
    F8 = args.kv_dtype in ("fp8", "int8")  # one-byte codes with per-K/V-head scales
    I8 = args.kv_dtype == "int8"
    if (P or T > 1 or F8) and args.kernel == "valu":
        print("paged, multi-token and fp8 calls run the matrix-core kernels only", file=sys.stderr)
        return 2
    if F8 and w.dtype != torch.bfloat16:
        print("an fp8 cache takes bf16 queries: pick a bf16 workload", file=sys.stderr)
        return 2
    WIN = args.window
    ROPE = args.rope
    if WIN < 0:
        print("--window takes a positive size (0: none)", file=sys.stderr)
        return 2
    if (WIN or ROPE) and args.kernel == "valu":
        print("the window and rotation calls run the matrix-core kernels only", file=sys.stderr)
        return 2
    if ROPE and (P or F8 or w.dtype != torch.bfloat16):
        print("--rope rotates rows of a contiguous bf16 cache", file=sys.stderr)
        return 2
    steps_in = []
    for r in range(reps):
        if F8:
            t = W.make_fp8_step(w, dev, T=T, layer=r, page_size=P, int8=I8)
        elif T > 1:
            t = W.make_multi_step(w, dev, T=T, layer=r, page_size=P)
        elif P:
            t = W.make_paged_step(w, dev, page_size=P, layer=r)
        else:
            t = W.make_step(w, dev, layer=r)
        if P and "k_cache" in t:
            del t["k_cache"], t["v_cache"]  # the pages hold the cache
        steps_in.append(t)
    cap = steps_in[0]["capacity"] if P else w.S
    t0 = steps_in[0]
    if WIN or I8:
        kk, vv = ("k_pages", "v_pages") if P else ("k_cache", "v_cache")
        nws = mqa.decode_ex_workspace_bytes(t0["q"], t0[kk], t0[vv], t0["seq_lens"],
                                            block_table=t0.get("block_table") if P else None,
                                            k_scale=t0.get("k_scale"), v_scale=t0.get("v_scale"),
                                            window=WIN, split_chunk=args.split_chunk)
    else:
        nws = mqa.decode_multi_workspace_bytes(w.b, T, w.h, w.g, cap, w.d, w.dtype,
                                               args.split_chunk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    cos_sin = None
    if ROPE:
        # the caller's table: angle pos * 10000^(-2i/d), fp32, [S][d/2][2]
        inv = np.power(10000.0, -2.0 * np.arange(w.d // 2, dtype=np.float64) / w.d)
        ang = np.arange(w.S, dtype=np.float64)[:, None] * inv[None, :]
        cos_sin = torch.from_numpy(np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)).to(dev)
    lens = steps_in[0]["seq_lens"].cpu().numpy().astype(np.int64)
    chunk = mqa.decode_resolve_chunk(w.b, w.h, w.g, cap, w.d, w.dtype, args.split_chunk)
    oshape = (w.b, T, w.h, w.d) if T > 1 else (w.b, w.h, w.d)
    outs = [torch.empty(oshape, dtype=torch.float32, device=dev) for _ in range(reps)]
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    kernel = {"auto": mqa.KERNEL_AUTO, "valu": mqa.KERNEL_VALU, "mfma": mqa.KERNEL_MFMA,
              "deterministic": mqa.KERNEL_MFMA_DETERMINISTIC}[args.kernel]
    if T > 1:
        schedule = mqa.decode_multi_schedule(w.b, T, w.h, w.g, cap, w.d, w.dtype, args.split_chunk)
    else:
        schedule = mqa.decode_schedule(w.b, w.h, w.g, cap, w.d, w.dtype, args.split_chunk, kernel)
    B = w.elem_bytes
    KB = 1 if F8 else B  # bytes per cached element
    # positions the step's tokens see: all L, or the window's (L - T + 1 - W, L)
    seen = [int(L) - (max(0, int(L) - T + 1 - WIN) if WIN else 0) for L in lens]
    kv_read = int(sum(2 * w.g * n * w.d * KB for n in seen))
    dec_bytes = kv_read + w.b * T * w.h * w.d * B + w.b * T * w.h * w.d * 4
    app_bytes = 2 * (w.b * T * w.g * w.d * (B + KB))  # new rows read, codes or rows written
    if F8:
        dec_bytes += 2 * w.g * 4  # the scales
        app_bytes += 2 * w.g * 4
    if P:
        first = [(max(0, int(L) - T + 1 - WIN) // P if WIN else 0) for L in lens]
        dec_bytes += 4 * int(sum(-(-int(L) // P) - f for L, f in zip(lens, first)))
        app_bytes += 4 * w.b * T
    if ROPE:
        app_bytes += 2 * w.b * T * w.h * w.d * B + 2 * w.b * T * (w.d // 2) * 8
    per_layer = dec_bytes + app_bytes
    step_bytes = per_layer * layers
    # token tau of a sequence of length L attends L - T + 1 + tau positions (at most W)
    def attended(L):
        n = [L - T + 1 + tau for tau in range(T)]
        return sum(min(x, WIN) if WIN else x for x in n)
    flops_per_step = 4 * w.h * w.d * layers * int(sum(attended(int(L)) for L in lens))

    def layer_call(r, ev=None):
        t = steps_in[r]
        kw = dict(out=outs[r], workspace=ws, split_chunk=args.split_chunk, err_flags=err)
        if F8:
            sc = (t["k_scale"], t["v_scale"])
            if P:
                append = mqa.append_kv_paged_int8 if I8 else mqa.append_kv_paged_fp8
                append(t["k_pages"], t["v_pages"], t["k_new"], t["v_new"], *sc, t["block_table"],
                       t["seq_lens"], err_flags=err)
            else:
                append = mqa.append_kv_int8 if I8 else mqa.append_kv_fp8
                append(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], *sc, t["seq_lens"],
                       err_flags=err)
        elif P:
            pages = (t["k_pages"], t["v_pages"])
            append = mqa.append_kv_paged_multi if T > 1 else mqa.append_kv_paged
            append(*pages, t["k_new"], t["v_new"], t["block_table"], t["seq_lens"], err_flags=err)
        elif ROPE:
            mqa.rope_q(t["q"], cos_sin, t["seq_lens"], err_flags=err)
            mqa.append_kv_rope(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], cos_sin,
                               t["seq_lens"], err_flags=err)
        else:
            append = mqa.append_kv_multi if T > 1 else mqa.append_kv
            append(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["seq_lens"], err_flags=err)
        if ev is not None:
            ev[0].record()
        if WIN or I8:
            kk, vv = ("k_pages", "v_pages") if P else ("k_cache", "v_cache")
            mqa.decode_attn_ex(t["q"], t[kk], t[vv], t["seq_lens"],
                               block_table=t.get("block_table") if P else None,
                               k_scale=t.get("k_scale"), v_scale=t.get("v_scale"), window=WIN, **kw)
        elif F8 and P:
            mqa.decode_attn_paged_fp8(t["q"], t["k_pages"], t["v_pages"], *sc, t["block_table"],
                                      t["seq_lens"], **kw)
        elif F8:
            mqa.decode_attn_fp8(t["q"], t["k_cache"], t["v_cache"], *sc, t["seq_lens"], **kw)
        elif P:
            decode = mqa.decode_attn_paged_multi if T > 1 else mqa.decode_attn_paged
            decode(t["q"], *pages, t["block_table"], t["seq_lens"], **kw)
        elif T > 1:
            mqa.decode_attn_multi(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], **kw)
        else:
            mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], kernel=kernel, **kw)
        if ev is not None:
            ev[1].record()

    def step(k, evs=None):
        if layers > 1:
            for l in range(layers):
                layer_call(l, None if evs is None else evs[l])
        else:
            layer_call(k % reps, None if evs is None else evs[0])

    # warmup
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, "device reported an error during warmup"

    # timed region: the step alone, exactly args.steps steps, with events at
    # the boundaries of `trials` consecutive trials (recorded on the stream,
    # so the steps run back to back as in one pass)
    ntr = max(1, min(args.trials, args.steps))
    bounds = [round(i * args.steps / ntr) for i in range(ntr + 1)]
    tev = [torch.cuda.Event(enable_timing=True) for _ in range(ntr + 1)]
    torch.cuda.synchronize()
    tev[0].record()
    for i in range(ntr):
        for k in range(bounds[i], bounds[i + 1]):
            step(k)
        tev[i + 1].record()
    torch.cuda.synchronize()
    ms_per_step = tev[0].elapsed_time(tev[-1]) / args.steps
    trial_ms = [tev[i].elapsed_time(tev[i + 1]) / (bounds[i + 1] - bounds[i]) for i in range(ntr)]

    # timed region again, with HIP events around every decode launch (same
    # stream). A spin kernel queued ahead of each step keeps the GPU busy while
    # Python issues the step's calls, so each event pair brackets the decode
    # kernels alone and not the host's issue time (which small launches would
    # otherwise show).
    spin = spin_cycles(torch, 40e-3 * max(1, layers))
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(layers)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        if spin:
            torch.cuda._sleep(spin)
        step(k, ev[k])
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for evk in ev for (a, b) in evk]
    dec_ms_avg = float(np.mean(dec_ms))
    assert int(err.item()) == 0, "device reported an error"

    graph = None if args.no_graph else graph_timing(torch, step, layers, reps, args.steps)
    assert int(err.item()) == 0, "device reported an error in the graph replays"
    hbm_copy = copy_gbs(torch, dev)
    launch_us = empty_launch_us(torch)

    if args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = dec_bytes / (dec_ms_avg * 1e-3) / 1e9
    traffic = None
    tag = (w.name + (f"-paged{P}" if P else "") + (f"-t{T}" if T > 1 else "")
           + (("-int8" if I8 else "-fp8") if F8 else "")
           + (f"-w{WIN}" if WIN else "") + ("-rope" if ROPE else ""))
    tf = os.path.join(ROOT, "profiles", f"decode_{tag}_traffic.json")
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if (rec.get("source_sha") == source_sha() and rec.get("split_chunk", 0) == args.split_chunk
                and args.kernel == "auto"):
            traffic = rec.get("bytes_per_launch")

    result = {
        "metric": "decode-attn µs/step + achieved HBM GB/s (% peak), bf16 b=64 h=64 g=8 ctx 4096",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "trials": {"n": ntr, "steps_each": [bounds[i + 1] - bounds[i] for i in range(ntr)],
                   "median_us_per_step": round(float(np.median(trial_ms)) * 1e3, 3),
                   "min_us_per_step": round(min(trial_ms) * 1e3, 3),
                   "max_us_per_step": round(max(trial_ms) * 1e3, 3)},
        "pct_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic: seeded N(0,1) q/K/V in HBM, no trained weights",
        "config": {"workload": w.name, "b": w.b, "h": w.h, "g": w.g, "d_h": w.d, "capacity": w.S,
                   "seq_lens": "fixed %d" % w.L if w.L else f"U[{w.L_lo},{w.L_hi}] (sum {int(lens.sum())})",
                   "layers": layers, "schedule": schedule,
                   "kv_layout": f"paged, {P}-row pages" if P else "contiguous",
                   "query_tokens": T,
                   "kv_dtype": ("int8" if I8 else "fp8 e4m3") + ", per-K/V-head scales" if F8 else "bf16",
                   "window": WIN or None, "rope_on_append": ROPE,
                   "split_chunk": chunk if schedule != "mfma-balanced" else None,
                   "cache_copies_rotated": reps,
                   "accumulate": "fp32", "out": "fp32"},
        "algorithmic_bytes_per_step": step_bytes,
        "flops_per_step": flops_per_step,
        "roofline": {
            "bound": "hbm",
            "kernel": ("mqa_decode_attn_ex" + (" (window)" if WIN else "") + (" (int8)" if I8 else "")
                       if WIN or I8 else
                       ("mqa_decode_attn" + ("_paged" if P else "")
                        + ("_fp8" if F8 else "_multi" if T > 1 else "")))
                      + " launch, schedule " + schedule,
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": dec_bytes,
            "us_per_launch": round(dec_ms_avg * 1e3, 3),
            "us_per_launch_median": round(float(np.median(dec_ms)) * 1e3, 3),
            "us_per_launch_min": round(min(dec_ms) * 1e3, 3),
            "us_per_launch_max": round(max(dec_ms) * 1e3, 3),
            "launches_timed": len(dec_ms),
        },
        "cpu_baseline": None,
        "graph": graph,
        "hbm_copy_gbs": hbm_copy,
        "launch_us": launch_us,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, steps_in[0], lens, per_layer, layers,
                                              args.cpu_seconds, P, T, F8, WIN, I8,
                                              args.cpu_threads)

    print(json.dumps(result), flush=True)
    return 0


def graph_timing(torch, step, layers, reps, steps):
    """Capture a whole number of steps (one per cache copy, or one step of
    every layer) in a HIP graph and time its replays; None if capture fails."""
    per = 1 if layers > 1 else reps
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for k in range(per):
                step(k)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(per):
                step(k)
        g.replay()
        torch.cuda.synchronize()
        n = max(1, steps // per)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / (n * per)
        return {"ms_per_step": round(ms, 6), "us_per_step": round(ms * 1e3, 3),
                "steps": n * per, "steps_per_graph": per}
    except RuntimeError as e:  # report, do not fail the bench line
        return {"error": str(e)[:200]}


def copy_gbs(torch, dev) -> float:
    """Read + write bytes per second of a 1 GiB device copy (best of 5)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del src, dst
    return round(2 * n / (best * 1e-3) / 1e9, 1)


def empty_launch_us(torch, n: int = 200):
    """µs per launch of n back-to-back empty kernels (torch.cuda._sleep(0)),
    issued eagerly and replayed from a graph; None where unavailable."""
    if not hasattr(torch.cuda, "_sleep"):
        return None

    def chain():
        for _ in range(n):
            torch.cuda._sleep(0)

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return round(a.elapsed_time(b) * 1e3 / n, 3)

    chain()
    res = {"eager": timed(chain)}
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            chain()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            chain()
        g.replay()
        res["graph"] = timed(g.replay)
    except RuntimeError:
        res["graph"] = None
    return res


def cpu_info() -> dict:
    """The host's CPU as /proc/cpuinfo and the OS describe it: model name(s)
    (the full strings), logical CPUs, sockets, and how many of the CPUs this
    process may run on."""
    models, sockets = [], set()
    try:
        for line in open("/proc/cpuinfo"):
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "model name" and val not in models:
                models.append(val)
            elif key == "physical id":
                sockets.add(val)
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    return {"model": "; ".join(models) or "unknown", "nproc": os.cpu_count(),
            "sockets": len(sockets) or None, "affinity": affinity}


def cpu_threads(requested: int) -> tuple[int, str]:
    """Threads for the CPU baseline and the rule that chose them."""
    if requested > 0:
        return requested, "--cpu-threads"
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        return int(omp), "OMP_NUM_THREADS (the host's CPU share for this process)"
    return cpu_info()["affinity"], "every CPU in the process's affinity mask"


def spin_cycles(torch, ms: float) -> int:
    """Argument of torch.cuda._sleep that keeps the GPU busy for about `ms`
    milliseconds (calibrated with events; 0 where the call is unavailable)."""
    if not hasattr(torch.cuda, "_sleep"):
        return 0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 1 << 20
    torch.cuda._sleep(n)  # first launch
    a.record()
    torch.cuda._sleep(n)
    b.record()
    torch.cuda.synchronize()
    per_ms = n / max(a.elapsed_time(b), 1e-3)
    return int(min(per_ms * ms, 1 << 40))


def cpu_baseline(w, t, lens, per_layer_bytes, layers, budget_s, page_size=0, T=1, F8=False,
                 window=0, I8=False, requested_threads=0):
    """The oracle (plain double loops) on the host cores, one layer's step."""
    import numpy as np

    import oracle
    import workloads as W

    nthreads, rule = cpu_threads(requested_threads)
    threads = [nthreads]  # the thread count run() uses (changed for the one-thread pass)
    scale = float(np.float32(1.0 / math.sqrt(w.d)))
    lens32 = lens.astype(np.int32)
    q = W.to_oracle(t["q"])
    if window or I8:  # the general call (an int8 cache is read through it)
        kk, vv = ("k_pages", "v_pages") if page_size else ("k_cache", "v_cache")
        conv = (lambda x: x.cpu().numpy()) if F8 else W.to_oracle
        kx, vx = conv(t[kk]), conv(t[vv])
        ks = t["k_scale"].cpu().numpy() if F8 else None
        vs = t["v_scale"].cpu().numpy() if F8 else None
        bt = t["block_table"].cpu().numpy() if page_size else None

        def run(n):
            kn, vn = (kx, vx) if page_size else (kx[:n].copy(), vx[:n].copy())
            oracle.decode_attn_ex(q[:n].copy(), kn, vn, lens32[:n], scale, window=window,
                                  k_scale=ks, v_scale=vs,
                                  block_table=None if bt is None else bt[:n].copy(),
                                  nthreads=threads[0])
    elif F8:
        ks, vs = t["k_scale"].cpu().numpy(), t["v_scale"].cpu().numpy()
        if page_size:
            kp, vp = t["k_pages"].cpu().numpy(), t["v_pages"].cpu().numpy()
            bt = t["block_table"].cpu().numpy()

            def run(n):
                oracle.decode_attn_paged_fp8(q[:n].copy(), kp, vp, ks, vs, bt[:n].copy(),
                                             lens32[:n], scale, nthreads=threads[0])
        else:
            kc, vc = t["k_cache"].cpu().numpy(), t["v_cache"].cpu().numpy()

            def run(n):
                oracle.decode_attn_fp8(q[:n].copy(), kc[:n].copy(), vc[:n].copy(), ks, vs,
                                       lens32[:n], scale, nthreads=threads[0])
    elif page_size:
        kp, vp = W.to_oracle(t["k_pages"]), W.to_oracle(t["v_pages"])
        bt = t["block_table"].cpu().numpy()
        paged = oracle.decode_attn_paged_multi if T > 1 else oracle.decode_attn_paged

        def run(n):
            paged(q[:n].copy(), kp, vp, bt[:n].copy(), lens32[:n], scale, nthreads=threads[0])
    else:
        kc, vc = W.to_oracle(t["k_cache"]), W.to_oracle(t["v_cache"])
        flat = oracle.decode_attn_multi if T > 1 else oracle.decode_attn

        def run(n):
            flat(q[:n].copy(), kc[:n].copy(), vc[:n].copy(), lens32[:n], scale, nthreads=threads[0])
    # bounded sample: the first sequences of the batch, sized to the budget
    # from a one-sequence probe
    seen = np.array([int(L) - (max(0, int(L) - T + 1 - window) if window else 0) for L in lens32])
    t0 = time.perf_counter()
    run(1)
    one = max(time.perf_counter() - t0, 1e-4) / max(int(seen[0]), 1)  # s per position seen
    nb = 1
    while nb < w.b and one * int(seen[:nb + 1].sum()) * 1.0 <= budget_s:
        nb += 1
    # a sample shorter than the budget is repeated (a steadier figure)
    t0 = time.perf_counter()
    run(nb)
    dt = time.perf_counter() - t0
    reps = max(1, min(50, int(budget_s / max(dt, 1e-3))))
    if reps > 1:
        t0 = time.perf_counter()
        for _ in range(reps):
            run(nb)
        dt = (time.perf_counter() - t0) / reps
    B = w.elem_bytes
    KB = 1 if F8 else B
    sample_bytes = int(sum(2 * w.g * int(n) * w.d * KB for n in seen[:nb])) + nb * T * w.h * w.d * (B + 4)
    gbs = sample_bytes / dt / 1e9
    # one thread, on the first sequence alone (bounded the same way)
    threads[0] = 1
    t0 = time.perf_counter()
    run(1)
    dt1 = time.perf_counter() - t0
    one_bytes = 2 * w.g * int(seen[0]) * w.d * KB + T * w.h * w.d * (B + 4)
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": f"decode attention of the first {nb} of {w.b} sequences of one layer "
                  f"({int(seen[:nb].sum())} positions seen), {dt:.2f} s wall per pass"
                  + (f", mean of {reps} passes" if reps > 1 else ""),
        "est_ms_per_step": round(1e3 * (per_layer_bytes * layers) / (gbs * 1e9), 3),
        "one_thread_gbs": round(one_bytes / dt1 / 1e9, 4),
        "threads": nthreads,
        "threads_rule": rule,
        "cpu": cpu_info(),
    }


if __name__ == "__main__":
    sys.exit(main())
