"""A decode step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library's calls only enqueue kernel launches on the caller's stream (no
memset, no allocation, no synchronisation when out and workspace are given),
so a caller may capture them. Each case captures append + decode once, then
replays the graph several times with eager work and synchronisations between
the replays, and checks every replay against the eager calls on the same
inputs: bitwise where the schedule is deterministic (fixed partitions),
within fp32 rounding of the merge order on the balanced schedule, within the
parity tolerance of the oracle for the general call.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import transformer_decode_attention_amd as mqa
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


def capture(fn):
    """Capture fn() into a graph after one eager run on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_check(g, out, check, eager_between):
    for k in range(REPLAYS):
        out.fill_(float("nan"))       # eager work between the replays
        eager_between()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(out, k)


@pytest.mark.parametrize("chunk", [256, 0])
def test_graph_replays_match_eager(chunk):
    """gqa-70b shape (16 sequences): fixed partitions (bitwise) and the
    balanced schedule (its last bits depend on which wave takes which step)."""
    w = W.shrink(W.WORKLOADS["gqa-70b"], b=16) if chunk else W.WORKLOADS["gqa-70b"]
    print(f"[graph] {w.name} b={w.b} chunk={chunk}", flush=True)
    t = W.make_step(w, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = mqa.decode_workspace(w.b, w.h, w.g, w.S, w.d, w.dtype, DEV, chunk)
    out = torch.empty((w.b, w.h, w.d), dtype=torch.float32, device=DEV)
    other = torch.empty_like(out)

    def step(o=out):
        mqa.append_kv(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["seq_lens"],
                      err_flags=err)
        mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], out=o, workspace=ws,
                        split_chunk=chunk, err_flags=err)

    step(other)  # eager reference (the append is idempotent: the same row each time)
    torch.cuda.synchronize()
    ref = other.clone()
    g = capture(step)

    def check(o, k):
        if chunk:
            assert torch.equal(o, ref), f"replay {k}"
        else:
            assert (o - ref).abs().max().item() <= 1e-5, f"replay {k}"

    replay_and_check(g, out, check, lambda: step(other))
    assert int(err.item()) == 0


def test_graph_general_call():
    """mqa_decode_attn_ex in a graph: four tokens, a sliding window, a paged
    fp8 cache; every replay against the oracle."""
    w = W.Workload("graph-ex", b=32, h=32, g=4, d=128, S=600, dtype=torch.bfloat16, seed=970,
                   L_lo=1, L_hi=600)
    T, P, window = 4, 16, 200
    print(f"[graph] {w.name} T={T} P={P} W={window} fp8", flush=True)
    t = W.make_fp8_step(w, DEV, T=T, page_size=P)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kw = dict(block_table=t["block_table"], k_scale=t["k_scale"], v_scale=t["v_scale"],
              window=window)
    ws = torch.empty(mqa.decode_ex_workspace_bytes(t["q"], t["k_pages"], t["v_pages"],
                                                   t["seq_lens"], **kw),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((w.b, T, w.h, w.d), dtype=torch.float32, device=DEV)

    def step():
        mqa.append_kv_paged_fp8(t["k_pages"], t["v_pages"], t["k_new"], t["v_new"], t["k_scale"],
                                t["v_scale"], t["block_table"], t["seq_lens"], err_flags=err)
        mqa.decode_attn_ex(t["q"], t["k_pages"], t["v_pages"], t["seq_lens"], out=out,
                           workspace=ws, err_flags=err, **kw)

    step()
    torch.cuda.synchronize()
    ref, rc = oracle.decode_attn_ex(
        W.to_oracle(t["q"]), t["k_pages"].cpu().numpy(), t["v_pages"].cpu().numpy(),
        t["seq_lens"].cpu().numpy(), float(np.float32(1.0 / math.sqrt(w.d))), window=window,
        k_scale=t["k_scale"].cpu().numpy(), v_scale=t["v_scale"].cpu().numpy(),
        block_table=t["block_table"].cpu().numpy(), nthreads=16)
    assert rc == oracle.OK
    g = capture(step)

    def check(o, k):
        got = o.cpu().double().numpy()
        err_ = np.abs(got - ref)
        rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
        assert np.isfinite(got).all(), f"replay {k}"
        assert err_.max() <= 2e-3 and (err_ / np.maximum(np.abs(ref), rms)).max() <= 2e-3, \
            f"replay {k}"

    scratch = torch.empty_like(out)
    replay_and_check(g, out, check,
                     lambda: mqa.decode_attn_ex(t["q"], t["k_pages"], t["v_pages"], t["seq_lens"],
                                                out=scratch, workspace=ws, **kw))
    assert int(err.item()) == 0
