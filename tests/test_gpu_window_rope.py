"""Parity of the sliding window (mqa_decode_attn_ex) and of the rotary
embedding calls (mqa_rope_q, mqa_append_kv_rope) against the CPU oracle.

Window: each case runs the general call on the GPU and oracle.decode_attn_ex
on the bytes read back, tolerance as everywhere (|gpu - ref| <= 2e-3 and
|gpu - ref| / max(|ref|, rms(ref row)) <= 2e-3). Rotation: the rotated rows
are bf16 values decided in fp32 by the same specified operations on both
sides, so they must be bit-exact. The cos/sin table is an input of the calls
(built by the caller); the tests build it with oracle.rope_table.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
import transformer_decode_attention_amd as mqa
import workloads as W

pytestmark = pytest.mark.gpu

ATOL = 2e-3
RTOL_ROW = 2e-3
NTHREADS = min(16, os.cpu_count() or 1)
DEV = "cuda:0"


def compare(out_gpu: torch.Tensor, ref: np.ndarray, what: str = "") -> None:
    got = out_gpu.detach().cpu().double().numpy()
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
    rel = err / np.maximum(np.abs(ref), rms)
    assert err.max() <= ATOL and rel.max() <= RTOL_ROW, f"{what}: abs {err.max()} rel {rel.max()}"


def wl(name, b, h, g, d, S, lo, hi, seed):
    return W.Workload(name, b=b, h=h, g=g, d=d, S=S, dtype=torch.bfloat16, seed=seed, L_lo=lo,
                      L_hi=hi)


def run_window(w, window, T=1, page_size=0, fp8=False, split_chunk=0):
    print(f"[window] {w.name} b={w.b} T={T} h={w.h} g={w.g} d={w.d} S={w.S} W={window} "
          f"P={page_size} fp8={fp8} chunk={split_chunk}", flush=True)
    if fp8:
        t = W.make_fp8_step(w, DEV, T=T, page_size=page_size)
    elif page_size:
        t = W.make_multi_step(w, DEV, T=T, page_size=page_size)
    else:
        t = W.make_multi_step(w, DEV, T=T) if T > 1 else W.make_step(w, DEV)
    kk, vv = ("k_pages", "v_pages") if page_size else ("k_cache", "v_cache")
    bt = t.get("block_table") if page_size else None
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ks, vs = (t["k_scale"], t["v_scale"]) if fp8 else (None, None)
    out = mqa.decode_attn_ex(t["q"], t[kk], t[vv], t["seq_lens"], block_table=bt, k_scale=ks,
                             v_scale=vs, window=window, split_chunk=split_chunk, err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    to_np = (lambda x: x.cpu().numpy()) if fp8 else W.to_oracle
    ref, rc = oracle.decode_attn_ex(
        W.to_oracle(t["q"]), to_np(t[kk]), to_np(t[vv]), t["seq_lens"].cpu().numpy(),
        float(np.float32(1.0 / math.sqrt(w.d))), window=window,
        k_scale=None if ks is None else ks.cpu().numpy(),
        v_scale=None if vs is None else vs.cpu().numpy(),
        block_table=None if bt is None else bt.cpu().numpy(), nthreads=NTHREADS)
    assert rc == oracle.OK
    compare(out, ref, f"{w.name} window {window}")


@pytest.mark.parametrize("window", [1, 37, 256, 5000])
def test_window_balanced(window):
    run_window(wl("win-bal", 64, 64, 8, 128, 1024, 1, 1024, 900 + window), window)


@pytest.mark.parametrize("window,T", [(100, 3), (33, 8)])
def test_window_several_tokens(window, T):
    run_window(wl("win-multi", 64, 32, 4, 128, 700, 1, 700, 910 + window), window, T=T)


@pytest.mark.parametrize("chunk", [0, 64])
def test_window_partitions(chunk):
    """Few units (fixed partitions): the partitions are counted from the
    window's first step, so they cover only what the window leaves."""
    run_window(wl("win-part", 4, 32, 1, 128, 3000, 1500, 3000, 920 + chunk), 300,
               split_chunk=chunk)


@pytest.mark.parametrize("window,T,chunk", [(77, 4, 0), (77, 4, 64), (1000, 2, 0), (5, 1, 0)])
def test_window_partitions_long_context(window, T, chunk):
    """MQA at long context, a window far shorter than the sequences (which
    start anywhere relative to the 32-position steps), several tokens."""
    run_window(wl("win-part-long", 3, 32, 1, 128, 9000, 1, 9000, 925 + window + T), window, T=T,
               split_chunk=chunk)


def test_window_paged_and_fp8():
    run_window(wl("win-paged", 64, 32, 4, 128, 800, 1, 800, 930), 200, page_size=16)
    run_window(wl("win-fp8", 64, 64, 8, 128, 1024, 1, 1024, 931), 300, fp8=True)
    run_window(wl("win-fp8-paged", 32, 32, 4, 64, 600, 1, 600, 932), 50, T=2, page_size=32,
               fp8=True)


def test_decode_ex_without_options_equals_the_plain_call():
    w = wl("ex-plain", 64, 64, 8, 128, 1024, 1, 1024, 940)
    t = W.make_step(w, DEV)
    a = mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], split_chunk=256)
    b = mqa.decode_attn_ex(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], split_chunk=256)
    torch.cuda.synchronize()
    assert torch.equal(a, b)  # the same kernels, fixed partitions: bitwise


@pytest.mark.parametrize("b,T,h,g,S,d", [(16, 3, 16, 4, 256, 128), (8, 1, 8, 8, 200, 64),
                                         (4, 5, 32, 1, 300, 64)])
def test_rope_q_and_append_bit_exact(b, T, h, g, S, d):
    print(f"[rope] b={b} T={T} h={h} g={g} S={S} d={d}", flush=True)
    cs = oracle.rope_table(10000.0, S, d)
    w = wl("rope", b, h, g, d, S, T, S, 950 + d + T)
    t = W.make_multi_step(w, DEV, T=T)
    lens = t["seq_lens"].cpu().numpy()
    q0 = W.to_oracle(t["q"])
    kc0, vc0 = W.to_oracle(t["k_cache"]), W.to_oracle(t["v_cache"])
    cs_dev = torch.from_numpy(cs).to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    mqa.rope_q(t["q"], cs_dev, t["seq_lens"], err_flags=err)
    mqa.append_kv_rope(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], cs_dev, t["seq_lens"],
                       err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    qr, rc = oracle.rope_q(q0, cs, lens)
    assert rc == oracle.OK
    assert np.array_equal(W.to_oracle(t["q"]), qr)
    assert oracle.append_kv_rope(kc0, vc0, W.to_oracle(t["k_new"]), W.to_oracle(t["v_new"]), cs,
                                 lens) == oracle.OK
    assert np.array_equal(W.to_oracle(t["k_cache"]), kc0)
    assert np.array_equal(W.to_oracle(t["v_cache"]), vc0)
    # and attention over the rotated step agrees with the oracle on the rotated bytes
    out = mqa.decode_attn_multi(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"])
    torch.cuda.synchronize()
    ref, _, rc = oracle.decode_attn_multi(qr, kc0, vc0, lens, float(np.float32(1 / math.sqrt(d))),
                                          nthreads=NTHREADS)
    compare(out, ref, "rotated step")


def test_rope_position_past_the_table_is_flagged():
    b, T, h, g, S, d = 4, 1, 8, 2, 64, 64
    cs = torch.from_numpy(oracle.rope_table(10000.0, 20, d)).to(DEV)  # positions 0..19 only
    w = wl("rope-short", b, h, g, d, S, 30, 40, 960)
    t = W.make_step(w, DEV)
    q0 = t["q"].clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    mqa.rope_q(t["q"], cs, t["seq_lens"], err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) & mqa.DEVERR_ROPE
    assert torch.equal(t["q"], q0)  # every position (>= 29) is past the table: untouched
