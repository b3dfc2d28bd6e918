"""Parity of the int8 cache path (through the C ABI) against the CPU oracle.

Each case draws a seeded int8 step (workloads.make_int8_step: codes, per-K/V
-head scales, bf16 q and new rows), runs the quantised append
(mqa_append_kv_int8 / _paged_int8) and the decode (mqa_decode_attn_ex with an
int8 cache) on the GPU, reads the codes back and runs the oracle on those
bytes. The append must be bit-exact (its codes are integers decided in fp32
on both sides: one correctly rounded division, nearest-even rounding); the
attention within |gpu - ref| <= 2e-3 and |gpu - ref| / max(|ref|, rms(ref
row)) <= 2e-3 of the double-precision result on the dequantised cache.
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


def run_int8(w: W.Workload, T: int = 1, page_size: int = 0, split_chunk: int = 0, window: int = 0):
    print(f"[int8] {w.name} b={w.b} T={T} h={w.h} g={w.g} d={w.d} S={w.S} P={page_size} "
          f"chunk={split_chunk} W={window}", flush=True)
    t = W.make_int8_step(w, DEV, T=T, page_size=page_size)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ks, vs = t["k_scale"], t["v_scale"]
    lens = t["seq_lens"].cpu().numpy()
    kk, vv = ("k_pages", "v_pages") if page_size else ("k_cache", "v_cache")
    bt = t.get("block_table") if page_size else None
    k0, v0 = t[kk].cpu().numpy(), t[vv].cpu().numpy()
    if page_size:
        mqa.append_kv_paged_int8(t[kk], t[vv], t["k_new"], t["v_new"], ks, vs, bt, t["seq_lens"],
                                 err_flags=err)
    else:
        mqa.append_kv_int8(t[kk], t[vv], t["k_new"], t["v_new"], ks, vs, t["seq_lens"],
                           err_flags=err)
    out = mqa.decode_attn_ex(t["q"], t[kk], t[vv], t["seq_lens"], block_table=bt, k_scale=ks,
                             v_scale=vs, window=window, split_chunk=split_chunk, err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    kn, vn = W.to_oracle(t["k_new"]), W.to_oracle(t["v_new"])
    ksn, vsn = ks.cpu().numpy(), vs.cpu().numpy()
    if page_size:
        assert oracle.append_kv_paged_int8(k0, v0, kn, vn, ksn, vsn, bt.cpu().numpy(),
                                           lens) == oracle.OK
    else:
        assert oracle.append_kv_int8(k0, v0, kn, vn, ksn, vsn, lens) == oracle.OK
    kc, vc = t[kk].cpu().numpy(), t[vv].cpu().numpy()
    # the quantised append: the same codes, byte for byte
    assert np.array_equal(kc, k0) and np.array_equal(vc, v0)
    ref, rc = oracle.decode_attn_ex(W.to_oracle(t["q"]), kc, vc, lens,
                                    float(np.float32(1.0 / math.sqrt(w.d))), window=window,
                                    k_scale=ksn, v_scale=vsn,
                                    block_table=None if bt is None else bt.cpu().numpy(),
                                    nthreads=NTHREADS)
    assert rc == oracle.OK
    compare(out, ref, f"{w.name} int8 T={T} P={page_size} W={window}")


@pytest.mark.parametrize("h,g,d", [(64, 8, 128), (32, 4, 64), (32, 32, 128)])
def test_int8_balanced(h, g, d):
    run_int8(wl("int8-bal", 64, h, g, d, 1024, 1, 1024, 1000 + h + g + d))


@pytest.mark.parametrize("h,g,d", [(32, 1, 128), (16, 2, 64)])
def test_int8_partitions(h, g, d):
    run_int8(wl("int8-part", 8, h, g, d, 2000, 1, 2000, 1020 + h + g + d))


@pytest.mark.parametrize("chunk", [64, 512])
def test_int8_fixed_partitions(chunk):
    run_int8(wl("int8-chunk", 16, 32, 8, 128, 1000, 1, 1000, 1030 + chunk), split_chunk=chunk)


@pytest.mark.parametrize("T", [2, 4])
def test_int8_multi_token(T):
    run_int8(wl("int8-multi", 64, 64, 8, 128, 700, 1, 700, 1040 + T), T=T)


def test_int8_many_blocks_on_partitions():
    """Four tokens of 32 heads sharing one K/V head (eight 16-row blocks):
    the partition kernel with wave pairs."""
    run_int8(wl("int8-pairs", 4, 32, 1, 128, 1500, 1, 1500, 1045), T=4)


@pytest.mark.parametrize("T,P", [(1, 16), (3, 32)])
def test_int8_paged(T, P):
    run_int8(wl("int8-paged", 64, 32, 4, 128, 800, 1, 800, 1050 + T + P), T=T, page_size=P)


def test_int8_window():
    run_int8(wl("int8-win", 64, 64, 8, 128, 1024, 1, 1024, 1060), window=300)
    run_int8(wl("int8-win-paged", 32, 32, 4, 64, 600, 1, 600, 1061), T=2, page_size=16, window=50)


def test_int8_append_saturates_and_flags_bad_lengths():
    """Values far beyond 127 * scale saturate to +-127 (never -128); a length
    past the capacity is skipped and flagged."""
    w = wl("int8-sat", 4, 8, 2, 64, 32, 10, 32, 1070)
    t = W.make_int8_step(w, DEV)
    t["k_new"][0] = 1e6
    t["v_new"][0] = -1e6
    lens = t["seq_lens"].clone()
    lens[2] = w.S + 1
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    k0 = t["k_cache"].clone()
    mqa.append_kv_int8(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["k_scale"],
                       t["v_scale"], lens, err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) & mqa.DEVERR_SEQLEN
    L0 = int(lens[0].item())
    assert (t["k_cache"][0, :, L0 - 1] == 127).all() and (t["v_cache"][0, :, L0 - 1] == -127).all()
    assert torch.equal(t["k_cache"][2], k0[2])


def test_int8_full_size():
    """gqa-70b shape (b=64, h=64, g=8, ragged up to 4096) over an int8 cache:
    every output against the oracle."""
    run_int8(W.WORKLOADS["gqa-70b"])
