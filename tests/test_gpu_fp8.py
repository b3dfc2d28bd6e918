"""Parity of the fp8 e4m3 cache path (through the C ABI) against the CPU oracle.

Each case draws a seeded fp8 step (workloads.make_fp8_step: codes, per-K/V-head
scales, bf16 q and new rows), runs the quantised append and the decode on the
GPU, reads the codes back and runs the oracle's fp8 functions on those bytes.
The append must be bit-exact (its codes are integers decided in fp32 on both
sides: one correctly rounded division, nearest-even rounding); the attention
within |gpu - ref| <= 2e-3 and |gpu - ref| / max(|ref|, rms(ref row)) <= 2e-3
of the double-precision result on the dequantised cache.
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


def bits(t: torch.Tensor) -> np.ndarray:
    return W.to_oracle(t)


def run_fp8(w: W.Workload, T: int = 1, page_size: int = 0, split_chunk: int = 0):
    print(f"[fp8] {w.name} b={w.b} T={T} h={w.h} g={w.g} d={w.d} S={w.S} P={page_size} "
          f"chunk={split_chunk}", flush=True)
    t = W.make_fp8_step(w, DEV, T=T, page_size=page_size)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ks, vs = t["k_scale"], t["v_scale"]
    lens = t["seq_lens"].cpu().numpy()
    sc = float(np.float32(1.0 / math.sqrt(w.d)))
    if page_size:
        kp0, vp0 = t["k_pages"].cpu().numpy(), t["v_pages"].cpu().numpy()
        bt = t["block_table"].cpu().numpy()
        mqa.append_kv_paged_fp8(t["k_pages"], t["v_pages"], t["k_new"], t["v_new"], ks, vs,
                                t["block_table"], t["seq_lens"], err_flags=err)
        out = mqa.decode_attn_paged_fp8(t["q"], t["k_pages"], t["v_pages"], ks, vs,
                                        t["block_table"], t["seq_lens"], split_chunk=split_chunk,
                                        err_flags=err)
        torch.cuda.synchronize()
        assert oracle.append_kv_paged_fp8(kp0, vp0, bits(t["k_new"]), bits(t["v_new"]),
                                          ks.cpu().numpy(), vs.cpu().numpy(), bt, lens) == oracle.OK
        kc, vc = t["k_pages"].cpu().numpy(), t["v_pages"].cpu().numpy()
        ref, rc = oracle.decode_attn_paged_fp8(bits(t["q"]), kc, vc, ks.cpu().numpy(),
                                               vs.cpu().numpy(), bt, lens, sc, nthreads=NTHREADS)
    else:
        kc0, vc0 = t["k_cache"].cpu().numpy(), t["v_cache"].cpu().numpy()
        mqa.append_kv_fp8(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], ks, vs,
                          t["seq_lens"], err_flags=err)
        out = mqa.decode_attn_fp8(t["q"], t["k_cache"], t["v_cache"], ks, vs, t["seq_lens"],
                                  split_chunk=split_chunk, err_flags=err)
        torch.cuda.synchronize()
        assert oracle.append_kv_fp8(kc0, vc0, bits(t["k_new"]), bits(t["v_new"]),
                                    ks.cpu().numpy(), vs.cpu().numpy(), lens) == oracle.OK
        kc, vc = t["k_cache"].cpu().numpy(), t["v_cache"].cpu().numpy()
        kp0, vp0 = kc0, vc0
        ref, rc = oracle.decode_attn_fp8(bits(t["q"]), kc, vc, ks.cpu().numpy(), vs.cpu().numpy(),
                                         lens, sc, nthreads=NTHREADS)
    assert int(err.item()) == 0
    # the quantised append: the same codes, byte for byte
    assert np.array_equal(kc, kp0) and np.array_equal(vc, vp0)
    assert rc == oracle.OK
    compare(out, ref, f"{w.name} fp8 T={T} P={page_size}")
    return t, out


def wl(name, b, h, g, d, S, lo, hi, seed):
    return W.Workload(name, b=b, h=h, g=g, d=d, S=S, dtype=torch.bfloat16, seed=seed, L_lo=lo,
                      L_hi=hi)


@pytest.mark.parametrize("h,g,d", [(64, 8, 128), (32, 4, 64), (32, 32, 128)])
def test_fp8_balanced(h, g, d):
    run_fp8(wl("fp8-bal", 64, h, g, d, 1024, 1, 1024, 800 + h + g + d))


@pytest.mark.parametrize("h,g,d", [(32, 1, 128), (16, 2, 64)])
def test_fp8_partitions(h, g, d):
    run_fp8(wl("fp8-part", 8, h, g, d, 2000, 1, 2000, 820 + h + g + d))


@pytest.mark.parametrize("chunk", [64, 512])
def test_fp8_fixed_partitions(chunk):
    run_fp8(wl("fp8-chunk", 16, 32, 8, 128, 1000, 1, 1000, 830 + chunk), split_chunk=chunk)


@pytest.mark.parametrize("T", [2, 4])
def test_fp8_multi_token(T):
    run_fp8(wl("fp8-multi", 64, 64, 8, 128, 700, 1, 700, 840 + T), T=T)


@pytest.mark.parametrize("T,P", [(1, 16), (3, 32)])
def test_fp8_paged(T, P):
    run_fp8(wl("fp8-paged", 64, 32, 4, 128, 800, 1, 800, 850 + T + P), T=T, page_size=P)


def test_fp8_append_saturates_and_flags_bad_lengths():
    """Values far beyond 448 * scale saturate to the largest code (never NaN);
    a length past the capacity is skipped and flagged."""
    w = wl("fp8-sat", 4, 8, 2, 64, 32, 10, 32, 860)
    t = W.make_fp8_step(w, DEV)
    t["k_new"][0] = 1e6
    t["v_new"][0] = -1e6
    lens = t["seq_lens"].clone()
    lens[2] = w.S + 1
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    k0 = t["k_cache"].clone()
    mqa.append_kv_fp8(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["k_scale"],
                      t["v_scale"], lens, err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) & mqa.DEVERR_SEQLEN
    L0 = int(lens[0].item())
    assert (t["k_cache"][0, :, L0 - 1] == 0x7E).all() and (t["v_cache"][0, :, L0 - 1] == 0xFE).all()
    assert torch.equal(t["k_cache"][2], k0[2])


def test_fp8_full_size():
    """gqa-70b shape (b=64, h=64, g=8, ragged up to 4096) over an fp8 cache:
    every output against the oracle."""
    run_fp8(W.WORKLOADS["gqa-70b"])
