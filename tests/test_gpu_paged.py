"""Parity of the paged-cache path (through the C ABI) against the CPU oracle.

Seeded inputs are scattered into randomly numbered pages (workloads.make_paged_step);
one step runs mqa_append_kv_paged + mqa_decode_attn_paged on the GPU, the
pages are read back, and the oracle's paged functions run on those bytes.
Tolerance as for the contiguous path: |gpu - ref| <= 2e-3 and
|gpu - ref| / max(|ref|, rms(ref row)) <= 2e-3; the append is bit-exact.
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


def paged_step(t: dict, split_chunk: int = 0):
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    mqa.append_kv_paged(t["k_pages"], t["v_pages"], t["k_new"], t["v_new"], t["block_table"],
                        t["seq_lens"], err_flags=err)
    out = mqa.decode_attn_paged(t["q"], t["k_pages"], t["v_pages"], t["block_table"],
                                t["seq_lens"], split_chunk=split_chunk, err_flags=err)
    torch.cuda.synchronize()
    return out, err


def oracle_paged(t: dict):
    d = t["q"].shape[-1]
    ref, rc = oracle.decode_attn_paged(W.to_oracle(t["q"]), W.to_oracle(t["k_pages"]),
                                       W.to_oracle(t["v_pages"]), t["block_table"].cpu().numpy(),
                                       t["seq_lens"].cpu().numpy(),
                                       float(np.float32(1.0 / math.sqrt(d))), nthreads=NTHREADS)
    return ref, rc


def check_paged(w: W.Workload, P: int, split_chunk: int = 0, share_prefix: bool = False):
    print(f"[paged] {w.name} b={w.b} h={w.h} g={w.g} d={w.d} S={w.S} P={P} chunk={split_chunk}",
          flush=True)
    t = W.make_paged_step(w, DEV, page_size=P, share_prefix=share_prefix)
    kp0, vp0 = W.to_oracle(t["k_pages"]), W.to_oracle(t["v_pages"])
    out, err = paged_step(t, split_chunk)
    assert int(err.item()) == 0
    # append: bit-exact against the oracle's paged append on the pre-step bytes
    bt, lens = t["block_table"].cpu().numpy(), t["seq_lens"].cpu().numpy()
    assert oracle.append_kv_paged(kp0, vp0, W.to_oracle(t["k_new"]), W.to_oracle(t["v_new"]),
                                  bt, lens) == oracle.OK
    assert W.to_oracle(t["k_pages"]).tobytes() == kp0.tobytes()
    assert W.to_oracle(t["v_pages"]).tobytes() == vp0.tobytes()
    ref, rc = oracle_paged(t)
    assert rc == oracle.OK
    compare(out, ref, f"{w.name} P={P}")
    return t, out


CASES = [
    # (b, h, g, d, S, L_lo, L_hi, page_size)
    (64, 64, 8, 128, 1024, 1, 1024, 16),    # many units: the balanced schedule
    (48, 32, 4, 64, 700, 1, 700, 32),       # d = 64, ragged tail pages
    (8, 32, 1, 128, 2048, 1500, 2048, 16),  # MQA, few units: fixed partitions
    (32, 64, 1, 128, 512, 1, 512, 64),      # G = 64: four head blocks
    (256, 16, 2, 128, 300, 1, 300, 16),     # many short sequences
]


@pytest.mark.parametrize("case", CASES)
def test_paged_matches_oracle(case):
    b, h, g, d, S, lo, hi, P = case
    w = W.Workload("paged", b=b, h=h, g=g, d=d, S=S, dtype=torch.bfloat16, seed=600 + b + h,
                   L_lo=lo, L_hi=hi)
    check_paged(w, P)


@pytest.mark.parametrize("chunk", [64, 256])
def test_paged_fixed_partitions(chunk):
    w = W.Workload("paged-fixed", b=16, h=32, g=8, d=128, S=1000, dtype=torch.bfloat16, seed=650,
                   L_lo=1, L_hi=1000)
    check_paged(w, 16, split_chunk=chunk)


def test_paged_shared_prefix_page():
    w = W.Workload("paged-share", b=64, h=32, g=4, d=128, S=800, dtype=torch.bfloat16, seed=660,
                   L_lo=100, L_hi=800)
    check_paged(w, 16, share_prefix=True)


def test_paged_equals_contiguous():
    """The same logical cache, paged or contiguous: the same attention (to rounding)."""
    w = W.Workload("paged-eq", b=64, h=64, g=8, d=128, S=1024, dtype=torch.bfloat16, seed=670,
                   L_lo=1, L_hi=1024)
    t = W.make_paged_step(w, DEV, page_size=16)
    a = mqa.decode_attn_paged(t["q"], t["k_pages"], t["v_pages"], t["block_table"], t["seq_lens"])
    c = mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"])
    torch.cuda.synchronize()
    assert (a - c).abs().max().item() <= 1e-5


def test_paged_bad_page_gives_nan_and_flag():
    """A referenced page id outside the pool: that (sequence, K/V head) group's
    rows are NaN, the flag is raised, the other sequences are exact."""
    w = W.Workload("paged-bad", b=32, h=16, g=2, d=128, S=512, dtype=torch.bfloat16, seed=680,
                   L_lo=200, L_hi=512)
    t = W.make_paged_step(w, DEV, page_size=16)
    num = t["k_pages"].shape[0]
    bt = t["block_table"].clone()
    bt[5, 3] = num + 7      # inside every length (L >= 200 > 3 * 16)
    bt[9, 0] = -1
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = mqa.decode_attn_paged(t["q"], t["k_pages"], t["v_pages"], bt, t["seq_lens"], err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) & mqa.DEVERR_PAGE
    o = out.cpu()
    assert torch.isnan(o[5]).all() and torch.isnan(o[9]).all()
    good = [i for i in range(w.b) if i not in (5, 9)]
    ref, rc = oracle_paged(t)
    assert rc == oracle.OK
    compare(out[good], ref[good], "good rows")
    # append with a bad page: flagged, nothing written there
    err.zero_()
    lens = t["seq_lens"].clone()
    bt2 = t["block_table"].clone()
    row_page = (int(lens[3].item()) - 1) // 16
    bt2[3, row_page] = num
    kp0 = t["k_pages"].clone()
    mqa.append_kv_paged(t["k_pages"], t["v_pages"], t["k_new"], t["v_new"], bt2, lens, err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) & mqa.DEVERR_PAGE
    assert torch.equal(t["k_pages"][int(t["block_table"][3, row_page])],
                       kp0[int(t["block_table"][3, row_page])])


def test_paged_full_size_sampled():
    """gqa-70b in 16-token pages (the default page size of [MQA blog] §3.3):
    every output against the oracle."""
    w = W.WORKLOADS["gqa-70b"]
    check_paged(w, 16)
