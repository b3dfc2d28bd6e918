"""Parity of the T-token (causal) path through the C ABI against the CPU oracle.

Each case draws a seeded step with T query tokens per sequence
(workloads.make_multi_step), runs mqa_append_kv_multi + mqa_decode_attn_multi
(or their paged forms) on the GPU, reads the cache back and runs the oracle's
T-token functions on those bytes. Tolerance as for one token: |gpu - ref| <=
2e-3 and |gpu - ref| / max(|ref|, rms(ref row)) <= 2e-3; the append is
bit-exact.
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


def scale_of(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


def run_and_check(w: W.Workload, T: int, page_size: int = 0, split_chunk: int = 0,
                  expect_schedule: str | None = None):
    S_cap = w.S if not page_size else -(-w.S // page_size) * page_size
    sched = mqa.decode_multi_schedule(w.b, T, w.h, w.g, S_cap, w.d, w.dtype, split_chunk)
    print(f"[multi] {w.name} b={w.b} T={T} h={w.h} g={w.g} d={w.d} S={w.S} P={page_size} "
          f"chunk={split_chunk} schedule={sched}", flush=True)
    if expect_schedule:
        assert sched == expect_schedule
    t = W.make_multi_step(w, DEV, T=T, page_size=page_size)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    lens = t["seq_lens"].cpu().numpy()
    if page_size:
        kc0, vc0 = W.to_oracle(t["k_pages"]), W.to_oracle(t["v_pages"])
        bt = t["block_table"].cpu().numpy()
        mqa.append_kv_paged_multi(t["k_pages"], t["v_pages"], t["k_new"], t["v_new"],
                                  t["block_table"], t["seq_lens"], err_flags=err)
        out = mqa.decode_attn_paged_multi(t["q"], t["k_pages"], t["v_pages"], t["block_table"],
                                          t["seq_lens"], split_chunk=split_chunk, err_flags=err)
        torch.cuda.synchronize()
        assert oracle.append_kv_paged_multi(kc0, vc0, W.to_oracle(t["k_new"]),
                                            W.to_oracle(t["v_new"]), bt, lens) == oracle.OK
        kc, vc = W.to_oracle(t["k_pages"]), W.to_oracle(t["v_pages"])
        ref, rc = oracle.decode_attn_paged_multi(W.to_oracle(t["q"]), kc, vc, bt, lens,
                                                 scale_of(w.d), nthreads=NTHREADS)
    else:
        kc0, vc0 = W.to_oracle(t["k_cache"]), W.to_oracle(t["v_cache"])
        mqa.append_kv_multi(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["seq_lens"],
                            err_flags=err)
        out = mqa.decode_attn_multi(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"],
                                    split_chunk=split_chunk, err_flags=err)
        torch.cuda.synchronize()
        assert oracle.append_kv_multi(kc0, vc0, W.to_oracle(t["k_new"]), W.to_oracle(t["v_new"]),
                                      lens) == oracle.OK
        kc, vc = W.to_oracle(t["k_cache"]), W.to_oracle(t["v_cache"])
        ref, _, rc = oracle.decode_attn_multi(W.to_oracle(t["q"]), kc, vc, lens, scale_of(w.d),
                                              nthreads=NTHREADS)
    assert int(err.item()) == 0
    # the append: bit-exact against the oracle's append on the pre-step bytes
    assert kc.tobytes() == kc0.tobytes() and vc.tobytes() == vc0.tobytes()
    assert rc == oracle.OK
    compare(out, ref, f"{w.name} T={T}")
    return t, out


def wl(name, b, h, g, d, S, lo, hi, seed):
    return W.Workload(name, b=b, h=h, g=g, d=d, S=S, dtype=torch.bfloat16, seed=seed, L_lo=lo,
                      L_hi=hi)


@pytest.mark.parametrize("T", [2, 4, 8])
def test_multi_balanced(T):
    """T tokens of 8 heads per K/V head: 16, 32, 64 query rows (1, 2, 4 blocks)."""
    w = wl("multi-gqa", 64, 64, 8, 128, 1024, 1, 1024, 700 + T)
    run_and_check(w, T, expect_schedule="mfma-balanced")


@pytest.mark.parametrize("T,h,g,d,sched", [(4, 32, 1, 128, "mfma-partitions"),
                                           (3, 32, 1, 128, "mfma-partitions"),
                                           (5, 16, 4, 64, "mfma-partitions"),
                                           (2, 64, 64, 128, "mfma-balanced")])
def test_multi_row_counts(T, h, g, d, sched):
    """Row counts T*G that are not multiples of 16 (96, 40, 2) and above 64
    (fixed partitions), MQA to MHA."""
    w = wl("multi-rows", 8, h, g, d, 700, 1, 700, 710 + T * h + g)
    run_and_check(w, T, expect_schedule=sched)


@pytest.mark.parametrize("chunk", [64, 128])
def test_multi_short_partitions(chunk):
    """Partitions shorter than a token's causal reach: some partitions hold no
    position for the earlier tokens (their partials are empty)."""
    w = wl("multi-chunk", 16, 32, 4, 128, 600, 60, 600, 720 + chunk)
    run_and_check(w, 8, split_chunk=chunk, expect_schedule="mfma-partitions")


def test_multi_lengths_equal_to_t():
    """Sequences as short as the step itself (a prompt chunk at the start)."""
    w = wl("multi-short", 300, 32, 4, 128, 64, 1, 12, 730)
    run_and_check(w, 8)


@pytest.mark.parametrize("T,P", [(5, 16), (4, 32)])
def test_multi_paged(T, P):
    """Paged cache; the T new tokens straddle page boundaries for some sequences."""
    w = wl("multi-paged", 64, 32, 4, 128, 800, 1, 800, 740 + T)
    run_and_check(w, T, page_size=P)


@pytest.mark.parametrize("T,h,g,S,b", [(32, 32, 8, 300, 8), (64, 16, 1, 500, 2), (48, 64, 64, 200, 4)])
def test_prompt_chunks(T, h, g, S, b):
    """Long prompt chunks (T = 32 .. 64 tokens: 128 to 3072 query rows per
    unit), causal within the chunk, lengths from T to the capacity."""
    w = wl("chunk", b, h, g, 128, S, T, S, 780 + T)
    run_and_check(w, T)


def test_multi_one_token_is_the_plain_decode():
    w = wl("multi-one", 64, 64, 8, 128, 1024, 1, 1024, 750)
    t = W.make_step(w, DEV)
    a = mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"])
    m = mqa.decode_attn_multi(t["q"].unsqueeze(1).contiguous(), t["k_cache"], t["v_cache"],
                              t["seq_lens"])
    torch.cuda.synchronize()
    assert (a - m[:, 0]).abs().max().item() <= 1e-5


def test_multi_length_below_t_gives_nan_and_flag():
    w = wl("multi-bad", 300, 16, 2, 128, 256, 20, 256, 760)
    T = 6
    t = W.make_multi_step(w, DEV, T=T)
    lens = t["seq_lens"].clone()
    lens[3] = T - 1
    lens[7] = w.S + 1
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    k0 = t["k_cache"][3].clone()
    mqa.append_kv_multi(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], lens, err_flags=err)
    out = mqa.decode_attn_multi(t["q"], t["k_cache"], t["v_cache"], lens, err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) & mqa.DEVERR_SEQLEN
    assert torch.equal(t["k_cache"][3], k0)
    o = out.cpu()
    assert torch.isnan(o[3]).all() and torch.isnan(o[7]).all()
    good = [i for i in range(w.b) if i not in (3, 7)]
    ref, _, rc = oracle.decode_attn_multi(W.to_oracle(t["q"]), W.to_oracle(t["k_cache"]),
                                          W.to_oracle(t["v_cache"]), lens.cpu().numpy(),
                                          scale_of(w.d), nthreads=NTHREADS)
    assert rc == oracle.BAD_LEN
    compare(out[good], ref[good], "valid rows")


def test_multi_full_size():
    """gqa-70b (b=64, h=64, g=8, ragged lengths up to 4096) verifying a draft of
    4 tokens: every output against the oracle."""
    run_and_check(W.WORKLOADS["gqa-70b"], 4, expect_schedule="mfma-balanced")
