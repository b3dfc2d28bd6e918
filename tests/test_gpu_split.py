"""The balanced schedule's weighted split on the GPU, at its edges.

The work-groups' ranges are equal shares of a weight that gives every
(sequence, K/V head) unit an allowance for closing its segment (StepSplit in
the HIP source); with an allowance the range boundaries move away from the
plain equal split of the steps, and the range that holds a cut unit's last
piece comes from the inverse formula. These cases put boundaries everywhere a
mistake in either would show: batches that mix one-step units (lengths 1 ..
32) and units shorter than the allowance with long ones, and invalid lengths
(below the T tokens, past the capacity) among them, on each kernel that
carries an allowance — two 16-row blocks per wave (four tokens of eight
heads), two blocks in each of two head groups (eight tokens), and the one-byte
caches. Valid rows are compared with the oracle at the usual bound
(|gpu - ref| <= 2e-3 and <= 2e-3 of max(|ref|, rms of the row)); invalid
sequences must come out NaN with MQA_DEVERR_SEQLEN raised.
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
S = 512


def mixed_lengths(b: int, T: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    kind = rng.random(b)
    lens = np.where(kind < 0.3, rng.integers(T, 9 + T, b),            # one step
                    np.where(kind < 0.6, rng.integers(9, 70, b),       # a few steps
                             rng.integers(100, S + 1, b)))              # long
    lens = np.maximum(lens, T)
    bad = rng.choice(b, size=max(2, b // 25), replace=False)
    lens[bad[0::2]] = T - 1 if T > 1 else 0                            # below the tokens
    lens[bad[1::2]] = S + 1                                            # past the capacity
    return lens.astype(np.int32)


@pytest.mark.parametrize("kind,T,b", [("bf16", 4, 200), ("bf16", 8, 100), ("fp8", 1, 160),
                                      ("int8", 2, 160), ("fp8", 4, 96)])
def test_weighted_split_edges(kind, T, b):
    h, g, d = 64, 8, 128
    print(f"[split] {kind} T={T} b={b}", flush=True)
    w = W.Workload(f"split-{kind}-{T}", b=b, h=h, g=g, d=d, S=S, dtype=torch.bfloat16,
                   seed=1500 + 10 * T + b, L_lo=1, L_hi=S)
    assert mqa.decode_multi_schedule(b, T, h, g, S, d, mqa.BF16) == "mfma-balanced"
    if kind == "bf16":
        t = W.make_multi_step(w, DEV, T=T)
    else:
        t = W.make_fp8_step(w, DEV, T=T, int8=(kind == "int8"))
    lens = mixed_lengths(b, T, w.seed)
    lens_d = torch.from_numpy(lens).to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ks, vs = t.get("k_scale"), t.get("v_scale")
    out = mqa.decode_attn_ex(t["q"], t["k_cache"], t["v_cache"], lens_d, k_scale=ks, v_scale=vs,
                             err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == mqa.DEVERR_SEQLEN
    valid = (lens >= T) & (lens <= S)
    got = out.detach().cpu().double().numpy()
    assert np.isnan(got[~valid]).all()
    kc = W.to_oracle(t["k_cache"]) if kind == "bf16" else t["k_cache"].cpu().numpy()
    vc = W.to_oracle(t["v_cache"]) if kind == "bf16" else t["v_cache"].cpu().numpy()
    ref, rc = oracle.decode_attn_ex(W.to_oracle(t["q"]), kc, vc, lens,
                                    float(np.float32(1.0 / math.sqrt(d))),
                                    k_scale=None if ks is None else ks.cpu().numpy(),
                                    v_scale=None if vs is None else vs.cpu().numpy(),
                                    nthreads=NTHREADS)
    assert rc == oracle.BAD_LEN
    got, ref = got[valid], ref[valid]
    assert np.isfinite(got).all()
    e = np.abs(got - ref)
    rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
    rel = e / np.maximum(np.abs(ref), rms)
    assert e.max() <= ATOL and rel.max() <= RTOL_ROW, f"abs {e.max()} rel {rel.max()}"
