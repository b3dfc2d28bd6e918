"""The partition combine over many partitions, ragged lengths and a reused workspace.

combine_kernel loads its first batch of partials before a sequence's length
is known and masks the partitions past that sequence's last one afterwards;
with more than four partitions per piece lane it keeps eight loads in flight
and loops over further batches. These cases reach every branch of it:
64 partitions of 128 rows (d = 128: one batch of eight per lane), 256
partitions of 64 rows (d = 64: two batches), lengths from 1 to the capacity
(a sequence with one partition leaves seven or fifteen of its lanes' first
loads masked), and a workspace that a call over full-length sequences has
just filled, so that every masked partial holds a stale, finite value of the
earlier call. Each output is compared with the oracle on the bytes read back:
|gpu - ref| <= 2e-3 and |gpu - ref| / max(|ref|, rms(ref row)) <= 2e-3.
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

DEV = "cuda:0"
NTHREADS = min(16, os.cpu_count() or 1)


def compare(out_gpu: torch.Tensor, ref: np.ndarray, what: str) -> None:
    got = out_gpu.detach().cpu().double().numpy()
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
    rel = err / np.maximum(np.abs(ref), rms)
    assert err.max() <= 2e-3 and rel.max() <= 2e-3, f"{what}: abs {err.max()} rel {rel.max()}"


@pytest.mark.parametrize("d,h,g,S,chunk,lens", [
    (128, 32, 1, 8192, 128, [1, 2, 127, 128, 129, 1000, 4097, 8191, 8192]),
    (64, 16, 2, 16384, 64, [1, 63, 64, 65, 640, 8193, 9000, 16383, 16384]),
])
def test_combine_many_partitions_ragged_reused_workspace(d, h, g, S, chunk, lens):
    b = len(lens)
    print(f"[combine] d={d} h={h} g={g} S={S} chunk={chunk} nsplit={S // chunk} b={b}", flush=True)
    w = W.Workload("combine", b=b, h=h, g=g, d=d, S=S, dtype=torch.bfloat16, seed=7100 + d,
                   L_lo=1, L_hi=S)
    t = W.make_step(w, DEV)
    ws = mqa.decode_workspace(b, h, g, S, d, torch.bfloat16, DEV, chunk)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    # fill every partial of the workspace with a full-length call
    full = torch.full((b,), S, dtype=torch.int32, device=DEV)
    mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], full, workspace=ws, split_chunk=chunk,
                    err_flags=err)
    # then the ragged lengths on the same workspace
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], seq, workspace=ws, split_chunk=chunk,
                          err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref, _, rc = oracle.decode_attn(W.to_oracle(t["q"]), W.to_oracle(t["k_cache"]),
                                    W.to_oracle(t["v_cache"]), np.array(lens, dtype=np.int32),
                                    float(np.float32(1.0 / math.sqrt(d))), nthreads=NTHREADS)
    assert rc == oracle.OK
    compare(out, ref, f"d={d} chunk={chunk}")
