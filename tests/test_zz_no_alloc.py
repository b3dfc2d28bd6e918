"""The entry point that allocates nothing (mqa_decode_attn_noalloc), on the GPU.

It is mqa_decode_attn with the workspace replaced by the library's own
scratch array. Called through the C ABI twice in a row, the second call with
a smaller input (so it runs other kernels over the first call's stale
scratch), it must give what mqa_decode_attn gives on the same inputs, within
the parity bound of every test (|d| <= 2e-3 and, relative to
max(|ref|, rms of the row), <= 2e-3). (The refusal of a call whose workspace
would exceed the scratch is checked on the CPU, in test_abi.py: it needs no
device, and a launch with such sizes on real buffers could fault.)
"""
from __future__ import annotations

import ctypes
import math

import numpy as np
import pytest
import torch

import transformer_decode_attention_amd as mqa
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def noalloc(t, out, err):
    """mqa_decode_attn_noalloc through the C ABI (ctypes, no binding logic)."""
    q, k, v, lens = t["q"], t["k_cache"], t["v_cache"], t["seq_lens"]
    b, h, d = q.shape
    g, S = k.shape[1], k.shape[2]
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    return mqa.lib().mqa_decode_attn_noalloc(
        p(q), p(k), p(v), p(lens), b, h, g, S, d, mqa.BF16, ctypes.c_float(1.0 / math.sqrt(d)),
        p(out), 0, p(err), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def close(got: torch.Tensor, ref: torch.Tensor, what: str):
    a, r = got.double().cpu().numpy(), ref.double().cpu().numpy()
    assert np.isfinite(a).all(), what
    e = np.abs(a - r)
    rms = np.sqrt((r ** 2).mean(axis=-1, keepdims=True))
    assert e.max() <= 2e-3 and (e / np.maximum(np.abs(r), rms)).max() <= 2e-3, (what, e.max())


def test_noalloc_matches_decode_attn_on_two_calls():
    big = W.WORKLOADS["gqa-70b"]                                   # balanced schedule
    small = W.shrink(W.WORKLOADS["mqa-1k"], b=4)                   # fixed partitions
    assert mqa.decode_schedule(big.b, big.h, big.g, big.S, big.d, big.dtype) == "mfma-balanced"
    assert mqa.decode_schedule(small.b, small.h, small.g, small.S, small.d, small.dtype) == \
        "mfma-partitions"
    for w in (big, small):
        print(f"[noalloc] {w.name} b={w.b} h={w.h} g={w.g} S={w.S}", flush=True)
        t = W.make_step(w, DEV)
        ref = mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"])
        out = torch.full((w.b, w.h, w.d), float("nan"), dtype=torch.float32, device=DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        st = noalloc(t, out, err)
        torch.cuda.synchronize()
        assert st == mqa.OK, mqa.status_string(st)
        assert int(err.item()) == 0
        close(out, ref, w.name)
