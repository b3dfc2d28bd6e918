"""Parity over seeded random combinations of every option.

Forty cases (MQA_COMBO_CASES) drawn from a fixed seed (MQA_COMBO_SEED), with
MQA_COMBO_LARGE=1 at larger capacities and batches:
head dimension, K/V heads and group size, query tokens, cache type (bf16,
fp8 or int8 codes), layout (contiguous or pages of 16 or 32 rows), sliding
window, automatic or fixed partitions, batch and ragged lengths. Each runs the matching append and the general
decode call (mqa_decode_attn_ex) on the GPU and compares against the oracle
on the bytes read back: the append bit-exact, the attention within |gpu -
ref| <= 2e-3 and |gpu - ref| / max(|ref|, rms(ref row)) <= 2e-3.
"""
from __future__ import annotations

import math
import os
import random

import numpy as np
import pytest
import torch

import oracle
import transformer_decode_attention_amd as mqa
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NTHREADS = min(16, os.cpu_count() or 1)


def draw_cases(n=40, seed=2024, large=False):
    """With large, capacities up to 5000 and batches up to 256 (halved while
    the oracle's multiply-adds would pass ~4e9, a few seconds per case, or a
    cache tensor 2e8 elements)."""
    rng = random.Random(seed)
    cases = []
    for k in range(n):
        d = rng.choice([64, 128])
        g = rng.choice([1, 2, 4, 8])
        G = rng.choice([1, 2, 4, 8, 16, 32])
        T = rng.choice([1, 1, 2, 3, 5])
        kv = rng.choice(["bf16", "fp8", "int8"])
        P = rng.choice([0, 0, 16, 32])
        S = rng.randint(max(T, 8), 5000 if large else 700)
        b = rng.choice([32, 64, 128, 256] if large else [1, 3, 17, 48, 96])
        window = rng.choice([0, 0, 1, rng.randint(2, 400)])
        chunk = rng.choice([0, 0, 64, 256])
        while large and b > 1 and (b * S * g * G * d * T > 4e9 or b * S * g * d > 2e8):
            b //= 2
        cases.append((k, d, g, G, T, kv, P, S, b, window, chunk))
    return cases


def append(t, kv, P, err):
    kk, vv = ("k_pages", "v_pages") if P else ("k_cache", "v_cache")
    args = (t[kk], t[vv], t["k_new"], t["v_new"])
    if kv == "bf16":
        if P:
            mqa.append_kv_paged_multi(*args, t["block_table"], t["seq_lens"], err_flags=err)
        else:
            mqa.append_kv_multi(*args, t["seq_lens"], err_flags=err)
        return
    sc = (t["k_scale"], t["v_scale"])
    fn = {("fp8", 0): mqa.append_kv_fp8, ("int8", 0): mqa.append_kv_int8,
          ("fp8", 1): mqa.append_kv_paged_fp8, ("int8", 1): mqa.append_kv_paged_int8}[(kv, int(bool(P)))]
    if P:
        fn(*args, *sc, t["block_table"], t["seq_lens"], err_flags=err)
    else:
        fn(*args, *sc, t["seq_lens"], err_flags=err)


def oracle_append(t0, kv, P, t):
    """The oracle's append on the pre-step bytes t0 (numpy, in place)."""
    kk, vv = ("k_pages", "v_pages") if P else ("k_cache", "v_cache")
    lens = t["seq_lens"].cpu().numpy()
    kn, vn = W.to_oracle(t["k_new"]), W.to_oracle(t["v_new"])
    bt = t["block_table"].cpu().numpy() if P else None
    if kv == "bf16":
        if P:
            return oracle.append_kv_paged_multi(t0[kk], t0[vv], kn, vn, bt, lens)
        return oracle.append_kv_multi(t0[kk], t0[vv], kn, vn, lens)
    ks, vs = t["k_scale"].cpu().numpy(), t["v_scale"].cpu().numpy()
    if kv == "fp8":
        if P:
            return oracle.append_kv_paged_fp8(t0[kk], t0[vv], kn, vn, ks, vs, bt, lens)
        return oracle.append_kv_fp8(t0[kk], t0[vv], kn, vn, ks, vs, lens)
    if P:
        return oracle.append_kv_paged_int8(t0[kk], t0[vv], kn, vn, ks, vs, bt, lens)
    return oracle.append_kv_int8(t0[kk], t0[vv], kn, vn, ks, vs, lens)


def host(x, kv):
    return W.to_oracle(x) if kv == "bf16" else x.cpu().numpy()


CASES = draw_cases(int(os.environ.get("MQA_COMBO_CASES", "40")),
                   int(os.environ.get("MQA_COMBO_SEED", "2024")),
                   os.environ.get("MQA_COMBO_LARGE", "0") == "1")


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"case{c[0]}")
def test_random_combination(case):
    k, d, g, G, T, kv, P, S, b, window, chunk = case
    h = g * G
    print(f"[combo] #{k} d={d} g={g} h={h} T={T} kv={kv} P={P} S={S} b={b} W={window} "
          f"chunk={chunk}", flush=True)
    w = W.Workload(f"combo{k}", b=b, h=h, g=g, d=d, S=S, dtype=torch.bfloat16, seed=5000 + 37 * k,
                   L_lo=T, L_hi=S)
    if kv == "bf16":
        t = W.make_multi_step(w, DEV, T=T, page_size=P)
    else:
        t = W.make_fp8_step(w, DEV, T=T, page_size=P, int8=(kv == "int8"))
    if T == 1 and t["q"].dim() == 3:
        t["q"] = t["q"].unsqueeze(1).contiguous()
        t["k_new"] = t["k_new"].unsqueeze(1).contiguous()
        t["v_new"] = t["v_new"].unsqueeze(1).contiguous()
    kk, vv = ("k_pages", "v_pages") if P else ("k_cache", "v_cache")
    t0 = {kk: host(t[kk], kv), vv: host(t[vv], kv)}
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    append(t, kv, P, err)
    out = mqa.decode_attn_ex(t["q"], t[kk], t[vv], t["seq_lens"],
                             block_table=t["block_table"] if P else None,
                             k_scale=t.get("k_scale"), v_scale=t.get("v_scale"), window=window,
                             split_chunk=chunk, err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert oracle_append(t0, kv, P, t) == oracle.OK
    kc, vc = host(t[kk], kv), host(t[vv], kv)
    assert np.array_equal(kc, t0[kk]) and np.array_equal(vc, t0[vv]), "append"
    ref, rc = oracle.decode_attn_ex(
        W.to_oracle(t["q"]), kc, vc, t["seq_lens"].cpu().numpy(),
        float(np.float32(1.0 / math.sqrt(d))), window=window,
        k_scale=None if kv == "bf16" else t["k_scale"].cpu().numpy(),
        v_scale=None if kv == "bf16" else t["v_scale"].cpu().numpy(),
        block_table=t["block_table"].cpu().numpy() if P else None, nthreads=NTHREADS)
    assert rc == oracle.OK
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all()
    e = np.abs(got - ref)
    rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
    assert e.max() <= 2e-3 and (e / np.maximum(np.abs(ref), rms)).max() <= 2e-3, \
        f"abs {e.max()} rel {(e / np.maximum(np.abs(ref), rms)).max()}"
