"""Pins of the CPU oracle against what the pages and the mathematics fix.

Sources (page title and section):
  [GQA notes]   ybb.press "分组查询注意力（GQA）与多查询注意力（MQA）深度实战"
  [MQA concept] compassingai.com "多查詢注意力"
  [MQA blog]    nanhubrain.csdn.net MQA article

Each pin is chosen so that a plausible slip in the oracle (a dropped scale, a
wrong head-to-group index, a missing normalisation, an off-by-one in the
attended length, a transposed operand) fails at least one of them; the mutant
tests at the end plant such slips in a copy of the oracle's source and check
that they are caught.
"""
from __future__ import annotations

import json
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def randn(*shape, scale=1.0):
    return (RNG.standard_normal(shape) * scale).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even) via torch; returns uint16 bits."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def sdpa_ref(q, k, v, lens, scale):
    """torch's scaled_dot_product_attention in float64 on the CPU, per sequence.

    q [b,h,d], k/v [b,g,S,d] float64; grouped heads via enable_gqa (torch
    repeats K/V heads with repeat_interleave, i.e. query head i uses K/V head
    i // (h/g)). A library routine, independent of the oracle's code.
    """
    b, h, d = q.shape
    g = k.shape[1]
    out = np.empty((b, h, d))
    for i in range(b):
        L = int(lens[i])
        qi = torch.from_numpy(q[i]).view(1, h, 1, d)
        ki = torch.from_numpy(np.ascontiguousarray(k[i, :, :L])).view(1, g, L, d)
        vi = torch.from_numpy(np.ascontiguousarray(v[i, :, :L])).view(1, g, L, d)
        o = torch.nn.functional.scaled_dot_product_attention(
            qi, ki, vi, scale=scale, enable_gqa=(g != h))
        out[i] = o.view(h, d).numpy()
    return out


# ---------------------------------------------------------------------------
# worked example and closed forms
# ---------------------------------------------------------------------------

def test_hand_example():
    """Brute force by hand on a 2-head, 2-position case ([GQA notes] §五)."""
    ex = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    q = np.array(ex["q"], np.float32)
    k = np.array(ex["k_cache"], np.float32)
    v = np.array(ex["v_cache"], np.float32)
    lens = np.array(ex["seq_lens"], np.int32)
    out, alpha, rc = oracle.decode_attn(q, k, v, lens, ex["scale"], want_alpha=True)
    assert rc == oracle.OK
    np.testing.assert_allclose(out, np.array(ex["out"]), rtol=0, atol=1e-6)
    np.testing.assert_allclose(alpha[:, :, :2], np.array(ex["alpha"]), rtol=0, atol=1e-7)


def test_kv_bytes_worked_examples():
    """Per-layer and 32-layer byte counts printed on the pages ([MQA concept] 技術原理)."""
    fx = json.load(open(os.path.join(GOLDEN, "kv_bytes.json")))
    for c in fx["cases"]:
        assert oracle.kv_bytes(c["layers"], c["g"], c["S"], c["d"], c["dtype_bytes"]) == c["bytes"], c["source"]
    for r in fx["ratios"]:
        mha = oracle.kv_bytes(1, r["h"], 4096, 128, 2)
        gqa = oracle.kv_bytes(1, r["g"], 4096, 128, 2)
        if "ratio" in r:
            assert mha / gqa == r["ratio"]
        else:
            assert gqa / mha == r["fraction"]


def test_length_one_returns_v0():
    """L = 1: the single weight is 1, so out = V_0 exactly."""
    q, k, v = randn(2, 4, 64), randn(2, 2, 8, 64), randn(2, 2, 8, 64)
    out, _, _ = oracle.decode_attn(q, k, v, np.array([1, 1], np.int32), 0.125)
    for i in range(2):
        for hq in range(4):
            np.testing.assert_array_equal(out[i, hq], v[i, hq // 2, 0].astype(np.float64))


def test_equal_v_rows_return_that_row():
    """Convex combination: all V rows = r gives out = r for any scores."""
    q, k = randn(3, 6, 64, scale=4.0), randn(3, 3, 50, 64)
    r = randn(3, 3, 1, 64)
    v = np.ascontiguousarray(np.broadcast_to(r, (3, 3, 50, 64)))
    out, _, _ = oracle.decode_attn(q, k, v, np.array([50, 17, 3], np.int32), 0.125)
    for i in range(3):
        for hq in range(6):
            np.testing.assert_allclose(out[i, hq], r[i, hq // 2, 0], rtol=0, atol=1e-12 + 1e-12 * np.abs(r).max())


def test_zero_k_gives_mean_of_v():
    """Zero keys: all scores 0, weights 1/L, out = mean of the first L V rows."""
    q, v = randn(2, 4, 128), randn(2, 1, 40, 128)
    k = np.zeros((2, 1, 40, 128), np.float32)
    lens = np.array([40, 23], np.int32)
    out, alpha, _ = oracle.decode_attn(q, k, v, lens, 0.088, want_alpha=True)
    for i in range(2):
        L = lens[i]
        mean = v[i, 0, :L].astype(np.float64).mean(axis=0)
        for hq in range(4):
            np.testing.assert_allclose(out[i, hq], mean, rtol=0, atol=1e-12)
            np.testing.assert_allclose(alpha[i, hq, :L], 1.0 / L, rtol=1e-14)


def test_weights_sum_to_one_and_vanish_past_length():
    q, k, v = randn(2, 8, 64, scale=3.0), randn(2, 2, 100, 64), randn(2, 2, 100, 64)
    lens = np.array([100, 31], np.int32)
    _, alpha, _ = oracle.decode_attn(q, k, v, lens, 0.125, want_alpha=True)
    np.testing.assert_allclose(alpha.sum(axis=2), 1.0, rtol=0, atol=1e-12)
    assert np.all(alpha[1, :, 31:] == 0.0)
    assert np.all(alpha >= 0.0)


# ---------------------------------------------------------------------------
# special cases that reduce to a library routine or a textbook loop
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("h,g", [(8, 8), (8, 1), (8, 2), (12, 4), (32, 8), (6, 3)])
def test_matches_torch_sdpa(h, g):
    """Any g: equals torch's SDPA (float64, CPU) with grouped K/V heads."""
    b, S, d = 3, 70, 64
    q, k, v = randn(b, h, d, scale=2.0), randn(b, g, S, d), randn(b, g, S, d)
    lens = np.array([70, 1, 45], np.int32)
    out, _, rc = oracle.decode_attn(q, k, v, lens, 0.125)
    assert rc == oracle.OK
    ref = sdpa_ref(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), lens, 0.125)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_g_equals_h_is_per_head_mha():
    """g = h is MHA ([GQA notes] §四): equals the textbook per-head routine."""
    h, L, d = 6, 33, 64
    q, k, v = randn(1, h, d), randn(1, h, L, d), randn(1, h, L, d)
    out, _, _ = oracle.decode_attn(q, k, v, np.array([L], np.int32), 0.125)
    ref = oracle.mha_per_head(q[0], k[0], v[0], 0.125)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-14)


# ---- paged cache ([MQA blog] §3.3: fixed-size pages, 16 tokens by default) ----

def _paged_from_contiguous(k, v, P, rng, extra_pages=5, share_prefix=False):
    """Scatter a contiguous cache [b, g, S, d] into randomly numbered pages of P
    rows (numpy indexing only); unused pages hold NaN."""
    b, g, S, d = k.shape
    maxp = -(-S // P)
    num = b * maxp + extra_pages
    ids = rng.permutation(num)[: b * maxp].reshape(b, maxp).astype(np.int32)
    if share_prefix:  # sequence 1 reuses sequence 0's first page
        ids[1, 0] = ids[0, 0]
    nan = np.float32("nan") if k.dtype == np.float32 else np.uint16(0x7FC0)
    kp = np.full((num, g, P, d), nan, k.dtype)
    vp = np.full((num, g, P, d), nan, v.dtype)
    for i in range(b):
        for p in range(maxp):
            rows = min(P, S - p * P)
            kp[ids[i, p], :, :rows] = k[i, :, p * P: p * P + rows]
            vp[ids[i, p], :, :rows] = v[i, :, p * P: p * P + rows]
    return kp, vp, ids


@pytest.mark.parametrize("P,h,g", [(16, 8, 2), (1, 4, 1), (7, 6, 3), (32, 8, 8)])
def test_paged_matches_gathered_sdpa(P, h, g):
    """Paged oracle = torch SDPA (float64) over the cache gathered back from
    random page numbers, and bitwise = the contiguous oracle."""
    rng = np.random.default_rng(P * 100 + h)
    b, S, d = 3, 70, 64
    q, k, v = randn(b, h, d, scale=2.0), randn(b, g, S, d), randn(b, g, S, d)
    lens = np.array([70, 17, 45], np.int32)
    kp, vp, bt = _paged_from_contiguous(k, v, P, rng)
    out, rc = oracle.decode_attn_paged(q, kp, vp, bt, lens, 0.125)
    assert rc == oracle.OK
    ref = sdpa_ref(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), lens, 0.125)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    flat, _, _ = oracle.decode_attn(q, k, v, lens, 0.125)
    assert np.array_equal(out, flat)


def test_paged_shared_prefix_page():
    """Two sequences may share a page (a common prefix): each reads it as its own."""
    rng = np.random.default_rng(5)
    b, h, g, S, d, P = 2, 4, 2, 48, 32, 16
    q, k, v = randn(b, h, d), randn(b, g, S, d), randn(b, g, S, d)
    k[1, :, :P], v[1, :, :P] = k[0, :, :P], v[0, :, :P]
    kp, vp, bt = _paged_from_contiguous(k, v, P, rng, share_prefix=True)
    lens = np.array([48, 40], np.int32)
    out, rc = oracle.decode_attn_paged(q, kp, vp, bt, lens, 0.2)
    assert rc == oracle.OK
    flat, _, _ = oracle.decode_attn(q, k, v, lens, 0.2)
    assert np.array_equal(out, flat)


def test_paged_entries_past_length_are_not_read():
    """Block-table entries past ceil(L/P) may be anything (here -1 and huge ids)."""
    rng = np.random.default_rng(6)
    b, h, g, S, d, P = 2, 4, 1, 64, 32, 16
    q, k, v = randn(b, h, d), randn(b, g, S, d), randn(b, g, S, d)
    kp, vp, bt = _paged_from_contiguous(k, v, P, rng)
    lens = np.array([17, 33], np.int32)
    bt[0, 2:] = -1
    bt[1, 3:] = 1 << 30
    out, rc = oracle.decode_attn_paged(q, kp, vp, bt, lens, 0.2)
    assert rc == oracle.OK and np.isfinite(out).all()
    flat, _, _ = oracle.decode_attn(q, k, v, lens, 0.2)
    assert np.array_equal(out, flat)


def test_paged_bad_page_is_flagged():
    """A page id outside [0, num_pages) among the attended positions: that
    sequence's rows are NaN and the status says so; the others are untouched."""
    rng = np.random.default_rng(7)
    b, h, g, S, d, P = 2, 4, 2, 32, 16, 16
    q, k, v = randn(b, h, d), randn(b, g, S, d), randn(b, g, S, d)
    kp, vp, bt = _paged_from_contiguous(k, v, P, rng)
    bt[1, 1] = kp.shape[0]
    lens = np.array([32, 20], np.int32)
    out, rc = oracle.decode_attn_paged(q, kp, vp, bt, lens, 0.25)
    assert rc & oracle.BAD_PAGE
    assert np.isnan(out[1]).all() and np.isfinite(out[0]).all()


def test_paged_append_writes_one_row():
    rng = np.random.default_rng(8)
    b, g, S, d, P = 3, 2, 40, 16, 16
    k, v = randn(b, g, S, d), randn(b, g, S, d)
    kp, vp, bt = _paged_from_contiguous(k, v, P, rng, extra_pages=2)
    kn, vn = randn(b, g, d), randn(b, g, d)
    lens = np.array([1, 16, 40], np.int32)
    kp0, vp0 = kp.copy(), vp.copy()
    assert oracle.append_kv_paged(kp, vp, kn, vn, bt, lens) == oracle.OK
    for i, L in enumerate(lens):
        page, row = bt[i, (L - 1) // P], (L - 1) % P
        assert np.array_equal(kp[page, :, row], kn[i]) and np.array_equal(vp[page, :, row], vn[i])
        kp0[page, :, row], vp0[page, :, row] = kn[i], vn[i]
    assert np.array_equal(kp, kp0, equal_nan=True) and np.array_equal(vp, vp0, equal_nan=True)
    bt[0, 0] = -3
    assert oracle.append_kv_paged(kp, vp, kn, vn, bt, lens) & oracle.BAD_PAGE


@pytest.mark.parametrize("h,g", [(8, 2), (12, 3), (16, 4)])
def test_group_map_is_repeat_interleave(h, g):
    """[GQA notes] §八: K/V heads repeated with repeat_interleave onto the query heads."""
    L, d = 25, 64
    q, k, v = randn(1, h, d), randn(1, g, L, d), randn(1, g, L, d)
    out, _, _ = oracle.decode_attn(q, k, v, np.array([L], np.int32), 0.125)
    G = h // g
    ref = oracle.mha_per_head(q[0], np.repeat(k[0], G, axis=0), np.repeat(v[0], G, axis=0), 0.125)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-14)
    # the other plausible map (head i -> K/V head i % g, i.e. tiling) must differ
    wrong = oracle.mha_per_head(q[0], np.tile(k[0], (G, 1, 1)), np.tile(v[0], (G, 1, 1)), 0.125)
    assert np.abs(wrong - out[0]).max() > 1e-3


def test_mqa_identical_queries_give_identical_heads():
    """g = 1 ([GQA notes] §三): all heads share one K/V, so equal q rows give equal outputs."""
    row = randn(1, 1, 128)
    q = np.ascontiguousarray(np.broadcast_to(row, (2, 16, 128)))
    k, v = randn(2, 1, 64, 128), randn(2, 1, 64, 128)
    out, _, _ = oracle.decode_attn(q, k, v, np.array([64, 20], np.int32), 0.088)
    for hq in range(16):
        np.testing.assert_array_equal(out[:, hq], out[:, 0])


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_permutation_of_positions():
    q, k, v = randn(1, 4, 64), randn(1, 1, 30, 64), randn(1, 1, 30, 64)
    perm = RNG.permutation(30)
    out1, _, _ = oracle.decode_attn(q, k, v, np.array([30], np.int32), 0.125)
    out2, _, _ = oracle.decode_attn(q, np.ascontiguousarray(k[:, :, perm]),
                                    np.ascontiguousarray(v[:, :, perm]), np.array([30], np.int32), 0.125)
    np.testing.assert_allclose(out1, out2, rtol=1e-12, atol=1e-14)


def test_shift_of_keys():
    """Adding one vector c to every key adds q.c to every score: softmax unchanged."""
    q = np.round(randn(1, 2, 64) * 4) / 4
    k = np.round(randn(1, 1, 20, 64) * 4) / 4
    c = np.round(randn(1, 1, 1, 64) * 4) / 4  # quarter-integers: k + c stays exact in fp32
    v = randn(1, 1, 20, 64)
    out1, _, _ = oracle.decode_attn(q, k, v, np.array([20], np.int32), 0.125)
    out2, _, _ = oracle.decode_attn(q, np.ascontiguousarray(k + c), v, np.array([20], np.int32), 0.125)
    np.testing.assert_allclose(out1, out2, rtol=1e-10, atol=1e-12)


def test_positions_past_length_are_never_read():
    q, k, v = randn(2, 4, 64), randn(2, 2, 40, 64), randn(2, 2, 40, 64)
    lens = np.array([25, 40], np.int32)
    out1, _, _ = oracle.decode_attn(q, k, v, lens, 0.125)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 25:] = np.nan
    v2[0, :, 25:] = np.inf
    out2, _, _ = oracle.decode_attn(q, k2, v2, lens, 0.125)
    np.testing.assert_array_equal(out1, out2)


@pytest.mark.parametrize("cuts", [[0, 64], [0, 1, 64], [0, 10, 20, 30, 64], [0, 63, 64], [0, 32, 32, 64]])
def test_shards_combine_to_the_whole(cuts):
    """Any partition of [0, L) into shards, merged by log-sum-exp, equals the whole row."""
    d, L = 64, 64
    q = randn(d, scale=3.0).astype(np.float64)
    K, V = randn(L, d).astype(np.float64), randn(L, d).astype(np.float64)
    ms, ls, os_ = [], [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        m, l, o = oracle.partial(q, K, V, 0.125, a, b)
        ms.append(m); ls.append(l); os_.append(o)
    merged = oracle.lse_combine(np.array(ms), np.array(ls), np.array(os_))
    whole = oracle.mha_per_head(q[None], K[None], V[None], 0.125)[0]
    np.testing.assert_allclose(merged, whole, rtol=1e-12, atol=1e-14)


def test_bf16_inputs_decode_exactly():
    """bfloat16 bits are widened exactly: bf16 input equals fp32 input of the same values."""
    q, k, v = randn(2, 8, 128), randn(2, 2, 33, 128), randn(2, 2, 33, 128)
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    lens = np.array([33, 9], np.int32)
    out_b, _, _ = oracle.decode_attn(qb, kb, vb, lens, 0.088)
    widen = lambda a: oracle.bf16_bits_to_f64(a).astype(np.float32)
    out_f, _, _ = oracle.decode_attn(widen(qb), widen(kb), widen(vb), lens, 0.088)
    np.testing.assert_array_equal(out_b, out_f)


def test_threads_do_not_change_results():
    q, k, v = randn(4, 8, 64), randn(4, 2, 50, 64), randn(4, 2, 50, 64)
    lens = np.array([50, 3, 17, 49], np.int32)
    o1, _, _ = oracle.decode_attn(q, k, v, lens, 0.125, nthreads=1)
    o4, _, _ = oracle.decode_attn(q, k, v, lens, 0.125, nthreads=4)
    np.testing.assert_array_equal(o1, o4)


# ---------------------------------------------------------------------------
# append and error reporting
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bf16", [False, True])
def test_append_writes_exactly_one_row_per_head(bf16):
    b, g, S, d = 3, 2, 10, 64
    kc, vc = randn(b, g, S, d), randn(b, g, S, d)
    kn, vn = randn(b, g, d), randn(b, g, d)
    if bf16:
        kc, vc, kn, vn = bf16_bits(kc), bf16_bits(vc), bf16_bits(kn), bf16_bits(vn)
    lens = np.array([1, 10, 4], np.int32)
    k2, v2 = kc.copy(), vc.copy()
    assert oracle.append_kv(k2, v2, kn, vn, lens) == oracle.OK
    ek, ev = kc.copy(), vc.copy()
    for i in range(b):
        ek[i, :, lens[i] - 1] = kn[i]
        ev[i, :, lens[i] - 1] = vn[i]
    assert k2.tobytes() == ek.tobytes() and v2.tobytes() == ev.tobytes()


def test_bad_lengths_are_reported_not_truncated():
    """[MQA blog] §4.3: running past the capacity must not truncate silently."""
    b, g, S, d = 3, 1, 8, 64
    kc, vc, kn, vn = randn(b, g, S, d), randn(b, g, S, d), randn(b, g, d), randn(b, g, d)
    lens = np.array([9, 0, 5], np.int32)
    k2, v2 = kc.copy(), vc.copy()
    assert oracle.append_kv(k2, v2, kn, vn, lens) == oracle.BAD_LEN
    np.testing.assert_array_equal(k2[:2], kc[:2])
    np.testing.assert_array_equal(k2[2, :, 4], kn[2])
    q = randn(b, 2, d)
    out, _, rc = oracle.decode_attn(q, kc, vc, lens, 0.125)
    assert rc == oracle.BAD_LEN
    assert np.isnan(out[:2]).all() and np.isfinite(out[2]).all()


def test_indivisible_heads_rejected():
    """[GQA notes] §十: h must be a multiple of g."""
    q, k, v = randn(1, 6, 64), randn(1, 4, 5, 64), randn(1, 4, 5, 64)
    _, _, rc = oracle.decode_attn(q, k, v, np.array([5], np.int32), 0.125)
    assert rc == oracle.BAD_SHAPE


# ---------------------------------------------------------------------------
# T query tokens per sequence with the causal mask ([GQA notes] §十 item 10)
# ---------------------------------------------------------------------------

def _causal_sdpa_last_rows(q_tok, k, v, L, scale, rng):
    """torch SDPA (float64) with is_causal=True over a full L-query problem whose
    last T query rows are q_tok [T, h, d] (the first L-T rows are arbitrary):
    row p of a causal L x L attention sees positions <= p, so the last T rows
    are the step's tokens at positions L-T .. L-1. k, v [g, >=L, d]."""
    T, h, d = q_tok.shape
    g = k.shape[0]
    qf = np.concatenate([rng.standard_normal((L - T, h, d)), q_tok], axis=0)  # [L, h, d]
    qt = torch.from_numpy(np.ascontiguousarray(qf.transpose(1, 0, 2))).view(1, h, L, d)
    kt = torch.from_numpy(np.ascontiguousarray(k[:, :L])).view(1, g, L, d)
    vt = torch.from_numpy(np.ascontiguousarray(v[:, :L])).view(1, g, L, d)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale, is_causal=True,
                                                         enable_gqa=(g != h))
    return o.view(h, L, d).numpy().transpose(1, 0, 2)[L - T:]  # [T, h, d]


@pytest.mark.parametrize("T,h,g", [(4, 8, 2), (3, 6, 6), (5, 8, 1)])
def test_multi_matches_causal_sdpa(T, h, g):
    """T tokens per sequence = the last T rows of torch's causal SDPA over the
    whole sequence (float64), for L > T and L = T (the whole prompt at once)."""
    rng = np.random.default_rng(T * 10 + h + g)
    b, S, d = 3, 40, 64
    q, k, v = randn(b, T, h, d, scale=2.0), randn(b, g, S, d), randn(b, g, S, d)
    lens = np.array([40, T, 23], np.int32)
    out, _, rc = oracle.decode_attn_multi(q, k, v, lens, 0.125)
    assert rc == oracle.OK
    for i in range(b):
        ref = _causal_sdpa_last_rows(q[i].astype(np.float64), k[i].astype(np.float64),
                                     v[i].astype(np.float64), int(lens[i]), 0.125, rng)
        np.testing.assert_allclose(out[i], ref, rtol=1e-10, atol=1e-12)


def test_multi_token_is_single_decode_over_its_prefix():
    """Token tau of a T-token step = the one-token decode (pinned above) of that
    token over the first L-T+1+tau positions; T = 1 is the one-token decode."""
    b, T, h, g, S, d = 2, 4, 8, 2, 30, 64
    q, k, v = randn(b, T, h, d), randn(b, g, S, d), randn(b, g, S, d)
    lens = np.array([30, 9], np.int32)
    out, _, rc = oracle.decode_attn_multi(q, k, v, lens, 0.125)
    assert rc == oracle.OK
    for tau in range(T):
        one, _, _ = oracle.decode_attn(np.ascontiguousarray(q[:, tau]), k, v, lens - T + 1 + tau, 0.125)
        np.testing.assert_array_equal(out[:, tau], one)
    one_tok, _, _ = oracle.decode_attn_multi(q[:, :1].copy(), k, v, lens, 0.125)
    flat, _, _ = oracle.decode_attn(np.ascontiguousarray(q[:, 0]), k, v, lens, 0.125)
    assert np.array_equal(one_tok[:, 0], flat)


def test_multi_weights_vanish_past_each_tokens_position():
    b, T, h, g, S, d = 1, 3, 4, 1, 12, 64
    q, k, v = randn(b, T, h, d), randn(b, g, S, d), randn(b, g, S, d)
    L = 10
    _, alpha, _ = oracle.decode_attn_multi(q, k, v, np.array([L], np.int32), 0.125, want_alpha=True)
    for tau in range(T):
        A = L - T + 1 + tau
        np.testing.assert_allclose(alpha[0, tau].sum(axis=-1), 1.0, rtol=1e-12)
        assert (alpha[0, tau, :, A:] == 0).all() and (alpha[0, tau, :, A - 1] > 0).all()


@pytest.mark.parametrize("bf16", [False, True])
def test_append_multi_writes_t_rows_per_head(bf16):
    b, T, g, S, d = 3, 3, 2, 10, 64
    kc, vc = randn(b, g, S, d), randn(b, g, S, d)
    kn, vn = randn(b, T, g, d), randn(b, T, g, d)
    if bf16:
        kc, vc, kn, vn = bf16_bits(kc), bf16_bits(vc), bf16_bits(kn), bf16_bits(vn)
    lens = np.array([3, 10, 7], np.int32)
    k2, v2 = kc.copy(), vc.copy()
    assert oracle.append_kv_multi(k2, v2, kn, vn, lens) == oracle.OK
    ek, ev = kc.copy(), vc.copy()
    for i in range(b):
        for tau in range(T):
            ek[i, :, lens[i] - T + tau] = kn[i, tau]
            ev[i, :, lens[i] - T + tau] = vn[i, tau]
    assert k2.tobytes() == ek.tobytes() and v2.tobytes() == ev.tobytes()


def test_multi_length_below_t_is_flagged():
    b, T, g, S, d = 2, 4, 1, 8, 64
    kc, vc = randn(b, g, S, d), randn(b, g, S, d)
    kn, vn = randn(b, T, g, d), randn(b, T, g, d)
    lens = np.array([3, 8], np.int32)
    k2, v2 = kc.copy(), vc.copy()
    assert oracle.append_kv_multi(k2, v2, kn, vn, lens) == oracle.BAD_LEN
    np.testing.assert_array_equal(k2[0], kc[0])
    out, _, rc = oracle.decode_attn_multi(randn(b, T, 2, d), kc, vc, lens, 0.125)
    assert rc == oracle.BAD_LEN
    assert np.isnan(out[0]).all() and np.isfinite(out[1]).all()


def test_paged_multi_matches_contiguous_multi():
    """Paged T-token decode = the contiguous one on the gathered cache (bitwise);
    the paged append writes T rows that may straddle a page boundary."""
    rng = np.random.default_rng(77)
    b, T, h, g, S, d, P = 3, 5, 8, 2, 48, 64, 16
    q, k, v = randn(b, T, h, d), randn(b, g, S, d), randn(b, g, S, d)
    lens = np.array([48, 18, 5], np.int32)  # 18: tokens at 13..17 straddle pages 0 and 1
    kp, vp, bt = _paged_from_contiguous(k, v, P, rng)
    out, rc = oracle.decode_attn_paged_multi(q, kp, vp, bt, lens, 0.125)
    assert rc == oracle.OK
    flat, _, _ = oracle.decode_attn_multi(q, k, v, lens, 0.125)
    assert np.array_equal(out, flat)
    kn, vn = randn(b, T, g, d), randn(b, T, g, d)
    assert oracle.append_kv_paged_multi(kp, vp, kn, vn, bt, lens) == oracle.OK
    assert oracle.append_kv_multi(k, v, kn, vn, lens) == oracle.OK
    for i in range(b):
        for t in range(int(lens[i])):
            page, row = bt[i, t // P], t % P
            np.testing.assert_array_equal(kp[page, :, row], k[i, :, t])
            np.testing.assert_array_equal(vp[page, :, row], v[i, :, t])


# ---------------------------------------------------------------------------
# fp8 e4m3 cache with per-K/V-head scales ([GQA notes] §十 item 7)
# ---------------------------------------------------------------------------

def _torch_fp8_values(codes: np.ndarray) -> np.ndarray:
    """Values of e4m3 codes by torch's float8_e4m3fn (a library decoder)."""
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_fp8_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = _torch_fp8_values(codes)
    got = np.array([oracle.fp8_decode(c) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert oracle.fp8_decode(0x7E) == 448.0 and oracle.fp8_decode(0x01) == 2.0 ** -9


def test_fp8_encode_matches_torch_in_range_and_saturates():
    rng = np.random.default_rng(8)
    reps = _torch_fp8_values(np.arange(256, dtype=np.uint8))
    finite = reps[np.isfinite(reps)]
    mids = (np.sort(np.unique(finite))[1:] + np.sort(np.unique(finite))[:-1]) / 2  # ties
    x = np.concatenate([finite, mids, rng.standard_normal(3000) * 30,
                        rng.standard_normal(1000) * 1e-3, [463.9, -463.9, 0.0, -0.0]])
    x = x.astype(np.float32)
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.fp8_encode(v) for v in x], np.uint8)
    assert np.array_equal(got, ref)
    # beyond the format: saturate at +-448 (torch's cast gives NaN there); NaN stays NaN
    for v, code in ((464.0, 0x7E), (1e30, 0x7E), (float("inf"), 0x7E), (-1e5, 0xFE),
                    (float("-inf"), 0xFE)):
        assert oracle.fp8_encode(v) == code
    assert oracle.fp8_encode(float("nan")) & 0x7F == 0x7F


def _fp8_case(rng, b, T, h, g, S, d):
    k = rng.integers(0, 256, (b, g, S, d), dtype=np.uint8)
    v = rng.integers(0, 256, (b, g, S, d), dtype=np.uint8)
    for c in (k, v):  # no NaN codes in a cache
        c[(c & 0x7F) == 0x7F] = 0x7E
    ks = (rng.uniform(0.005, 0.05, g)).astype(np.float32)
    vs = (rng.uniform(0.005, 0.05, g)).astype(np.float32)
    q = bf16_bits(randn(b, T, h, d))
    return q, k, v, ks, vs


@pytest.mark.parametrize("T,h,g", [(1, 8, 2), (1, 4, 4), (3, 8, 1), (1, 12, 3)])
def test_fp8_decode_matches_sdpa_on_dequantised_cache(T, h, g):
    """fp8 decode = torch SDPA (float64) on the cache dequantised by torch's
    e4m3 decoder times the head's scale; causal last-T rows for T > 1."""
    rng = np.random.default_rng(T * 100 + h * 10 + g)
    b, S, d = 3, 40, 64
    q, k, v, ks, vs = _fp8_case(rng, b, T, h, g, S, d)
    lens = np.array([40, T + 3, 17], np.int32)
    out, rc = oracle.decode_attn_fp8(q, k, v, ks, vs, lens, 0.125)
    assert rc == oracle.OK
    kd = _torch_fp8_values(k) * ks[None, :, None, None].astype(np.float64)
    vd = _torch_fp8_values(v) * vs[None, :, None, None].astype(np.float64)
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).double().numpy()
    for i in range(b):
        ref = _causal_sdpa_last_rows(qd[i], kd[i], vd[i], int(lens[i]), 0.125, rng)
        np.testing.assert_allclose(out[i], ref, rtol=1e-10, atol=1e-12)


def test_fp8_paged_matches_contiguous():
    rng = np.random.default_rng(81)
    b, T, h, g, S, d, P = 3, 2, 8, 2, 48, 64, 16
    q, k, v, ks, vs = _fp8_case(rng, b, T, h, g, S, d)
    lens = np.array([48, 18, 5], np.int32)
    kp, vp, bt = _paged_from_contiguous(k, v, P, rng)
    kp[np.isnan(kp.astype(np.float32))] = 0  # (uint8 pages carry no NaN marker)
    out, rc = oracle.decode_attn_paged_fp8(q, kp, vp, ks, vs, bt, lens, 0.125)
    assert rc == oracle.OK
    flat, _ = oracle.decode_attn_fp8(q, k, v, ks, vs, lens, 0.125)
    assert np.array_equal(out, flat)
    kn, vn = bf16_bits(randn(b, T, g, d)), bf16_bits(randn(b, T, g, d))
    assert oracle.append_kv_paged_fp8(kp, vp, kn, vn, ks, vs, bt, lens) == oracle.OK
    assert oracle.append_kv_fp8(k, v, kn, vn, ks, vs, lens) == oracle.OK
    for i in range(b):
        for t in range(int(lens[i])):
            np.testing.assert_array_equal(kp[bt[i, t // P], :, t % P], k[i, :, t])
            np.testing.assert_array_equal(vp[bt[i, t // P], :, t % P], v[i, :, t])


@pytest.mark.parametrize("T", [1, 3])
def test_fp8_append_quantises_with_the_head_scale(T):
    """Codes of the appended rows = torch's e4m3 cast of (x / scale) in float32
    (in range), at positions L-T .. L-1; every other byte untouched."""
    rng = np.random.default_rng(90 + T)
    b, g, S, d = 3, 2, 12, 64
    k = rng.integers(0, 126, (b, g, S, d), dtype=np.uint8)
    v = rng.integers(0, 126, (b, g, S, d), dtype=np.uint8)
    ks = np.array([0.01, 0.03], np.float32)
    vs = np.array([0.02, 0.012], np.float32)  # |x / scale| stays below 448
    kn, vn = randn(b, T, g, d), randn(b, T, g, d)
    lens = np.array([T, 12, 7], np.int32)
    k2, v2 = k.copy(), v.copy()
    assert oracle.append_kv_fp8(k2, v2, kn, vn, ks, vs, lens) == oracle.OK
    ek, ev = k.copy(), v.copy()
    cast = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i in range(b):
        for tau in range(T):
            pos = lens[i] - T + tau
            ek[i, :, pos] = cast((torch.from_numpy(kn[i, tau]) / torch.from_numpy(ks)[:, None]).numpy())
            ev[i, :, pos] = cast((torch.from_numpy(vn[i, tau]) / torch.from_numpy(vs)[:, None]).numpy())
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)


# ---------------------------------------------------------------------------
# int8 cache with per-K/V-head scales (the pages' INT8 K/V)
# ---------------------------------------------------------------------------

def test_int8_decode_is_twos_complement():
    """All 256 codes against torch's int8 reading of the same bytes."""
    codes = np.arange(256, dtype=np.uint8).view(np.int8)
    ref = torch.from_numpy(codes.copy()).double().numpy()
    got = np.array([oracle.int8_decode(int(c)) for c in codes])
    assert np.array_equal(got, ref)
    assert oracle.int8_decode(-1) == -1.0 and oracle.int8_decode(-128) == -128.0


def test_int8_encode_matches_torch_round_and_saturates():
    """Nearest integer with ties to even (torch.round), clamped to +-127; the
    ties k + 0.5 and the saturation edges explicitly; NaN to 0."""
    rng = np.random.default_rng(13)
    xs = np.concatenate([rng.uniform(-140, 140, 4000), np.arange(-130, 131) + 0.5,
                         [126.49, 126.5, 127.5, 128.0, -127.5, -128.0, -1e30, 1e30, 0.0, -0.0]])
    xs = xs.astype(np.float32)
    ref = torch.round(torch.from_numpy(xs)).clamp(-127, 127).to(torch.int8).numpy()
    got = np.array([oracle.int8_encode(x) for x in xs], np.int8)
    assert np.array_equal(got, ref)
    assert oracle.int8_encode(float("nan")) == 0
    assert oracle.int8_encode(-128.0) == -127  # -128 is never produced


def _int8_case(rng, b, T, h, g, S, d):
    k = rng.integers(-127, 128, (b, g, S, d), dtype=np.int8)
    v = rng.integers(-127, 128, (b, g, S, d), dtype=np.int8)
    ks = (rng.uniform(0.005, 0.03, g)).astype(np.float32)
    vs = (rng.uniform(0.005, 0.03, g)).astype(np.float32)
    q = bf16_bits(randn(b, T, h, d))
    return q, k, v, ks, vs


@pytest.mark.parametrize("T,h,g,W", [(1, 8, 2, 0), (3, 8, 1, 0), (1, 12, 3, 0), (2, 8, 2, 9)])
def test_int8_decode_matches_sdpa_on_dequantised_cache(T, h, g, W):
    """int8 decode (through the general call) = torch SDPA (float64) on the
    codes times the head's scale; causal last-T rows; a window where given."""
    rng = np.random.default_rng(T * 100 + h * 10 + g + W)
    b, S, d = 3, 40, 64
    q, k, v, ks, vs = _int8_case(rng, b, T, h, g, S, d)
    lens = np.array([40, T + 3, 17], np.int32)
    out, rc = oracle.decode_attn_ex(q, k, v, lens, 0.125, window=W, k_scale=ks, v_scale=vs)
    assert rc == oracle.OK
    kd = torch.from_numpy(k).double().numpy() * ks[None, :, None, None].astype(np.float64)
    vd = torch.from_numpy(v).double().numpy() * vs[None, :, None, None].astype(np.float64)
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).double().numpy()
    for i in range(b):
        if W == 0:
            ref = _causal_sdpa_last_rows(qd[i], kd[i], vd[i], int(lens[i]), 0.125, rng)
            np.testing.assert_allclose(out[i], ref, rtol=1e-10, atol=1e-12)
        else:
            for tau in range(T):
                A = int(lens[i]) - T + 1 + tau
                a0 = max(0, A - W)
                ref = _sdpa_rows(qd[i, tau], kd[i, :, a0:A], vd[i, :, a0:A], 0.125)
                np.testing.assert_allclose(out[i, tau], ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("T", [1, 3])
def test_int8_append_quantises_with_the_head_scale(T):
    """Codes of the appended rows = torch.round(x / scale) clamped to +-127
    (the division in float32), at positions L-T .. L-1, contiguous and paged;
    every other byte untouched. Large values saturate."""
    rng = np.random.default_rng(95 + T)
    b, g, S, d, P = 3, 2, 32, 64, 16
    k = rng.integers(-127, 128, (b, g, S, d), dtype=np.int8)
    v = rng.integers(-127, 128, (b, g, S, d), dtype=np.int8)
    ks = np.array([0.01, 0.03], np.float32)
    vs = np.array([0.02, 0.012], np.float32)
    kn, vn = randn(b, T, g, d, scale=1.5), randn(b, T, g, d, scale=1.5)  # some beyond 127 * scale
    lens = np.array([T, 32, 7], np.int32)
    kp, vp, bt = _paged_from_contiguous(k.astype(np.float32), v.astype(np.float32), P, rng)
    kp = np.nan_to_num(kp).astype(np.int8)
    vp = np.nan_to_num(vp).astype(np.int8)
    k2, v2 = k.copy(), v.copy()
    assert oracle.append_kv_int8(k2, v2, kn, vn, ks, vs, lens) == oracle.OK
    assert oracle.append_kv_paged_int8(kp, vp, kn, vn, ks, vs, bt, lens) == oracle.OK
    ek, ev = k.copy(), v.copy()
    q8 = lambda x, sc: torch.round(torch.from_numpy(x) / torch.from_numpy(sc)[:, None]).clamp(-127, 127).to(torch.int8).numpy()
    for i in range(b):
        for tau in range(T):
            pos = lens[i] - T + tau
            ek[i, :, pos] = q8(kn[i, tau], ks)
            ev[i, :, pos] = q8(vn[i, tau], vs)
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)
    assert (np.abs(ek.astype(np.int32)) == 127).any()  # the saturation was exercised
    for i in range(b):
        for t in range(int(lens[i])):
            np.testing.assert_array_equal(kp[bt[i, t // P], :, t % P], k2[i, :, t])
            np.testing.assert_array_equal(vp[bt[i, t // P], :, t % P], v2[i, :, t])


# ---------------------------------------------------------------------------
# sliding window ([MQA concept] 玩家對比: GQA + SWA) and rotary positions
# ---------------------------------------------------------------------------

def _sdpa_rows(q_rows, k, v, scale):
    """torch SDPA (float64) of query rows [h, d] over k, v [g, n, d]."""
    h, d = q_rows.shape
    g, n, _ = k.shape
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.ascontiguousarray(q_rows)).view(1, h, 1, d),
        torch.from_numpy(np.ascontiguousarray(k)).view(1, g, n, d),
        torch.from_numpy(np.ascontiguousarray(v)).view(1, g, n, d), scale=scale,
        enable_gqa=(g != h))
    return o.view(h, d).numpy()


@pytest.mark.parametrize("T,W", [(1, 5), (1, 32), (3, 7), (2, 1)])
def test_window_matches_sdpa_on_the_window(T, W):
    """Each token sees only its last W positions: torch SDPA over that slice."""
    b, h, g, S, d = 3, 8, 2, 40, 64
    q, k, v = randn(b, T, h, d), randn(b, g, S, d), randn(b, g, S, d)
    lens = np.array([40, T + 2, 23], np.int32)
    out, rc = oracle.decode_attn_ex(q, k, v, lens, 0.125, window=W)
    assert rc == oracle.OK
    for i in range(b):
        for tau in range(T):
            A = int(lens[i]) - T + 1 + tau
            a0 = max(0, A - W)
            ref = _sdpa_rows(q[i, tau].astype(np.float64), k[i, :, a0:A].astype(np.float64),
                             v[i, :, a0:A].astype(np.float64), 0.125)
            np.testing.assert_allclose(out[i, tau], ref, rtol=1e-10, atol=1e-12)


def test_window_special_cases():
    b, h, g, S, d = 2, 4, 1, 20, 64
    q, k, v = randn(b, h, d), randn(b, g, S, d), randn(b, g, S, d)
    lens = np.array([20, 9], np.int32)
    full, _, _ = oracle.decode_attn(q, k, v, lens, 0.125)
    wide, _ = oracle.decode_attn_ex(q, k, v, lens, 0.125, window=20)
    assert np.array_equal(full, wide)  # a window at least the length changes nothing
    one, _ = oracle.decode_attn_ex(q, k, v, lens, 0.125, window=1)
    for i in range(b):  # a window of one position returns that position's value row
        np.testing.assert_allclose(one[i], np.broadcast_to(v[i, 0, lens[i] - 1], (h, d)), rtol=1e-12)
    # fp8 and paged forms of the general call agree with the dedicated ones
    rng = np.random.default_rng(5)
    qb, kc, vc, ks, vs = _fp8_case(rng, b, 1, h, g, S, d)
    f8, _ = oracle.decode_attn_fp8(qb, kc, vc, ks, vs, lens, 0.125)
    ex, _ = oracle.decode_attn_ex(qb, kc, vc, lens, 0.125, k_scale=ks, v_scale=vs)
    assert np.array_equal(f8, ex)
    kp, vp, bt = _paged_from_contiguous(k, v, 16, rng)
    pg, _ = oracle.decode_attn_paged(q, kp, vp, bt, lens, 0.125)
    ex2, _ = oracle.decode_attn_ex(q, kp, vp, lens, 0.125, block_table=bt)
    assert np.array_equal(pg, ex2)


def _bf16_val(bits_arr):
    return torch.from_numpy(np.ascontiguousarray(bits_arr).view(np.int16)).view(torch.bfloat16).double().numpy()


def test_rope_table_closed_forms():
    d, base = 64, 10000.0
    t = oracle.rope_table(base, 50, d)
    p = np.arange(50)
    np.testing.assert_array_equal(t[:, 0, 0], np.cos(p).astype(np.float32))  # pair 0: angle p
    np.testing.assert_array_equal(t[:, 0, 1], np.sin(p).astype(np.float32))
    th = base ** (-2.0 * np.arange(d // 2) / d)
    np.testing.assert_array_equal(t[1, :, 0], np.cos(th).astype(np.float32))
    np.testing.assert_array_equal(t[7, :, 1], np.sin(7 * th).astype(np.float32))
    assert (t[0, :, 0] == 1).all() and (t[0, :, 1] == 0).all()


def test_rope_rotation_properties():
    """Position 0 is the identity; each pair (i, i + d/2) keeps its length;
    rotated dot products depend only on the distance of the positions."""
    d = 64
    t = oracle.rope_table(10000.0, 200, d)
    x = bf16_bits(randn(6, d))
    assert np.array_equal(oracle.rope_rows(x, np.zeros(6, np.int32), t), x)
    # a unit vector in element i turns towards element i + d/2: (cos, sin) of the pair's angle
    for i in (0, 5, d // 2 - 1):
        e = np.zeros((1, d), np.float32)
        e[0, i] = 1.0
        r = _bf16_val(oracle.rope_rows(bf16_bits(e), np.array([37], np.int32), t))[0]
        expect = np.zeros(d)
        expect[i], expect[i + d // 2] = t[37, i, 0], t[37, i, 1]
        np.testing.assert_allclose(r, expect, rtol=2 ** -8, atol=1e-30)
    pos = np.array([0, 3, 17, 64, 150, 199], np.int32)
    y = _bf16_val(oracle.rope_rows(x, pos, t))
    xv = _bf16_val(x)
    n0 = xv[:, :d // 2] ** 2 + xv[:, d // 2:] ** 2
    n1 = y[:, :d // 2] ** 2 + y[:, d // 2:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=2e-2, atol=1e-3)  # bf16 rounding of the results
    # the pair convention: (i, i + d/2) -- adjacent pairs (2i, 2i+1) would not keep these norms
    qrow, krow = bf16_bits(randn(1, d)), bf16_bits(randn(1, d))
    dots = []
    for p1, p2 in ((10, 4), (56, 50), (199, 193), (106, 100)):  # distance 6 each time
        a = _bf16_val(oracle.rope_rows(qrow, np.array([p1], np.int32), t))[0]
        b_ = _bf16_val(oracle.rope_rows(krow, np.array([p2], np.int32), t))[0]
        dots.append(a @ b_)
    far = _bf16_val(oracle.rope_rows(krow, np.array([180], np.int32), t))[0] @ \
        _bf16_val(oracle.rope_rows(qrow, np.array([10], np.int32), t))[0]
    assert np.ptp(dots) < 0.05 * np.abs(dots).max() + 0.05
    assert abs(far - dots[0]) > 0.05  # another distance, another product


def test_rope_append_and_q():
    rng = np.random.default_rng(12)
    b, T, g, S, d, h = 3, 2, 2, 16, 64, 4
    t = oracle.rope_table(10000.0, S, d)
    kc, vc = bf16_bits(randn(b, g, S, d)), bf16_bits(randn(b, g, S, d))
    kn, vn = bf16_bits(randn(b, T, g, d)), bf16_bits(randn(b, T, g, d))
    lens = np.array([2, 16, 9], np.int32)
    k2, v2 = kc.copy(), vc.copy()
    assert oracle.append_kv_rope(k2, v2, kn, vn, t, lens) == oracle.OK
    ek, ev = kc.copy(), vc.copy()
    for i in range(b):
        for tau in range(T):
            pos = lens[i] - T + tau
            ek[i, :, pos] = oracle.rope_rows(kn[i, tau], np.full(g, pos, np.int32), t)
            ev[i, :, pos] = vn[i, tau]
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)
    q = bf16_bits(randn(b, T, h, d))
    qr, rc = oracle.rope_q(q, t, lens)
    assert rc == oracle.OK
    for i in range(b):
        for tau in range(T):
            pos = np.full(h, lens[i] - T + tau, np.int32)
            assert np.array_equal(qr[i, tau], oracle.rope_rows(q[i, tau], pos, t))
    del rng


# ---------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle's source must fail a pin above
# ---------------------------------------------------------------------------

MUTANTS = {
    "group map i % g": ("int j = hq / G;", "int j = hq % J->g;"),
    "scale dropped": ("s[t] = J->scale * dot;", "s[t] = dot;"),
    "attended length off by one": ("for (int t = a0; t < A; t++) {\n        double dot", "for (int t = a0; t < A - 1; t++) {\n        double dot"),
    "window one position short": ("? A - J->window : 0;", "? A - J->window + 1 : 0;"),
    "window ignored": ("int a0 = (J->window > 0 && A > J->window)", "int a0 = (0 && A > J->window)"),
    "rope pairs adjacent": ("float b = (float)elem(row, (size_t)(i + hd), ORACLE_BF16);", "float b = (float)elem(row, (size_t)(i ^ 1), ORACLE_BF16);"),
    "rope sine sign flipped": ("float ra = ac - bs, rb = bc + as;", "float ra = ac + bs, rb = bc - as;"),
    "rope angle exponent over d/2": ("double th = pow(base, -2.0 * i / d);", "double th = pow(base, -1.0 * i / d);"),
    "causal mask dropped": ("int A = L - J->T + 1 + tau;", "int A = L;"),
    "token order reversed": ("int A = L - J->T + 1 + tau;", "int A = L - tau;"),
    "every token uses the first token's query": ("size_t qoff = (size_t)row * d;", "size_t qoff = ((size_t)i * J->T * J->h + hq) * d;"),
    "appended tokens reversed": ("* S + (size_t)(L - T + tau)) * row;", "* S + (size_t)(L - 1 - tau)) * row;"),
    "fp8 exponent bias off by one": ("(1.0 + m / 8.0) * ldexp(1.0, e - 7)", "(1.0 + m / 8.0) * ldexp(1.0, e - 8)"),
    "fp8 subnormal scale wrong": ("(m / 8.0) * ldexp(1.0, -6)", "(m / 8.0) * ldexp(1.0, -7)"),
    "fp8 ties rounded away from zero": ("int sm = (int)nearbyintf(fr * 16.0f);", "int sm = (int)roundf(fr * 16.0f);"),
    "key scale ignored": ("double ks = J->k_scale ? (double)J->k_scale[j] : 1.0;", "double ks = 1.0;"),
    "value scale of the key": ("double vs = J->v_scale ? (double)J->v_scale[j] : 1.0;", "double vs = J->k_scale ? (double)J->k_scale[j] : 1.0;"),
    "quantised by multiplying": ("float y = x / scale;", "float y = x * scale;"),
    "int8 ties rounded away from zero": ("float r = nearbyintf(f);", "float r = roundf(f);"),
    "int8 saturates one step too far": ("if (r > 127.0f) r = 127.0f;", "if (r > 128.0f) r = 128.0f;"),
    "int8 codes read as unsigned": ("return oracle_int8_decode(((const int8_t *)base)[idx]);", "return oracle_int8_decode((int8_t)((const uint8_t *)base)[idx] & 0x7F);"),
    "no normalisation": ("for (int t = a0; t < A; t++) s[t] /= Z;", ""),
    "key and value swapped": ("elem(J->v, (size_t)kv_row(J, i, j, t) + x, J->dtype));\n        o[x]", "elem(J->k, (size_t)kv_row(J, i, j, t) + x, J->dtype));\n        o[x]"),
    "page looked up one position late": ("(size_t)i * J->max_pages + t / J->page_size]", "(size_t)i * J->max_pages + (t + 1) / J->page_size]"),
    "row within the page ignored": ("J->page_size + t % J->page_size) * J->d", "J->page_size) * J->d"),
    "query index transposed": ("elem(J->q, qoff + x, J->q_dtype)", "elem(J->q, (size_t)x * J->h + hq, J->q_dtype)"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert old in src, f"mutation anchor for '{name}' not found"
    path = tmp_path / (re.sub(r"\W+", "_", name) + ".c")
    path.write_text(src.replace(old, new, 1))
    (tmp_path / "oracle.h").write_text(open(os.path.join(os.path.dirname(oracle.__file__), "oracle.h")).read())
    so = str(path)[:-2] + ".so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", so, str(path), "-lm"], check=True)
    return so


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistakes_are_caught(tmp_path, name, monkeypatch):
    import ctypes
    so = _build_mutant(tmp_path, name, *MUTANTS[name])
    mutant = ctypes.CDLL(so)
    real = oracle.lib()
    # reuse the argument declarations of the real library
    for fn in ("oracle_decode_attn", "oracle_mha_per_head", "oracle_decode_attn_paged",
               "oracle_decode_attn_multi", "oracle_decode_attn_paged_multi",
               "oracle_append_kv_multi", "oracle_append_kv_paged_multi",
               "oracle_fp8_e4m3_decode", "oracle_fp8_e4m3_encode", "oracle_decode_attn_fp8",
               "oracle_decode_attn_paged_fp8", "oracle_append_kv_fp8", "oracle_append_kv_paged_fp8",
               "oracle_decode_attn_ex", "oracle_rope_table", "oracle_rope_rows", "oracle_rope_q",
               "oracle_append_kv_rope", "oracle_int8_decode", "oracle_int8_encode",
               "oracle_append_kv_int8", "oracle_append_kv_paged_int8"):
        getattr(mutant, fn).argtypes = getattr(real, fn).argtypes
        getattr(mutant, fn).restype = getattr(real, fn).restype
    monkeypatch.setattr(oracle, "_lib", mutant)
    caught = []
    for pin in (test_hand_example, lambda: test_matches_torch_sdpa(12, 4),
                lambda: test_matches_torch_sdpa(8, 8),
                lambda: test_paged_matches_gathered_sdpa(16, 8, 2),
                lambda: test_multi_matches_causal_sdpa(4, 8, 2),
                lambda: test_append_multi_writes_t_rows_per_head(False),
                test_fp8_decode_matches_torch, test_fp8_encode_matches_torch_in_range_and_saturates,
                lambda: test_fp8_decode_matches_sdpa_on_dequantised_cache(1, 8, 2),
                lambda: test_fp8_append_quantises_with_the_head_scale(1),
                lambda: test_window_matches_sdpa_on_the_window(3, 7), test_window_special_cases,
                test_rope_table_closed_forms, test_rope_rotation_properties,
                test_int8_decode_is_twos_complement,
                test_int8_encode_matches_torch_round_and_saturates,
                lambda: test_int8_decode_matches_sdpa_on_dequantised_cache(1, 8, 2, 0),
                lambda: test_int8_append_quantises_with_the_head_scale(1)):
        try:
            pin()
        except AssertionError:
            caught.append(pin)
    assert caught, f"mutant '{name}' passed every pin"
