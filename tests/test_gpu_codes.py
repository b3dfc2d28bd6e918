"""The one-byte caches over their whole code space, on the GPU.

A quantised KV cache is to be validated on its own ([GQA notes] §十 item 7),
so every code a cache can hold is made to reach the output here: the 254
finite fp8 e4m3 codes (0x7F and 0xFF are NaN: subnormals with exponent field 0,
both zeros, and the 256..448 binade included) and all 256 int8 codes
(-128 .. 127, -128 included although the append never writes it).

* Values, exactly. With one visible position its softmax weight is exactly 1,
  so out = v_scale * value(code): one fp32 rounding of a product of two exact
  fp32 numbers on the GPU, the double product rounded once to fp32 in the
  oracle. The row of V enumerates the codes; GPU and oracle must agree bit for
  bit.
* Keys, through the scores. Two visible positions: position 0 with zero codes
  in K and V, position 1 with the code under test in column x of K and V = 1
  (code of 1.0). Query head hq is one-hot in column x(hq), its value chosen so
  that the score of position 1 is about +-1; then out = v_scale * sigmoid(s1)
  and a key decoded wrongly by a factor of 2 (one exponent step) or one
  mantissa step moves out far beyond 2e-3. GPU against the oracle at the
  usual bound.

Every case runs on the fixed partitions (16 units) and the balanced schedule
(256 units), contiguous and paged (pages of 16 rows). Rows past the visible
positions hold NaN codes (fp8) or -128 (int8) and are never read. The inputs
are built with torch's own fp8 and int8 readings (a library, independent of
both the kernels and the oracle).
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
import transformer_decode_attention_amd as mqa

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL = 2e-3
RTOL_ROW = 2e-3
NTHREADS = min(16, os.cpu_count() or 1)
H, G, D, S = 32, 2, 128, 32   # h/g = 16: one matrix block per unit

FP8_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
INT8_CODES = np.arange(-128, 128, dtype=np.int16).astype(np.int8)


def code_values(codes: np.ndarray) -> np.ndarray:
    """What torch reads each code as (float64)."""
    t = torch.from_numpy(codes.copy())
    if codes.dtype == np.uint8:
        t = t.view(torch.float8_e4m3fn)
    return t.double().numpy()


def pad_code(kind: str):
    return (np.uint8(0x7F), np.uint8(0x38)) if kind == "fp8" else (np.int8(-128), np.int8(1))


def build(kind: str, b: int, what: str, seed: int):
    """Caches [b, G, S, D] of codes, q [b, H, D] bf16, lengths and scales.
    what = "values": L = 1, V row 0 walks the code list; "keys": L = 2, K row 1
    holds one code under test per query head."""
    rng = np.random.default_rng(seed)
    codes = FP8_CODES if kind == "fp8" else INT8_CODES
    nan_code, one_code = pad_code(kind)
    k = np.full((b, G, S, D), nan_code, codes.dtype)
    v = np.full((b, G, S, D), nan_code, codes.dtype)
    ks = (0.25 + 1.5 * rng.random(G)).astype(np.float32)
    vs = (0.25 + 1.5 * rng.random(G)).astype(np.float32)
    if kind == "int8":
        ks /= 32
        vs /= 32
    q = np.zeros((b, H, D), np.float32)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    if what == "values":
        L = 1
        k[:, :, 0, :] = 0
        start = rng.integers(0, len(codes))
        for u in range(b * G):
            i, j = divmod(u, G)
            v[i, j, 0, :] = codes[(start + u * D + np.arange(D)) % len(codes)]
        q[:] = rng.standard_normal(q.shape)
    else:
        L = 2
        k[:, :, 0, :] = 0
        v[:, :, 0, :] = 0
        v[:, :, 1, :] = one_code
        k[:, :, 1, :] = codes[rng.integers(0, len(codes), (b, G, D))]  # not looked at by q
        vals = code_values(codes)
        Gh = H // G
        for u in range(b * G):
            i, j = divmod(u, G)
            for hh in range(Gh):
                c = (u * Gh + hh) % len(codes)
                x = (hh * 7 + u) % D          # the column this head looks at
                k[i, j, 1, x] = codes[c]
                val = vals[c] * ks[j]
                q[i, j * Gh + hh, x] = 1.0 if val == 0 else 1.0 / (scale * val)
    lens = np.full(b, L, np.int32)
    return k, v, ks, vs, q, lens, scale


def paged(c: np.ndarray, P: int = 16):
    """The same cache cut into pages of P rows, page ids reversed in the pool."""
    b, g, s, d = c.shape
    maxp = s // P
    pages = c.reshape(b, g, maxp, P, d).transpose(0, 2, 1, 3, 4).reshape(b * maxp, g, P, d)
    ids = np.arange(b * maxp, dtype=np.int32)[::-1].copy()
    pool = np.empty_like(pages)
    pool[ids] = pages
    return np.ascontiguousarray(pool), ids.reshape(b, maxp)


def run(kind: str, b: int, what: str, page: bool, seed: int):
    print(f"[codes] {kind} {what} b={b} paged={page}", flush=True)
    k, v, ks, vs, q, lens, scale = build(kind, b, what, seed)
    bt = None
    if page:
        k, bt = paged(k)
        v, _ = paged(v)
    qt = torch.from_numpy(q).to(torch.bfloat16)
    q_bits = qt.view(torch.int16).numpy().view(np.uint16)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = mqa.decode_attn_ex(qt.to(DEV), dev(k), dev(v), dev(lens),
                             block_table=None if bt is None else dev(bt),
                             k_scale=dev(ks), v_scale=dev(vs), err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref, rc = oracle.decode_attn_ex(q_bits, k, v, lens, scale, k_scale=ks, v_scale=vs,
                                    block_table=bt, nthreads=NTHREADS)
    assert rc == oracle.OK
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all()
    if what == "values":
        want = ref.astype(np.float32).astype(np.float64)  # the oracle's one rounding to fp32
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[0]}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"
        # and they are the scaled code values (every code reached the output)
        vals = code_values(v if bt is None else build(kind, b, what, seed)[1])
        assert np.array_equal(want[:, 0, :], (vals[:, 0, 0, :] * vs[0]).astype(np.float32).astype(np.float64))
    else:
        e = np.abs(got - ref)
        rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
        assert e.max() <= ATOL and (e / np.maximum(np.abs(ref), rms)).max() <= RTOL_ROW, \
            f"abs {e.max()} rel {(e / np.maximum(np.abs(ref), rms)).max()}"
        # the scores were about +-1: outputs spread between sigmoid(-1) and sigmoid(1)
        assert (ref[:, :, 0] / np.repeat(vs, H // G)[None, :] > 0.2).all()


@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("what", ["values", "keys"])
@pytest.mark.parametrize("b", [8, 128])
@pytest.mark.parametrize("page", [False, True])
def test_code_space(kind, what, b, page):
    sched = mqa.decode_multi_schedule(b, 1, H, G, S, D, mqa.BF16)
    assert sched == ("mfma-balanced" if b * G >= 256 else "mfma-partitions")
    run(kind, b, what, page, seed=1200 + 3 * b + (what == "keys") + 7 * page + 11 * (kind == "int8"))


def test_every_code_is_covered():
    """The unit and head walks above touch every code (CPU-side check of the
    construction, run with the GPU cases)."""
    for kind in ("fp8", "int8"):
        codes = FP8_CODES if kind == "fp8" else INT8_CODES
        for what in ("values", "keys"):
            k, v, *_ = build(kind, 8, what, 5)
            seen = set((v[:, :, 0, :] if what == "values" else k[:, :, 1, :]).ravel().tolist())
            assert seen >= set(codes.tolist()), (kind, what)
