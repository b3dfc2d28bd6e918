"""Properties of the library's host-side queries over random shapes (CPU).

The size and schedule queries of the C ABI (workspace bytes, partition
length, schedule name, the general call's size query) run on the host and
launch nothing, so they are checked here on any machine: valid shapes get a
positive workspace and a partition length that is a positive multiple of 64
no longer than the capacity rounded up; invalid shapes (h not a multiple of
g, d outside {64, 128}, a head's rows reaching 2 GiB, T above S, bad
split_chunk) get 0 / -1; the general call's query equals the dedicated
one for the same shape; the decode calls return their host-detected errors
before any launch.
"""
from __future__ import annotations

import ctypes

import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import transformer_decode_attention_amd as mqa  # noqa: E402

FAKE = 0x10000        # an aligned, never dereferenced address
MISALIGNED = 0x10008

SETTINGS = settings(max_examples=300, deadline=None, derandomize=True)


@st.composite
def shapes(draw, valid=True):
    g = draw(st.sampled_from([1, 2, 4, 8, 16, 32]))
    G = draw(st.sampled_from([1, 2, 3, 4, 8, 16, 32, 64]))
    h = g * G
    d = draw(st.sampled_from([64, 128]))
    S = draw(st.integers(1, 40000))
    b = draw(st.integers(1, 1500))
    T = draw(st.integers(1, min(S, 16)))
    chunk = draw(st.sampled_from([0, 0, 64, 128, 512, 4096]))
    return b, T, h, g, S, d, chunk


@SETTINGS
@given(shapes())
def test_valid_shapes_get_a_workspace_and_a_chunk(shape):
    b, T, h, g, S, d, chunk = shape
    L = mqa.lib()
    c = L.mqa_decode_resolve_chunk(b, h, g, S, d, mqa.BF16, chunk)
    assert c > 0 and c % 64 == 0
    if chunk:
        assert c == chunk
    else:
        assert c <= -(-S // 64) * 64
    n1 = L.mqa_decode_workspace_bytes(b, h, g, S, d, mqa.BF16, chunk)
    nT = L.mqa_decode_multi_workspace_bytes(b, T, h, g, S, d, mqa.BF16, chunk)
    assert n1 > 0 and nT > 0
    if T == 1:
        assert nT == n1
    assert L.mqa_decode_schedule(b, h, g, S, d, mqa.BF16, chunk, 0) >= 0
    assert L.mqa_decode_multi_schedule(b, T, h, g, S, d, mqa.BF16, chunk) >= 0
    # the general call's size query: the same figure for the same shape
    desc = mqa.DecodeDesc()
    desc.b, desc.T, desc.h, desc.g, desc.d, desc.S = b, T, h, g, d, S
    desc.kv_dtype, desc.split_chunk = mqa.BF16, chunk
    assert L.mqa_decode_ex_workspace_bytes(ctypes.byref(desc)) == nT
    desc.kv_dtype = mqa.INT8
    assert L.mqa_decode_ex_workspace_bytes(ctypes.byref(desc)) == nT


@SETTINGS
@given(shapes(), st.sampled_from(["h_not_multiple", "d", "slab", "T", "chunk"]))
def test_invalid_shapes_are_refused(shape, what):
    b, T, h, g, S, d, chunk = shape
    if what == "h_not_multiple":
        g = g if g > 1 else 2
        h = g * 3 + 1
    elif what == "d":
        d = 96
    elif what == "slab":
        S = (1 << 31) // (2 * d)  # one head's bf16 rows reach 2 GiB
    elif what == "T":
        T = S + 1
    else:
        chunk = 100  # not a multiple of 64
    L = mqa.lib()
    if what != "T":
        assert L.mqa_decode_workspace_bytes(b, h, g, S, d, mqa.BF16, chunk) == 0
        assert L.mqa_decode_resolve_chunk(b, h, g, S, d, mqa.BF16, chunk) == -1
    assert L.mqa_decode_multi_workspace_bytes(b, T, h, g, S, d, mqa.BF16, chunk) == 0
    desc = mqa.DecodeDesc()
    desc.b, desc.T, desc.h, desc.g, desc.d, desc.S = b, T, h, g, d, S
    desc.kv_dtype, desc.split_chunk = mqa.BF16, chunk
    assert L.mqa_decode_ex_workspace_bytes(ctypes.byref(desc)) == 0
    # the decode itself refuses before launching anything
    desc.q = desc.k = desc.v = desc.seq_lens = desc.out = desc.workspace = FAKE
    desc.workspace_bytes = 1 << 40
    assert L.mqa_decode_attn_ex(ctypes.byref(desc), None) != mqa.OK


@SETTINGS
@given(shapes())
def test_host_errors_come_before_any_launch(shape):
    """Valid shapes with a NULL or misaligned pointer, or a workspace one
    byte short: the status is returned at once (nothing is enqueued)."""
    b, T, h, g, S, d, chunk = shape
    L = mqa.lib()
    need = L.mqa_decode_multi_workspace_bytes(b, T, h, g, S, d, mqa.BF16, chunk)
    args = lambda q=FAKE, ws=FAKE, nws=need: (q, FAKE, FAKE, FAKE, b, T, h, g, S, d, mqa.BF16,
                                              ctypes.c_float(0.1), FAKE, ws, nws, chunk, None,
                                              None)
    assert L.mqa_decode_attn_multi(*args(q=None)) == mqa.ERR_NULL
    assert L.mqa_decode_attn_multi(*args(q=MISALIGNED)) == mqa.ERR_ALIGN
    assert L.mqa_decode_attn_multi(*args(nws=need - 1)) == mqa.ERR_WORKSPACE
