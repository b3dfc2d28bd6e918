"""The C ABI of libmqa_decode.so, checked without a GPU.

Loads the library, checks that it exports every function include/mqa_decode.h
declares, and exercises the host-side argument checks, which return before
anything is enqueued (no HIP call is made on these paths). No kernel runs.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest
import torch

import transformer_decode_attention_amd as mqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mqa_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mqa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(mqa.EXPORTS)
    lib = mqa.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_schedule_choice():
    # many ragged (sequence, K/V head) units in bf16: the balanced schedule
    assert mqa.decode_schedule(64, 64, 8, 4096, 128, mqa.BF16) == "mfma-balanced"
    # few units (MQA, small batch): fixed partitions on the matrix cores
    assert mqa.decode_schedule(4, 32, 1, 32768, 128, mqa.BF16) == "mfma-partitions"
    # an explicit partition length, or the vector-ALU kernel, or fp32
    assert mqa.decode_schedule(64, 64, 8, 4096, 128, mqa.BF16, 512) == "mfma-partitions"
    assert mqa.decode_schedule(64, 64, 8, 4096, 128, mqa.BF16, 0, mqa.KERNEL_VALU) == "valu-partitions"
    assert mqa.decode_schedule(1, 8, 1, 129, 64, mqa.F32) == "valu-partitions"
    with pytest.raises(ValueError):
        mqa.decode_schedule(1, 8, 1, 129, 64, mqa.F32, 0, mqa.KERNEL_MFMA)


def test_status_strings():
    for s in range(8):
        assert mqa.status_string(s)
    assert mqa.status_string(0) == "ok"
    assert "unknown" in mqa.status_string(99)


def test_kv_bytes_formula():
    # 2 * layers * g * S * d * bytes; the h/g shrink at h=32 (compassingai 技術原理)
    assert mqa.kv_bytes(1, 32, 8192, 128, 2) == 134217728
    assert mqa.kv_bytes(32, 1, 8192, 128, 2) == 134217728
    assert mqa.kv_bytes(80, 64, 4096, 128, 2) == 10737418240
    assert mqa.kv_bytes(1, 32, 8192, 128, 2) // mqa.kv_bytes(1, 1, 8192, 128, 2) == 32


def test_chunk_resolution_and_workspace():
    # explicit chunk is kept; automatic chunk is a multiple of 64 within [256, S rounded up]
    assert mqa.decode_resolve_chunk(64, 64, 8, 4096, 128, mqa.BF16, 512) == 512
    for (b, h, g, S) in [(64, 64, 8, 4096), (4, 32, 1, 32768), (1, 8, 1, 129), (16, 32, 32, 8192)]:
        c = mqa.decode_resolve_chunk(b, h, g, S, 128, mqa.BF16, 0)
        assert c % 64 == 0 and 64 <= c <= (S + 63) // 64 * 64
        nsplit = -(-S // c)
        ws = mqa.decode_workspace_bytes(b, h, g, S, 128, mqa.BF16, 0)
        assert ws >= b * h * nsplit * (128 + 2) * 4
    # invalid arguments: -1 / 0
    assert mqa.decode_resolve_chunk(1, 6, 4, 10, 64, mqa.F32, 0) == -1     # h % g
    assert mqa.decode_resolve_chunk(1, 8, 1, 10, 96, mqa.F32, 0) == -1     # d
    assert mqa.decode_resolve_chunk(1, 8, 1, 10, 64, mqa.F32, 100) == -1   # chunk not /64
    assert mqa.decode_workspace_bytes(0, 8, 1, 10, 64, mqa.F32, 0) == 0


FAKE = ctypes.c_void_p(0x10000)      # 16-byte aligned, never dereferenced: rejected first
MISALIGNED = ctypes.c_void_p(0x10008)


def decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, b=2, h=8, g=2, S=64, d=128, dt=mqa.BF16,
             scale=0.088, out=FAKE, ws=FAKE, ws_bytes=0, chunk=0)
    a.update(kw)
    return mqa.lib().mqa_decode_attn(a["q"], a["k"], a["v"], a["lens"], a["b"], a["h"], a["g"],
                                     a["S"], a["d"], a["dt"], ctypes.c_float(a["scale"]), a["out"],
                                     a["ws"], a["ws_bytes"], a["chunk"], None, None)


def append(**kw):
    a = dict(k=FAKE, v=FAKE, kn=FAKE, vn=FAKE, lens=FAKE, b=2, g=2, S=64, d=128, dt=mqa.BF16)
    a.update(kw)
    return mqa.lib().mqa_append_kv(a["k"], a["v"], a["kn"], a["vn"], a["lens"], a["b"], a["g"],
                                   a["S"], a["d"], a["dt"], None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), mqa.ERR_NULL),
    (dict(lens=None), mqa.ERR_NULL),
    (dict(out=None), mqa.ERR_NULL),
    (dict(h=6, g=4), mqa.ERR_SHAPE),           # h not a multiple of g
    (dict(b=0), mqa.ERR_SHAPE),
    (dict(S=0), mqa.ERR_SHAPE),
    (dict(S=1 << 23), mqa.ERR_SHAPE),         # one head's bf16 rows reach 2 GiB
    (dict(d=96), mqa.ERR_UNSUPPORTED),
    (dict(dt=7), mqa.ERR_UNSUPPORTED),
    (dict(chunk=100), mqa.ERR_UNSUPPORTED),
    (dict(chunk=-64), mqa.ERR_UNSUPPORTED),
    (dict(k=MISALIGNED), mqa.ERR_ALIGN),
    (dict(out=MISALIGNED), mqa.ERR_ALIGN),
    (dict(ws=None, ws_bytes=1 << 30), mqa.ERR_WORKSPACE),
    (dict(ws_bytes=16), mqa.ERR_WORKSPACE),
])
def test_decode_rejects_bad_arguments_before_launch(kw, status):
    assert decode(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), mqa.ERR_NULL),
    (dict(lens=None), mqa.ERR_NULL),
    (dict(g=0), mqa.ERR_SHAPE),
    (dict(d=32), mqa.ERR_UNSUPPORTED),
    (dict(vn=MISALIGNED), mqa.ERR_ALIGN),
])
def test_append_rejects_bad_arguments_before_launch(kw, status):
    assert append(**kw) == status


def test_python_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 8, 64)
    k = torch.zeros(1, 1, 16, 64)
    with pytest.raises(ValueError):
        mqa.decode_attn(q, k, k, torch.ones(1, dtype=torch.int32))


def test_product_path_does_not_touch_the_oracle():
    """The package imports nothing from oracle/ and names no oracle symbol."""
    pkg = os.path.join(ROOT, "transformer_decode_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle_" not in text and "liboracle" not in text, f


def paged_decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, b=2, h=8, g=2, P=16, maxp=4, num=8,
             d=128, dt=mqa.BF16, scale=0.088, out=FAKE, ws=FAKE, ws_bytes=1 << 30, chunk=0)
    a.update(kw)
    return mqa.lib().mqa_decode_attn_paged(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["b"],
                                           a["h"], a["g"], a["P"], a["maxp"], a["num"], a["d"],
                                           a["dt"], ctypes.c_float(a["scale"]), a["out"], a["ws"],
                                           a["ws_bytes"], a["chunk"], None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), mqa.ERR_NULL),
    (dict(P=8), mqa.ERR_SHAPE),            # pages are multiples of 16 rows
    (dict(P=24), mqa.ERR_SHAPE),
    (dict(maxp=0), mqa.ERR_SHAPE),
    (dict(num=0), mqa.ERR_SHAPE),
    (dict(h=6, g=4), mqa.ERR_SHAPE),
    (dict(dt=mqa.F32), mqa.ERR_UNSUPPORTED),  # paged reads run the bf16 matrix-core kernels
    (dict(d=96), mqa.ERR_UNSUPPORTED),
    (dict(v=MISALIGNED), mqa.ERR_ALIGN),
    (dict(ws_bytes=16), mqa.ERR_WORKSPACE),
])
def test_paged_decode_rejects_bad_arguments_before_launch(kw, status):
    assert paged_decode(**kw) == status


def test_paged_workspace_bytes():
    n = mqa.decode_paged_workspace_bytes(64, 64, 8, 16, 256, 128, mqa.BF16)
    assert n == mqa.decode_workspace_bytes(64, 64, 8, 16 * 256, 128, mqa.BF16)
    assert mqa.decode_paged_workspace_bytes(64, 64, 8, 24, 256, 128, mqa.BF16) == 0


def multi_decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, b=2, T=4, h=8, g=2, S=64, d=128, dt=mqa.BF16,
             scale=0.088, out=FAKE, ws=FAKE, ws_bytes=1 << 30, chunk=0)
    a.update(kw)
    return mqa.lib().mqa_decode_attn_multi(a["q"], a["k"], a["v"], a["lens"], a["b"], a["T"],
                                           a["h"], a["g"], a["S"], a["d"], a["dt"],
                                           ctypes.c_float(a["scale"]), a["out"], a["ws"],
                                           a["ws_bytes"], a["chunk"], None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), mqa.ERR_NULL),
    (dict(T=0), mqa.ERR_SHAPE),
    (dict(T=65), mqa.ERR_SHAPE),             # more tokens than the capacity
    (dict(dt=mqa.F32), mqa.ERR_UNSUPPORTED),  # several tokens: matrix-core kernels, bf16
    (dict(h=6, g=4), mqa.ERR_SHAPE),
    (dict(out=MISALIGNED), mqa.ERR_ALIGN),
    (dict(ws_bytes=16), mqa.ERR_WORKSPACE),
])
def test_multi_decode_rejects_bad_arguments_before_launch(kw, status):
    assert multi_decode(**kw) == status


def test_multi_append_rejects_bad_arguments_before_launch():
    L = mqa.lib()
    assert L.mqa_append_kv_multi(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0, 2, 64, 128, mqa.BF16, None,
                                 None) == mqa.ERR_SHAPE
    assert L.mqa_append_kv_multi(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 65, 2, 64, 128, mqa.BF16, None,
                                 None) == mqa.ERR_SHAPE
    assert L.mqa_append_kv_multi(FAKE, None, FAKE, FAKE, FAKE, 2, 4, 2, 64, 128, mqa.BF16, None,
                                 None) == mqa.ERR_NULL


def test_multi_workspace_and_schedule():
    # T = 1 is the one-token call
    assert mqa.decode_multi_workspace_bytes(64, 1, 64, 8, 4096, 128, mqa.BF16) == \
        mqa.decode_workspace_bytes(64, 64, 8, 4096, 128, mqa.BF16)
    assert mqa.decode_multi_schedule(64, 1, 64, 8, 4096, 128, mqa.BF16) == "mfma-balanced"
    # T tokens of G heads: T*G query rows per K/V head; up to 64 on the balanced schedule
    assert mqa.decode_multi_schedule(64, 4, 64, 8, 4096, 128, mqa.BF16) == "mfma-balanced"
    assert mqa.decode_multi_schedule(64, 8, 64, 8, 4096, 128, mqa.BF16) == "mfma-balanced"
    assert mqa.decode_multi_schedule(64, 9, 64, 8, 4096, 128, mqa.BF16) == "mfma-partitions"
    assert mqa.decode_multi_schedule(8, 4, 32, 1, 1024, 128, mqa.BF16) == "mfma-partitions"
    assert mqa.decode_multi_workspace_bytes(64, 4, 64, 8, 4096, 128, mqa.F32) == 0
    n1 = mqa.decode_multi_workspace_bytes(8, 1, 32, 1, 1024, 128, mqa.BF16, 256)
    n4 = mqa.decode_multi_workspace_bytes(8, 4, 32, 1, 1024, 128, mqa.BF16, 256)
    assert n1 == 8 * 32 * 4 * (128 * 4 + 8)  # partials (o, m, l) of 4 partitions per row
    assert n4 == 4 * n1                        # one set per query token


def fp8_decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, lens=FAKE, b=2, T=1, h=8, g=2, S=64, d=128,
             scale=0.088, out=FAKE, ws=FAKE, ws_bytes=1 << 30, chunk=0)
    a.update(kw)
    return mqa.lib().mqa_decode_attn_fp8(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["lens"], a["b"],
                                         a["T"], a["h"], a["g"], a["S"], a["d"],
                                         ctypes.c_float(a["scale"]), a["out"], a["ws"], a["ws_bytes"],
                                         a["chunk"], None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), mqa.ERR_NULL),
    (dict(vs=None), mqa.ERR_NULL),
    (dict(T=0), mqa.ERR_SHAPE),
    (dict(T=65), mqa.ERR_SHAPE),
    (dict(d=96), mqa.ERR_UNSUPPORTED),
    (dict(h=6, g=4), mqa.ERR_SHAPE),
    (dict(k=MISALIGNED), mqa.ERR_ALIGN),
    (dict(ks=ctypes.c_void_p(0x10002)), mqa.ERR_ALIGN),
    (dict(ws_bytes=16), mqa.ERR_WORKSPACE),
])
def test_fp8_decode_rejects_bad_arguments_before_launch(kw, status):
    assert fp8_decode(**kw) == status


def test_fp8_append_rejects_bad_arguments_before_launch():
    L = mqa.lib()
    assert L.mqa_append_kv_fp8(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 2, 1, 2, 64, 128, None,
                               None) == mqa.ERR_NULL
    assert L.mqa_append_kv_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0, 2, 64, 128, None,
                               None) == mqa.ERR_SHAPE
    assert L.mqa_append_kv_fp8(FAKE, MISALIGNED, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, 2, 64, 128,
                               None, None) == mqa.ERR_ALIGN
    assert L.mqa_append_kv_paged_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 2, 1, 2, 16, 4,
                                     8, 128, None, None) == mqa.ERR_NULL
    assert L.mqa_append_kv_paged_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, 2, 16, 0,
                                     8, 128, None, None) == mqa.ERR_SHAPE


def test_decode_desc_layout_matches_the_header(tmp_path):
    """The ctypes mirror of mqa_decode_desc has the C struct's offsets and size
    (a small C program built with the host compiler prints them)."""
    src = tmp_path / "layout.c"
    fields = [f[0] for f in mqa.DecodeDesc._fields_]
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"mqa_decode.h\"\n"
                   "int main(void) {\n"
                   + "".join(f'  printf("%zu\\n", offsetof(mqa_decode_desc, {f}));\n' for f in fields)
                   + '  printf("%zu\\n", sizeof(mqa_decode_desc));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I", "/opt/rocm/include",
                        "-o", str(exe), str(src)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("host compiler cannot include the HIP runtime header: " + r.stderr[:200])
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [getattr(mqa.DecodeDesc, f).offset for f in fields] + [ctypes.sizeof(mqa.DecodeDesc)]
    assert got == want


def ex_desc(**kw):
    d = mqa.DecodeDesc()
    d.q = d.k = d.v = d.seq_lens = d.out = d.workspace = 0x10000
    d.b, d.T, d.h, d.g, d.d, d.S = 2, 1, 8, 2, 128, 64
    d.kv_dtype, d.window, d.split_chunk, d.scale = mqa.BF16, 0, 0, 0.088
    d.workspace_bytes = 1 << 30
    for k_, v_ in kw.items():
        setattr(d, k_, v_)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), mqa.ERR_NULL),
    (dict(window=-1), mqa.ERR_SHAPE),
    (dict(kv_dtype=7), mqa.ERR_UNSUPPORTED),
    (dict(kv_dtype=mqa.F32, T=2), mqa.ERR_UNSUPPORTED),
    (dict(kv_dtype=mqa.F32, window=4), mqa.ERR_UNSUPPORTED),
    (dict(kv_dtype=mqa.FP8_E4M3), mqa.ERR_NULL),              # no scales
    (dict(block_table=0x10000, page_size=24, max_pages=4, num_pages=8), mqa.ERR_SHAPE),
    (dict(T=65), mqa.ERR_SHAPE),
    (dict(workspace_bytes=16), mqa.ERR_WORKSPACE),
    (dict(out=0x10008), mqa.ERR_ALIGN),
])
def test_decode_ex_rejects_bad_arguments_before_launch(kw, status):
    d = ex_desc(**kw)
    assert mqa.lib().mqa_decode_attn_ex(ctypes.byref(d), None) == status


def test_decode_ex_workspace_matches_the_dedicated_calls():
    L = mqa.lib()
    d = ex_desc(b=64, h=64, g=8, S=4096)
    assert L.mqa_decode_ex_workspace_bytes(ctypes.byref(d)) == \
        mqa.decode_workspace_bytes(64, 64, 8, 4096, 128, mqa.BF16)
    d = ex_desc(b=64, h=64, g=8, S=4096, T=4)
    assert L.mqa_decode_ex_workspace_bytes(ctypes.byref(d)) == \
        mqa.decode_multi_workspace_bytes(64, 4, 64, 8, 4096, 128, mqa.BF16)
    # a window: partitions cover at most W + T + 30 positions (from the
    # window's first 32-position step to the end), and no more than S
    d = ex_desc(b=4, h=32, g=1, S=32768, T=4, window=100)
    assert L.mqa_decode_ex_workspace_bytes(ctypes.byref(d)) == \
        mqa.decode_multi_workspace_bytes(4, 4, 32, 1, 134, 128, mqa.BF16)
    d = ex_desc(b=4, h=32, g=1, S=120, T=4, window=100)
    assert L.mqa_decode_ex_workspace_bytes(ctypes.byref(d)) == \
        mqa.decode_multi_workspace_bytes(4, 4, 32, 1, 120, 128, mqa.BF16)


def test_decode_ex_workspace_query_reads_sizes_only():
    """The size query takes a descriptor whose data pointers are unset, and
    still rejects bad shapes (0 bytes)."""
    L = mqa.lib()
    full = ex_desc(b=64, h=64, g=8, S=4096, T=2, window=512)
    bare = ex_desc(b=64, h=64, g=8, S=4096, T=2, window=512, q=None, k=None, v=None,
                   seq_lens=None, out=None, workspace=None, kv_dtype=mqa.FP8_E4M3)
    n = L.mqa_decode_ex_workspace_bytes(ctypes.byref(full))
    assert n > 0 and L.mqa_decode_ex_workspace_bytes(ctypes.byref(bare)) == n
    assert L.mqa_decode_ex_workspace_bytes(ctypes.byref(ex_desc(q=None, window=-1))) == 0
    assert L.mqa_decode_ex_workspace_bytes(ctypes.byref(ex_desc(out=None, T=65))) == 0
    # the decode itself still checks the pointers
    assert L.mqa_decode_attn_ex(ctypes.byref(bare), None) == mqa.ERR_NULL


def test_int8_calls_reject_bad_arguments_before_launch():
    """The int8 cache through the general call needs its scales; the int8
    appends check like the fp8 ones."""
    L = mqa.lib()
    assert L.mqa_decode_attn_ex(ctypes.byref(ex_desc(kv_dtype=mqa.INT8)), None) == mqa.ERR_NULL
    d = ex_desc(kv_dtype=mqa.INT8, k_scale=0x10002, v_scale=0x10000)
    assert L.mqa_decode_attn_ex(ctypes.byref(d), None) == mqa.ERR_ALIGN
    assert L.mqa_decode_ex_workspace_bytes(ctypes.byref(ex_desc(kv_dtype=mqa.INT8))) == \
        L.mqa_decode_ex_workspace_bytes(ctypes.byref(ex_desc(kv_dtype=mqa.FP8_E4M3)))
    assert L.mqa_append_kv_int8(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 2, 1, 2, 64, 128, None,
                                None) == mqa.ERR_NULL
    assert L.mqa_append_kv_int8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0, 2, 64, 128, None,
                                None) == mqa.ERR_SHAPE
    assert L.mqa_append_kv_paged_int8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, 2, 16,
                                      4, 0, 128, None, None) == mqa.ERR_SHAPE


def test_rope_calls_reject_bad_arguments_before_launch():
    L = mqa.lib()
    assert L.mqa_rope_q(FAKE, None, 16, FAKE, 2, 1, 8, 128, None, None) == mqa.ERR_NULL
    assert L.mqa_rope_q(FAKE, FAKE, 0, FAKE, 2, 1, 8, 128, None, None) == mqa.ERR_SHAPE
    assert L.mqa_rope_q(FAKE, FAKE, 16, FAKE, 2, 1, 8, 96, None, None) == mqa.ERR_UNSUPPORTED
    assert L.mqa_rope_q(MISALIGNED, FAKE, 16, FAKE, 2, 1, 8, 128, None, None) == mqa.ERR_ALIGN
    assert L.mqa_append_kv_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, 2, 0, 2, 64, 128, None,
                                None) == mqa.ERR_SHAPE
    assert L.mqa_append_kv_rope(FAKE, FAKE, FAKE, FAKE, None, 16, FAKE, 2, 1, 2, 64, 128, None,
                                None) == mqa.ERR_NULL


def test_err_flags_is_checked_before_any_launch():
    """err_flags must be None or a contiguous int32 device tensor on the
    call's device: a host tensor (whose pointer the kernels would OR bits
    into) or another dtype is refused with ValueError by the binding."""
    like = torch.zeros(4)
    assert mqa._err(None, like) is None
    for bad in (torch.zeros(1, dtype=torch.int32), torch.zeros(1, dtype=torch.int64),
                torch.zeros(0, dtype=torch.int32), [0]):
        with pytest.raises(ValueError):
            mqa._err(bad, like)


def test_noalloc_host_errors_need_no_device():
    """The no-allocation entry point refuses NULL pointers, bad sizes and a call
    needing more scratch than it holds before any HIP call (no GPU here)."""
    L = mqa.lib()
    fake = ctypes.c_void_p(0x10000)
    args = lambda q=fake, b=4, S=1024: (q, fake, fake, fake, b, 32, 8, S, 128, mqa.BF16,
                                        ctypes.c_float(0.1), fake, 0, None, None)
    assert L.mqa_decode_attn_noalloc(*args(q=None)) == mqa.ERR_NULL
    assert L.mqa_decode_attn_noalloc(*args(b=0)) == mqa.ERR_SHAPE
    assert mqa.decode_workspace_bytes(4096, 32, 8, 32768, 128, mqa.BF16) > 64 << 20
    assert L.mqa_decode_attn_noalloc(*args(b=4096, S=32768)) == mqa.ERR_SCRATCH
