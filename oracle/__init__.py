"""Plain CPU oracle for decode attention over a shared-head KV cache.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product path
(``transformer_decode_attention_amd``) never imports, loads or calls it, and
the two share no code: the C source here includes nothing from the HIP
library, and this module imports nothing from the product package.

The arithmetic lives in ``oracle.c`` (double precision, plain loops). This
module is ctypes marshalling over numpy arrays only. Element type codes:
``F32 = 0`` (binary32) and ``BF16 = 1`` (bfloat16 stored as uint16 bits).

Sources, cited by page title and section:
  [GQA notes] ybb.press "分组查询注意力（GQA）与多查询注意力（MQA）深度实战",
              §一/§七 (KV bytes), §四/§五 (grouped math), §八 (cache write).
  [MQA blog]  nanhubrain.csdn.net MQA article §2.2 (append on the sequence axis),
              §3.3 (paged cache, 16 tokens per page).
  [GQA notes] §十 item 10 (the causal mask stays per query position when several
              query tokens attend at once), §十 item 7 (a quantised KV cache), §十 item 6
              (position encoding applied per head).
  [MQA concept] 玩家對比 (GQA with a sliding window).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32 = 0
BF16 = 1
FP8_E4M3 = 2
INT8 = 3
OK = 0
BAD_LEN = 1
BAD_SHAPE = 2
BAD_PAGE = 4

_HERE = os.path.dirname(os.path.abspath(__file__))
BUILD_PATH = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIB: load another build of oracle.c instead (the sanitizer test's)
LIB_PATH = os.environ.get("ORACLE_LIB") or BUILD_PATH
_SRC = os.path.join(_HERE, "oracle.c")


def build() -> str:
    """Compile oracle.c with the host C compiler (gcc) into liboracle.so."""
    tmp = BUILD_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fPIC",
           "-shared", "-pthread", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, BUILD_PATH)
    return BUILD_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            if LIB_PATH != BUILD_PATH:
                raise ImportError(f"ORACLE_LIB={LIB_PATH} does not exist")
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, dp = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_double)
        L.oracle_append_kv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32]
        L.oracle_append_kv.restype = i32
        L.oracle_decode_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                         i32, ctypes.c_float, vp, vp, i32]
        L.oracle_decode_attn.restype = i32
        L.oracle_mha_per_head.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_double, vp]
        L.oracle_mha_per_head.restype = None
        L.oracle_partial.argtypes = [vp, vp, vp, i32, ctypes.c_double, i32, i32, dp, dp, vp]
        L.oracle_partial.restype = None
        L.oracle_lse_combine.argtypes = [i32, vp, vp, vp, i32, vp]
        L.oracle_lse_combine.restype = None
        L.oracle_decode_attn_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                               i32, i32, i32, ctypes.c_float, vp, i32]
        L.oracle_decode_attn_paged.restype = i32
        L.oracle_append_kv_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                             i32, i32]
        L.oracle_append_kv_paged.restype = i32
        L.oracle_append_kv_multi.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32]
        L.oracle_append_kv_multi.restype = i32
        L.oracle_decode_attn_multi.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                               i32, ctypes.c_float, vp, vp, i32]
        L.oracle_decode_attn_multi.restype = i32
        L.oracle_decode_attn_paged_multi.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                     i32, i32, i32, i32, i32, ctypes.c_float,
                                                     vp, i32]
        L.oracle_decode_attn_paged_multi.restype = i32
        L.oracle_append_kv_paged_multi.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                   i32, i32, i32, i32]
        L.oracle_append_kv_paged_multi.restype = i32
        L.oracle_fp8_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_fp8_e4m3_decode.restype = ctypes.c_double
        L.oracle_fp8_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_fp8_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_decode_attn_fp8.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                             i32, ctypes.c_float, vp, i32]
        L.oracle_decode_attn_fp8.restype = i32
        L.oracle_decode_attn_paged_fp8.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                                   i32, i32, i32, i32, i32, ctypes.c_float, vp, i32]
        L.oracle_decode_attn_paged_fp8.restype = i32
        L.oracle_append_kv_fp8.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32]
        L.oracle_append_kv_fp8.restype = i32
        L.oracle_append_kv_paged_fp8.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32,
                                                 i32, i32, i32, i32]
        L.oracle_append_kv_paged_fp8.restype = i32
        L.oracle_int8_decode.argtypes = [ctypes.c_int8]
        L.oracle_int8_decode.restype = ctypes.c_double
        L.oracle_int8_encode.argtypes = [ctypes.c_float]
        L.oracle_int8_encode.restype = ctypes.c_int8
        L.oracle_append_kv_int8.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32]
        L.oracle_append_kv_int8.restype = i32
        L.oracle_append_kv_paged_int8.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, i32,
                                                  i32, i32, i32, i32, i32]
        L.oracle_append_kv_paged_int8.restype = i32
        L.oracle_decode_attn_ex.argtypes = [vp, i32, vp, vp, i32, vp, vp, vp, i32, i32, i32, vp,
                                            i32, i32, i32, i32, i32, i32, i32, ctypes.c_float, vp,
                                            i32]
        L.oracle_decode_attn_ex.restype = i32
        L.oracle_rope_table.argtypes = [ctypes.c_double, i32, i32, vp]
        L.oracle_rope_table.restype = None
        L.oracle_rope_rows.argtypes = [vp, vp, vp, i32, i32]
        L.oracle_rope_rows.restype = None
        L.oracle_rope_q.argtypes = [vp, vp, vp, i32, i32, i32, i32]
        L.oracle_rope_q.restype = i32
        L.oracle_append_kv_rope.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32]
        L.oracle_append_kv_rope.restype = i32
        L.oracle_kv_bytes.argtypes = [i32, i32, ctypes.c_int64, i32, i32]
        L.oracle_kv_bytes.restype = ctypes.c_uint64
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype in (np.uint16, np.int16):
        return BF16
    raise TypeError(f"oracle takes float32 or bfloat16 bits (uint16), got {a.dtype}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def append_kv(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray,
              v_new: np.ndarray, seq_lens: np.ndarray) -> int:
    """In place: row seq_lens[i]-1 of every head of sequence i gets k_new/v_new.

    k_cache, v_cache: [b, g, S, d] (float32 or bf16 bits); k_new, v_new: [b, g, d].
    Returns the oracle status bits (BAD_LEN if some length is outside [1, S]).
    """
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    b, g, S, d = k_cache.shape
    sl = _c(seq_lens.astype(np.int32))
    return lib().oracle_append_kv(_ptr(k_cache), _ptr(v_cache), _ptr(_c(k_new)),
                                  _ptr(_c(v_new)), _ptr(sl), b, g, S, d,
                                  _dtype_code(k_cache))


def decode_attn(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                seq_lens: np.ndarray, scale: float, want_alpha: bool = False,
                nthreads: int = 1):
    """Plain-definition decode attention in double.

    q: [b, h, d]; k_cache, v_cache: [b, g, S, d]; seq_lens: [b] (attended
    lengths). Returns (out [b, h, d] float64, alpha [b, h, S] or None, status).
    """
    b, h, d = q.shape
    _, g, S, _ = k_cache.shape
    dt = _dtype_code(k_cache)
    assert _dtype_code(q) == dt and _dtype_code(v_cache) == dt
    out = np.empty((b, h, d), np.float64)
    alpha = np.empty((b, h, S), np.float64) if want_alpha else None
    sl = _c(seq_lens.astype(np.int32))
    rc = lib().oracle_decode_attn(_ptr(_c(q)), _ptr(_c(k_cache)), _ptr(_c(v_cache)),
                                  _ptr(sl), b, h, g, S, d, dt, ctypes.c_float(scale),
                                  _ptr(out), _ptr(alpha), int(nthreads))
    return out, alpha, rc


def decode_attn_paged(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray,
                      block_table: np.ndarray, seq_lens: np.ndarray, scale: float,
                      nthreads: int = 1):
    """Decode attention over a paged cache, in double.

    q: [b, h, d]; k_pages, v_pages: [num_pages, g, page_size, d]; block_table:
    [b, max_pages] int32 page ids; seq_lens: [b]. Returns (out [b, h, d], status).
    """
    b, h, d = q.shape
    num_pages, g, P, _ = k_pages.shape
    max_pages = block_table.shape[1]
    dt = _dtype_code(k_pages)
    assert _dtype_code(q) == dt and _dtype_code(v_pages) == dt
    out = np.empty((b, h, d), np.float64)
    bt = _c(block_table.astype(np.int32))
    sl = _c(seq_lens.astype(np.int32))
    rc = lib().oracle_decode_attn_paged(_ptr(_c(q)), _ptr(_c(k_pages)), _ptr(_c(v_pages)),
                                        _ptr(bt), _ptr(sl), b, h, g, P, max_pages, num_pages,
                                        d, dt, ctypes.c_float(scale), _ptr(out), int(nthreads))
    return out, rc


def append_kv_paged(k_pages: np.ndarray, v_pages: np.ndarray, k_new: np.ndarray,
                    v_new: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray) -> int:
    """In place: row (L-1) % page_size of page block_table[i][(L-1) // page_size]
    of every K/V head of sequence i gets k_new/v_new. Returns the status bits."""
    assert k_pages.flags.c_contiguous and v_pages.flags.c_contiguous
    num_pages, g, P, d = k_pages.shape
    b = k_new.shape[0]
    bt = _c(block_table.astype(np.int32))
    sl = _c(seq_lens.astype(np.int32))
    return lib().oracle_append_kv_paged(_ptr(k_pages), _ptr(v_pages), _ptr(_c(k_new)),
                                        _ptr(_c(v_new)), _ptr(bt), _ptr(sl), b, g, P,
                                        bt.shape[1], num_pages, d, _dtype_code(k_pages))


def append_kv_multi(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray,
                    v_new: np.ndarray, seq_lens: np.ndarray) -> int:
    """In place: token tau of k_new/v_new [b, T, g, d] goes to position
    seq_lens[i]-T+tau of every K/V head of sequence i. Returns the status bits."""
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    b, g, S, d = k_cache.shape
    T = k_new.shape[1]
    sl = _c(seq_lens.astype(np.int32))
    return lib().oracle_append_kv_multi(_ptr(k_cache), _ptr(v_cache), _ptr(_c(k_new)),
                                        _ptr(_c(v_new)), _ptr(sl), b, T, g, S, d,
                                        _dtype_code(k_cache))


def decode_attn_multi(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                      seq_lens: np.ndarray, scale: float, want_alpha: bool = False,
                      nthreads: int = 1):
    """T query tokens per sequence with the causal mask, in double.

    q: [b, T, h, d] (token tau at position seq_lens[i]-T+tau); k_cache, v_cache:
    [b, g, S, d]. Returns (out [b, T, h, d] float64, alpha [b, T, h, S] or None, status).
    """
    b, T, h, d = q.shape
    _, g, S, _ = k_cache.shape
    dt = _dtype_code(k_cache)
    assert _dtype_code(q) == dt and _dtype_code(v_cache) == dt
    out = np.empty((b, T, h, d), np.float64)
    alpha = np.empty((b, T, h, S), np.float64) if want_alpha else None
    sl = _c(seq_lens.astype(np.int32))
    rc = lib().oracle_decode_attn_multi(_ptr(_c(q)), _ptr(_c(k_cache)), _ptr(_c(v_cache)),
                                        _ptr(sl), b, T, h, g, S, d, dt, ctypes.c_float(scale),
                                        _ptr(out), _ptr(alpha), int(nthreads))
    return out, alpha, rc


def decode_attn_paged_multi(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray,
                            block_table: np.ndarray, seq_lens: np.ndarray, scale: float,
                            nthreads: int = 1):
    """decode_attn_multi over a paged cache. Returns (out [b, T, h, d], status)."""
    b, T, h, d = q.shape
    num_pages, g, P, _ = k_pages.shape
    dt = _dtype_code(k_pages)
    assert _dtype_code(q) == dt and _dtype_code(v_pages) == dt
    out = np.empty((b, T, h, d), np.float64)
    bt = _c(block_table.astype(np.int32))
    sl = _c(seq_lens.astype(np.int32))
    rc = lib().oracle_decode_attn_paged_multi(_ptr(_c(q)), _ptr(_c(k_pages)),
                                              _ptr(_c(v_pages)), _ptr(bt), _ptr(sl), b, T, h,
                                              g, P, bt.shape[1], num_pages, d, dt,
                                              ctypes.c_float(scale), _ptr(out), int(nthreads))
    return out, rc


def append_kv_paged_multi(k_pages: np.ndarray, v_pages: np.ndarray, k_new: np.ndarray,
                          v_new: np.ndarray, block_table: np.ndarray,
                          seq_lens: np.ndarray) -> int:
    """append_kv_multi into a paged cache. Returns the status bits."""
    assert k_pages.flags.c_contiguous and v_pages.flags.c_contiguous
    num_pages, g, P, d = k_pages.shape
    b, T = k_new.shape[:2]
    bt = _c(block_table.astype(np.int32))
    sl = _c(seq_lens.astype(np.int32))
    return lib().oracle_append_kv_paged_multi(_ptr(k_pages), _ptr(v_pages), _ptr(_c(k_new)),
                                              _ptr(_c(v_new)), _ptr(bt), _ptr(sl), b, T, g,
                                              P, bt.shape[1], num_pages, d,
                                              _dtype_code(k_pages))


# ---- fp8 e4m3 cache with per-K/V-head scales ([GQA notes] §十 item 7) ----

def fp8_decode(code: int) -> float:
    """Value of one e4m3 code (OCP E4M3FN)."""
    return float(lib().oracle_fp8_e4m3_decode(int(code)))


def fp8_encode(x: float) -> int:
    """e4m3 code of a float32 value: nearest, ties to even, saturating at +-448."""
    return int(lib().oracle_fp8_e4m3_encode(float(np.float32(x))))


def _f32(a):
    return _c(np.asarray(a, np.float32))


def decode_attn_fp8(q: np.ndarray, k_codes: np.ndarray, v_codes: np.ndarray,
                    k_scale: np.ndarray, v_scale: np.ndarray, seq_lens: np.ndarray,
                    scale: float, nthreads: int = 1):
    """Decode attention over an fp8 cache (values code * scale[j]), in double.

    q: [b, h, d] or [b, T, h, d] (float32 or bf16 bits); k_codes, v_codes:
    [b, g, S, d] uint8; k_scale, v_scale: [g]. Returns (out shaped like q, status).
    """
    q4 = q if q.ndim == 4 else q[:, None]
    b, T, h, d = q4.shape
    _, g, S, _ = k_codes.shape
    assert k_codes.dtype == np.uint8 and v_codes.dtype == np.uint8
    out = np.empty((b, T, h, d), np.float64)
    sl = _c(seq_lens.astype(np.int32))
    rc = lib().oracle_decode_attn_fp8(_ptr(_c(q4)), _dtype_code(q4), _ptr(_c(k_codes)),
                                      _ptr(_c(v_codes)), _ptr(_f32(k_scale)), _ptr(_f32(v_scale)),
                                      _ptr(sl), b, T, h, g, S, d, ctypes.c_float(scale), _ptr(out),
                                      int(nthreads))
    return (out if q.ndim == 4 else out[:, 0]), rc


def decode_attn_paged_fp8(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray,
                          k_scale: np.ndarray, v_scale: np.ndarray, block_table: np.ndarray,
                          seq_lens: np.ndarray, scale: float, nthreads: int = 1):
    """decode_attn_fp8 over a paged cache [num_pages, g, page_size, d] of codes."""
    q4 = q if q.ndim == 4 else q[:, None]
    b, T, h, d = q4.shape
    num_pages, g, P, _ = k_pages.shape
    out = np.empty((b, T, h, d), np.float64)
    bt = _c(block_table.astype(np.int32))
    sl = _c(seq_lens.astype(np.int32))
    rc = lib().oracle_decode_attn_paged_fp8(_ptr(_c(q4)), _dtype_code(q4), _ptr(_c(k_pages)),
                                            _ptr(_c(v_pages)), _ptr(_f32(k_scale)),
                                            _ptr(_f32(v_scale)), _ptr(bt), _ptr(sl), b, T, h, g,
                                            P, bt.shape[1], num_pages, d, ctypes.c_float(scale),
                                            _ptr(out), int(nthreads))
    return (out if q.ndim == 4 else out[:, 0]), rc


def append_kv_fp8(k_codes: np.ndarray, v_codes: np.ndarray, k_new: np.ndarray,
                  v_new: np.ndarray, k_scale: np.ndarray, v_scale: np.ndarray,
                  seq_lens: np.ndarray) -> int:
    """In place: the new rows ([b, g, d] or [b, T, g, d], float32 or bf16 bits)
    quantised with the head's scale into positions L-T .. L-1. Returns the status."""
    assert k_codes.flags.c_contiguous and v_codes.flags.c_contiguous
    kn = k_new if k_new.ndim == 4 else k_new[:, None]
    vn = v_new if v_new.ndim == 4 else v_new[:, None]
    b, g, S, d = k_codes.shape
    T = kn.shape[1]
    sl = _c(seq_lens.astype(np.int32))
    return lib().oracle_append_kv_fp8(_ptr(k_codes), _ptr(v_codes), _ptr(_c(kn)), _ptr(_c(vn)),
                                      _dtype_code(kn), _ptr(_f32(k_scale)), _ptr(_f32(v_scale)),
                                      _ptr(sl), b, T, g, S, d)


def append_kv_paged_fp8(k_pages: np.ndarray, v_pages: np.ndarray, k_new: np.ndarray,
                        v_new: np.ndarray, k_scale: np.ndarray, v_scale: np.ndarray,
                        block_table: np.ndarray, seq_lens: np.ndarray) -> int:
    """append_kv_fp8 into a paged cache."""
    assert k_pages.flags.c_contiguous and v_pages.flags.c_contiguous
    kn = k_new if k_new.ndim == 4 else k_new[:, None]
    vn = v_new if v_new.ndim == 4 else v_new[:, None]
    num_pages, g, P, d = k_pages.shape
    b, T = kn.shape[:2]
    bt = _c(block_table.astype(np.int32))
    sl = _c(seq_lens.astype(np.int32))
    return lib().oracle_append_kv_paged_fp8(_ptr(k_pages), _ptr(v_pages), _ptr(_c(kn)),
                                            _ptr(_c(vn)), _dtype_code(kn), _ptr(_f32(k_scale)),
                                            _ptr(_f32(v_scale)), _ptr(bt), _ptr(sl), b, T, g, P,
                                            bt.shape[1], num_pages, d)


# ---- int8 cache with per-K/V-head scales (the pages' INT8 K/V) ----

def int8_decode(code: int) -> float:
    """Value of one int8 code before the head's scale (two's complement)."""
    return float(lib().oracle_int8_decode(int(code)))


def int8_encode(x: float) -> int:
    """int8 code of a float32 value: nearest, ties to even, saturating at +-127, NaN -> 0."""
    return int(lib().oracle_int8_encode(float(np.float32(x))))


def append_kv_int8(k_codes: np.ndarray, v_codes: np.ndarray, k_new: np.ndarray,
                   v_new: np.ndarray, k_scale: np.ndarray, v_scale: np.ndarray,
                   seq_lens: np.ndarray) -> int:
    """append_kv_fp8 with int8 codes ([b, g, S, d] int8)."""
    assert k_codes.dtype == np.int8 and v_codes.dtype == np.int8
    assert k_codes.flags.c_contiguous and v_codes.flags.c_contiguous
    kn = k_new if k_new.ndim == 4 else k_new[:, None]
    vn = v_new if v_new.ndim == 4 else v_new[:, None]
    b, g, S, d = k_codes.shape
    T = kn.shape[1]
    sl = _c(seq_lens.astype(np.int32))
    return lib().oracle_append_kv_int8(_ptr(k_codes), _ptr(v_codes), _ptr(_c(kn)), _ptr(_c(vn)),
                                       _dtype_code(kn), _ptr(_f32(k_scale)), _ptr(_f32(v_scale)),
                                       _ptr(sl), b, T, g, S, d)


def append_kv_paged_int8(k_pages: np.ndarray, v_pages: np.ndarray, k_new: np.ndarray,
                         v_new: np.ndarray, k_scale: np.ndarray, v_scale: np.ndarray,
                         block_table: np.ndarray, seq_lens: np.ndarray) -> int:
    """append_kv_int8 into a paged cache [num_pages, g, page_size, d] of int8 codes."""
    assert k_pages.dtype == np.int8 and v_pages.dtype == np.int8
    assert k_pages.flags.c_contiguous and v_pages.flags.c_contiguous
    kn = k_new if k_new.ndim == 4 else k_new[:, None]
    vn = v_new if v_new.ndim == 4 else v_new[:, None]
    num_pages, g, P, d = k_pages.shape
    b, T = kn.shape[:2]
    bt = _c(block_table.astype(np.int32))
    sl = _c(seq_lens.astype(np.int32))
    return lib().oracle_append_kv_paged_int8(_ptr(k_pages), _ptr(v_pages), _ptr(_c(kn)),
                                             _ptr(_c(vn)), _dtype_code(kn), _ptr(_f32(k_scale)),
                                             _ptr(_f32(v_scale)), _ptr(bt), _ptr(sl), b, T, g, P,
                                             bt.shape[1], num_pages, d)


# ---- every option at once; rotary position embedding ----

def decode_attn_ex(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens: np.ndarray,
                   scale: float, window: int = 0, k_scale=None, v_scale=None,
                   block_table=None, nthreads: int = 1):
    """Decode with every option: q [b, h, d] or [b, T, h, d]; k, v contiguous
    [b, g, S, d] or pages [num_pages, g, P, d] (with block_table [b, max_pages]);
    float32, bf16 bits (uint16), fp8 codes (uint8) or int8 codes (int8), the codes
    with k_scale, v_scale [g];
    window > 0: a query at position p sees only t in (p - window, p].
    Returns (out shaped like q, status)."""
    q4 = q if q.ndim == 4 else q[:, None]
    b, T, h, d = q4.shape
    if k.dtype in (np.uint8, np.int8):
        kvd = FP8_E4M3 if k.dtype == np.uint8 else INT8
        ks, vs = _f32(k_scale), _f32(v_scale)
    else:
        kvd = _dtype_code(k)
        ks = vs = None
    g = k.shape[1]
    if block_table is not None:
        bt = _c(block_table.astype(np.int32))
        P, maxp, num, S = k.shape[2], bt.shape[1], k.shape[0], 0
    else:
        bt, P, maxp, num, S = None, 0, 0, 0, k.shape[2]
    out = np.empty((b, T, h, d), np.float64)
    sl = _c(seq_lens.astype(np.int32))
    rc = lib().oracle_decode_attn_ex(_ptr(_c(q4)), _dtype_code(q4), _ptr(_c(k)), _ptr(_c(v)), kvd,
                                     _ptr(ks), _ptr(vs), _ptr(bt), P, maxp, num, _ptr(sl), b, T,
                                     h, g, S, d, int(window), ctypes.c_float(scale), _ptr(out),
                                     int(nthreads))
    return (out if q.ndim == 4 else out[:, 0]), rc


def rope_table(base: float, n_pos: int, d: int) -> np.ndarray:
    """cos_sin [n_pos, d/2, 2] float32 of the rotary angles p * base^(-2i/d)."""
    t = np.empty((n_pos, d // 2, 2), np.float32)
    lib().oracle_rope_table(float(base), int(n_pos), int(d), _ptr(t))
    return t


def rope_rows(x: np.ndarray, pos: np.ndarray, cos_sin: np.ndarray) -> np.ndarray:
    """A rotated copy of bf16 rows x [..., d] (uint16 bits) at positions pos [n rows]."""
    y = _c(x.copy()).reshape(-1, x.shape[-1])
    lib().oracle_rope_rows(_ptr(y), _ptr(_c(pos.astype(np.int32))), _ptr(_c(cos_sin)),
                           y.shape[0], y.shape[1])
    return y.reshape(x.shape)


def rope_q(q: np.ndarray, cos_sin: np.ndarray, seq_lens: np.ndarray):
    """A rotated copy of q [b, h, d] or [b, T, h, d] (bf16 bits), token tau at
    position L - T + tau. Returns (q', status)."""
    q4 = _c((q if q.ndim == 4 else q[:, None]).copy())
    b, T, h, d = q4.shape
    rc = lib().oracle_rope_q(_ptr(q4), _ptr(_c(cos_sin)), _ptr(_c(seq_lens.astype(np.int32))),
                             b, T, h, d)
    return (q4 if q.ndim == 4 else q4[:, 0]), rc


def append_kv_rope(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray,
                   v_new: np.ndarray, cos_sin: np.ndarray, seq_lens: np.ndarray) -> int:
    """In place (bf16 bits): keys rotated at their positions, values as they are."""
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    kn = k_new if k_new.ndim == 4 else k_new[:, None]
    vn = v_new if v_new.ndim == 4 else v_new[:, None]
    b, g, S, d = k_cache.shape
    return lib().oracle_append_kv_rope(_ptr(k_cache), _ptr(v_cache), _ptr(_c(kn)), _ptr(_c(vn)),
                                       _ptr(_c(cos_sin)), _ptr(_c(seq_lens.astype(np.int32))),
                                       b, kn.shape[1], g, S, d)


def mha_per_head(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Textbook MHA for one sequence: q [h, d], K and V [h, L, d] (float64)."""
    q = _c(q.astype(np.float64))
    K = _c(K.astype(np.float64))
    V = _c(V.astype(np.float64))
    h, L, d = K.shape
    out = np.empty((h, d), np.float64)
    lib().oracle_mha_per_head(_ptr(q), _ptr(K), _ptr(V), h, L, d, float(scale), _ptr(out))
    return out


def partial(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, t0: int, t1: int):
    """Shard [t0, t1) of one query row: returns (m, l, o_unnormalised[d])."""
    q = _c(q.astype(np.float64))
    K = _c(K.astype(np.float64))
    V = _c(V.astype(np.float64))
    d = q.shape[0]
    m, l = ctypes.c_double(), ctypes.c_double()
    o = np.empty(d, np.float64)
    lib().oracle_partial(_ptr(q), _ptr(K), _ptr(V), d, float(scale), t0, t1,
                         ctypes.byref(m), ctypes.byref(l), _ptr(o))
    return m.value, l.value, o


def lse_combine(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Combine n shards (m [n], l [n], o [n, d]) into the normalised output [d]."""
    m = _c(np.asarray(m, np.float64))
    l = _c(np.asarray(l, np.float64))
    o = _c(np.asarray(o, np.float64))
    n, d = o.shape
    out = np.empty(d, np.float64)
    lib().oracle_lse_combine(n, _ptr(m), _ptr(l), _ptr(o), d, _ptr(out))
    return out


def kv_bytes(layers: int, g: int, S: int, d: int, dtype_bytes: int) -> int:
    """2 * layers * g * S * d * dtype_bytes ([GQA notes] §一, §七)."""
    return int(lib().oracle_kv_bytes(layers, g, S, d, dtype_bytes))


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
