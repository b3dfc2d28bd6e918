"""Decode attention over a shared-head KV cache on MI355X (gfx950).

Thin Python binding over the C ABI of ``libmqa_decode.so`` (declared in
``include/mqa_decode.h``). Every step of the path runs in the library's HIP
kernels; this module only checks tensor metadata and marshals pointers,
sizes and the current HIP stream. PyTorch supplies device memory and streams.

Entry points (same names as the C ABI, without the ``mqa_`` prefix):
  append_kv(k_cache, v_cache, k_new, v_new, seq_lens, err_flags=None)
  decode_attn(q, k_cache, v_cache, seq_lens, scale=None, out=None,
              workspace=None, split_chunk=0, err_flags=None) -> out
  decode_workspace_bytes(b, h, g, S, d, dtype, split_chunk=0)
  decode_workspace(b, h, g, S, d, dtype, device, split_chunk=0) -> uint8 tensor
  decode_resolve_chunk(b, h, g, S, d, dtype, split_chunk=0)
  append_kv_paged(k_pages, v_pages, k_new, v_new, block_table, seq_lens, err_flags=None)
  decode_attn_paged(q, k_pages, v_pages, block_table, seq_lens, scale=None, out=None,
                    workspace=None, split_chunk=0, err_flags=None) -> out
  decode_paged_workspace_bytes(b, h, g, page_size, max_pages, d, dtype, split_chunk=0)
  append_kv_multi(k_cache, v_cache, k_new, v_new, seq_lens, err_flags=None)
  decode_attn_multi(q, k_cache, v_cache, seq_lens, ...) -> out      (q [b, T, h, d])
  append_kv_paged_multi(k_pages, v_pages, k_new, v_new, block_table, seq_lens, err_flags=None)
  decode_attn_paged_multi(q, k_pages, v_pages, block_table, seq_lens, ...) -> out
  decode_multi_workspace_bytes(b, T, h, g, S, d, dtype, split_chunk=0)
  decode_multi_schedule(b, T, h, g, S, d, dtype, split_chunk=0)
  append_kv_fp8 / decode_attn_fp8 / append_kv_paged_fp8 / decode_attn_paged_fp8:
      the same over a cache of fp8 e4m3 codes (uint8 or float8_e4m3fn tensors)
      with per-K/V-head scales k_scale, v_scale (float32 [g]); q and new rows bf16
  decode_attn_ex(q, k, v, seq_lens, block_table=None, k_scale=None, v_scale=None, window=0, ...)
      every option at once (layout, cache type, tokens, sliding window)
  rope_q(q, cos_sin, seq_lens) / append_kv_rope(k_cache, v_cache, k_new, v_new, cos_sin, seq_lens)
      rotary position embedding of the queries / of the keys on append
  kv_bytes(layers, g, S, d, dtype_bytes)
  status_string(status)

There is no CPU fallback: if the library is missing, the first call raises
ImportError. Build it with ``python -m transformer_decode_attention_amd.build``.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "append_kv", "decode_attn", "decode_workspace_bytes", "decode_workspace", "decode_resolve_chunk",
    "decode_schedule", "kv_bytes", "status_string", "MQAError", "LIB_PATH", "DEVERR_SEQLEN",
    "DEVERR_PAGE", "append_kv_paged", "decode_attn_paged", "decode_paged_workspace_bytes",
    "append_kv_multi", "decode_attn_multi", "append_kv_paged_multi", "decode_attn_paged_multi",
    "decode_multi_workspace_bytes", "decode_multi_schedule", "append_kv_fp8", "decode_attn_fp8",
    "append_kv_paged_fp8", "decode_attn_paged_fp8", "decode_attn_ex", "decode_ex_workspace_bytes",
    "rope_q", "append_kv_rope", "append_kv_int8", "append_kv_paged_int8",
    "DEVERR_ROPE", "DEVERR_STALL", "FP8_E4M3", "INT8", "decode_attn_noalloc",
]

# MQA_DECODE_LIB: load another build of the library instead of the in-tree one
# (for instance the host-only sanitizer build of the CPU tests)
LIB_PATH = os.environ.get("MQA_DECODE_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmqa_decode.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH = range(8)
F32, BF16, FP8_E4M3, INT8 = 0, 1, 2, 3
DEVERR_SEQLEN = 1
DEVERR_PAGE = 2
DEVERR_ROPE = 4
DEVERR_STALL = 8

KERNEL_AUTO, KERNEL_VALU, KERNEL_MFMA, KERNEL_MFMA_DETERMINISTIC = 0, 1, 2, 3

EXPORTS = (
    "mqa_append_kv", "mqa_decode_workspace_bytes", "mqa_decode_resolve_chunk",
    "mqa_decode_attn", "mqa_decode_attn_kernel", "mqa_decode_schedule", "mqa_status_string",
    "mqa_kv_bytes", "mqa_append_kv_paged", "mqa_decode_paged_workspace_bytes",
    "mqa_decode_attn_paged", "mqa_append_kv_multi", "mqa_decode_multi_workspace_bytes",
    "mqa_decode_multi_schedule", "mqa_decode_attn_multi", "mqa_append_kv_paged_multi",
    "mqa_decode_attn_paged_multi", "mqa_append_kv_fp8", "mqa_append_kv_paged_fp8",
    "mqa_decode_attn_fp8", "mqa_decode_attn_paged_fp8", "mqa_decode_ex_workspace_bytes",
    "mqa_decode_attn_ex", "mqa_rope_q", "mqa_append_kv_rope", "mqa_append_kv_int8",
    "mqa_append_kv_paged_int8", "mqa_decode_attn_noalloc",
)


class DecodeDesc(ctypes.Structure):
    """mqa_decode_desc of include/mqa_decode.h, field for field."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("err_flags", ctypes.c_void_p),
                ("b", ctypes.c_int), ("T", ctypes.c_int), ("h", ctypes.c_int), ("g", ctypes.c_int),
                ("d", ctypes.c_int), ("S", ctypes.c_int), ("page_size", ctypes.c_int),
                ("max_pages", ctypes.c_int), ("num_pages", ctypes.c_int),
                ("kv_dtype", ctypes.c_int), ("window", ctypes.c_int),
                ("split_chunk", ctypes.c_int), ("scale", ctypes.c_float)]
SCHEDULES = {0: "valu-partitions", 1: "mfma-partitions", 2: "mfma-balanced"}


class MQAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m transformer_decode_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.mqa_append_kv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    L.mqa_append_kv.restype = i32
    L.mqa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.mqa_decode_workspace_bytes.restype = ctypes.c_size_t
    L.mqa_decode_resolve_chunk.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.mqa_decode_resolve_chunk.restype = i32
    L.mqa_decode_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, ctypes.c_float,
                                  vp, vp, ctypes.c_size_t, i32, vp, vp]
    L.mqa_decode_attn.restype = i32
    L.mqa_decode_attn_kernel.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                         ctypes.c_float, vp, vp, ctypes.c_size_t, i32, vp, i32,
                                         vp]
    L.mqa_decode_attn_kernel.restype = i32
    L.mqa_decode_attn_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                          ctypes.c_float, vp, i32, vp, vp]
    L.mqa_decode_attn_noalloc.restype = i32
    L.mqa_decode_schedule.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    L.mqa_decode_schedule.restype = i32
    L.mqa_status_string.argtypes = [i32]
    L.mqa_status_string.restype = ctypes.c_char_p
    L.mqa_kv_bytes.argtypes = [i32, i32, i64, i32, i32]
    L.mqa_kv_bytes.restype = ctypes.c_uint64
    L.mqa_append_kv_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                      vp, vp]
    L.mqa_append_kv_paged.restype = i32
    L.mqa_decode_paged_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    L.mqa_decode_paged_workspace_bytes.restype = ctypes.c_size_t
    L.mqa_decode_attn_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                        i32, ctypes.c_float, vp, vp, ctypes.c_size_t, i32, vp, vp]
    L.mqa_decode_attn_paged.restype = i32
    L.mqa_append_kv_multi.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
    L.mqa_append_kv_multi.restype = i32
    L.mqa_decode_multi_workspace_bytes.argtypes = [i32] * 8
    L.mqa_decode_multi_workspace_bytes.restype = ctypes.c_size_t
    L.mqa_decode_multi_schedule.argtypes = [i32] * 8
    L.mqa_decode_multi_schedule.restype = i32
    L.mqa_decode_attn_multi.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                        ctypes.c_float, vp, vp, ctypes.c_size_t, i32, vp, vp]
    L.mqa_decode_attn_multi.restype = i32
    L.mqa_append_kv_paged_multi.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                            i32, i32, i32, vp, vp]
    L.mqa_append_kv_paged_multi.restype = i32
    L.mqa_decode_attn_paged_multi.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                              i32, i32, i32, ctypes.c_float, vp, vp,
                                              ctypes.c_size_t, i32, vp, vp]
    L.mqa_decode_attn_paged_multi.restype = i32
    L.mqa_append_kv_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    L.mqa_append_kv_fp8.restype = i32
    L.mqa_append_kv_paged_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                          i32, i32, vp, vp]
    L.mqa_append_kv_paged_fp8.restype = i32
    L.mqa_append_kv_int8.argtypes = L.mqa_append_kv_fp8.argtypes
    L.mqa_append_kv_int8.restype = i32
    L.mqa_append_kv_paged_int8.argtypes = L.mqa_append_kv_paged_fp8.argtypes
    L.mqa_append_kv_paged_int8.restype = i32
    L.mqa_decode_attn_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                      ctypes.c_float, vp, vp, ctypes.c_size_t, i32, vp, vp]
    L.mqa_decode_attn_fp8.restype = i32
    L.mqa_decode_attn_paged_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                            i32, i32, i32, ctypes.c_float, vp, vp, ctypes.c_size_t,
                                            i32, vp, vp]
    L.mqa_decode_attn_paged_fp8.restype = i32
    L.mqa_decode_ex_workspace_bytes.argtypes = [ctypes.POINTER(DecodeDesc)]
    L.mqa_decode_ex_workspace_bytes.restype = ctypes.c_size_t
    L.mqa_decode_attn_ex.argtypes = [ctypes.POINTER(DecodeDesc), vp]
    L.mqa_decode_attn_ex.restype = i32
    L.mqa_rope_q.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, vp, vp]
    L.mqa_rope_q.restype = i32
    L.mqa_append_kv_rope.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, vp, vp]
    L.mqa_append_kv_rope.restype = i32
    return L


_lib_handle: ctypes.CDLL | None = None


def lib() -> ctypes.CDLL:
    """The loaded libmqa_decode.so (loaded on first use; raises if missing)."""
    global _lib_handle
    if _lib_handle is None:
        _lib_handle = _load()
    return _lib_handle


def status_string(status: int) -> str:
    return lib().mqa_status_string(int(status)).decode()


def kv_bytes(layers: int, g: int, S: int, d: int, dtype_bytes: int) -> int:
    return int(lib().mqa_kv_bytes(layers, g, S, d, dtype_bytes))


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {dt} (bfloat16 or float32)")


def decode_workspace_bytes(b, h, g, S, d, dtype, split_chunk: int = 0) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(lib().mqa_decode_workspace_bytes(b, h, g, S, d, code, split_chunk))


def decode_workspace(b, h, g, S, d, dtype, device, split_chunk: int = 0) -> torch.Tensor:
    """A workspace for these sizes (its contents on entry are ignored)."""
    n = decode_workspace_bytes(b, h, g, S, d, dtype, split_chunk)
    if n == 0:
        raise ValueError("invalid sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode_resolve_chunk(b, h, g, S, d, dtype, split_chunk: int = 0) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(lib().mqa_decode_resolve_chunk(b, h, g, S, d, code, split_chunk))


def decode_schedule(b, h, g, S, d, dtype, split_chunk: int = 0, kernel: int = 0) -> str:
    """Name of the schedule mqa_decode_attn_kernel runs for these arguments."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    v = int(lib().mqa_decode_schedule(b, h, g, S, d, code, split_chunk, kernel))
    if v < 0:
        raise ValueError("invalid arguments")
    return SCHEDULES[v]


def _ptr(t) -> ctypes.c_void_p | None:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _err(err_flags: torch.Tensor | None, like: torch.Tensor) -> ctypes.c_void_p | None:
    """Pointer to the device error word, checked before any launch: None, or a
    contiguous int32 device tensor of at least one element on the same device
    as the call's tensors (the kernels OR flag bits into its first element, so
    a host pointer or a narrower word there would fault the device)."""
    if err_flags is None:
        return None
    if not isinstance(err_flags, torch.Tensor):
        raise ValueError("err_flags must be a torch.Tensor or None")
    if not err_flags.is_cuda:
        raise ValueError("err_flags must be a device tensor")
    if err_flags.device != like.device:
        raise ValueError(f"err_flags is on {err_flags.device}, the call's tensors on {like.device}")
    if err_flags.dtype != torch.int32:
        raise ValueError("err_flags must be int32")
    if err_flags.numel() < 1 or not err_flags.is_contiguous():
        raise ValueError("err_flags must be a contiguous int32 tensor of at least one element")
    return ctypes.c_void_p(err_flags.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def append_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
              v_new: torch.Tensor, seq_lens: torch.Tensor,
              err_flags: torch.Tensor | None = None) -> None:
    """Write k_new/v_new [b,g,d] into row seq_lens[i]-1 of k_cache/v_cache [b,g,S,d]."""
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new),
                 ("v_new", v_new), ("seq_lens", seq_lens)):
        _dev(t, n)
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must both be [b, g, S, d]")
    b, g, S, d = k_cache.shape
    if k_new.shape != (b, g, d) or v_new.shape != (b, g, d):
        raise ValueError("k_new and v_new must be [b, g, d]")
    if not (k_cache.dtype == v_cache.dtype == k_new.dtype == v_new.dtype):
        raise TypeError("caches and new rows must share one dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (b,):
        raise ValueError("seq_lens must be int32 [b]")
    st = lib().mqa_append_kv(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                            _ptr(seq_lens), b, g, S, d, _dtype_code(k_cache.dtype),
                            _err(err_flags, k_cache), _stream(k_cache.device))
    if st != OK:
        raise MQAError(st, "mqa_append_kv")


def decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                seq_lens: torch.Tensor, scale: float | None = None,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                split_chunk: int = 0, err_flags: torch.Tensor | None = None,
                kernel: int = KERNEL_AUTO) -> torch.Tensor:
    """Decode attention: q [b,h,d], caches [b,g,S,d], seq_lens int32 [b] -> out fp32 [b,h,d].

    kernel: KERNEL_AUTO (mqa_decode_attn), or KERNEL_VALU / KERNEL_MFMA /
    KERNEL_MFMA_DETERMINISTIC (mqa_decode_attn_kernel with that choice; the
    last gives bitwise identical results call after call).
    """
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens)):
        _dev(t, n)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [b, h, d]; k_cache and v_cache [b, g, S, d]")
    b, h, d = q.shape
    bb, g, S, dd = k_cache.shape
    if bb != b or dd != d:
        raise ValueError("q and the caches disagree on b or d")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and the caches must share one dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (b,):
        raise ValueError("seq_lens must be int32 [b]")
    code = _dtype_code(q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((b, h, d), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or out.shape != (b, h, d):
        raise ValueError("out must be float32 [b, h, d]")
    _dev(out, "out")
    if workspace is None:
        workspace = decode_workspace(b, h, g, S, d, code, q.device, split_chunk)
    _dev(workspace, "workspace")
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), b, h, g, S, d, code,
            ctypes.c_float(scale), _ptr(out), _ptr(workspace),
            workspace.numel() * workspace.element_size(), split_chunk, _err(err_flags, q))
    if kernel == KERNEL_AUTO:
        st = lib().mqa_decode_attn(*args, _stream(q.device))
        where = "mqa_decode_attn"
    else:
        st = lib().mqa_decode_attn_kernel(*args, int(kernel), _stream(q.device))
        where = "mqa_decode_attn_kernel"
    if st != OK:
        raise MQAError(st, where)
    return out


def decode_attn_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        seq_lens: torch.Tensor, out: torch.Tensor, scale: float | None = None,
                        split_chunk: int = 0, err_flags: torch.Tensor | None = None) -> torch.Tensor:
    """decode_attn without a workspace (mqa_decode_attn_noalloc: the library's
    own scratch on the current device, nothing allocated); `out` (float32
    [b, h, d]) is the caller's."""
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens),
                 ("out", out)):
        _dev(t, n)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [b, h, d]; k_cache and v_cache [b, g, S, d]")
    b, h, d = q.shape
    bb, g, S, dd = k_cache.shape
    if bb != b or dd != d:
        raise ValueError("q and the caches disagree on b or d")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and the caches must share one dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (b,):
        raise ValueError("seq_lens must be int32 [b]")
    if out.dtype != torch.float32 or out.shape != (b, h, d):
        raise ValueError("out must be float32 [b, h, d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().mqa_decode_attn_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), b, h,
                                       g, S, d, _dtype_code(q.dtype), ctypes.c_float(scale),
                                       _ptr(out), split_chunk, _err(err_flags, q),
                                       _stream(q.device))
    if st != OK:
        raise MQAError(st, "mqa_decode_attn_noalloc")
    return out


# ---- paged cache: pages [num_pages, g, page_size, d], block_table int32 [b, max_pages] ----

def _check_pages(k_pages, v_pages, block_table, seq_lens):
    for n, t in (("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
                 ("seq_lens", seq_lens)):
        _dev(t, n)
    if k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages and v_pages must both be [num_pages, g, page_size, d]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [b, max_pages]")
    b = block_table.shape[0]
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (b,):
        raise ValueError("seq_lens must be int32 [b]")
    return k_pages.shape, b, block_table.shape[1]


def append_kv_paged(k_pages: torch.Tensor, v_pages: torch.Tensor, k_new: torch.Tensor,
                    v_new: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                    err_flags: torch.Tensor | None = None) -> None:
    """Write k_new/v_new [b,g,d] into row (L-1) % page_size of page block_table[i][(L-1) // page_size]."""
    (num_pages, g, P, d), b, max_pages = _check_pages(k_pages, v_pages, block_table, seq_lens)
    for n, t in (("k_new", k_new), ("v_new", v_new)):
        _dev(t, n)
    if k_new.shape != (b, g, d) or v_new.shape != (b, g, d):
        raise ValueError("k_new and v_new must be [b, g, d]")
    if not (k_pages.dtype == v_pages.dtype == k_new.dtype == v_new.dtype):
        raise TypeError("pages and new rows must share one dtype")
    st = lib().mqa_append_kv_paged(_ptr(k_pages), _ptr(v_pages), _ptr(k_new), _ptr(v_new),
                                   _ptr(block_table), _ptr(seq_lens), b, g, P, max_pages,
                                   num_pages, d, _dtype_code(k_pages.dtype), _err(err_flags, k_pages),
                                   _stream(k_pages.device))
    if st != OK:
        raise MQAError(st, "mqa_append_kv_paged")


def decode_paged_workspace_bytes(b, h, g, page_size, max_pages, d, dtype, split_chunk: int = 0) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(lib().mqa_decode_paged_workspace_bytes(b, h, g, page_size, max_pages, d, code,
                                                      split_chunk))


def decode_attn_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                      block_table: torch.Tensor, seq_lens: torch.Tensor,
                      scale: float | None = None, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, split_chunk: int = 0,
                      err_flags: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention over a paged cache -> out fp32 [b,h,d]."""
    (num_pages, g, P, d), b, max_pages = _check_pages(k_pages, v_pages, block_table, seq_lens)
    _dev(q, "q")
    if q.dim() != 3 or q.shape[0] != b or q.shape[2] != d:
        raise ValueError("q must be [b, h, d] matching the pages and the block table")
    if not (q.dtype == k_pages.dtype == v_pages.dtype):
        raise TypeError("q and the pages must share one dtype")
    h = q.shape[1]
    code = _dtype_code(q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((b, h, d), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or out.shape != (b, h, d):
        raise ValueError("out must be float32 [b, h, d]")
    _dev(out, "out")
    if workspace is None:
        n = decode_paged_workspace_bytes(b, h, g, P, max_pages, d, code, split_chunk)
        if n == 0:
            raise ValueError("invalid sizes")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    st = lib().mqa_decode_attn_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                     _ptr(seq_lens), b, h, g, P, max_pages, num_pages, d, code,
                                     ctypes.c_float(scale), _ptr(out), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), split_chunk,
                                     _err(err_flags, q), _stream(q.device))
    if st != OK:
        raise MQAError(st, "mqa_decode_attn_paged")
    return out


# ---- several query tokens per sequence (q [b, T, h, d], causal) ----

def decode_multi_workspace_bytes(b, T, h, g, S, d, dtype, split_chunk: int = 0) -> int:
    """Workspace bytes of a T-token decode (S: capacity, page_size * max_pages when paged)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(lib().mqa_decode_multi_workspace_bytes(b, T, h, g, S, d, code, split_chunk))


def decode_multi_schedule(b, T, h, g, S, d, dtype, split_chunk: int = 0) -> str:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    v = int(lib().mqa_decode_multi_schedule(b, T, h, g, S, d, code, split_chunk))
    if v < 0:
        raise ValueError("invalid arguments")
    return SCHEDULES[v]


def append_kv_multi(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
                    v_new: torch.Tensor, seq_lens: torch.Tensor,
                    err_flags: torch.Tensor | None = None) -> None:
    """Token tau of k_new/v_new [b, T, g, d] -> cache position seq_lens[i] - T + tau."""
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new), ("v_new", v_new),
                 ("seq_lens", seq_lens)):
        _dev(t, n)
    b, g, S, d = k_cache.shape
    if v_cache.shape != k_cache.shape or k_new.dim() != 4 or k_new.shape[0] != b \
            or k_new.shape[2:] != (g, d) or v_new.shape != k_new.shape:
        raise ValueError("caches [b, g, S, d] and new rows [b, T, g, d] must match")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (b,):
        raise ValueError("seq_lens must be int32 [b]")
    if not (k_cache.dtype == v_cache.dtype == k_new.dtype == v_new.dtype):
        raise TypeError("caches and new rows must share one dtype")
    st = lib().mqa_append_kv_multi(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                                   _ptr(seq_lens), b, k_new.shape[1], g, S, d,
                                   _dtype_code(k_cache.dtype), _err(err_flags, k_cache),
                                   _stream(k_cache.device))
    if st != OK:
        raise MQAError(st, "mqa_append_kv_multi")


def _multi_out(q, out, workspace, nbytes):
    b, T, h, d = q.shape
    if out is None:
        out = torch.empty((b, T, h, d), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or out.shape != (b, T, h, d):
        raise ValueError("out must be float32 [b, T, h, d]")
    _dev(out, "out")
    if workspace is None:
        if nbytes == 0:
            raise ValueError("invalid sizes")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    return out, workspace


def decode_attn_multi(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      seq_lens: torch.Tensor, scale: float | None = None,
                      out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      split_chunk: int = 0, err_flags: torch.Tensor | None = None) -> torch.Tensor:
    """T query tokens per sequence with the causal mask -> out fp32 [b, T, h, d]."""
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens)):
        _dev(t, n)
    b, g, S, d = k_cache.shape
    if q.dim() != 4 or q.shape[0] != b or q.shape[3] != d or v_cache.shape != k_cache.shape:
        raise ValueError("q [b, T, h, d] and caches [b, g, S, d] must match")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (b,):
        raise ValueError("seq_lens must be int32 [b]")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and the caches must share one dtype")
    T, h = q.shape[1], q.shape[2]
    code = _dtype_code(q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, workspace = _multi_out(q, out, workspace,
                                decode_multi_workspace_bytes(b, T, h, g, S, d, code, split_chunk))
    st = lib().mqa_decode_attn_multi(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), b, T,
                                     h, g, S, d, code, ctypes.c_float(scale), _ptr(out),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     split_chunk, _err(err_flags, q), _stream(q.device))
    if st != OK:
        raise MQAError(st, "mqa_decode_attn_multi")
    return out


def append_kv_paged_multi(k_pages: torch.Tensor, v_pages: torch.Tensor, k_new: torch.Tensor,
                          v_new: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                          err_flags: torch.Tensor | None = None) -> None:
    """append_kv_multi into a paged cache."""
    (num_pages, g, P, d), b, max_pages = _check_pages(k_pages, v_pages, block_table, seq_lens)
    for n, t in (("k_new", k_new), ("v_new", v_new)):
        _dev(t, n)
    if k_new.dim() != 4 or k_new.shape[0] != b or k_new.shape[2:] != (g, d) \
            or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [b, T, g, d]")
    if not (k_pages.dtype == v_pages.dtype == k_new.dtype == v_new.dtype):
        raise TypeError("pages and new rows must share one dtype")
    st = lib().mqa_append_kv_paged_multi(_ptr(k_pages), _ptr(v_pages), _ptr(k_new), _ptr(v_new),
                                         _ptr(block_table), _ptr(seq_lens), b, k_new.shape[1], g,
                                         P, max_pages, num_pages, d, _dtype_code(k_pages.dtype),
                                         _err(err_flags, k_pages), _stream(k_pages.device))
    if st != OK:
        raise MQAError(st, "mqa_append_kv_paged_multi")


def decode_attn_paged_multi(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                            block_table: torch.Tensor, seq_lens: torch.Tensor,
                            scale: float | None = None, out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, split_chunk: int = 0,
                            err_flags: torch.Tensor | None = None) -> torch.Tensor:
    """decode_attn_multi over a paged cache -> out fp32 [b, T, h, d]."""
    (num_pages, g, P, d), b, max_pages = _check_pages(k_pages, v_pages, block_table, seq_lens)
    _dev(q, "q")
    if q.dim() != 4 or q.shape[0] != b or q.shape[3] != d:
        raise ValueError("q must be [b, T, h, d] matching the pages and the block table")
    if not (q.dtype == k_pages.dtype == v_pages.dtype):
        raise TypeError("q and the pages must share one dtype")
    T, h = q.shape[1], q.shape[2]
    code = _dtype_code(q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, workspace = _multi_out(q, out, workspace,
                                decode_multi_workspace_bytes(b, T, h, g, P * max_pages, d, code,
                                                             split_chunk))
    st = lib().mqa_decode_attn_paged_multi(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                           _ptr(seq_lens), b, T, h, g, P, max_pages, num_pages, d,
                                           code, ctypes.c_float(scale), _ptr(out), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           split_chunk, _err(err_flags, q), _stream(q.device))
    if st != OK:
        raise MQAError(st, "mqa_decode_attn_paged_multi")
    return out


# ---- fp8 e4m3 cache with per-K/V-head scales (q and new rows bf16) ----

_FP8_TYPES = (torch.uint8,) + ((torch.float8_e4m3fn,) if hasattr(torch, "float8_e4m3fn") else ())


def _check_fp8(k, v, k_scale, v_scale, g, int8: bool = False):
    for n, t in (("k cache", k), ("v cache", v), ("k_scale", k_scale), ("v_scale", v_scale)):
        _dev(t, n)
    if int8:
        if k.dtype != torch.int8 or v.dtype != k.dtype:
            raise TypeError("an int8 cache is int8 codes")
    elif k.dtype not in _FP8_TYPES or v.dtype != k.dtype:
        raise TypeError("an fp8 cache is uint8 or float8_e4m3fn codes")
    for n, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
        if sc.dtype != torch.float32 or sc.shape != (g,) or not sc.is_contiguous():
            raise ValueError(f"{n} must be contiguous float32 [g]")


def _rows4(x, name):
    _dev(x, name)
    if x.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16")
    return x if x.dim() == 4 else x.unsqueeze(1)


def _append_codes(fn, int8, k_cache, v_cache, k_new, v_new, k_scale, v_scale, seq_lens,
                  err_flags):
    b, g, S, d = k_cache.shape
    _check_fp8(k_cache, v_cache, k_scale, v_scale, g, int8)
    kn, vn = _rows4(k_new, "k_new"), _rows4(v_new, "v_new")
    if kn.shape[0] != b or kn.shape[2:] != (g, d) or vn.shape != kn.shape or v_cache.shape != k_cache.shape:
        raise ValueError("cache [b, g, S, d] and new rows [b, (T,) g, d] must match")
    _dev(seq_lens, "seq_lens")
    st = getattr(lib(), fn)(_ptr(k_cache), _ptr(v_cache), _ptr(kn), _ptr(vn), _ptr(k_scale),
                            _ptr(v_scale), _ptr(seq_lens), b, kn.shape[1], g, S, d,
                            _err(err_flags, k_cache), _stream(k_cache.device))
    if st != OK:
        raise MQAError(st, fn)


def _append_codes_paged(fn, int8, k_pages, v_pages, k_new, v_new, k_scale, v_scale, block_table,
                        seq_lens, err_flags):
    num_pages, g, P, d = k_pages.shape
    _check_fp8(k_pages, v_pages, k_scale, v_scale, g, int8)
    kn, vn = _rows4(k_new, "k_new"), _rows4(v_new, "v_new")
    for n, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        _dev(t, n)
    b, max_pages = block_table.shape
    st = getattr(lib(), fn)(_ptr(k_pages), _ptr(v_pages), _ptr(kn), _ptr(vn), _ptr(k_scale),
                            _ptr(v_scale), _ptr(block_table), _ptr(seq_lens), b, kn.shape[1], g,
                            P, max_pages, num_pages, d, _err(err_flags, k_pages), _stream(k_pages.device))
    if st != OK:
        raise MQAError(st, fn)


def append_kv_fp8(k_cache, v_cache, k_new, v_new, k_scale, v_scale, seq_lens, err_flags=None):
    """k_new/v_new bf16 [b, g, d] or [b, T, g, d] -> e4m3(x / scale[j]) at positions L-T .. L-1."""
    _append_codes("mqa_append_kv_fp8", False, k_cache, v_cache, k_new, v_new, k_scale, v_scale,
                  seq_lens, err_flags)


def append_kv_paged_fp8(k_pages, v_pages, k_new, v_new, k_scale, v_scale, block_table, seq_lens,
                        err_flags=None):
    """append_kv_fp8 into pages [num_pages, g, page_size, d] of codes."""
    _append_codes_paged("mqa_append_kv_paged_fp8", False, k_pages, v_pages, k_new, v_new, k_scale,
                        v_scale, block_table, seq_lens, err_flags)


def append_kv_int8(k_cache, v_cache, k_new, v_new, k_scale, v_scale, seq_lens, err_flags=None):
    """k_new/v_new bf16 -> int8 codes round-half-even(x / scale[j]) clamped to +-127
    at positions L-T .. L-1 of an int8 cache [b, g, S, d]."""
    _append_codes("mqa_append_kv_int8", True, k_cache, v_cache, k_new, v_new, k_scale, v_scale,
                  seq_lens, err_flags)


def append_kv_paged_int8(k_pages, v_pages, k_new, v_new, k_scale, v_scale, block_table, seq_lens,
                         err_flags=None):
    """append_kv_int8 into pages [num_pages, g, page_size, d] of int8 codes."""
    _append_codes_paged("mqa_append_kv_paged_int8", True, k_pages, v_pages, k_new, v_new, k_scale,
                        v_scale, block_table, seq_lens, err_flags)


def decode_attn_fp8(q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale=None, out=None,
                    workspace=None, split_chunk: int = 0, err_flags=None):
    """Decode over an fp8 cache -> out fp32 shaped like q ([b, h, d] or [b, T, h, d])."""
    b, g, S, d = k_cache.shape
    _check_fp8(k_cache, v_cache, k_scale, v_scale, g)
    q4 = _rows4(q, "q")
    _dev(seq_lens, "seq_lens")
    T, h = q4.shape[1], q4.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o4 = None if out is None else (out if out.dim() == 4 else out.unsqueeze(1))
    o4, workspace = _multi_out(q4, o4, workspace,
                               decode_multi_workspace_bytes(b, T, h, g, S, d, BF16, split_chunk))
    st = lib().mqa_decode_attn_fp8(_ptr(q4), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                   _ptr(v_scale), _ptr(seq_lens), b, T, h, g, S, d,
                                   ctypes.c_float(scale), _ptr(o4), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), split_chunk,
                                   _err(err_flags, q), _stream(q.device))
    if st != OK:
        raise MQAError(st, "mqa_decode_attn_fp8")
    return o4 if q.dim() == 4 else o4[:, 0]


def decode_attn_paged_fp8(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, scale=None,
                          out=None, workspace=None, split_chunk: int = 0, err_flags=None):
    """decode_attn_fp8 over pages [num_pages, g, page_size, d] of codes."""
    num_pages, g, P, d = k_pages.shape
    _check_fp8(k_pages, v_pages, k_scale, v_scale, g)
    q4 = _rows4(q, "q")
    for n, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        _dev(t, n)
    b, max_pages = block_table.shape
    T, h = q4.shape[1], q4.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o4 = None if out is None else (out if out.dim() == 4 else out.unsqueeze(1))
    o4, workspace = _multi_out(q4, o4, workspace,
                               decode_multi_workspace_bytes(b, T, h, g, P * max_pages, d, BF16,
                                                            split_chunk))
    st = lib().mqa_decode_attn_paged_fp8(_ptr(q4), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                         _ptr(v_scale), _ptr(block_table), _ptr(seq_lens), b, T, h,
                                         g, P, max_pages, num_pages, d, ctypes.c_float(scale),
                                         _ptr(o4), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), split_chunk,
                                         _err(err_flags, q), _stream(q.device))
    if st != OK:
        raise MQAError(st, "mqa_decode_attn_paged_fp8")
    return o4 if q.dim() == 4 else o4[:, 0]


# ---- every option at once; rotary position embedding ----

def _ex_desc(q4, k, v, seq_lens, block_table, k_scale, v_scale, window, scale, split_chunk):
    for n, t in (("q", q4), ("k", k), ("v", v), ("seq_lens", seq_lens)):
        _dev(t, n)
    b, T, h, d = q4.shape
    g = k.shape[1]
    if k.dtype in _FP8_TYPES:
        kvd = FP8_E4M3
        _check_fp8(k, v, k_scale, v_scale, g)
    elif k.dtype == torch.int8:
        kvd = INT8
        _check_fp8(k, v, k_scale, v_scale, g, int8=True)
    else:
        kvd = _dtype_code(k.dtype)
    desc = DecodeDesc()
    desc.q, desc.k, desc.v, desc.seq_lens = _ptr(q4), _ptr(k), _ptr(v), _ptr(seq_lens)
    desc.b, desc.T, desc.h, desc.g, desc.d = b, T, h, g, d
    if block_table is not None:
        _dev(block_table, "block_table")
        desc.block_table = _ptr(block_table)
        desc.page_size, desc.max_pages, desc.num_pages = k.shape[2], block_table.shape[1], k.shape[0]
    else:
        desc.S = k.shape[2]
    if kvd in (FP8_E4M3, INT8):
        desc.k_scale, desc.v_scale = _ptr(k_scale), _ptr(v_scale)
    desc.kv_dtype, desc.window, desc.split_chunk = kvd, int(window), int(split_chunk)
    desc.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    return desc


def decode_ex_workspace_bytes(q, k, v, seq_lens, block_table=None, k_scale=None, v_scale=None,
                              window=0, split_chunk: int = 0) -> int:
    """Workspace bytes decode_attn_ex needs for these operands
    (mqa_decode_ex_workspace_bytes; raises on invalid arguments)."""
    q4 = q if q.dim() == 4 else q.unsqueeze(1)
    desc = _ex_desc(q4, k, v, seq_lens, block_table, k_scale, v_scale, window, None, split_chunk)
    n = int(lib().mqa_decode_ex_workspace_bytes(ctypes.byref(desc)))
    if n == 0:
        raise ValueError("invalid arguments")
    return n


def decode_attn_ex(q, k, v, seq_lens, block_table=None, k_scale=None, v_scale=None, window=0,
                   scale=None, out=None, workspace=None, split_chunk: int = 0, err_flags=None):
    """Decode with every option (mqa_decode_attn_ex): q [b, h, d] or [b, T, h, d];
    k, v contiguous [b, g, S, d] or pages [num_pages, g, P, d] with block_table
    [b, max_pages]; a bf16, f32, fp8 (uint8 / float8_e4m3fn codes) or int8 (int8
    codes) cache, the codes with k_scale, v_scale [g]; window > 0: sliding window.
    Returns out shaped like q."""
    q4 = q if q.dim() == 4 else q.unsqueeze(1)
    b, T, h, d = q4.shape
    desc = _ex_desc(q4, k, v, seq_lens, block_table, k_scale, v_scale, window, scale, split_chunk)
    o4 = None if out is None else (out if out.dim() == 4 else out.unsqueeze(1))
    if o4 is None:
        o4 = torch.empty((b, T, h, d), dtype=torch.float32, device=q.device)
    _dev(o4, "out")
    desc.out = _ptr(o4)
    if workspace is None:
        n = int(lib().mqa_decode_ex_workspace_bytes(ctypes.byref(desc)))
        if n == 0:
            raise ValueError("invalid arguments")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    desc.workspace = _ptr(workspace)
    desc.workspace_bytes = workspace.numel() * workspace.element_size()
    desc.err_flags = _err(err_flags, q)
    st = lib().mqa_decode_attn_ex(ctypes.byref(desc), _stream(q.device))
    if st != OK:
        raise MQAError(st, "mqa_decode_attn_ex")
    return o4 if q.dim() == 4 else o4[:, 0]


def _cos_sin(cs, d):
    _dev(cs, "cos_sin")
    if cs.dtype != torch.float32 or cs.dim() != 3 or cs.shape[1:] != (d // 2, 2):
        raise ValueError("cos_sin must be float32 [n_pos, d/2, 2]")
    return cs.shape[0]


def rope_q(q, cos_sin, seq_lens, err_flags=None):
    """Rotate q ([b, h, d] or [b, T, h, d], bf16) in place at positions L - T + tau."""
    q4 = _rows4(q, "q")
    _dev(seq_lens, "seq_lens")
    b, T, h, d = q4.shape
    n_pos = _cos_sin(cos_sin, d)
    st = lib().mqa_rope_q(_ptr(q4), _ptr(cos_sin), n_pos, _ptr(seq_lens), b, T, h, d,
                          _err(err_flags, q), _stream(q.device))
    if st != OK:
        raise MQAError(st, "mqa_rope_q")
    return q


def append_kv_rope(k_cache, v_cache, k_new, v_new, cos_sin, seq_lens, err_flags=None):
    """append_kv_multi with the keys rotated at their positions (bf16 cache)."""
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens)):
        _dev(t, n)
    kn, vn = _rows4(k_new, "k_new"), _rows4(v_new, "v_new")
    b, g, S, d = k_cache.shape
    if k_cache.dtype != torch.bfloat16 or v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise TypeError("the rotated append takes a bf16 cache")
    if kn.shape[0] != b or kn.shape[2:] != (g, d) or vn.shape != kn.shape:
        raise ValueError("new rows must be [b, (T,) g, d]")
    n_pos = _cos_sin(cos_sin, d)
    st = lib().mqa_append_kv_rope(_ptr(k_cache), _ptr(v_cache), _ptr(kn), _ptr(vn), _ptr(cos_sin),
                                  n_pos, _ptr(seq_lens), b, kn.shape[1], g, S, d, _err(err_flags, k_cache),
                                  _stream(k_cache.device))
    if st != OK:
        raise MQAError(st, "mqa_append_kv_rope")
