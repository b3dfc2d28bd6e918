"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Every case: seeded synthetic inputs on the GPU, one step through
mqa_append_kv + mqa_decode_attn, the exact bytes read back, the oracle run on
them, and an element-by-element comparison.

Tolerance (attention; fp32 accumulate, bf16 or fp32 inputs): for every output
element, |gpu - ref| <= 2e-3 and |gpu - ref| / max(|ref|, rms(ref row)) <= 2e-3,
where the row is out[i, hq, :]. The append must be bit-exact.
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


def compare(out_gpu: torch.Tensor, ref: np.ndarray, what: str = "") -> dict:
    got = out_gpu.detach().cpu().double().numpy()
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
    rel = err / np.maximum(np.abs(ref), rms)
    stats = {"max_abs": float(err.max()), "max_rel_row": float(rel.max())}
    assert stats["max_abs"] <= ATOL and stats["max_rel_row"] <= RTOL_ROW, f"{what}: {stats}"
    return stats


def run_step(t: dict, split_chunk: int = 0, scale: float | None = None,
             kernel: int = mqa.KERNEL_AUTO):
    """append + decode on the device; returns (out, err_flags)."""
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    mqa.append_kv(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["seq_lens"], err_flags=err)
    out = mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], scale=scale,
                          split_chunk=split_chunk, err_flags=err, kernel=kernel)
    torch.cuda.synchronize()
    return out, err


def oracle_ref(t: dict, scale: float | None = None):
    d = t["q"].shape[-1]
    s = np.float32(1.0 / math.sqrt(d)) if scale is None else np.float32(scale)
    ref, _, rc = oracle.decode_attn(W.to_oracle(t["q"]), W.to_oracle(t["k_cache"]),
                                    W.to_oracle(t["v_cache"]), t["seq_lens"].cpu().numpy(),
                                    float(s), nthreads=NTHREADS)
    return ref, rc


def check_case(w: W.Workload, split_chunk: int = 0, layer: int = 0, q_scale: float = 1.0,
               kernel: int = mqa.KERNEL_AUTO):
    print(f"[case] {w.name} b={w.b} h={w.h} g={w.g} d={w.d} S={w.S} chunk={split_chunk} "
          f"kernel={kernel}", flush=True)
    t = W.make_step(w, DEV, layer)
    if q_scale != 1.0:
        t["q"] = (t["q"].float() * q_scale).to(w.dtype)
    kc0, vc0 = W.to_oracle(t["k_cache"]), W.to_oracle(t["v_cache"])
    out, err = run_step(t, split_chunk, kernel=kernel)
    assert int(err.item()) == 0
    # append: bit-exact against the oracle's append on the pre-step bytes
    assert oracle.append_kv(kc0, vc0, W.to_oracle(t["k_new"]), W.to_oracle(t["v_new"]),
                            t["seq_lens"].cpu().numpy()) == oracle.OK
    assert W.to_oracle(t["k_cache"]).tobytes() == kc0.tobytes()
    assert W.to_oracle(t["v_cache"]).tobytes() == vc0.tobytes()
    ref, rc = oracle_ref(t)
    assert rc == oracle.OK
    return compare(out, ref, w.name)


# ---------------------------------------------------------------------------
# the configured workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny-mqa", "mqa-1k", "gqa-70b", "gqa-70b-full", "gqa-70b-tp8",
                                  "gqa-70b-dp8", "mqa-32k"])
def test_workload_full_size(name):
    print(check_case(W.WORKLOADS[name]), flush=True)


@pytest.mark.parametrize("name", ["sweep-g1", "sweep-g8", "sweep-g32"])
@pytest.mark.parametrize("layer", [0, 17, 31])
def test_sweep_layers(name, layer):
    print(check_case(W.WORKLOADS[name], layer=layer), flush=True)


# ---------------------------------------------------------------------------
# shapes, ragged lengths, partitions
# ---------------------------------------------------------------------------

SHAPES = [
    # (h, g, d, dtype): every head grouping the kernels distinguish
    (8, 1, 64, torch.float32), (8, 8, 64, torch.float32), (16, 4, 128, torch.float32),
    (12, 4, 128, torch.bfloat16), (40, 2, 128, torch.bfloat16), (64, 8, 64, torch.bfloat16),
    (32, 1, 128, torch.bfloat16), (32, 16, 128, torch.bfloat16), (6, 6, 128, torch.bfloat16),
    (24, 8, 64, torch.float32), (48, 3, 128, torch.bfloat16),
]


KERNELS = [mqa.KERNEL_AUTO, mqa.KERNEL_VALU]


@pytest.mark.parametrize("kernel", KERNELS, ids=["auto", "valu"])
@pytest.mark.parametrize("h,g,d,dtype", SHAPES)
def test_shapes_with_ragged_lengths(h, g, d, dtype, kernel):
    # lengths around tile (64) and partition (256) edges, 1 and the capacity
    lens = [1, 2, 63, 64, 65, 255, 256, 257, 300, 511, 513, 700]
    w = W.Workload(f"shape-h{h}-g{g}-d{d}", b=len(lens), h=h, g=g, d=d, S=700, dtype=dtype,
                   seed=77)
    t = W.make_step(w, DEV)
    t["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    if kernel == mqa.KERNEL_VALU and dtype == torch.float32:
        pytest.skip("fp32 always runs the vector-ALU kernel (covered by 'auto')")
    for chunk in (256, 0):
        out, err = run_step(t, chunk, kernel=kernel)
        assert int(err.item()) == 0
        ref, _ = oracle_ref(t)
        compare(out, ref, f"{w.name} chunk={chunk}")


@pytest.mark.parametrize("kernel", KERNELS, ids=["auto", "valu"])
@pytest.mark.parametrize("chunk", [64, 128, 512, 4096])
def test_partition_length_sweep(chunk, kernel):
    """Every partition length gives the oracle's result (pins the LSE combine)."""
    w = W.shrink(W.WORKLOADS["gqa-70b"], b=8)
    check_case(w, split_chunk=chunk, kernel=kernel)


@pytest.mark.parametrize("name", ["gqa-70b", "mqa-32k"])
def test_vector_alu_kernel_full_size(name):
    """The vector-ALU kernel on bf16 workloads (the automatic choice there is MFMA)."""
    print(check_case(W.WORKLOADS[name], kernel=mqa.KERNEL_VALU), flush=True)


def test_mfma_kernel_rejects_fp32():
    w = W.Workload("f32", b=1, h=8, g=1, d=64, S=64, dtype=torch.float32, seed=1)
    t = W.make_step(w, DEV)
    with pytest.raises(mqa.MQAError):
        mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], kernel=mqa.KERNEL_MFMA)


@pytest.mark.parametrize("kernel", KERNELS, ids=["auto", "valu"])
def test_peaky_softmax(kernel):
    """q scaled by 8: near one-hot weights, large score range (many rescales)."""
    check_case(W.shrink(W.WORKLOADS["gqa-70b"], b=8), q_scale=8.0, kernel=kernel)
    check_case(W.shrink(W.WORKLOADS["mqa-32k"], b=1, S=4096, L=4096), q_scale=8.0, kernel=kernel)


def test_scale_argument_is_used():
    w = W.shrink(W.WORKLOADS["mqa-1k"], b=2)
    t = W.make_step(w, DEV)
    out, _ = run_step(t, scale=0.3)
    ref, _ = oracle_ref(t, scale=0.3)
    compare(out, ref, "scale=0.3")


# ---------------------------------------------------------------------------
# invariants on the device
# ---------------------------------------------------------------------------

def _nan_tail_pair(t: dict):
    """The step's caches twice: rows >= L zero, and rows >= L NaN."""
    lens = t["seq_lens"].cpu().tolist()
    kz, vz = t["k_cache"].clone(), t["v_cache"].clone()
    kn, vn = t["k_cache"].clone(), t["v_cache"].clone()
    for i, L in enumerate(lens):
        kz[i, :, L:] = 0
        vz[i, :, L:] = 0
        kn[i, :, L:] = float("nan")
        vn[i, :, L:] = float("nan")
    return (kz, vz), (kn, vn)


def test_rows_past_length_are_never_read():
    """NaN in every cache row >= L: the output is finite and bit for bit the
    output with zeros there (the rows are never read; one read as 0 instead of
    skipped would not give NaN, but would move the result). Fixed partitions
    (this shape), and the balanced schedule in its bitwise-reproducible mode."""
    w = W.Workload("tail", b=6, h=16, g=2, d=128, S=1024, dtype=torch.bfloat16, seed=91)
    assert mqa.decode_schedule(w.b, w.h, w.g, w.S, w.d, w.dtype) == "mfma-partitions"
    t = W.make_step(w, DEV)
    t["seq_lens"] = torch.tensor([1, 64, 65, 500, 1000, 1024], dtype=torch.int32, device=DEV)
    run_step(t)  # append first so row L-1 holds k_new
    (kz, vz), (kn, vn) = _nan_tail_pair(t)
    oz = mqa.decode_attn(t["q"], kz, vz, t["seq_lens"])
    on = mqa.decode_attn(t["q"], kn, vn, t["seq_lens"])
    torch.cuda.synchronize()
    assert torch.isfinite(on).all()
    assert torch.equal(oz, on)
    # the balanced schedule: 256 units of ragged lengths
    w = W.Workload("tail-bal", b=128, h=16, g=2, d=128, S=1024, dtype=torch.bfloat16, seed=92,
                   L_lo=1, L_hi=1024)
    assert mqa.decode_schedule(w.b, w.h, w.g, w.S, w.d, w.dtype) == "mfma-balanced"
    t = W.make_step(w, DEV)
    run_step(t)
    (kz, vz), (kn, vn) = _nan_tail_pair(t)
    det = mqa.KERNEL_MFMA_DETERMINISTIC
    oz = mqa.decode_attn(t["q"], kz, vz, t["seq_lens"], kernel=det)
    on = mqa.decode_attn(t["q"], kn, vn, t["seq_lens"], kernel=det)
    torch.cuda.synchronize()
    assert torch.isfinite(on).all()
    assert torch.equal(oz, on)


# Bound on the difference between two calls of the default balanced schedule,
# whose waves claim steps as they go (so which wave sums which steps, and from
# which reference max, varies with timing). For an output element
# o = sum_t a_t v_t / sum_t a_t, each call's result differs from the exact one
# by at most (n u + 2^-18) sum_t alpha_t |v_t| to first order: u = 2^-24 for
# each of the n <= L/32 fp32 additions of step results and merges into a
# running sum, and 2^-18 relative for a weight p split into bf16 hi + lo (lo
# rounds the exact remainder p - hi, |p - hi| <= 2^-9 p). With L <= 4096,
# n u <= 2^-17, so two calls differ by at most 2 (2^-17 + 2^-18) < 2^-15 of
# sum_t alpha_t |v_t|.
RUN_TWICE_BOUND = 2.0 ** -15


def test_deterministic():
    """Fixed partitions (explicit split_chunk) and the balanced schedule in its
    bitwise-reproducible mode give identical bits call after call; the default
    balanced schedule repeats within RUN_TWICE_BOUND * sum_t alpha_t |v_t| of
    each element (alpha from the oracle)."""
    w = W.shrink(W.WORKLOADS["gqa-70b"], b=16)
    t = W.make_step(w, DEV)
    a = mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], split_chunk=512)
    b = mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], split_chunk=512)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    w = W.shrink(W.WORKLOADS["gqa-70b"], b=32)  # 256 units
    t = W.make_step(w, DEV)
    assert mqa.decode_schedule(w.b, w.h, w.g, w.S, w.d, w.dtype) == "mfma-balanced"
    det = mqa.KERNEL_MFMA_DETERMINISTIC
    outs = [mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], kernel=det)
            for _ in range(3)]
    a = mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"])
    b = mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"])
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    scale = float(np.float32(1.0 / math.sqrt(w.d)))
    ref, alpha, rc = oracle.decode_attn(W.to_oracle(t["q"]), W.to_oracle(t["k_cache"]),
                                        W.to_oracle(t["v_cache"]), t["seq_lens"].cpu().numpy(),
                                        scale, want_alpha=True, nthreads=NTHREADS)
    assert rc == oracle.OK
    v = torch.from_numpy(oracle.bf16_bits_to_f64(W.to_oracle(t["v_cache"]))).abs()  # [b, g, S, d]
    al = torch.from_numpy(alpha).view(w.b, w.g, w.h // w.g, w.S)                   # [b, g, G, S]
    spread = torch.matmul(al, v).reshape(w.b, w.h, w.d).numpy()                     # sum_t a_t |v_t|
    diff = (a - b).abs().double().cpu().numpy()
    assert (diff <= RUN_TWICE_BOUND * spread).all(), float((diff / spread).max())
    # both modes are the same attention
    compare(outs[0], ref, "deterministic mode")
    compare(a, ref, "default mode")


def test_constant_v_and_zero_k():
    """V = 1 gives 1; K = 0 gives the mean of the first L rows of V."""
    w = W.Workload("closed", b=4, h=32, g=4, d=128, S=2048, dtype=torch.bfloat16, seed=5)
    t = W.make_step(w, DEV)
    t["seq_lens"] = torch.tensor([1, 100, 1500, 2048], dtype=torch.int32, device=DEV)
    ones = torch.ones_like(t["v_cache"])
    out = mqa.decode_attn(t["q"], t["k_cache"], ones, t["seq_lens"])
    torch.cuda.synchronize()
    assert (out - 1).abs().max().item() <= 1e-6
    zk = torch.zeros_like(t["k_cache"])
    out = mqa.decode_attn(t["q"], zk, t["v_cache"], t["seq_lens"])
    torch.cuda.synchronize()
    for i, L in enumerate(t["seq_lens"].cpu().tolist()):
        mean = t["v_cache"][i, :, :L].double().mean(dim=1)          # [g, d]
        ref = mean.repeat_interleave(w.G, dim=0).cpu().numpy()     # [h, d]
        got = out[i].double().cpu().numpy()
        assert np.abs(got - ref).max() <= 1e-5


# ---------------------------------------------------------------------------
# append and device-side errors
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_append_bit_exact_with_sentinels(dtype):
    """Whole-buffer comparison, with sentinel bands before and after each cache."""
    b, g, S, d = 5, 3, 37, 128
    n = b * g * S * d
    band = 4096
    w = W.Workload("append", b=b, h=g, g=g, d=d, S=S, dtype=dtype, seed=11)
    t = W.make_step(w, DEV)
    t["seq_lens"] = torch.tensor([1, 37, 20, 2, 36], dtype=torch.int32, device=DEV)
    bufs = []
    for name in ("k_cache", "v_cache"):
        buf = torch.full((n + 2 * band,), 7.0, dtype=dtype, device=DEV)
        buf[band:band + n] = t[name].reshape(-1)
        bufs.append(buf)
    kview = bufs[0][band:band + n].view(b, g, S, d)
    vview = bufs[1][band:band + n].view(b, g, S, d)
    k0, v0 = W.to_oracle(kview), W.to_oracle(vview)
    before = [W.to_oracle(x) for x in bufs]
    mqa.append_kv(kview, vview, t["k_new"], t["v_new"], t["seq_lens"])
    torch.cuda.synchronize()
    assert oracle.append_kv(k0, v0, W.to_oracle(t["k_new"]), W.to_oracle(t["v_new"]),
                            t["seq_lens"].cpu().numpy()) == oracle.OK
    after = [W.to_oracle(x) for x in bufs]
    for x0, x1, exp in zip(before, after, (k0, v0)):
        assert x1[:band].tobytes() == x0[:band].tobytes()
        assert x1[band + n:].tobytes() == x0[band + n:].tobytes()
        assert x1[band:band + n].tobytes() == exp.reshape(-1).tobytes()


def test_out_of_range_lengths_flag_and_nan():
    w = W.Workload("badlen", b=4, h=8, g=2, d=64, S=100, dtype=torch.bfloat16, seed=3)
    t = W.make_step(w, DEV)
    t["seq_lens"] = torch.tensor([50, 0, 101, 100], dtype=torch.int32, device=DEV)
    kc0 = t["k_cache"].clone()
    out, err = run_step(t)
    assert int(err.item()) & mqa.DEVERR_SEQLEN
    assert torch.isnan(out[1]).all() and torch.isnan(out[2]).all()
    assert torch.isfinite(out[0]).all() and torch.isfinite(out[3]).all()
    # append skipped the bad sequences entirely
    assert torch.equal(t["k_cache"][1], kc0[1]) and torch.equal(t["k_cache"][2], kc0[2])
    ref, rc = oracle_ref(t)
    assert rc == oracle.BAD_LEN
    got = out.double().cpu().numpy()
    for i in (0, 3):
        assert np.abs(got[i] - ref[i]).max() <= ATOL


# ---------------------------------------------------------------------------
# balanced schedule (bf16, automatic partitioning): unit boundaries cut by
# work-group ranges in every way
# ---------------------------------------------------------------------------

def _check_lens(w: W.Workload, lens, split_chunk=0, kernel=mqa.KERNEL_AUTO):
    t = W.make_step(w, DEV)
    t["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, err = run_step(t, split_chunk, kernel=kernel)
    assert int(err.item()) == 0
    ref, _ = oracle_ref(t)
    return compare(out, ref, w.name)


@pytest.mark.parametrize("chunk", [0, 256])
def test_lengths_at_step_and_partition_edges(chunk):
    """Lengths at the edges of the 32-position steps (31, 32, 33), of a
    partition of C positions (C-1, C, C+1) and of the capacity (S-1, S), with
    1: fixed partitions (C = 256) and the balanced schedule (C = 0)."""
    S = 1000
    edges = [1, 2, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 512, 513, S - 1, S]
    b = 256  # enough (sequence, K/V head) units for the balanced schedule
    lens = [edges[i % len(edges)] for i in range(b)]
    w = W.Workload("edges", b=b, h=16, g=2, d=128, S=S, dtype=torch.bfloat16, seed=28)
    if chunk == 0:
        assert mqa.decode_schedule(w.b, w.h, w.g, w.S, w.d, w.dtype) == "mfma-balanced"
    print(_check_lens(w, lens, split_chunk=chunk), flush=True)


def test_paged_lengths_at_page_edges():
    """Paged cache (16-row pages): lengths at page and step edges."""
    S, P = 200, 16
    edges = [1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 199, 200]
    b = 128
    w = W.Workload("page-edges", b=b, h=16, g=2, d=128, S=S, dtype=torch.bfloat16, seed=29)
    t = W.make_paged_step(w, DEV, page_size=P)
    t["seq_lens"] = torch.tensor([edges[i % len(edges)] for i in range(b)], dtype=torch.int32,
                                 device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = mqa.decode_attn_paged(t["q"], t["k_pages"], t["v_pages"], t["block_table"],
                                t["seq_lens"], err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    d = w.d
    ref, rc = oracle.decode_attn_paged(W.to_oracle(t["q"]), W.to_oracle(t["k_pages"]),
                                       W.to_oracle(t["v_pages"]), t["block_table"].cpu().numpy(),
                                       t["seq_lens"].cpu().numpy(),
                                       float(np.float32(1.0 / math.sqrt(d))), nthreads=NTHREADS)
    assert rc == oracle.OK
    compare(out, ref, "page edges")


def test_many_short_sequences():
    """Units far smaller than a work-group's range (many units per range)."""
    gen = torch.Generator().manual_seed(8)
    lens = torch.randint(1, 101, (1000,), generator=gen).tolist()
    w = W.Workload("short", b=1000, h=16, g=2, d=128, S=100, dtype=torch.bfloat16, seed=21)
    _check_lens(w, lens)


def test_one_long_sequence_many_pieces():
    """One long unit among 255 tiny ones: cut into hundreds of pieces."""
    lens = [1 + (k * 7) % 50 for k in range(255)] + [8192]
    w = W.Workload("long", b=256, h=16, g=1, d=128, S=8192, dtype=torch.bfloat16, seed=22)
    _check_lens(w, lens)


@pytest.mark.parametrize("h,g,d,b", [(64, 2, 128, 128), (32, 1, 64, 256), (64, 1, 128, 256),
                                     (128, 2, 128, 128)])
def test_head_blocks(h, g, d, b):
    """G = 32 / 64 (several 16-head blocks per work-group) and G = 64 across two groups."""
    gen = torch.Generator().manual_seed(h + g + b)
    lens = torch.randint(1, 301, (b,), generator=gen).tolist()
    w = W.Workload(f"hb-h{h}-g{g}", b=b, h=h, g=g, d=d, S=300, dtype=torch.bfloat16, seed=23)
    _check_lens(w, lens)


@pytest.mark.parametrize("h,g,d", [(64, 1, 128), (32, 1, 64), (128, 2, 128)])
def test_few_units_many_heads(h, g, d):
    """Few (sequence, K/V head) units with 32-64 heads each: fixed partitions."""
    w = W.Workload(f"few-h{h}-g{g}", b=3, h=h, g=g, d=d, S=3000, dtype=torch.bfloat16, seed=25)
    _check_lens(w, [3000, 1, 1777])


def test_largest_head_slab():
    """The largest cache the kernels take: one K/V head of 2^23 - 32 bf16 rows
    of d = 128 (just under 2 GiB, the limit of their 32-bit offsets), every
    position attended, the new row appended at the last one."""
    S = (1 << 23) - 32
    w = W.Workload("max-slab", b=1, h=8, g=1, d=128, S=S, dtype=torch.bfloat16, seed=27, L=S)
    print(check_case(w), flush=True)


def test_balanced_schedule_at_its_sequence_limit():
    """1024 sequences (the most the balanced schedule takes) with ragged lengths."""
    gen = torch.Generator().manual_seed(10)
    lens = torch.randint(1, 161, (1024,), generator=gen).tolist()
    w = W.Workload("b1024", b=1024, h=16, g=2, d=128, S=160, dtype=torch.bfloat16, seed=26)
    assert mqa.decode_schedule(w.b, w.h, w.g, w.S, w.d, w.dtype) == "mfma-balanced"
    _check_lens(w, lens)


def test_large_batch_uses_fixed_partitions():
    """More sequences than the balanced schedule takes: the fixed partitions serve it."""
    gen = torch.Generator().manual_seed(9)
    lens = torch.randint(1, 41, (1100,), generator=gen).tolist()
    w = W.Workload("b1100", b=1100, h=8, g=1, d=64, S=40, dtype=torch.bfloat16, seed=24)
    _check_lens(w, lens)


def test_workspace_reused_across_shapes_and_kernels():
    """One workspace for many calls of different shapes and paths; its contents
    on entry are ignored (it starts as NaN bytes and is refilled between
    calls), and partials never collide."""
    big = mqa.decode_workspace(256, 64, 8, 4096, 128, torch.bfloat16, DEV)
    big.fill_(0xFF)  # NaN as float
    cases = [
        (W.Workload("r1", b=64, h=64, g=8, d=128, S=2048, dtype=torch.bfloat16, seed=31), 0, mqa.KERNEL_AUTO),
        (W.Workload("r2", b=256, h=16, g=2, d=64, S=700, dtype=torch.bfloat16, seed=32), 0, mqa.KERNEL_AUTO),
        (W.Workload("r3", b=8, h=32, g=1, d=128, S=3000, dtype=torch.bfloat16, seed=33), 512, mqa.KERNEL_AUTO),
        (W.Workload("r4", b=64, h=64, g=8, d=128, S=2048, dtype=torch.bfloat16, seed=34), 0, mqa.KERNEL_VALU),
    ]
    for rep in range(2):
        for w, chunk, kernel in cases:
            gen = torch.Generator().manual_seed(rep * 100 + w.seed)
            t = W.make_step(w, DEV)
            t["seq_lens"] = torch.randint(1, w.S + 1, (w.b,), generator=gen, dtype=torch.int32).to(DEV)
            out = mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], workspace=big,
                                  split_chunk=chunk, kernel=kernel)
            torch.cuda.synchronize()
            ref, _ = oracle_ref(t)
            compare(out, ref, f"{w.name} rep {rep}")
            big.fill_(0xFF if rep == 0 else 0x7F)


def test_err_flags_checked_before_any_launch():
    """A device err_flags of another dtype, an empty one or a strided one is
    refused by the binding before anything is enqueued."""
    w = W.Workload("errflags", b=2, h=8, g=2, d=64, S=64, dtype=torch.bfloat16, seed=93, L=40)
    t = W.make_step(w, DEV)
    for bad in (torch.zeros(1, dtype=torch.int64, device=DEV),
                torch.zeros(0, dtype=torch.int32, device=DEV),
                torch.zeros(4, dtype=torch.int32, device=DEV)[::2]):
        with pytest.raises(ValueError):
            mqa.append_kv(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["seq_lens"],
                          err_flags=bad)
        with pytest.raises(ValueError):
            mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], err_flags=bad)
    ok = torch.zeros(1, dtype=torch.int32, device=DEV)
    mqa.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], err_flags=ok)
    torch.cuda.synchronize()
    assert int(ok.item()) == 0
