"""Seeded synthetic workloads for decode attention over a shared-head KV cache.

Input generation only: shapes, seeds and value distributions. No step of the
method is computed here; both the HIP path (through the tests and the bench)
and the oracle consume what these generators produce.

The configurations mirror the workload shapes on the pages (cited by title and
section):
  tiny-mqa   b=1, h=8, g=1, d=64, 128 cached + 1 appended, fp32
             (freeguideonline "多查询注意力 MQA", §5: d_model=512, h=8, d_k=64)
  mqa-1k     b=8, h=32, g=1, d=128, L=1024, bf16
             (nanhubrain.csdn.net MQA article §2.1/§4.3: 32 heads, 1024 positions, batch 8)
  gqa-70b    b=64, h=64, g=8, d=128, ragged L ~ U[1024, 4096], capacity 4096, bf16
             (ybb.press GQA/MQA notes §一 and §七: LLaMA-2-70B-like h=64, g=8,
             4K context, 64 concurrent sequences)
  gqa-70b-full  the same with every L = 4096
  gqa-70b-tp8   one GPU's share of gqa-70b when the heads are split 8 ways
             (b=64, h=8, g=1, the same lengths): one K/V head and its 8 query heads
  gqa-70b-dp8   one GPU's share when the sequences are split 8 ways instead
             (b=8, h=64, g=8; lengths U[1024, 4096] drawn for 8 sequences)
  mqa-32k    b=4, h=32, g=1, d=128, L=32768, bf16 (same notes §一: context of 32K)
  sweep-g{1,8,32}  32 layers of b=16, h=32, d=128, L=8192, bf16, g in {1, 8, 32}
             (compassingai "多查詢注意力", 技術原理: d_model=4096, h=32, seq 8192, 32 layers)

Values: q, K, V, k_new, v_new are i.i.d. N(0, 1), drawn in fp32 with torch's
seeded generator and rounded (round-to-nearest-even) to the cache dtype. The
whole cache capacity is filled; the step's append then overwrites row L_i-1.
seq_lens holds the post-append lengths. Seeds: base = 1000 * k for the k-th
configuration; streams q +1, k_cache +2, v_cache +3, k_new +4, v_new +5,
seq_lens +6 (a CPU generator), layer l adds 100 * l.

Several query tokens per sequence (make_multi_step): q [b, T, h, d] and
k_new/v_new [b, T, g, d] drawn like the one-token ones (streams +8, +9, +10),
lengths raised to at least T.

fp8 caches (make_fp8_step): codes drawn bit by bit on the device, not
converted from values: sign uniform, exponent field 7 + round(N(0, 1.5))
clipped to [0, 15] (magnitudes around 1, as quantised N(0, 1) data, with
subnormals and the top binade among them), mantissa uniform, the NaN pattern
(exponent 15, mantissa 7) moved to mantissa 6 (stream +11); per-K/V-head
scales U[0.25, 1] for K and for V (stream +12, CPU); q and the new rows as
above (bf16). int8 caches (make_int8_step): codes N(0, 32) rounded and
clamped to -128 .. 127 (stream +13), scales U[1/48, 1/24] (stream +14).

Paged variants (make_paged_step): the same values scattered into pages of
page_size rows with page ids drawn as a random permutation (CPU generator,
stream +7) of b * ceil(S / page_size) + extra_pages pages; pages no sequence
uses hold NaN.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    b: int
    h: int
    g: int
    d: int
    S: int                 # cache capacity (rows per K/V head)
    dtype: torch.dtype
    seed: int
    L: int | None = None   # fixed attended length; None -> ragged U[L_lo, L_hi]
    L_lo: int = 0
    L_hi: int = 0
    layers: int = 1

    @property
    def G(self) -> int:
        return self.h // self.g

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == torch.bfloat16 else 4


WORKLOADS = {
    "tiny-mqa": Workload("tiny-mqa", b=1, h=8, g=1, d=64, S=129, dtype=torch.float32,
                         seed=1000, L=129),
    "mqa-1k": Workload("mqa-1k", b=8, h=32, g=1, d=128, S=1024, dtype=torch.bfloat16,
                       seed=2000, L=1024),
    "gqa-70b": Workload("gqa-70b", b=64, h=64, g=8, d=128, S=4096, dtype=torch.bfloat16,
                        seed=3000, L=None, L_lo=1024, L_hi=4096),
    "gqa-70b-full": Workload("gqa-70b-full", b=64, h=64, g=8, d=128, S=4096,
                             dtype=torch.bfloat16, seed=3000, L=4096),
    "gqa-70b-tp8": Workload("gqa-70b-tp8", b=64, h=8, g=1, d=128, S=4096, dtype=torch.bfloat16,
                            seed=3000, L=None, L_lo=1024, L_hi=4096),
    "gqa-70b-dp8": Workload("gqa-70b-dp8", b=8, h=64, g=8, d=128, S=4096, dtype=torch.bfloat16,
                            seed=3000, L=None, L_lo=1024, L_hi=4096),
    "mqa-32k": Workload("mqa-32k", b=4, h=32, g=1, d=128, S=32768, dtype=torch.bfloat16,
                        seed=4000, L=32768),
    "sweep-g1": Workload("sweep-g1", b=16, h=32, g=1, d=128, S=8192, dtype=torch.bfloat16,
                         seed=5000, L=8192, layers=32),
    "sweep-g8": Workload("sweep-g8", b=16, h=32, g=8, d=128, S=8192, dtype=torch.bfloat16,
                         seed=5000, L=8192, layers=32),
    "sweep-g32": Workload("sweep-g32", b=16, h=32, g=32, d=128, S=8192,
                          dtype=torch.bfloat16, seed=5000, L=8192, layers=32),
}


def shrink(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    return replace(w, **kw)


def seq_lens(w: Workload) -> torch.Tensor:
    """Post-append lengths [b] (int32, CPU)."""
    if w.L is not None:
        return torch.full((w.b,), w.L, dtype=torch.int32)
    gen = torch.Generator().manual_seed(w.seed + 6)
    return torch.randint(w.L_lo, w.L_hi + 1, (w.b,), generator=gen, dtype=torch.int32)


def _normal(shape, seed: int, dtype: torch.dtype, device) -> torch.Tensor:
    gen = torch.Generator(device=device).manual_seed(seed)
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(dtype)


def make_step(w: Workload, device="cpu", layer: int = 0) -> dict:
    """One layer's inputs for one decode step.

    Returns q [b,h,d], k_cache/v_cache [b,g,S,d] (every row filled), k_new and
    v_new [b,g,d], seq_lens int32 [b] (post-append), all on `device`.
    """
    base = w.seed + 100 * layer
    return {
        "q": _normal((w.b, w.h, w.d), base + 1, w.dtype, device),
        "k_cache": _normal((w.b, w.g, w.S, w.d), base + 2, w.dtype, device),
        "v_cache": _normal((w.b, w.g, w.S, w.d), base + 3, w.dtype, device),
        "k_new": _normal((w.b, w.g, w.d), base + 4, w.dtype, device),
        "v_new": _normal((w.b, w.g, w.d), base + 5, w.dtype, device),
        "seq_lens": seq_lens(w).to(device),
    }


def to_oracle(t: torch.Tensor):
    """Host numpy view the oracle takes: float32 as is, bfloat16 as uint16 bits."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def make_paged_step(w: Workload, device="cpu", page_size: int = 16, layer: int = 0,
                    extra_pages: int = 3, share_prefix: bool = False) -> dict:
    """make_step's values in a paged layout.

    Returns the make_step dict plus k_pages/v_pages [num_pages, g, page_size, d],
    block_table int32 [b, max_pages] and the capacity page_size * max_pages.
    With share_prefix, sequence 1 uses sequence 0's first page (its first
    page_size rows are set equal to sequence 0's before the scatter).
    """
    t = make_step(w, device, layer)
    b, g, S, d = t["k_cache"].shape
    P = page_size
    maxp = -(-S // P)
    num = b * maxp + extra_pages
    gen = torch.Generator().manual_seed(w.seed + 100 * layer + 7)
    ids = torch.randperm(num, generator=gen)[: b * maxp].view(b, maxp).to(torch.int32)
    if share_prefix and b > 1:
        ids[1, 0] = ids[0, 0]
        for name in ("k_cache", "v_cache"):
            t[name][1, :, :P] = t[name][0, :, :P]
    pages = {}
    for name in ("k_cache", "v_cache"):
        c = t[name]
        padded = torch.full((b, g, maxp * P, d), float("nan"), dtype=c.dtype, device=device)
        padded[:, :, :S] = c
        per_page = padded.view(b, g, maxp, P, d).permute(0, 2, 1, 3, 4).reshape(b * maxp, g, P, d)
        dst = torch.full((num, g, P, d), float("nan"), dtype=c.dtype, device=device)
        dst[ids.view(-1).long().to(device)] = per_page
        pages[name] = dst
    t["k_pages"], t["v_pages"] = pages["k_cache"], pages["v_cache"]
    t["block_table"] = ids.to(device)
    t["page_size"] = P
    t["capacity"] = maxp * P
    return t


def make_multi_step(w: Workload, device="cpu", T: int = 4, layer: int = 0,
                    page_size: int = 0) -> dict:
    """A step with T query tokens per sequence (a verified draft, a prompt chunk).

    The make_step (or make_paged_step, page_size > 0) dict with q [b, T, h, d],
    k_new/v_new [b, T, g, d], and seq_lens (post-append, so counting the T new
    tokens) raised to at least T.
    """
    t = make_paged_step(w, device, page_size, layer) if page_size else make_step(w, device, layer)
    base = w.seed + 100 * layer
    t["q"] = _normal((w.b, T, w.h, w.d), base + 8, w.dtype, device)
    t["k_new"] = _normal((w.b, T, w.g, w.d), base + 9, w.dtype, device)
    t["v_new"] = _normal((w.b, T, w.g, w.d), base + 10, w.dtype, device)
    t["seq_lens"] = torch.clamp(t["seq_lens"], min=T)
    t["T"] = T
    return t


def make_int8_step(w: Workload, device="cpu", T: int = 1, layer: int = 0,
                   page_size: int = 0) -> dict:
    """make_fp8_step over an int8 cache (codes N(0, 32) rounded, clamped to
    -128 .. 127; scales U[1/48, 1/24] per K/V head)."""
    return make_fp8_step(w, device, T, layer, page_size, int8=True)


def make_fp8_step(w: Workload, device="cpu", T: int = 1, layer: int = 0,
                  page_size: int = 0, int8: bool = False) -> dict:
    """A step over an fp8 e4m3 cache: k_cache/v_cache uint8 codes [b, g, S, d]
    (or k_pages/v_pages with block_table), k_scale/v_scale float32 [g], q bf16
    [b, h, d] (T = 1) or [b, T, h, d], k_new/v_new bf16 [b, g, d] or [b, T, g, d],
    seq_lens (post-append, at least T). With int8 the codes are int8."""
    base = w.seed + 100 * layer
    gen = torch.Generator(device=device).manual_seed(base + (13 if int8 else 11))
    shape = (w.b, w.g, w.S, w.d)

    def codes():
        kw = dict(generator=gen, device=device)
        if int8:  # N(0, 32) rounded and clamped to the code range: N(0,1)-like values at scale ~1/32
            return torch.round(torch.randn(shape, **kw) * 32).clamp(-128, 127).to(torch.int8)
        sign = torch.randint(0, 2, shape, dtype=torch.uint8, **kw)
        # exponent field 7 + N(0, 1.5) over the whole range 0 .. 15 (0: subnormals,
        # 15: the 256 .. 448 binade), mantissa uniform; the NaN pattern (15, 7)
        # becomes (15, 6), the largest finite code
        expo = (7 + torch.round(torch.randn(shape, **kw) * 1.5)).clamp(0, 15).to(torch.uint8)
        mant = torch.randint(0, 8, shape, dtype=torch.uint8, **kw)
        mant = torch.where((expo == 15) & (mant == 7), torch.full_like(mant, 6), mant)
        return (sign << 7) | (expo << 3) | mant

    k, v = codes(), codes()
    sgen = torch.Generator().manual_seed(base + (14 if int8 else 12))
    lo, span = (1 / 48, 1 / 48) if int8 else (0.25, 0.75)
    t = {
        "k_cache": k, "v_cache": v,
        "k_scale": (lo + span * torch.rand(w.g, generator=sgen)).to(device),
        "v_scale": (lo + span * torch.rand(w.g, generator=sgen)).to(device),
        "seq_lens": torch.clamp(seq_lens(w), min=T).to(device),
    }
    if T == 1:
        t["q"] = _normal((w.b, w.h, w.d), base + 1, torch.bfloat16, device)
        t["k_new"] = _normal((w.b, w.g, w.d), base + 4, torch.bfloat16, device)
        t["v_new"] = _normal((w.b, w.g, w.d), base + 5, torch.bfloat16, device)
    else:
        t["q"] = _normal((w.b, T, w.h, w.d), base + 8, torch.bfloat16, device)
        t["k_new"] = _normal((w.b, T, w.g, w.d), base + 9, torch.bfloat16, device)
        t["v_new"] = _normal((w.b, T, w.g, w.d), base + 10, torch.bfloat16, device)
    t["T"] = T
    if page_size:
        P = page_size
        b, g, S, d = shape
        maxp = -(-S // P)
        num = b * maxp + 3
        pgen = torch.Generator().manual_seed(base + 7)
        ids = torch.randperm(num, generator=pgen)[: b * maxp].view(b, maxp).to(torch.int32)
        for name, c in (("k_pages", k), ("v_pages", v)):
            padded = torch.zeros((b, g, maxp * P, d), dtype=c.dtype, device=device)
            padded[:, :, :S] = c
            per_page = padded.view(b, g, maxp, P, d).permute(0, 2, 1, 3, 4).reshape(b * maxp, g, P, d)
            # unused pages: NaN codes (fp8), the largest code (int8)
            dst = torch.full((num, g, P, d), 127 if int8 else 0x7F, dtype=c.dtype, device=device)
            dst[ids.view(-1).long().to(device)] = per_page
            t[name] = dst
        del t["k_cache"], t["v_cache"]
        t["block_table"] = ids.to(device)
        t["page_size"] = P
        t["capacity"] = maxp * P
    return t
