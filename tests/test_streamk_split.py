"""CPU model of how the balanced schedule splits the work between work-groups.

Every valid (sequence, K/V head) unit weighs its steps plus an allowance of C
steps for closing its segment; the units are laid end to end, the allowance
before the steps, and work-group w takes the weights [TW w / nwg,
TW (w + 1) / nwg) of the total TW, with every step whose weight falls inside
(a boundary inside an allowance falls at the unit's first step). The kernel
(StepSplit in the HIP source) finds the sequence that holds a range's end
(here by a binary search over the per-sequence prefix sums, there by every
thread checking its share of the sequences) and the range that holds a given
step by the inverse formula; this model restates both and checks, over random
ragged batches with invalid lengths among them, that
  * the ranges cover the steps in order, each exactly once, none empty
    (ranges of at least kStreamMinSteps weights);
  * the owner formula names the range that holds each step;
  * each range's weight is its share of the total to within C;
  * C = 0 is the plain equal split of the steps.
"""
from __future__ import annotations

import os
import random
import re

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "transformer_decode_attention_amd", "csrc", "mqa_decode.hip")


def kernel_constant(name: str) -> int:
    m = re.search(rf"constexpr int {name} = ([^;]+);", open(SRC).read())
    assert m, name
    return int(eval(m.group(1), {}, {}))


MIN_STEPS = kernel_constant("kStreamMinSteps")


def seq_steps(L: int, S: int) -> int:
    return 0 if (L < 1 or L > S) else (L + 31) // 32


class Split:
    def __init__(self, lens, S, g, nwg, C):
        self.C, self.g, self.nwg, self.b = C, g, nwg, len(lens)
        self.n = [seq_steps(L, S) for L in lens]
        self.pre, self.vpre = [0], [0]
        for n in self.n:
            self.pre.append(self.pre[-1] + g * n)
            self.vpre.append(self.vpre[-1] + (n > 0))
        self.T = self.pre[-1]

    def useq(self, i):
        return self.pre[i] + self.C * self.g * self.vpre[i]

    def start(self, w):
        if self.C == 0:
            return self.T * w // self.nwg
        TW = self.useq(self.b)
        wb = TW * w // self.nwg
        if wb >= TW:
            return self.T
        lo, hi = 0, self.b
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if self.useq(mid) <= wb:
                lo = mid
            else:
                hi = mid
        n = self.n[lo]
        off = wb - self.useq(lo)
        j, o = divmod(off, n + self.C)
        return self.pre[lo] + j * n + max(0, o - self.C)

    def owner(self, i, j, o):
        TW = self.useq(self.b)
        x = self.useq(i) + j * (self.n[i] + self.C) + self.C + o
        return ((x + 1) * self.nwg - 1) // TW


def random_batch(rng):
    b = rng.randint(1, 120)
    S = rng.choice([64, 1000, 4096])
    lens = []
    for _ in range(b):
        r = rng.random()
        lens.append(0 if r < 0.05 else S + 1 if r < 0.08 else rng.randint(1, S))
    return lens, S, rng.choice([1, 2, 8])


@pytest.mark.parametrize("C", [0, 1, 2, 3, 4, 6])
def test_ranges_partition_the_steps_and_owner_agrees(C):
    rng = random.Random(300 + C)
    n = 0
    while n < 300:
        lens, S, g = random_batch(rng)
        sp = Split(lens, S, g, 1, C)
        if sp.T < MIN_STEPS:
            continue
        n += 1
        nwg = rng.randint(1, min(300, sp.T // MIN_STEPS))
        sp.nwg = nwg
        bounds = [sp.start(w) for w in range(nwg + 1)]
        assert bounds[0] == 0 and bounds[-1] == sp.T
        assert all(a < b_ for a, b_ in zip(bounds, bounds[1:])), "an empty or reversed range"
        if C == 0:
            assert bounds == [sp.T * w // nwg for w in range(nwg + 1)]
        TW = sp.useq(sp.b)
        units_starting = [0] * nwg
        w = 0
        for i, ni in enumerate(sp.n):
            for j in range(g if ni else 0):
                for o in range(ni):
                    x = sp.pre[i] + j * ni + o
                    while not (bounds[w] <= x < bounds[w + 1]):
                        w += 1
                    assert sp.owner(i, j, o) == w, (i, j, o)
                    if o == 0:
                        units_starting[w] += 1
        for w in range(nwg):
            weight = bounds[w + 1] - bounds[w] + C * units_starting[w]
            share = TW * (w + 1) // nwg - TW * w // nwg
            assert abs(weight - share) <= C, (w, weight, share)


def test_kernel_allowances():
    """The allowances the kernel gives its variants: none for the one-block
    bf16 kernel (its segment closes cost a fraction of a step), a few steps
    where closes were measured dear."""
    src = open(SRC).read()
    m = re.search(r"constexpr int kSegC = KV::kF8 \? (\d+) : NHB == 2 \? \(SHARED \? (\d+) : (\d+)\) : (\d+);",
                  src)
    assert m, "the allowance expression changed; update this model"
    f8, two_shared, two, one = map(int, m.groups())
    assert one == 0 and all(0 < c < MIN_STEPS for c in (f8, two_shared, two))
