"""CPU model of the balanced schedule's claim protocol (no GPU).

In the balanced decode kernel the waves of one head block share the steps of
a work-group's range: each claims the next step from an LDS counter (the
range's last segment first, then the rest from its start), keeps a running
state while its claims stay in one unit (a sequence's K/V head), and when a
claim leaves the unit it either passes the segment's record on (all of the
segment was its own) or parks its state in its LDS slot and adds
(steps, its bit) to the segment's record; the wave whose addition completes
the segment merges the parked states, frees their slots and releases the
record to the segment kRing later. Its waits (for a slot, for a record) are
bounded: a wait that runs out marks the work-group broken, raises
MQA_DEVERR_STALL and makes its rows NaN.

This model runs the same protocol, with the kernel's constants read from the
kernel source, as Python generators that yield at every LDS access, under
random interleavings (uniform, and with one wave starved), and checks that
  * no interleaving deadlocks or reaches the wait bound,
  * every segment of the range gets exactly one result, and it holds each of
    the segment's steps exactly once (from whichever waves computed them);
and that a protocol with a planted mistake (a record never released, a slot
never freed) ends with every wait bounded, the stall flag raised and the
broken work-group's results marked, instead of spinning forever. The same
checks run the bitwise-reproducible variant (fixed claims, merges in wave
order), which must also merge every segment identically in every
interleaving.
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
    return int(eval(m.group(1), {}, {}))  # literals such as 16 or 1 << 22


RING = kernel_constant("kRing")
WAVES = kernel_constant("kStreamWaves")
MIN_STEPS = kernel_constant("kStreamMinSteps")


def range_start(w: int, T: int, nwg: int) -> int:
    return T * w // nwg


class Stalled(Exception):
    pass


class WorkGroup:
    """One work-group's range [x0, x1) over units laid end to end (unit u has
    steps [start[u], start[u] + n[u])), one head block of `wph` waves."""

    def __init__(self, lens, x0, x1, wph, ring, cap, mutant=None, det=False):
        self.lens, self.x0, self.x1, self.wph, self.ring, self.cap = lens, x0, x1, wph, ring, cap
        self.mutant = mutant
        self.det = det               # fixed round-robin claims, merges in wave order
        self.nclaims = [0] * wph
        self.start = [0]
        for n in lens:
            self.start.append(self.start[-1] + n)
        self.cursor = 0
        self.rec_tag = list(range(ring))
        self.rec_val = [0] * ring
        self.slot_busy = [0] * wph
        self.slot = [None] * wph
        self.broken = False
        self.flags = 0
        self.results = {}  # segment start -> (steps, written while broken)
        self.orders = {}   # segment start -> the merge as ((wave, its steps), ...) in order
        u_last = self.unit_of(x1 - 1)
        self.xl = max(x0, self.start[u_last])
        self.len_last = x1 - self.xl
        self.ord0 = self.unit_of(x0)
        self.max_spin = 0

    def unit_of(self, t):
        lo, hi = 0, len(self.lens)
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if self.start[mid] <= t:
                lo = mid
            else:
                hi = mid
        return lo

    def claim(self, w):
        if self.det:
            c = w + self.wph * self.nclaims[w]
            self.nclaims[w] += 1
        else:
            c = self.cursor
            self.cursor += 1
        if c >= self.x1 - self.x0:
            return self.x1
        return self.xl + c if c < self.len_last else self.x0 + (c - self.len_last)

    def wait(self, cond):
        """Poll cond at most `cap` times (one poll per scheduling turn)."""
        n = 0
        while not cond():
            n += 1
            self.max_spin = max(self.max_spin, n)
            if n == self.cap:
                self.broken = True
                self.flags |= 8
                return
            yield "wait", cond

    def finish(self, w, u, mine):
        seg_s, seg_e = max(self.x0, self.start[u]), min(self.x1, self.start[u + 1])
        sn = 0 if seg_s == self.xl else u - self.ord0 + 1
        e = sn % self.ring
        if len(mine) == seg_e - seg_s:
            yield from self.wait(lambda: self.rec_tag[e] == sn)
            if self.mutant != "keep_record":
                self.rec_tag[e] = sn + self.ring
            yield "step", None
            self.emit(seg_s, mine, ((w, frozenset(mine)),))
            return
        yield from self.wait(lambda: self.slot_busy[w] == 0)
        self.slot[w] = set(mine)
        yield "step", None
        self.slot_busy[w] = 1
        yield "step", None
        yield from self.wait(lambda: self.rec_tag[e] == sn)
        add = (len(mine) << 8) | (1 << w)
        old = self.rec_val[e]
        self.rec_val[e] = old + add  # one atomic add
        yield "step", None
        now = old + add
        if (now >> 8) != seg_e - seg_s:
            return  # not the last: the state waits in the slot
        self.slot_busy[w] = 0
        # (the order of the merge: with det from an empty state, every parked
        # state in wave order, this wave's own included)
        merged, order = (set(), []) if self.det else (set(mine), [(w, frozenset(mine))])
        bits = now & 0xFF & ~(0 if self.det else 1 << w)
        for ww in range(self.wph):
            if bits >> ww & 1:
                got = self.slot[ww]
                assert got is not None and not (merged & got), "a step merged twice"
                merged |= got
                order.append((ww, frozenset(got)))
                yield "step", None
                if self.mutant != "keep_slot":
                    self.slot_busy[ww] = 0
                yield "step", None
        self.rec_val[e] = 0
        yield "step", None
        if self.mutant != "keep_record":
            self.rec_tag[e] = sn + self.ring
        yield "step", None
        self.emit(seg_s, merged, tuple(order))

    def emit(self, seg_s, steps, order=None):
        assert seg_s not in self.results, f"segment at {seg_s} written twice"
        self.results[seg_s] = (frozenset(steps), self.broken)
        self.orders[seg_s] = order

    def wave(self, w):
        t = self.claim(w)
        yield "step", None
        if t >= self.x1:
            return
        u = self.unit_of(t)
        mine = {t}
        while True:
            tn = self.claim(w)
            yield "step", None
            more = tn < self.x1
            if not more or self.unit_of(tn) != u:
                yield from self.finish(w, u, mine)
                mine = set()
                if not more:
                    return
                u = self.unit_of(tn)
            mine.add(tn)

    def segments(self):
        segs = {}
        for u in range(self.unit_of(self.x0), self.unit_of(self.x1 - 1) + 1):
            s, e = max(self.x0, self.start[u]), min(self.x1, self.start[u + 1])
            segs[s] = frozenset(range(s, e))
        return segs


def run(wg: WorkGroup, rng: random.Random, starve: int | None = None, max_turns=10 ** 7):
    """Interleave the waves at random; starve: that wave gets 1/20 of the
    turns the others get. Raises on a deadlock (every live wave waiting on a
    condition no other wave can make true is reported by the wait bound)."""
    waves = {w: wg.wave(w) for w in range(wg.wph)}
    for _ in range(max_turns):
        if not waves:
            return
        ids = list(waves)
        if starve is not None and starve in waves and len(ids) > 1 and rng.random() > 0.05:
            ids.remove(starve)
        w = rng.choice(ids)
        try:
            next(waves[w])
        except StopIteration:
            del waves[w]
    raise AssertionError("the model did not finish")


def random_case(rng: random.Random):
    nunits = rng.randint(1, 12)
    lens = [rng.choice([1, 2, 3, rng.randint(1, 40), rng.randint(30, 130)]) for _ in range(nunits)]
    T = sum(lens)
    nwg = max(1, min(rng.randint(1, 40), T // MIN_STEPS if rng.random() < 0.7 else T))
    w = rng.randrange(nwg)
    x0, x1 = range_start(w, T, nwg), range_start(w + 1, T, nwg)
    return lens, x0, x1


@pytest.mark.parametrize("ring,wph", [(RING, WAVES), (RING, 1), (RING, 2), (RING, 8), (2, WAVES),
                                      (2, 8), (1, WAVES)])
def test_protocol_completes_and_merges_every_step_once(ring, wph):
    rng = random.Random(1000 * ring + wph)
    n = 0
    while n < 400:
        lens, x0, x1 = random_case(rng)
        if x1 <= x0:
            continue
        n += 1
        wg = WorkGroup(lens, x0, x1, wph, ring, cap=10 ** 6)
        run(wg, rng, starve=rng.randrange(wph) if rng.random() < 0.3 else None)
        assert wg.flags == 0 and not wg.broken, (lens, x0, x1, "a wait ran out")
        want = wg.segments()
        got = {s: steps for s, (steps, _) in wg.results.items()}
        assert got == want, (lens, x0, x1)


def test_kernel_constants():
    """The model runs the kernel's own ring size and wave count, and the wait
    bound in the kernel is far above any legitimate wait in the model."""
    assert RING == 16 and WAVES == 4 and MIN_STEPS >= 1
    cap = kernel_constant("kSpinCap")
    worst = 0
    rng = random.Random(7)
    for _ in range(200):
        lens, x0, x1 = random_case(rng)
        if x1 <= x0:
            continue
        wg = WorkGroup(lens, x0, x1, WAVES, RING, cap=10 ** 6)
        run(wg, rng, starve=0)
        worst = max(worst, wg.max_spin)
    assert worst * 1000 < cap, (worst, cap)


@pytest.mark.parametrize("mutant", ["keep_record", "keep_slot"])
def test_planted_protocol_mistake_is_bounded_and_flagged(mutant):
    """A record never passed on, or a slot never freed, would make the next
    user spin forever; with the bound every wait ends, the stall flag is
    raised and every result written after it carries the broken mark."""
    rng = random.Random(11)
    hit = 0
    for _ in range(300):
        lens, x0, x1 = random_case(rng)
        if x1 <= x0:
            continue
        wg = WorkGroup(lens, x0, x1, WAVES, 2, cap=200, mutant=mutant)
        run(wg, rng)  # finishes: no wait outlives the bound
        if wg.flags:
            hit += 1
            assert wg.broken
            # a segment left unfinished by the mistake has no result; every
            # result written after the stall is marked (NaN rows on the GPU)
            stalled_after = [s for s, (_, b) in wg.results.items() if b]
            assert len(wg.results) < len(wg.segments()) or stalled_after
    assert hit > 0, "the planted mistake never caused a stall"


@pytest.mark.parametrize("ring,wph", [(RING, WAVES), (RING, 8), (2, WAVES), (1, 2)])
def test_fixed_claims_complete_and_merge_in_one_order(ring, wph):
    """The bitwise-reproducible mode (MQA_KERNEL_MFMA_DETERMINISTIC): the same
    protocol with each wave's claims dealt round robin never deadlocks either,
    and every segment is merged from the same wave states in the same order
    whatever the interleaving (so the fp32 sums repeat bit for bit)."""
    rng = random.Random(77 + ring * 10 + wph)
    n = 0
    while n < 150:
        lens, x0, x1 = random_case(rng)
        if x1 <= x0:
            continue
        n += 1
        seen = None
        for rep in range(4):
            wg = WorkGroup(lens, x0, x1, wph, ring, cap=10 ** 6, det=True)
            run(wg, rng, starve=rng.randrange(wph) if rep % 2 else None)
            assert wg.flags == 0
            assert {s: st for s, (st, _) in wg.results.items()} == wg.segments()
            if seen is None:
                seen = wg.orders
            else:
                assert wg.orders == seen, (lens, x0, x1)
