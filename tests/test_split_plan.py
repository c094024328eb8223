"""Host-side model of the work-balanced GQA split (no GPU).

The split kernel walks its run of 128-position units the way ``first_item``
and ``next_item`` do in gqa_decode.hip, taking the run's units of one
(sequence, KV head) pair as one segment stored in slot ``w + b*h_kv + j``;
the merge finds a pair's slots from the sequence lengths alone. This file
restates both walks in Python and checks, over random batches, windows and
grid sizes, the properties the two kernels rely on: every unit of every pair
is covered exactly once, slots are distinct and inside the workspace's
``groups + B*h_kv`` slots, and the merge's lookup names exactly the slots the
kernel wrote (skipping work-groups whose run is empty).
"""

import random

import pytest

UNIT = 128


def _units(n, window):
    lo = max(0, n - window) if window > 0 else 0
    return (n - lo + UNIT - 1) // UNIT


def _kernel_walk(units, h_kv, groups):
    """(b, j) -> [(work-group, first unit, end unit)], as the kernel walks its runs."""
    B = len(units)
    U = sum(units) * h_kv
    segs, slots = {}, set()
    for w in range(groups):
        lo, hi = U * w // groups, U * (w + 1) // groups
        if hi <= lo:
            continue
        base, b = 0, 0
        while base + units[b] * h_kv <= lo:
            base += units[b] * h_kv
            b += 1
        off = lo - base
        np_ = units[b]
        j, p, left = off // np_, off % np_, hi - lo
        while left > 0 and b < B:
            ln = min(np_ - p, left)                 # the segment: the run's units of (b, j)
            segs.setdefault((b, j), []).append((w, p, p + ln))
            slot = w + b * h_kv + j
            assert slot not in slots and slot < groups + B * h_kv
            slots.add(slot)
            if left <= ln:
                break
            left -= ln
            p = 0                                   # the segment ended the pair: next pair
            j += 1
            if j == h_kv:
                j, b = 0, b + 1
                while b < B and units[b] == 0:
                    b += 1
                if b < B:
                    np_ = units[b]
    return segs


def _merge_lookup(units, h_kv, groups, b, j):
    """The work-groups whose slots the merge reads for pair (b, j)."""
    U = sum(units) * h_kv
    if units[b] == 0:
        return []
    base = sum(units[:b]) * h_kv + j * units[b]
    holder = lambda u: ((u + 1) * groups - 1) // U
    held = lambda w: U * (w + 1) // groups > U * w // groups
    return [w for w in range(holder(base), holder(base + units[b] - 1) + 1) if held(w)]


@pytest.mark.parametrize("seed", range(6))
def test_split_covers_every_unit_once_and_merge_finds_the_slots(seed):
    rng = random.Random(seed)
    for _ in range(300):
        B = rng.randint(1, 70)
        h_kv = rng.choice([1, 2, 4, 8])
        groups = rng.choice([1, 3, 7, 64, 256, 512])
        window = rng.choice([0, 0, 100, 4096])
        lens = [rng.choice([0, 1, 127, 128, 129, rng.randint(0, 40000)]) for _ in range(B)]
        units = [_units(n, window) for n in lens]
        segs = _kernel_walk(units, h_kv, groups)
        for b in range(B):
            for j in range(h_kv):
                got = sorted(segs.get((b, j), []), key=lambda s: s[1])
                covered = [u for (_, a, c) in got for u in range(a, c)]
                assert covered == list(range(units[b]))
                assert _merge_lookup(units, h_kv, groups, b, j) == [w for (w, _, _) in got]


def test_decode_step_shapes_split_evenly():
    """At a 70B-shaped ragged batch every work-group streams the same number
    of units give or take one, and combines once per pair it touches: at most
    one more than its units divided by the shortest pair's."""
    rng = random.Random(0)
    lens = [rng.randint(1024, 32768) for _ in range(16)]
    units = [_units(n, 0) for n in lens]
    segs = _kernel_walk(units, 8, 512)
    per_wg, pieces_per_wg = {}, {}
    for pieces in segs.values():
        for (w, a, c) in pieces:
            per_wg[w] = per_wg.get(w, 0) + (c - a)
            pieces_per_wg[w] = pieces_per_wg.get(w, 0) + 1
    assert len(per_wg) == 512
    assert max(per_wg.values()) - min(per_wg.values()) <= 1
    bound = -(-max(per_wg.values()) // min(units)) + 1
    assert max(pieces_per_wg.values()) <= bound
