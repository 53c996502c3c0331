"""Invariants of the split-KV schedule, on the host model of the device rule.

The GPU tests check that the device writes exactly what this model computes.
"""

import numpy as np
import pytest

from sched_model import schedule, partition_items


def _check(seqlens, num_parts, c0):
    meta, splits, n = schedule(seqlens, num_parts, c0)
    batch = len(seqlens)
    # ordered, contiguous, covering
    prev_end = (0, 0)
    seen = []
    for p, m in enumerate(meta):
        assert (m[0], m[1]) == prev_end
        prev_end = (m[2], m[3])
        assert (m[0], m[1]) <= (m[2], m[3])
        seen += partition_items(m, n)
    assert prev_end == (batch, 0)
    expect = [(b, j) for b in range(batch) for j in range(n[b])]
    assert seen == expect  # every page slot exactly once, in order
    # split counts: partitions touching each sequence
    touch = [0] * batch
    for m in meta:
        for b in sorted({b for b, _ in partition_items(m, n)}):
            touch[b] += 1
    assert [splits[b + 1] - splits[b] for b in range(batch)] == touch
    assert splits[0] == 0 and splits[batch] == sum(touch)
    assert splits[batch] <= batch + num_parts - 1
    # first_split: index of this partition among those touching b_begin
    seen_count = [0] * batch
    for m in meta:
        items = partition_items(m, n)
        if not items:
            continue
        b0 = items[0][0]
        assert m[4] == seen_count[b0]
        for b in sorted({b for b, _ in items}):
            seen_count[b] += 1
    # balance: cost of a partition (c0 per sequence segment + pages) <= q + c0
    q = meta[0][5]
    for m in meta:
        items = partition_items(m, n)
        segs = len({b for b, _ in items})
        assert len(items) + c0 * segs <= q + c0
    return meta, splits


@pytest.mark.parametrize("seqlens", [
    [0], [1], [63], [64], [65], [131072],
    [4096] * 64,
    [0, 0, 0, 5],
    [1, 63, 64, 65, 127, 128, 4097],
    [131072] + [1024] * 15,
    [1024] * 15 + [131072],
    list(range(0, 3000, 37)),
])
@pytest.mark.parametrize("num_parts", [1, 3, 64, 256, 1024])
@pytest.mark.parametrize("c0", [1, 3])
def test_schedule_invariants(seqlens, num_parts, c0):
    _check(seqlens, num_parts, c0)


def test_schedule_random():
    rng = np.random.Generator(np.random.PCG64(5))
    for _ in range(50):
        batch = int(rng.integers(1, 40))
        L = rng.integers(0, 9000, size=batch)
        _check(list(L), int(rng.integers(1, 300)), int(rng.integers(1, 5)))


def test_long_sequence_is_spread():
    # one 131072-token sequence among short ones is cut into many pieces
    meta, splits = _check([131072] + [2048] * 15, 256, 3)
    assert splits[1] - splits[0] > 100
