"""The block map's schedule column as the GPU tests expect it (parity_util.expected_schedule),
pinned on hand-worked cases and on the properties the header states: full tiles first, in
contiguous runs per XCD (position i runs on XCD i % 8), then partial tiles tallest first."""
import numpy as np

from parity_util import expected_schedule


def tiles_of(heights):
    """A tile list {group, row_begin, row_end} with the given heights (one group per tile)."""
    rows, t = [], 0
    for g, h in enumerate(heights):
        rows.append((g, t, t + h))
        t += h
    return np.array(rows, dtype=np.int64)


def test_hand_worked_ten_full_tiles():
    # 10 full tiles t0..t9 and partial tiles of 50 (t10) and 70 (t11) rows.
    # 10 = 8 * 1 + 2: runs 0 and 1 hold two tiles ({t0, t1}, {t2, t3}), runs 2..7 one
    # (t4 .. t9); the r-th tile of run x sits at position 8r + x.
    sched = expected_schedule(tiles_of([128] * 10 + [50, 70]))
    assert sched.tolist() == [0, 2, 4, 5, 6, 7, 8, 9, 1, 3, 11, 10]


def test_hand_worked_fewer_full_tiles_than_xcds():
    # 3 full tiles: runs 0..2 hold one each, positions 0..2; then heights 90, 90, 5
    sched = expected_schedule(tiles_of([90, 128, 5, 128, 90, 128]))
    assert sched.tolist() == [1, 3, 5, 0, 4, 2]


def test_hand_worked_no_full_tiles():
    sched = expected_schedule(tiles_of([3, 7, 7, 1]))
    assert sched.tolist() == [1, 2, 0, 3]


def test_properties_on_random_block_maps():
    rng = np.random.default_rng(7)
    for _ in range(300):
        n = int(rng.integers(1, 200))
        heights = np.where(rng.random(n) < 0.5, 128, rng.integers(1, 128, n))
        tiles = tiles_of(heights.tolist())
        sched = expected_schedule(tiles)
        assert sorted(sched.tolist()) == list(range(n))
        full = [i for i in range(n) if heights[i] == 128]
        F = len(full)
        assert sorted(sched[:F].tolist()) == full
        lengths = []
        for x in range(8):
            run = sched[x:F:8].tolist()
            lengths.append(len(run))
            # a run is consecutive among the full tiles, in tile order
            if run:
                k = full.index(run[0])
                assert run == full[k:k + len(run)]
        assert max(lengths) - min(lengths) <= 1
        assert lengths == sorted(lengths, reverse=True)
        # runs follow one another in tile order: run x ends where run x + 1 starts
        starts = [full.index(sched[x]) for x in range(8) if x < F]
        assert starts == sorted(starts)
        rest = sched[F:].tolist()
        assert rest == sorted(rest, key=lambda i: (-int(heights[i]), i))
