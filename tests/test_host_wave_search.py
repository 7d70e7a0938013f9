"""Host model of the kernels' wave-wide list lookup (upper_index_wave in
csrc/moba_device.h): a tile finds the routed list it belongs to as the largest L
with tile_offsets[L] <= tile. The model re-enacts its rounds (64 evenly spaced
entries read per round, the highest lane at or below x narrows the range) and must
agree with a plain bisection on every x, for offset arrays with empty lists
(repeated offsets), one list, and list counts around the 64 and 4096 round
boundaries."""
import bisect

import numpy as np


def wave_search(offs, n, x):
    lo, length, rounds = 0, n, 0
    while length > 1:
        step = (length + 63) // 64
        lanes = np.arange(64)
        inside = lanes * step < length
        vals = offs[np.minimum(lo + lanes * step, n - 1)]
        ok = inside & (vals <= x)
        assert ok[0], "the answer must lie at or after the range's first entry"
        assert not np.any(ok[1:] & ~ok[:-1]), "lanes at or below x form a prefix"
        hl = int(np.nonzero(ok)[0].max())
        lo += hl * step
        length = min(step, length - hl * step)
        rounds += 1
    return lo, rounds


def _offsets(rng, n, empty_frac):
    sizes = rng.integers(1, 9, size=n)
    sizes[rng.random(n) < empty_frac] = 0
    offs = np.zeros(n + 1, dtype=np.int64)
    offs[1:] = np.cumsum(sizes)
    return offs


def test_wave_search_matches_bisection():
    rng = np.random.default_rng(5)
    for n in (1, 2, 63, 64, 65, 100, 4095, 4096, 4097, 5120, 20000):
        for empty_frac in (0.0, 0.3, 0.9):
            offs = _offsets(rng, n, empty_frac)
            total = int(offs[n])
            if total == 0:
                continue
            xs = np.unique(np.concatenate([rng.integers(0, total, size=300),
                                           [0, total - 1], offs[:n][offs[:n] < total]]))
            max_rounds = 0
            for x in xs:
                got, rounds = wave_search(offs, n, int(x))
                # largest L in [0, n) with offs[L] <= x
                want = bisect.bisect_right(offs[:n].tolist(), int(x)) - 1
                assert got == want, (n, empty_frac, int(x), got, want)
                max_rounds = max(max_rounds, rounds)
            # two rounds (two dependent loads) up to 4096 lists, three beyond
            assert max_rounds <= (0 if n == 1 else 1 if n <= 64 else 2 if n <= 4096 else 3)
