"""Host model of the screened gate's packed-value lists (CPU only).

The screened pass keeps, per lane, the best topk-1 scores of its stream as plain
float values: each score carries its place in the stream (16 * chunk + position)
in its CB low mantissa bits (8 for sequences of up to 512 blocks, 12 up to 8192,
13 beyond), the list is updated with max / med3 only, and the blocks are decoded
from the bits at the end. This re-enacts those steps in numpy, bit for bit, and
checks them against a brute-force sort of the same packed values (kept set,
order, and the best value left out), with exact ties, masked candidates and
short streams, and checks the bound the screen adds for the packing (less than
2^(CB-23) of each score).
"""
import numpy as np
import pytest

MASKED = np.float32(-3.4028234663852886e38)


def pack(s, code, cb=8):
    b = np.asarray(s, dtype=np.float32).view(np.uint32)
    keep = np.uint32((0xFFFFFFFF << cb) & 0xFFFFFFFF)
    return ((b & keep) | np.uint32(code)).view(np.float32)


def med3(a, b, c):
    return np.float32(sorted([a, b, c])[1])


def lane_model(scores, kb, ks, cb=8):
    """scores: [chunks, 16] fp32 (MASKED for blocks past the candidates)."""
    tl = [np.float32(-np.inf)] * kb
    out = np.float32(-np.inf)
    for st in range(scores.shape[0]):
        for e in range(16):
            sc = pack(scores[st, e], 16 * st + e, cb)
            out = med3(out, tl[kb - 1], sc)
            for p in range(kb - 1, 0, -1):
                tl[p] = med3(tl[p - 1], tl[p], sc)
            tl[0] = max(tl[0], sc)
    kept = []
    for p in range(kb):
        real = tl[p] > -1e38
        if p < ks:
            kept.append(int(tl[p].view(np.uint32) & ((1 << cb) - 1)) if real else None)
        elif real:
            out = max(out, tl[p])
    if not out > -1e38:
        out = np.float32(-np.inf)
    return kept, out


@pytest.mark.parametrize("kb,ks,cb", [(2, 2, 8), (4, 3, 8), (4, 4, 8), (8, 7, 8), (12, 11, 8),
                                      (16, 16, 8), (2, 2, 12), (4, 3, 12), (2, 1, 13),
                                      (4, 4, 13)])
def test_packed_lists_match_a_sort(kb, ks, cb):
    rng = np.random.default_rng(kb * 100 + ks + cb)
    max_chunks = (1 << cb) // 16
    trials = 300 if cb == 8 else 40
    for trial in range(trials):
        # long streams too for the wider codes (the last trial the longest)
        nchunks = max_chunks if trial == trials - 1 else int(rng.integers(1, min(max_chunks, 48) + 1))
        s = rng.standard_normal((nchunks, 16)).astype(np.float32) * np.float32(rng.choice([1, 30]))
        if trial % 3 == 0:                       # exact ties
            s = np.round(s * 2) / np.float32(2)
        ncand = int(rng.integers(1, nchunks * 16 + 1))
        flat = s.reshape(-1)
        flat[ncand:] = MASKED
        kept, out = lane_model(s, kb, ks, cb)
        packed = np.array([pack(flat[c], c, cb) for c in range(flat.size)], dtype=np.float32)
        real = np.nonzero(flat > -1e38)[0]
        order = real[np.argsort(-packed[real].astype(np.float64), kind="stable")]
        want = [int(c) for c in order[:ks]] + [None] * max(0, ks - order.size)
        assert kept == want, (trial, kept, want)
        left = packed[order[ks:]]
        want_out = left.max() if left.size else np.float32(-np.inf)
        assert out == want_out
        # packed values are distinct, so the kept set is unique
        assert np.unique(packed[real]).size == real.size


@pytest.mark.parametrize("cb", [8, 12, 13])
def test_packing_moves_a_score_by_less_than_its_bound(cb):
    rng = np.random.default_rng(3 + cb)
    s = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-6, 6, 20000)).astype(np.float32)
    code = rng.integers(0, 1 << cb, s.size)
    p = np.array([pack(x, c, cb) for x, c in zip(s, code)], dtype=np.float32)
    x = s.astype(np.float64)
    assert np.all(np.abs(p.astype(np.float64) - x) < 2.0 ** (cb - 23) * np.abs(x))
    # the masked value stays finite and below every real score
    top = (1 << cb) - 1
    assert np.isfinite(pack(MASKED, top, cb)) and pack(MASKED, top, cb) < -1e38
