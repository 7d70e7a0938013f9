"""Host model of the screened gate's packed-value lists (CPU only).

The screened pass keeps, per lane, the best topk-1 scores of its stream as plain
float values: each score carries its place in the stream (16 * chunk + position)
in its 8 low mantissa bits, the list is updated with max / med3 only, and the
blocks are decoded from the bits at the end. This re-enacts those steps in
numpy, bit for bit, and checks them against a brute-force sort of the same
packed values (kept set, order, and the best value left out), with exact ties,
masked candidates and short streams, and checks the bound the screen adds for
the packing (less than 2^-15 of each score).
"""
import numpy as np
import pytest

MASKED = np.float32(-3.4028234663852886e38)


def pack(s, code):
    b = np.asarray(s, dtype=np.float32).view(np.uint32)
    return ((b & np.uint32(0xFFFFFF00)) | np.uint32(code)).view(np.float32)


def med3(a, b, c):
    return np.float32(sorted([a, b, c])[1])


def lane_model(scores, kb, ks):
    """scores: [chunks, 16] fp32 (MASKED for blocks past the candidates)."""
    tl = [np.float32(-np.inf)] * kb
    out = np.float32(-np.inf)
    for st in range(scores.shape[0]):
        for e in range(16):
            sc = pack(scores[st, e], 16 * st + e)
            out = med3(out, tl[kb - 1], sc)
            for p in range(kb - 1, 0, -1):
                tl[p] = med3(tl[p - 1], tl[p], sc)
            tl[0] = max(tl[0], sc)
    kept = []
    for p in range(kb):
        real = tl[p] > -1e38
        if p < ks:
            kept.append(int(tl[p].view(np.uint32) & 0xFF) if real else None)
        elif real:
            out = max(out, tl[p])
    if not out > -1e38:
        out = np.float32(-np.inf)
    return kept, out


@pytest.mark.parametrize("kb,ks", [(2, 2), (4, 3), (4, 4), (8, 7), (12, 11), (16, 16)])
def test_packed_lists_match_a_sort(kb, ks):
    rng = np.random.default_rng(kb * 100 + ks)
    for trial in range(300):
        nchunks = int(rng.integers(1, 17))
        s = rng.standard_normal((nchunks, 16)).astype(np.float32) * np.float32(rng.choice([1, 30]))
        if trial % 3 == 0:                       # exact ties
            s = np.round(s * 2) / np.float32(2)
        ncand = int(rng.integers(1, nchunks * 16 + 1))
        flat = s.reshape(-1)
        flat[ncand:] = MASKED
        kept, out = lane_model(s, kb, ks)
        packed = np.array([pack(flat[c], c) for c in range(flat.size)], dtype=np.float32)
        real = np.nonzero(flat > -1e38)[0]
        order = real[np.argsort(-packed[real].astype(np.float64), kind="stable")]
        want = [int(c) for c in order[:ks]] + [None] * max(0, ks - order.size)
        assert kept == want, (trial, kept, want)
        left = packed[order[ks:]]
        want_out = left.max() if left.size else np.float32(-np.inf)
        assert out == want_out
        # packed values are distinct, so the kept set is unique
        assert np.unique(packed[real]).size == real.size


def test_packing_moves_a_score_by_less_than_2_to_the_minus_15():
    rng = np.random.default_rng(3)
    s = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-6, 6, 100000)).astype(np.float32)
    code = rng.integers(0, 256, s.size)
    p = np.array([pack(x, c) for x, c in zip(s[:20000], code[:20000])], dtype=np.float32)
    x = s[:20000].astype(np.float64)
    assert np.all(np.abs(p.astype(np.float64) - x) < 2.0 ** -15 * np.abs(x))
    # the masked value stays finite and below every real score
    assert np.isfinite(pack(MASKED, 255)) and pack(MASKED, 255) < -1e38
