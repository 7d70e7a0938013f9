"""Numpy brute force of MoBA prefill, written as a dense attention mask.

Test helper, independent of the oracle's C code. It follows the mask-based
formulation (MoBA: Mixture of Block Attention for Long-Context LLMs, README,
"Implementation Details": the naive implementation materialises the attention
mask): build the full [S, S] boolean mask of every head literally, then run a
masked dense softmax. Only for tiny inputs: it is O(S^2) in memory and time.
"""
import numpy as np


def brute_force(q, k, v, seqlens, block, topk, scale=None, sel_in=None, return_margin=False):
    """out, lse, sel (and, with return_margin, the gate margin of every row: the
    lowest kept score minus the highest score left out, +inf when no past block is
    left out). With sel_in [T, Hq, topk-1] (-1 padded) the mask takes those past
    blocks instead of the gated ones."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((T, hq, d))
    lse = np.zeros((T, hq))
    sel = np.full((T, hq, max(topk - 1, 0)), -1, dtype=np.int32)
    margin = np.full((T, hq), np.inf)
    start = 0
    for S in seqlens:
        if S == 0:
            continue
        sl = slice(start, start + S)
        nb = -(-S // block)
        pos = np.arange(S)
        blk = pos // block
        # pooled keys: arithmetic mean of each block's rows, [nb, hkv, d]
        kbar = np.stack([k[sl][b * block:min((b + 1) * block, S)].mean(axis=0)
                         for b in range(nb)])
        own = (blk[:, None] == blk[None, :]) & (pos[None, :] <= pos[:, None])
        for h in range(hq):
            g = h // group
            qh = q[sl, h]
            gate = qh @ kbar[:, g].T                       # [S, nb]
            mask = own.copy()
            for t in range(S):
                cand = np.arange(blk[t])                   # past blocks only
                order = np.lexsort((cand, -gate[t, cand]))  # score desc, index asc
                if sel_in is not None:
                    given = np.asarray(sel_in[start + t, h])
                    chosen = np.sort(given[given >= 0])
                else:
                    chosen = np.sort(cand[order[:topk - 1]]) if topk > 1 else cand[:0]
                sel[start + t, h, :len(chosen)] = chosen
                mask[t] |= np.isin(blk, chosen)
                kept = cand[order[:topk - 1]] if topk > 1 else cand[:0]
                left = cand[order[max(topk - 1, 0):]]
                if len(left) and len(kept):
                    margin[start + t, h] = gate[t, kept].min() - gate[t, left].max()
            logits = scale * (qh @ k[sl, g].T)
            logits[~mask] = -np.inf
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            den = p.sum(axis=1, keepdims=True)
            out[sl, h] = (p @ v[sl, g]) / den
            lse[sl, h] = (m + np.log(den))[:, 0]
        start += S
    if return_margin:
        return out, lse, sel, margin
    return out, lse, sel
