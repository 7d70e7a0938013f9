"""Seeded synthetic inputs for MoBA prefill: Llama-shaped Q/K/V with planted needles.

This module only builds inputs. It holds none of MoBA's arithmetic (no pooling,
gating, top-k or attention), so the GPU library's tests and the CPU oracle can
both draw from it without sharing any of the method's code.

Recipe (the pages give none; no trained weights or datasets are available):
  * Q, K, V ~ N(0, 1), drawn in fp32 from a seeded torch generator, then the
    planted terms are added, then everything is cast (round to nearest even) to
    the working dtype.
  * Needles. For each (sequence, kv-head g) a set of needle blocks is chosen:
    blocks 0 .. topk-2, then every m-th block after them, at most head_dim in
    total. Needle number r gets code c_r, column r of a seeded random orthogonal
    matrix, so the codes are orthonormal. Every key row of needle block b gets
    beta * c_b added.
  * Targets. For query block i >= 1 and each q-head h of group g, the target set
    J*(i, h) is a random subset of size min(topk-1, i) of the needle blocks
    before i (for i <= topk-1 that is every earlier block). Every query row of
    block i, head h gets alpha * sum_{b in J*} c_b added.
Because the codes are orthonormal the planted terms do not interfere: a target
block scores about alpha*beta higher than any other candidate, far above the
noise, so the top-(topk-1) choice is well separated. The intended targets are
returned so that a selection can be checked on every row at any size.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}

# The five workloads: tiny fp32 check, a Llama-3.1-8B-shaped layer at 32K, a packed
# varlen batch, one 1M-token sequence, and fine-grained blocks at 256K; and the
# per-GPU head shard of a 10M-token sequence.
CONFIGS = {
    "tiny": dict(seqlens=[2048], hq=1, hkv=1, d=64, block=256, topk=3, dtype="f32"),
    "llama32k": dict(seqlens=[32768], hq=32, hkv=8, d=128, block=2048, topk=3, dtype="bf16"),
    "varlen131k": dict(seqlens=[16384, 32768, 65536, 19456], hq=32, hkv=8, d=128, block=2048,
                       topk=3, dtype="bf16"),
    "1m": dict(seqlens=[1048576], hq=32, hkv=8, d=128, block=2048, topk=3, dtype="bf16"),
    "fine256k": dict(seqlens=[262144], hq=32, hkv=8, d=128, block=512, topk=12, dtype="bf16"),
    # one GPU's share of a 10M-token (10 x 2^20) layer of the same shape split by kv head
    # over 8 GPUs: 4 q heads and their kv head, 5,120 blocks
    "10m_shard": dict(seqlens=[10485760], hq=4, hkv=1, d=128, block=2048, topk=3,
                      dtype="bf16"),
}


@dataclass
class Inputs:
    q: torch.Tensor             # [T, Hq, D]
    k: torch.Tensor             # [T, Hkv, D]
    v: torch.Tensor             # [T, Hkv, D]
    cu_seqlens: torch.Tensor    # [N+1] int32, on the CPU
    block: int
    topk: int
    targets: torch.Tensor | None = None   # [T, Hq, topk-1] int32 on the CPU, -1 padded
    meta: dict = field(default_factory=dict)

    @property
    def seqlens(self):
        cu = self.cu_seqlens.tolist()
        return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]


def cu_seqlens_of(seqlens) -> torch.Tensor:
    cu = [0]
    for s in seqlens:
        cu.append(cu[-1] + int(s))
    return torch.tensor(cu, dtype=torch.int32)


def block_of_token(seqlens, block: int) -> tuple[torch.Tensor, list[int]]:
    """Global block id of every packed token, and the first global block id per sequence."""
    ids, base, bases = [], 0, []
    for s in seqlens:
        nb = (s + block - 1) // block
        bases.append(base)
        ids.append(base + torch.arange(s, dtype=torch.int64) // block)
        base += nb
    return (torch.cat(ids) if ids else torch.zeros(0, dtype=torch.int64)), bases


def needle_blocks(num_blocks: int, topk: int, d: int) -> list[int]:
    """Blocks 0..topk-2, then every m-th block after them, at most d in all."""
    first = min(topk - 1, num_blocks)
    needles = list(range(first))
    rest = num_blocks - first
    if rest > 0:
        room = d - first
        if room <= 0:
            raise ValueError("head_dim too small to plant topk-1 orthogonal needles")
        step = max(1, math.ceil(rest / room))
        needles += list(range(first, num_blocks, step))
    return needles


def _plants(seqlens, hq, hkv, d, block, topk, alpha, beta, gen):
    """Per-block planted terms for Q and K and the per-block target sets (CPU fp32)."""
    group = hq // hkv
    nsel_max = max(topk - 1, 0)
    pq, pk, tg = [], [], []
    for s in seqlens:
        nb = (s + block - 1) // block
        pq_n = torch.zeros(nb, hq, d, dtype=torch.float64)
        pk_n = torch.zeros(nb, hkv, d, dtype=torch.float64)
        tg_n = torch.full((nb, hq, nsel_max), -1, dtype=torch.int32)
        if nb > 0 and nsel_max > 0:
            needles = needle_blocks(nb, topk, d)
            for g in range(hkv):
                basis, _ = torch.linalg.qr(torch.randn(d, d, generator=gen, dtype=torch.float64))
                code = {b: basis[:, r] for r, b in enumerate(needles)}
                for b in needles:
                    pk_n[b, g] = beta * code[b]
                for i in range(1, nb):
                    past = [b for b in needles if b < i]
                    nsel = min(nsel_max, i)
                    for hh in range(group):
                        h = g * group + hh
                        pick = torch.randperm(len(past), generator=gen)[:nsel].tolist()
                        chosen = sorted(past[p] for p in pick)
                        for b in chosen:
                            pq_n[i, h] += alpha * code[b]
                        tg_n[i, h, :nsel] = torch.tensor(chosen, dtype=torch.int32)
        pq.append(pq_n.float())
        pk.append(pk_n.float())
        tg.append(tg_n)
    return torch.cat(pq), torch.cat(pk), torch.cat(tg)


def make_inputs(seqlens, hq, hkv, d, block, topk, dtype="bf16", seed=0, device="cpu",
                plant=True, alpha=16.0, beta=4.0, chunk_tokens=32768) -> Inputs:
    """Seeded Q/K/V for one packed batch, optionally with planted needles."""
    seqlens = [int(s) for s in seqlens]
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    tdt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    T = sum(seqlens)
    dev = torch.device(device)
    gen_struct = torch.Generator(device="cpu").manual_seed(seed)
    gen_bulk = torch.Generator(device=dev).manual_seed(seed + 1)
    cu = cu_seqlens_of(seqlens)
    blk, _ = block_of_token(seqlens, block)
    targets = None
    if plant and topk > 1:
        pq, pk, tg = _plants(seqlens, hq, hkv, d, block, topk, alpha, beta, gen_struct)
        pq, pk = pq.to(dev), pk.to(dev)
        targets = tg[blk] if T > 0 else tg[:0]
    q = torch.empty(T, hq, d, dtype=tdt, device=dev)
    k = torch.empty(T, hkv, d, dtype=tdt, device=dev)
    v = torch.empty(T, hkv, d, dtype=tdt, device=dev)
    blk_dev = blk.to(dev)
    for a in range(0, T, chunk_tokens):
        b = min(T, a + chunk_tokens)
        for name, dst, heads in (("q", q, hq), ("k", k, hkv), ("v", v, hkv)):
            x = torch.randn(b - a, heads, d, generator=gen_bulk, device=dev, dtype=torch.float32)
            if targets is not None and name == "q":
                x += pq[blk_dev[a:b]]
            if targets is not None and name == "k":
                x += pk[blk_dev[a:b]]
            dst[a:b] = x.to(tdt)
    meta = dict(seed=seed, alpha=alpha, beta=beta, plant=plant, dtype=str(dtype))
    return Inputs(q=q, k=k, v=v, cu_seqlens=cu, block=block, topk=topk, targets=targets,
                  meta=meta)


def make_grad(shape, dtype="bf16", seed=0, device="cpu", mean=0.0,
              chunk_rows=32768) -> torch.Tensor:
    """Seeded upstream gradient dO ~ N(mean, 1) of the given [T, H, D] shape."""
    tdt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    dev = torch.device(device)
    gen = torch.Generator(device=dev).manual_seed(seed + 7)
    g = torch.empty(tuple(shape), dtype=tdt, device=dev)
    for a in range(0, shape[0], chunk_rows):
        b = min(shape[0], a + chunk_rows)
        x = torch.randn((b - a,) + tuple(shape[1:]), generator=gen, device=dev,
                        dtype=torch.float32)
        g[a:b] = (x + mean).to(tdt)
    return g


def make_config(name: str, seed=0, device="cpu", **over) -> Inputs:
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    return make_inputs(cfg["seqlens"], cfg["hq"], cfg["hkv"], cfg["d"], cfg["block"],
                       cfg["topk"], dtype=cfg["dtype"], seed=seed, device=device,
                       **{k: v for k, v in over.items() if k in ("plant", "alpha", "beta")})


def make_10m_full(seed=0, device="cpu", groups=8) -> Inputs:
    """A full-width 10M-token layer: the 10m_shard recipe for each of `groups` kv
    groups (seed + g for group g; 4 q heads and 1 kv head each), laid out as one
    [T, 4 * groups, D] / [T, groups, D] batch. Group g holds q heads 4g .. 4g+3 and
    kv head g, exactly the g-th head share of the layer."""
    base = CONFIGS["10m_shard"]
    T, d, G = sum(base["seqlens"]), base["d"], base["hq"]
    tdt = DTYPES[base["dtype"]]
    dev = torch.device(device)
    q = torch.empty(T, G * groups, d, dtype=tdt, device=dev)
    k = torch.empty(T, groups, d, dtype=tdt, device=dev)
    v = torch.empty(T, groups, d, dtype=tdt, device=dev)
    targets = torch.empty(T, G * groups, base["topk"] - 1, dtype=torch.int32)
    for g in range(groups):
        part = make_config("10m_shard", seed=seed + g, device=device)
        q[:, G * g:G * (g + 1)] = part.q
        k[:, g] = part.k[:, 0]
        v[:, g] = part.v[:, 0]
        targets[:, G * g:G * (g + 1)] = part.targets
        del part
    meta = dict(seed=seed, groups=groups, recipe="10m_shard per kv group")
    return Inputs(q=q, k=k, v=v, cu_seqlens=cu_seqlens_of(base["seqlens"]), block=base["block"],
                  topk=base["topk"], targets=targets, meta=meta)


def sample_tokens(seqlens, block: int, n_tokens: int, seed: int = 0,
                  every_block: bool = False) -> np.ndarray:
    """Seeded sample of packed token indices for sampled-row checks.

    Always includes: the first and last token of every sequence, the first and last
    token of blocks 0, 1 and 2 of every sequence (rows with fewer than topk-1 past
    blocks), and the first token of each sequence's last block; with every_block, also
    one uniformly drawn token of every block of every sequence. The rest, up to
    n_tokens, are drawn uniformly over all tokens. Sorted, unique.
    """
    rng = np.random.default_rng(seed)
    fixed, start = [], 0
    T = int(sum(seqlens))
    for s in seqlens:
        if s > 0:
            fixed += [start, start + s - 1]
            for b in range(3):
                if b * block < s:
                    fixed += [start + b * block, start + min((b + 1) * block, s) - 1]
            fixed.append(start + ((s - 1) // block) * block)
            if every_block:
                nb = (s + block - 1) // block
                lo = np.arange(nb, dtype=np.int64) * block
                hi = np.minimum(lo + block, s)
                fixed += (start + lo + rng.integers(0, hi - lo)).tolist()
        start += s
    picked = np.unique(np.asarray(fixed, dtype=np.int64))
    want = min(int(n_tokens), T)
    while picked.size < want:          # uniform extras until n_tokens distinct tokens
        picked = np.unique(np.concatenate([picked, rng.integers(0, T, size=want - picked.size)]))
    return picked.astype(np.int32)
