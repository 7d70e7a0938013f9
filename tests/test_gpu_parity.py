"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (from the workload definition): selected block ids bit-exact; outputs
within max-abs 1e-4 for fp32 inputs and 2e-2 for bf16 inputs of the fp64
oracle; pooled keys within 1e-6 (fp32 sums of at most a few thousand O(1)
terms, divided by the block length); integer routing lists bit-exact.

Small cases run every row through the oracle; the full-size workloads run in
the same launch configuration as the benchmark and are checked on sampled rows
against the oracle, plus on every row against the planted-needle targets.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_causal_amd as moba
import oracle
from synth_inputs import CONFIGS, make_config, make_inputs, sample_tokens

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def _say(msg):
    print("\n[case] " + msg, flush=True)
    sys.stdout.flush()


def _to_gpu(inp):
    inp.q, inp.k, inp.v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    return inp


def _run(inp, **kw):
    out, sel, lse = moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk,
                                      return_sel=True, return_lse=True, **kw)
    torch.cuda.synchronize()
    return out, sel, lse


def _check_all_rows(inp, out, sel, lse, tol):
    ref = oracle.all_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk)
    np.testing.assert_array_equal(sel.cpu().numpy(), ref["sel"])
    err = np.abs(out.float().cpu().numpy() - ref["out"]).max()
    assert err <= tol, "max-abs error %.3g > %.3g" % (err, tol)
    lerr = np.abs(lse.cpu().numpy() - ref["lse"]).max()
    assert lerr <= 1e-3, "lse error %.3g" % lerr
    return err


SMALL = [
    # name, seqlens, hq, hkv, d, block, topk, dtype
    ("tiny-fp32", CONFIGS["tiny"]["seqlens"], 1, 1, 64, 256, 3, "f32"),
    ("gqa-varlen-bf16", [1000, 64, 0, 2300, 129], 8, 2, 128, 256, 3, "bf16"),
    ("gqa-d64-bf16", [1536, 700], 4, 1, 64, 128, 4, "bf16"),
    ("fine-blocks-bf16", [3000], 4, 2, 128, 64, 12, "bf16"),
    ("own-block-only-bf16", [1000, 333], 8, 8, 128, 128, 1, "bf16"),
    ("topk-covers-all-bf16", [1100], 4, 4, 64, 128, 16, "bf16"),
    ("g8-heads-bf16", [900], 16, 2, 128, 192, 3, "bf16"),
    ("g3-heads-f32", [700, 450], 6, 2, 64, 64, 3, "f32"),
    ("gqa-fp32", [1200, 300], 4, 2, 128, 128, 5, "f32"),
    # more than 512 blocks in a sequence: the screened gate's best-first lists
    ("many-blocks-k3-bf16", [40000, 900], 2, 1, 64, 64, 3, "bf16"),
    ("many-blocks-k5-bf16", [36000], 4, 2, 128, 64, 5, "bf16"),
    # three q heads per kv head with 16-bit D = 128: own-block tiles of one head,
    # three selected parts merged two and then one at a time
    ("g3-heads-k4-bf16", [1500, 700, 97], 6, 2, 128, 128, 4, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_forward_small_all_rows(case):
    name, seqlens, hq, hkv, d, block, topk, dt = case
    _say("%s seqlens=%s hq=%d hkv=%d d=%d block=%d topk=%d %s" % (name, seqlens, hq, hkv, d,
                                                                  block, topk, dt))
    inp = _to_gpu(make_inputs(seqlens, hq, hkv, d, block, topk, dtype=dt, seed=21))
    out, sel, lse = _run(inp)
    _check_all_rows(inp, out, sel, lse, TOL[inp.q.dtype])
    if inp.targets is not None:
        np.testing.assert_array_equal(sel.cpu().numpy(), inp.targets.numpy())


def test_forward_unplanted_random_inputs():
    # plain N(0,1): selections are decided by noise; compare where the fp64
    # margin is clear of fp32 rounding, and outputs on those rows
    _say("unplanted bf16 [2048, 517] hq=8 hkv=2 d=128 block=128 topk=3")
    inp = _to_gpu(make_inputs([2048, 517], 8, 2, 128, 128, 3, dtype="bf16", seed=5, plant=False))
    out, sel, lse = _run(inp)
    ref = oracle.all_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk)
    clear = ref["margin"] > 1e-3
    assert clear.mean() > 0.99
    np.testing.assert_array_equal(sel.cpu().numpy()[clear], ref["sel"][clear])
    err = np.abs(out.float().cpu().numpy() - ref["out"])[clear].max()
    assert err <= 2e-2


def test_gate_near_ties_match_oracle():
    """Pooled keys that differ only by small steps in one coordinate: the scores
    of competing blocks differ by ~1e-3, far below what the single bf16 pass
    of the screened gate can resolve, but far above fp32 rounding. Those rows
    must go through the exact gate and still pick the oracle's blocks."""
    _say("gate near ties bf16 [1024, 700] hq=2 hkv=1 d=128 block=64 topk=3")
    seqlens, block, d = [1024, 700], 64, 128
    inp = make_inputs(seqlens, 2, 1, d, block, 3, dtype="bf16", seed=9, plant=False)
    g = torch.Generator().manual_seed(10)
    base = torch.randn(block, 1, d, generator=g)
    base[:, :, 0] = 0.0
    k = []
    for s in seqlens:
        nb = (s + block - 1) // block
        for j in range(nb):
            blk = base.clone()
            blk[:, :, 0] = (j + 1) * 2.0 ** -10        # exact in bf16, same for every token
            k.append(blk[:min(block, s - j * block)])
    inp.k = torch.cat(k).to(torch.bfloat16).contiguous()
    inp = _to_gpu(inp)
    out, sel, lse = _run(inp)
    ref = oracle.all_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk)
    m = ref["margin"][np.isfinite(ref["margin"])]
    assert m.size and np.median(m) < 0.05          # the cut is far inside the single-pass error
    # rows whose fp64 margin is clear of fp32-grade rounding (|q_0| not tiny)
    clear = ref["margin"] > 1e-4
    assert clear.mean() > 0.85
    np.testing.assert_array_equal(sel.cpu().numpy()[clear], ref["sel"][clear])
    err = np.abs(out.float().cpu().numpy() - ref["out"])[clear].max()
    assert err <= 2e-2, err


@pytest.mark.parametrize("topk", [3, 6])
def test_gate_exact_ties_pick_lowest_blocks(topk):
    """Every block of every sequence has the same keys, so every past block scores
    the same for a row: the tie rule alone decides, and each row must keep its
    min(topk-1, i) lowest past blocks (the oracle's selection), on the screened
    path (topk 3) and on the exact gate (topk 6)."""
    _say("gate exact ties bf16 [1000, 650] hq=4 hkv=2 d=128 block=64 topk=%d" % topk)
    seqlens, block, d = [1000, 650], 64, 128
    inp = make_inputs(seqlens, 4, 2, d, block, topk, dtype="bf16", seed=12, plant=False)
    g = torch.Generator().manual_seed(13)
    base = torch.randn(block, 2, d, generator=g)
    k = []
    for s in seqlens:
        for j in range((s + block - 1) // block):
            k.append(base[:min(block, s - j * block)])
    inp.k = torch.cat(k).to(torch.bfloat16).contiguous()
    inp = _to_gpu(inp)
    out, sel, lse = _run(inp)
    ref = oracle.all_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk)
    np.testing.assert_array_equal(sel.cpu().numpy(), ref["sel"])
    # the rule by itself: ascending lowest blocks, -1 padded
    sel_np = sel.cpu().numpy()
    start = 0
    for s in seqlens:
        tok = np.arange(s)
        i = tok // block
        want = np.full((s, topk - 1), -1, dtype=np.int32)
        for c in range(topk - 1):
            want[:, c] = np.where(c < i, c, -1)
        for h in range(4):
            np.testing.assert_array_equal(sel_np[start:start + s, h], want)
        start += s
    err = np.abs(out.float().cpu().numpy() - ref["out"]).max()
    assert err <= 2e-2, err


def test_pool_matches_oracle():
    for seqlens, hkv, d, block, dt in (([2048], 1, 64, 256, "f32"), ([1000, 0, 2300, 129], 2,
                                                                       128, 256, "bf16"),
                                       ([4096], 8, 128, 2048, "bf16")):
        _say("pool seqlens=%s hkv=%d d=%d block=%d %s" % (seqlens, hkv, d, block, dt))
        inp = _to_gpu(make_inputs(seqlens, hkv, hkv, d, block, 3, dtype=dt, seed=3))
        kbar = moba.moba_block_pool(inp.k, inp.cu_seqlens, block)
        torch.cuda.synchronize()
        ref = oracle.pool(inp.k, inp.cu_seqlens, block)
        np.testing.assert_allclose(kbar.cpu().numpy(), ref, rtol=1e-6, atol=1e-6)


def _host_route(sel, seqlens, hq, hkv, block):
    """Stable counting sort of sel into per-(global block, kv-head) lists (numpy)."""
    T, _, ks = sel.shape
    group = hq // hkv
    base, start, gblk = [], 0, np.zeros(T, dtype=np.int64)
    nb_total = 0
    for s in seqlens:
        nb = (s + block - 1) // block
        gblk[start:start + s] = nb_total
        nb_total += nb
        start += s
    lists = [[] for _ in range(nb_total * hkv)]
    for t in range(T):
        for h in range(hq):
            for sl in range(ks):
                j = sel[t, h, sl]
                if j >= 0:
                    lists[(gblk[t] + j) * hkv + h // group].append((t * hq + h) * ks + sl)
    offs = np.zeros(len(lists) + 1, dtype=np.int64)
    for i, l in enumerate(lists):
        offs[i + 1] = offs[i] + len(l)
    ent = np.array([e for l in lists for e in l], dtype=np.int64)
    return offs, ent


def test_route_matches_host_counting_sort():
    seqlens, hq, hkv, d, block, topk = [1500, 77, 2100], 8, 2, 64, 64, 5
    _say("route seqlens=%s hq=%d hkv=%d block=%d topk=%d" % (seqlens, hq, hkv, block, topk))
    inp = _to_gpu(make_inputs(seqlens, hq, hkv, d, block, topk, dtype="bf16", seed=9))
    _, sel, _ = _run(inp)
    offs, ent = moba.moba_route(sel, inp.cu_seqlens, hkv, d, torch.bfloat16, block, topk)
    torch.cuda.synchronize()
    ref_offs, ref_ent = _host_route(sel.cpu().numpy(), seqlens, hq, hkv, block)
    np.testing.assert_array_equal(offs.cpu().numpy(), ref_offs)
    np.testing.assert_array_equal(ent.cpu().numpy(), ref_ent)


def test_deterministic_repeat():
    _say("determinism gqa-varlen-bf16")
    inp = _to_gpu(make_inputs([1000, 2300], 8, 2, 128, 256, 3, dtype="bf16", seed=4))
    a = _run(inp)
    b = _run(inp)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_dense_causal_matches_oracle_small():
    for seqlens, hq, hkv, d, dt in (([700, 0, 333], 4, 2, 128, "bf16"), ([513], 2, 1, 64, "f32"),
                                    ([300], 16, 2, 128, "bf16")):
        _say("dense seqlens=%s hq=%d hkv=%d d=%d %s" % (seqlens, hq, hkv, d, dt))
        inp = _to_gpu(make_inputs(seqlens, hq, hkv, d, 256, 3, dtype=dt, seed=2))
        out, lse = moba.moba_dense_causal_forward(inp.q, inp.k, inp.v, inp.cu_seqlens,
                                                  return_lse=True)
        torch.cuda.synchronize()
        T = sum(seqlens)
        tt, hh = np.repeat(np.arange(T), hq), np.tile(np.arange(hq), T)
        ref = oracle.causal_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, tt, hh)
        err = np.abs(out.float().cpu().numpy().reshape(-1, d) - ref["out"]).max()
        assert err <= TOL[inp.q.dtype], err
        np.testing.assert_allclose(lse.cpu().numpy().reshape(-1), ref["lse"], atol=1e-3)


def test_block_longer_than_sequence_equals_dense():
    _say("moba with one block per sequence vs dense, bf16")
    inp = _to_gpu(make_inputs([500, 1024], 8, 2, 128, 1024, 3, dtype="bf16", seed=8, plant=False))
    out = moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, 1024, 3)
    dense = moba.moba_dense_causal_forward(inp.q, inp.k, inp.v, inp.cu_seqlens)
    torch.cuda.synchronize()
    assert (out.float() - dense.float()).abs().max().item() <= 2e-2


def test_hybrid_switch_runs_each_path():
    """moba_attention_forward: sparse mode is moba_forward, full mode is the dense
    causal kernel (bitwise), and a two-layer sparse-then-full stack matches the
    oracle layer by layer."""
    _say("hybrid switch, gqa varlen bf16")
    inp = _to_gpu(make_inputs([1000, 64, 2300], 8, 2, 128, 256, 3, dtype="bf16", seed=21))
    sparse = moba.moba_attention(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk)
    full, lse_full = moba.moba_attention(inp.q, inp.k, inp.v, inp.cu_seqlens, 0, 0, full=True,
                                         return_lse=True)
    ref_sparse = moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk)
    ref_full, ref_lse = moba.moba_dense_causal_forward(inp.q, inp.k, inp.v, inp.cu_seqlens,
                                                       return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(sparse, ref_sparse)
    assert torch.equal(full, ref_full) and torch.equal(lse_full, ref_lse)
    # layer 2 (full) takes layer 1's (sparse) output as its query, as a stack would
    q2 = sparse.contiguous()
    out2 = moba.moba_attention(q2, inp.k, inp.v, inp.cu_seqlens, 0, 0, full=True)
    torch.cuda.synchronize()
    ref1 = oracle.all_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk)
    err1 = np.abs(sparse.float().cpu().numpy() - ref1["out"]).max()
    assert err1 <= TOL[inp.q.dtype], err1
    T, hq, d = q2.shape
    tt, hh = np.repeat(np.arange(T), hq), np.tile(np.arange(hq), T)
    ref2 = oracle.causal_rows(q2, inp.k, inp.v, inp.cu_seqlens, tt, hh)
    err2 = np.abs(out2.float().cpu().numpy().reshape(-1, d) - ref2["out"]).max()
    assert err2 <= TOL[inp.q.dtype], err2


# --- full-size workloads, benchmark launch configuration, sampled rows --------

FULL = ["llama32k", "varlen131k", "fine256k", "1m", "10m_shard"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(name):
    cfg = CONFIGS[name]
    _say("full-size %s %s" % (name, cfg))
    inp = make_config(name, seed=0, device="cuda")
    out, sel, lse = _run(inp)
    # every row: the planted targets
    sel_h = sel.cpu()
    assert torch.equal(sel_h, inp.targets), "selection differs from planted targets"
    # sampled rows: the oracle
    toks = sample_tokens(inp.seqlens, inp.block, 48, seed=1)
    hq = cfg["hq"]
    tt, hh = np.repeat(toks, hq), np.tile(np.arange(hq), len(toks))
    ref = oracle.rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk, tt, hh)
    m = ref["margin"]
    assert np.all(m[np.isfinite(m)] >= 0.5)
    np.testing.assert_array_equal(sel_h.numpy()[tt, hh], ref["sel"])
    got = out[torch.as_tensor(tt, device="cuda"), torch.as_tensor(hh, device="cuda")]
    err = np.abs(got.float().cpu().numpy() - ref["out"]).max()
    assert err <= 2e-2, err
    lgot = lse[torch.as_tensor(tt, device="cuda"), torch.as_tensor(hh, device="cuda")]
    assert np.abs(lgot.cpu().numpy() - ref["lse"]).max() <= 1e-3


def test_dense_full_32k_sampled_rows():
    _say("dense full-size llama32k")
    inp = make_config("llama32k", seed=0, device="cuda")
    out = moba.moba_dense_causal_forward(inp.q, inp.k, inp.v, inp.cu_seqlens)
    torch.cuda.synchronize()
    toks = sample_tokens(inp.seqlens, inp.block, 16, seed=2)
    tt, hh = np.repeat(toks, 32), np.tile(np.arange(32), len(toks))
    ref = oracle.causal_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, tt, hh)
    got = out[torch.as_tensor(tt, device="cuda"), torch.as_tensor(hh, device="cuda")]
    err = np.abs(got.float().cpu().numpy() - ref["out"]).max()
    assert err <= 2e-2, err
