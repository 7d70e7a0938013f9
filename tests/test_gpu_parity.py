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
from synth_inputs import CONFIGS, make_10m_full, make_config, make_inputs, sample_tokens

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
    # every past block kept in the first sequence and in the second's first 16
    # blocks; the second's 18 blocks keep the batch on the MoBA kernels
    ("topk-covers-all-bf16", [1100, 2200], 4, 4, 64, 128, 16, "bf16"),
    ("g8-heads-bf16", [900], 16, 2, 128, 192, 3, "bf16"),
    ("g3-heads-f32", [700, 450], 6, 2, 64, 64, 3, "f32"),
    ("gqa-fp32", [1200, 300], 4, 2, 128, 128, 5, "f32"),
    # more than 512 blocks in a sequence: the screened gate's 12-bit codes
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


U32 = 2.0 ** -23      # one fp32 ulp at 1: rounding of any kind (nearest or toward zero)


def _gamma(n):
    return n * U32 / (1 - n * U32)


def _gate_error_bound(inp, q_rows, heads):
    """Per (row, block) bound E on |GPU gate score - fp64 score| for the GPU's
    arithmetic: each pooled key is a sum of L <= block fp32 values divided by L
    (|error| <= gamma_L mean|k| + 2u|Kbar| per coordinate), scored as a sum of at
    most 3D exact bf16 x bf16 (or fp32) products accumulated in fp32
    (gamma_3D sum |q||Kbar|). Returns (scores [n, NB] fp64 over the row's
    sequence-global blocks, bound [n, NB])."""
    kbar = oracle.pool(inp.k, inp.cu_seqlens, inp.block)                  # [NB, hkv, d] fp64
    kabs = oracle.pool(inp.k.abs(), inp.cu_seqlens, inp.block)            # mean |k|
    L = []
    for S in inp.seqlens:
        L += [min(inp.block, S - b * inp.block) for b in range((S + inp.block - 1) // inp.block)]
    L = np.asarray(L, dtype=np.float64)[:, None, None]
    delta = _gamma(L) * kabs + 2 * U32 * np.abs(kbar)                      # [NB, hkv, d]
    d = kbar.shape[2]
    g = heads // (inp.q.shape[1] // inp.k.shape[1])
    qa = np.abs(q_rows)
    kg, dg = kbar[:, g, :], delta[:, g, :]                                 # [NB, n, d]
    scores = np.einsum("nd,bnd->nb", q_rows, kg)
    bound = np.einsum("nd,bnd->nb", qa, dg) + _gamma(3 * d) * np.einsum(
        "nd,bnd->nb", qa, np.abs(kg) + dg)
    return scores, bound


def _check_rows_exact_or_valid(inp, out, sel, tokens, heads, tol, min_equal):
    """Every listed row: where the GPU's selection equals the oracle's, its output
    against the oracle's; elsewhere (scores tied within rounding) the GPU's kept set
    must be a valid top-(topk-1) under the fp64 scores within the GPU's error bound
    (right count, distinct past blocks, ascending, no kept score below a dropped one
    by more than their two bounds), and its output must match the oracle evaluated
    on the GPU's own selection."""
    ks = inp.topk - 1
    ref = oracle.rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk, tokens, heads)
    got_sel = sel[torch.as_tensor(tokens, device=sel.device),
                  torch.as_tensor(heads, device=sel.device)].cpu().numpy().reshape(-1, ks)
    got_out = out[torch.as_tensor(tokens, device=out.device),
                  torch.as_tensor(heads, device=out.device)].float().cpu().numpy()
    same = (got_sel == ref["sel"]).all(axis=1)
    assert same.mean() >= min_equal, "only %.4f of rows select as the oracle" % same.mean()
    err = np.abs(got_out[same] - ref["out"][same]).max() if same.any() else 0.0
    assert err <= tol, "max-abs error %.3g > %.3g on rows selecting as the oracle" % (err, tol)
    diff = np.nonzero(~same)[0]
    if diff.size == 0:
        return 0
    cu = inp.cu_seqlens.numpy()
    seq = np.searchsorted(cu, tokens[diff], side="right") - 1
    local = tokens[diff] - cu[seq]
    i = local // inp.block
    blk0 = np.cumsum([0] + [(S + inp.block - 1) // inp.block for S in inp.seqlens])[seq]
    qd = oracle._f32(inp.q[torch.as_tensor(tokens[diff]), torch.as_tensor(heads[diff])])
    scores, bound = _gate_error_bound(inp, qd.astype(np.float64), heads[diff])
    for r in range(diff.size):
        kept = got_sel[diff[r]]
        ids = kept[kept >= 0]
        assert ids.size == min(ks, i[r]) and (kept[ids.size:] == -1).all(), (r, kept)
        assert (np.diff(ids) > 0).all() and (ids >= 0).all() and (ids < i[r]).all(), (r, kept)
        cand = np.arange(i[r])
        drop = np.setdiff1d(cand, ids)
        if drop.size == 0:
            continue
        sk, sd = scores[r, blk0[r] + ids], scores[r, blk0[r] + drop]
        ek, ed = bound[r, blk0[r] + ids], bound[r, blk0[r] + drop]
        worst = (sk[:, None] - sd[None, :]) + (ek[:, None] + ed[None, :])
        assert (worst >= 0).all(), "row %d keeps %s although a dropped block scores higher " \
            "beyond the error bound (%.3g)" % (r, ids, worst.min())
    alt = oracle.rows_given_sel(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk,
                                tokens[diff], heads[diff], got_sel[diff])
    err = np.abs(got_out[diff] - alt["out"]).max()
    assert err <= tol, "max-abs error %.3g > %.3g on rows with a tied selection" % (err, tol)
    return diff.size


def _all_rows_index(inp):
    T, hq = inp.q.shape[0], inp.q.shape[1]
    return (np.repeat(np.arange(T, dtype=np.int32), hq), np.tile(np.arange(hq, dtype=np.int32), T))


def test_forward_unplanted_random_inputs():
    # plain N(0,1): selections are decided by noise, so a few rows tie within
    # rounding; every row is checked, tied ones for validity
    _say("unplanted bf16 [2048, 517] hq=8 hkv=2 d=128 block=128 topk=3")
    inp = _to_gpu(make_inputs([2048, 517], 8, 2, 128, 128, 3, dtype="bf16", seed=5, plant=False))
    out, sel, lse = _run(inp)
    tt, hh = _all_rows_index(inp)
    n = _check_rows_exact_or_valid(inp, out, sel, tt, hh, 2e-2, min_equal=0.99)
    print("rows with a tied, valid selection: %d of %d" % (n, tt.size))


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
    # rows whose fp64 margin is clear of fp32-grade rounding (|q_0| not tiny) select
    # as the oracle; every other row must keep a valid top-(topk-1) set
    clear = ref["margin"] > 1e-4
    assert clear.mean() > 0.85
    np.testing.assert_array_equal(sel.cpu().numpy()[clear], ref["sel"][clear])
    tt, hh = _all_rows_index(inp)
    n = _check_rows_exact_or_valid(inp, out, sel, tt, hh, 2e-2, min_equal=0.85)
    print("rows with a tied, valid selection: %d of %d" % (n, tt.size))


@pytest.mark.parametrize("seqlens,hq,hkv,d,topk,plant", [
    ([600000], 4, 1, 128, 3, True),      # 9,375 blocks: 13-bit codes
    ([600000], 2, 1, 128, 5, False),     # the same, unplanted, topk - 1 = 4
    ([70000, 40000], 2, 2, 64, 4, True),  # 1,094 and 625 blocks: 12-bit codes, D = 64
    ([40000], 4, 2, 128, 3, False),      # 625 blocks, unplanted: flagged tiles
    ([40000], 4, 2, 128, 13, True),      # 625 blocks, twelve kept: 12-bit codes
    ([600000], 2, 1, 128, 9, False),     # 9,375 blocks, eight kept, unplanted
])
def test_many_blocks_wide_codes(seqlens, hq, hkv, d, topk, plant):
    """Sequences of more than 512 blocks (block 64): the screened pass packs wider
    codes (12 bits up to 8,192 blocks, 13 beyond) into the scores, so its screen
    bound is looser. Planted inputs with up to four targets must still select them
    on every row; 1,024 sampled tokens x every q head (each sequence's first and
    last tokens and its early blocks among them) against the oracle, tied rows
    for validity."""
    _say("many blocks bf16 %s hq=%d hkv=%d d=%d block=64 topk=%d plant=%s"
         % (seqlens, hq, hkv, d, topk, plant))
    inp = make_inputs(seqlens, hq, hkv, d, 64, topk, dtype="bf16", seed=21, device="cuda",
                      plant=plant)
    out, sel, lse = _run(inp)
    if plant and topk <= 5:
        # (with twelve planted blocks the weakest can score below a noise block,
        # so there only the oracle decides)
        assert torch.equal(sel.cpu(), inp.targets), "selection differs from planted targets"
    toks = sample_tokens(seqlens, 64, 1024, seed=3, every_block=False)
    tt, hh = np.repeat(toks, hq), np.tile(np.arange(hq), len(toks))
    n = _check_rows_exact_or_valid(inp, out, sel, tt, hh, 2e-2, min_equal=0.97)
    print("rows with a tied, valid selection: %d of %d" % (n, tt.size))


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


FORCED = [
    # name, seqlens, hq, hkv, d, block, topk, dtype: no sequence longer than topk blocks
    ("gqa-varlen-bf16", [1000, 0, 517, 64], 8, 2, 128, 256, 4, "bf16"),
    ("one-block-each-f32", [200, 64, 131], 4, 2, 64, 256, 2, "f32"),
    ("topk-equals-blocks-bf16", [2048, 1500], 4, 1, 128, 512, 4, "bf16"),
]


@pytest.mark.parametrize("case", FORCED, ids=[c[0] for c in FORCED])
def test_forced_selection_runs_dense_kernel(case):
    """When no sequence has more than topk blocks every row keeps all of its past
    blocks, and the forward runs the dense causal kernel with the forced
    selection: every row against the oracle, and the stage timers show the dense
    launch and no pool, gate or selected-block launch."""
    name, seqlens, hq, hkv, d, block, topk, dt = case
    _say("forced selection %s seqlens=%s hq=%d hkv=%d d=%d block=%d topk=%d %s"
         % (name, seqlens, hq, hkv, d, block, topk, dt))
    inp = _to_gpu(make_inputs(seqlens, hq, hkv, d, block, topk, dtype=dt, seed=31))
    moba.moba_timing_enable(True)
    moba.moba_timing_read()
    out, sel, lse = _run(inp)
    st = moba.moba_timing_read()
    moba.moba_timing_enable(False)
    assert st["attn_dense"][1] == 1
    assert st["pool"][1] == 0 and st["attn_selected"][1] == 0 and st["attn_self"][1] == 0
    _check_all_rows(inp, out, sel, lse, TOL[inp.q.dtype])


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


def test_binding_rejects_bad_arguments_before_launch():
    """Each inconsistent argument raises ValueError in the binding before anything
    is enqueued: the caller's output buffers keep their contents."""
    _say("binding argument checks on the GPU")
    inp = _to_gpu(make_inputs([700, 333], 4, 2, 128, 128, 3, dtype="bf16", seed=6))
    T = inp.q.shape[0]
    out = torch.full_like(inp.q, 7.0)
    cu_long = torch.tensor([0, 700, T + 64], dtype=torch.int32)
    with pytest.raises(ValueError, match="cu_seqlens"):
        moba.moba_forward(inp.q, inp.k, inp.v, cu_long, 128, 3, out=out)
    with pytest.raises(ValueError, match="cu_seqlens"):
        moba.moba_dense_causal_forward(inp.q, inp.k, inp.v, cu_long, out=out)
    with pytest.raises(ValueError, match="out"):
        moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, 128, 3, out=out[:-1])
    with pytest.raises(ValueError, match="out"):
        moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, 128, 3, out=out.float())
    with pytest.raises(ValueError, match="workspace"):
        moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, 128, 3, out=out,
                          workspace=torch.empty(1024, dtype=torch.uint8, device="cuda"))
    o2, sel, lse = moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, 128, 3,
                                     return_sel=True, return_lse=True)
    dq = torch.full_like(inp.q, 7.0)
    with pytest.raises(ValueError, match="dq"):
        moba.moba_backward(inp.q, inp.k, inp.v, o2, lse, o2, sel, inp.cu_seqlens, 128, 3,
                           dq=dq.float())
    with pytest.raises(ValueError, match="cu_seqlens"):
        moba.moba_backward(inp.q, inp.k, inp.v, o2, lse, o2, sel, cu_long, 128, 3, dq=dq)
    # decoding: caches shorter than cu_k says, pooled-key cache too small
    cu_k, cu_q = [0, 700, T], [0, 1, 2]
    q_new = inp.q[torch.tensor([699, T - 1], device="cuda")].contiguous()
    kbar = torch.zeros(2 * 6, 2, 128, dtype=torch.float32, device="cuda")
    dec_out = torch.full_like(q_new, 7.0)
    with pytest.raises(ValueError, match="k_cache"):
        moba.moba_decode(q_new, inp.k[:-1], inp.v[:-1], cu_q, cu_k, 128, 3, kbar, 6, out=dec_out)
    with pytest.raises(ValueError, match="kbar_cache"):
        moba.moba_decode(q_new, inp.k, inp.v, cu_q, cu_k, 128, 3, kbar[:-1], 6, out=dec_out)
    with pytest.raises(ValueError, match="kbar_cache"):
        moba.moba_kbar_append(inp.k, cu_k, [0, 0], 128, 6, kbar[:-1])
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((dq == 7.0).all()) and bool((dec_out == 7.0).all())


def test_large_values_within_the_fp16_part_range():
    """bf16 inputs keep their selected-block parts in fp16: values up to the stated
    limit |v| <= 65504 must come out right (relative to max|v|: bf16 output
    rounding 2^-9, fp16 part rounding 2^-11)."""
    _say("bf16 with max|v| = 6e4")
    inp = make_inputs([1500, 700], 8, 2, 128, 128, 4, dtype="bf16", seed=14)
    v = inp.v.float()
    inp.v = (v / v.abs().max() * 60000.0).to(torch.bfloat16).contiguous()
    assert float(inp.v.float().abs().max()) <= 65504.0
    inp = _to_gpu(inp)
    out, sel, lse = _run(inp)
    ref = oracle.all_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk)
    np.testing.assert_array_equal(sel.cpu().numpy(), ref["sel"])
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - ref["out"]).max()
    assert err <= 2.0 ** -8 * 60000.0, err


@pytest.mark.parametrize("case", [
    # shapes whose kv-group workspace is the smaller (many selected parts per row)
    ("bf16-gqa2-varlen-k6", [1000, 64, 0, 2300, 129], 8, 4, 128, 128, 6, "bf16"),
    ("f32-gqa2-d64-k5", [700, 450], 4, 2, 64, 64, 5, "f32"),
    ("bf16-gqa3-k6", [1500, 97], 6, 2, 128, 128, 6, "bf16"),
    # no sequence longer than topk blocks: each group takes the dense kernel and
    # the forced selection
    ("bf16-gqa2-forced-k6", [640, 64, 0, 300], 8, 4, 128, 128, 6, "bf16"),
], ids=lambda c: c[0])
def test_kv_group_mode_equals_one_pass(case):
    """A workspace below moba_workspace_bytes runs the kv groups one after another
    (slabs gathered, the same stages, outputs scattered back): the same rows, so
    out, sel and lse are bitwise those of one pass over all heads."""
    name, seqlens, hq, hkv, d, block, topk, dt = case
    _say("kv-group mode %s" % name)
    inp = _to_gpu(make_inputs(seqlens, hq, hkv, d, block, topk, dtype=dt, seed=23))
    full = moba.moba_workspace_bytes(inp.cu_seqlens, hq, hkv, d, inp.q.dtype, block, topk)
    small = moba.moba_workspace_bytes_min(inp.cu_seqlens, hq, hkv, d, inp.q.dtype, block, topk)
    assert small < full
    a = _run(inp)
    ws = torch.empty(small, dtype=torch.uint8, device="cuda")
    b = _run(inp, workspace=ws)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    _check_all_rows(inp, b[0], b[1], b[2], TOL[inp.q.dtype])


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
    # sampled rows: the oracle, on 4,096 tokens x every q head (at least one token of
    # every block, the first and last tokens of blocks 0-2 and of every sequence)
    toks = sample_tokens(inp.seqlens, inp.block, 4096, seed=1, every_block=True)
    print("oracle rows: %d tokens x %d heads" % (len(toks), cfg["hq"]), flush=True)
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


def test_full_width_10m_by_kv_group():
    """A full-width 10M-token layer (32 q heads, 8 kv heads, 5,120 blocks) through
    moba_forward itself: one pass over all heads would need more than the GPU's
    memory, so the forward runs kv group by kv group inside the library. Every
    row's selection equals the planted targets; sampled rows (one token of every
    block and more, all 32 heads) match the oracle, evaluated per kv group on that
    group's keys."""
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    _say("full-width 10M layer, kv-group mode")
    inp = make_10m_full(seed=0, device="cuda")
    T, hq, d = inp.q.shape
    hkv = inp.k.shape[1]
    G = hq // hkv
    full = moba.moba_workspace_bytes_min(inp.cu_seqlens, hq, hkv, d, inp.q.dtype, inp.block,
                                         inp.topk)
    print("workspace (kv-group mode): %.1f GB" % (full / 1e9), flush=True)
    out, sel, lse = moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk,
                                      return_sel=True, return_lse=True, by_kv_group=True)
    torch.cuda.synchronize()
    sel_h = sel.cpu()
    assert torch.equal(sel_h, inp.targets), "selection differs from planted targets"
    toks = sample_tokens(inp.seqlens, inp.block, 4096, seed=1, every_block=True)
    tt_dev = torch.as_tensor(toks, dtype=torch.long, device="cuda")
    worst = 0.0
    for g in range(hkv):
        kf = oracle._f32(inp.k[:, g:g + 1])
        vf = oracle._f32(inp.v[:, g:g + 1])
        qg = inp.q[:, G * g:G * (g + 1)]
        tt, hh = np.repeat(toks, G), np.tile(np.arange(G), len(toks))
        qr = oracle._f32(qg[tt_dev][:, :, :].reshape(-1, d))
        ref = oracle.rows(qr, kf, vf, inp.cu_seqlens, inp.block, inp.topk, tt, hh,
                          num_q_heads=G)
        m = ref["margin"]
        assert np.all(m[np.isfinite(m)] >= 0.5)
        np.testing.assert_array_equal(sel_h.numpy()[tt, G * g + hh], ref["sel"])
        got = out[tt_dev][:, G * g:G * (g + 1)].float().cpu().numpy().reshape(-1, d)
        err = np.abs(got - ref["out"]).max()
        worst = max(worst, err)
        assert err <= 2e-2, (g, err)
        lg = lse[tt_dev][:, G * g:G * (g + 1)].cpu().numpy().reshape(-1)
        assert np.abs(lg - ref["lse"]).max() <= 1e-3
        del kf, vf
        print("kv group %d: %d rows, max-abs error %.3g" % (g, len(tt), err), flush=True)
    del inp, out, sel, lse
    gc.collect()
    torch.cuda.empty_cache()
