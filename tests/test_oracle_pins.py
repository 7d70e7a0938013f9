"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped own-block
prefix, an off-by-one in the causal boundary, a wrong head grouping, a sign
error in the gate, mean vs sum pooling, a wrong softmax scale, the own block
counted or not counted in top-k, ties broken the other way) fails at least one:

* brute force: a literal dense [S, S] mask in numpy (tests/brute.py);
* closed forms through torch's scaled_dot_product_attention in fp64 (a library
  routine): top-k covering every past block gives full causal attention; top-k
  of 1 gives block-diagonal causal attention; a block as long as the sequence
  gives dense causal attention;
* closed forms by hand: zero queries give a uniform average over the attended
  set with lse = log |A|; a hand-worked fixture (tests/golden);
* selection invariants, tie-break on exactly equal scores, pooled-key closed
  forms, and the planted-needle targets of the input generator.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from brute import brute_force
from synth_inputs import cu_seqlens_of, make_config, make_inputs, sample_tokens

HERE = os.path.dirname(os.path.abspath(__file__))


def _np(x):
    return x.to(torch.float64).numpy()


def _sdpa_causal(q, k, v, scale):
    """torch SDPA in fp64 for one head: q,k,v [S, d] numpy -> (out, lse)."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=scale)
    return out[0, 0].numpy()


def _rand_inputs(seqlens, hq, hkv, d, seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    T = sum(seqlens)
    q = torch.randn(T, hq, d, generator=g).to(dtype)
    k = torch.randn(T, hkv, d, generator=g).to(dtype)
    v = torch.randn(T, hkv, d, generator=g).to(dtype)
    return q, k, v, cu_seqlens_of(seqlens)


BRUTE_CASES = [
    # seqlens, hq, hkv, d, block, topk
    ([2048], 1, 1, 64, 256, 3),                # the tiny workload's shape
    ([300, 512, 0, 77, 1000], 4, 2, 16, 64, 3),  # varlen, empty sequence, partial blocks, GQA
    ([640], 2, 1, 8, 64, 1),                   # own block only
    ([640], 2, 2, 8, 64, 30),                  # top-k beyond the block count
    ([513, 129], 6, 3, 8, 64, 5),              # G = 2, k-1 = 4
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_oracle_matches_dense_mask_brute_force(oracle_mod, case):
    seqlens, hq, hkv, d, block, topk = case
    q, k, v, cu = _rand_inputs(seqlens, hq, hkv, d, seed=len(seqlens) * 7 + d)
    ref_out, ref_lse, ref_sel, ref_margin = brute_force(_np(q), _np(k), _np(v), seqlens, block,
                                                        topk, return_margin=True)
    res = oracle_mod.all_rows(q, k, v, cu, block, topk)
    np.testing.assert_array_equal(res["sel"], ref_sel)
    np.testing.assert_allclose(res["out"], ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["lse"], ref_lse, rtol=1e-13, atol=1e-12)
    # the margin (lowest kept score minus highest score left out) decides which
    # rows a GPU test compares by selection; the brute force computes it from its
    # own dense score matrix
    fin = np.isfinite(ref_margin)
    np.testing.assert_array_equal(np.isfinite(res["margin"]), fin)
    np.testing.assert_allclose(res["margin"][fin], ref_margin[fin], rtol=0, atol=1e-12)
    if topk > 1 and fin.any():
        assert (ref_margin[fin] > 0).all()          # random scores: no exact ties


def _random_valid_selection(seqlens, hq, block, topk, seed):
    """For every row, a random set of min(topk-1, i) distinct past blocks (not the
    gated ones), ascending, -1 padded."""
    rng = np.random.default_rng(seed)
    ks = topk - 1
    rows = []
    for S in seqlens:
        for t in range(S):
            i = t // block
            for _ in range(hq):
                c = np.sort(rng.choice(i, size=min(ks, i), replace=False)) if i else []
                rows.append(list(c) + [-1] * (ks - len(c)))
    return np.asarray(rows, dtype=np.int32).reshape(sum(seqlens), hq, ks)


@pytest.mark.parametrize("case", [([700, 0, 333], 4, 2, 16, 64, 4), ([1024], 2, 1, 8, 128, 3)])
def test_rows_given_sel_matches_brute_force(oracle_mod, case):
    """Attention over a forced selection (what a GPU's near-tied choice is checked
    against): the brute force's dense mask built from the same forced blocks."""
    seqlens, hq, hkv, d, block, topk = case
    q, k, v, cu = _rand_inputs(seqlens, hq, hkv, d, seed=77)
    sel = _random_valid_selection(seqlens, hq, block, topk, seed=5)
    ref_out, ref_lse, _ = brute_force(_np(q), _np(k), _np(v), seqlens, block, topk, sel_in=sel)
    T = sum(seqlens)
    tt, hh = np.repeat(np.arange(T), hq), np.tile(np.arange(hq), T)
    res = oracle_mod.rows_given_sel(q, k, v, cu, block, topk, tt, hh, sel.reshape(T * hq, -1))
    np.testing.assert_allclose(res["out"].reshape(T, hq, d), ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["lse"].reshape(T, hq), ref_lse, rtol=1e-13, atol=1e-12)
    # on its own gated selection it is the full oracle (blocks summed in ascending
    # order instead of the order taken: equal up to fp64 rounding)
    full = oracle_mod.rows(q, k, v, cu, block, topk, tt, hh)
    again = oracle_mod.rows_given_sel(q, k, v, cu, block, topk, tt, hh, full["sel"])
    np.testing.assert_allclose(again["out"], full["out"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(again["lse"], full["lse"], rtol=1e-14, atol=1e-13)
    # ids that are not distinct past blocks are refused
    bad = sel.reshape(T * hq, -1).copy()
    r = int(np.nonzero((tt // block) == 2)[0][0])     # a row in block 2
    bad[r, 0] = 2                                       # its own block
    with pytest.raises(ValueError):
        oracle_mod.rows_given_sel(q, k, v, cu, block, topk, tt, hh, bad)
    bad[r, :2] = [1, 1]                                 # a duplicate
    with pytest.raises(ValueError):
        oracle_mod.rows_given_sel(q, k, v, cu, block, topk, tt, hh, bad)


def test_planted_tiny_matches_brute_force_and_targets(oracle_mod):
    inp = make_config("tiny", seed=0)
    ref_out, ref_lse, ref_sel = brute_force(_np(inp.q), _np(inp.k), _np(inp.v),
                                            inp.seqlens, inp.block, inp.topk)
    res = oracle_mod.all_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk)
    np.testing.assert_array_equal(res["sel"], ref_sel)
    np.testing.assert_array_equal(res["sel"], inp.targets.numpy())
    np.testing.assert_allclose(res["out"], ref_out, rtol=0, atol=1e-12)
    # the gate margin the workload promises: >= 0.5 wherever a choice is made
    blocks = (np.arange(2048) // 256)[:, None]
    has_choice = blocks > inp.topk - 1
    assert np.all(res["margin"][np.broadcast_to(has_choice, res["margin"].shape)] >= 0.5)


def test_full_attention_when_topk_covers_all_blocks(oracle_mod):
    # README: MoBA switches seamlessly to full attention; with every past block
    # selected the key set of token t is {0..t}.
    seqlens, hq, hkv, d, block = [700, 333], 4, 2, 16, 64
    q, k, v, cu = _rand_inputs(seqlens, hq, hkv, d, seed=3)
    res = oracle_mod.all_rows(q, k, v, cu, block, topk=64)
    scale = 1 / math.sqrt(d)
    start = 0
    for S in seqlens:
        for h in range(hq):
            ref = _sdpa_causal(_np(q[start:start + S, h]), _np(k[start:start + S, h // 2]),
                               _np(v[start:start + S, h // 2]), scale)
            np.testing.assert_allclose(res["out"][start:start + S, h], ref, atol=1e-12, rtol=0)
        start += S


def test_own_block_only_is_block_diagonal_causal(oracle_mod):
    seqlens, hq, hkv, d, block = [300], 2, 1, 8, 64
    q, k, v, cu = _rand_inputs(seqlens, hq, hkv, d, seed=4)
    res = oracle_mod.all_rows(q, k, v, cu, block, topk=1)
    scale = 1 / math.sqrt(d)
    for h in range(hq):
        for b0 in range(0, 300, block):
            b1 = min(b0 + block, 300)
            ref = _sdpa_causal(_np(q[b0:b1, h]), _np(k[b0:b1, 0]), _np(v[b0:b1, 0]), scale)
            np.testing.assert_allclose(res["out"][b0:b1, h], ref, atol=1e-12, rtol=0)


def test_block_as_long_as_sequence_is_dense_causal(oracle_mod):
    seqlens, hq, hkv, d = [200, 150], 2, 2, 8
    q, k, v, cu = _rand_inputs(seqlens, hq, hkv, d, seed=5)
    res = oracle_mod.all_rows(q, k, v, cu, block=256, topk=3)
    dense = oracle_mod.causal_rows(q, k, v, cu, np.repeat(np.arange(350), hq),
                                   np.tile(np.arange(hq), 350))
    scale = 1 / math.sqrt(d)
    start = 0
    for S in seqlens:
        for h in range(hq):
            ref = _sdpa_causal(_np(q[start:start + S, h]), _np(k[start:start + S, h]),
                               _np(v[start:start + S, h]), scale)
            np.testing.assert_allclose(res["out"][start:start + S, h], ref, atol=1e-12, rtol=0)
        start += S
    np.testing.assert_allclose(dense["out"].reshape(350, hq, d), res["out"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(dense["lse"].reshape(350, hq), res["lse"], atol=1e-12, rtol=0)


def test_zero_queries_average_uniformly_over_the_attended_set(oracle_mod):
    # q = 0: every gate score ties at 0 (lowest blocks win) and every logit is 0,
    # so out is the plain mean of V over A and lse = log |A|.
    seqlens, hq, hkv, d, block, topk = [450], 2, 1, 4, 64, 3
    _, k, v, cu = _rand_inputs(seqlens, hq, hkv, d, seed=6)
    q = torch.zeros(450, hq, d)
    res = oracle_mod.all_rows(q, k, v, cu, block, topk)
    vv = _np(v)[:, 0]
    for t in range(450):
        i = t // block
        chosen = list(range(min(topk - 1, i)))
        keys = list(range(i * block, t + 1))
        for j in chosen:
            keys += list(range(j * block, (j + 1) * block))
        for h in range(hq):
            assert list(res["sel"][t, h][res["sel"][t, h] >= 0]) == chosen
            np.testing.assert_allclose(res["out"][t, h], vv[keys].mean(axis=0), atol=1e-13)
            assert abs(res["lse"][t, h] - math.log(len(keys))) < 1e-13


def test_ties_break_toward_lower_block_index(oracle_mod):
    # every block holds the same keys, so all pooled keys and all scores are equal
    seqlens, hq, hkv, d, block, topk = [512], 2, 1, 8, 64, 4
    q, _, v, cu = _rand_inputs(seqlens, hq, hkv, d, seed=7)
    base = torch.randn(block, hkv, d, generator=torch.Generator().manual_seed(8))
    k = base.repeat(512 // block, 1, 1)
    res = oracle_mod.all_rows(q, k, v, cu, block, topk)
    for t in range(512):
        n = min(topk - 1, t // block)
        for h in range(hq):
            assert list(res["sel"][t, h]) == list(range(n)) + [-1] * (topk - 1 - n)


def test_selection_invariants(oracle_mod):
    seqlens, hq, hkv, d, block, topk = [1000, 64, 1], 4, 1, 8, 64, 4
    q, k, v, cu = _rand_inputs(seqlens, hq, hkv, d, seed=9)
    res = oracle_mod.all_rows(q, k, v, cu, block, topk)
    start = 0
    for S in seqlens:
        for t in range(S):
            i = t // block
            for h in range(hq):
                s = res["sel"][start + t, h]
                kept = s[s >= 0]
                assert len(kept) == min(topk - 1, i)          # count
                assert np.all(s[len(kept):] == -1)            # padding at the end
                assert np.all(kept < i) and np.all(kept >= 0)  # past blocks only
                assert np.all(np.diff(kept) > 0)              # ascending, no duplicates
        start += S


def test_pool_closed_forms(oracle_mod):
    seqlens, hkv, d, block = [300, 128], 2, 3, 128
    T = sum(seqlens)
    # constant keys within each block: the pooled key is that constant
    blk_val = torch.tensor([5.0, -1.5, 0.25, 7.0])
    blk_id = torch.tensor([0] * 128 + [1] * 128 + [2] * 44 + [3] * 128)
    k = blk_val[blk_id][:, None, None].expand(T, hkv, d).contiguous()
    kb = oracle_mod.pool(k, cu_seqlens_of(seqlens), block)
    np.testing.assert_array_equal(kb[:, 0, 0], blk_val.numpy())
    # a linear ramp within the partial final block: its mean uses the true length
    ramp = torch.arange(T, dtype=torch.float32)[:, None, None].expand(T, hkv, d).contiguous()
    kb = oracle_mod.pool(ramp, cu_seqlens_of(seqlens), block)
    assert kb[2, 1, 2] == (256 + 299) / 2
    assert kb[3, 0, 0] == (300 + 427) / 2
    # linearity (dyadic values, so 2*k1 - 3*k2 is exact in fp32)
    g = torch.Generator().manual_seed(10)
    k1 = torch.randint(-64, 64, (T, hkv, d), generator=g).float() / 8
    k2 = torch.randint(-64, 64, (T, hkv, d), generator=g).float() / 8
    lhs = oracle_mod.pool(2 * k1 - 3 * k2, cu_seqlens_of(seqlens), block)
    rhs = 2 * oracle_mod.pool(k1, cu_seqlens_of(seqlens), block) - \
        3 * oracle_mod.pool(k2, cu_seqlens_of(seqlens), block)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)


def test_hand_worked_fixture(oracle_mod):
    fx = json.load(open(os.path.join(HERE, "golden", "hand_d1_s8_b2.json")))
    q = torch.tensor(fx["q"]).reshape(8, 1, 1)
    k = torch.tensor(fx["k"]).reshape(8, 1, 1)
    v = torch.tensor(fx["v"]).reshape(8, 1, 1)
    env = {"e": math.e, "log": math.log, "__builtins__": {}}
    for case in fx["cases"]:
        res = oracle_mod.all_rows(q, k, v, cu_seqlens_of([8]), fx["block"], case["topk"])
        np.testing.assert_array_equal(res["sel"][:, 0], np.array(case["sel"]))
        out = np.array([eval(x, env) for x in case["out"]])
        lse = np.array([eval(x, env) for x in case["lse"]])
        np.testing.assert_allclose(res["out"][:, 0, 0], out, atol=1e-14, rtol=1e-14)
        np.testing.assert_allclose(res["lse"][:, 0], lse, atol=1e-14, rtol=1e-14)


def test_planted_gqa_targets_and_margin(oracle_mod):
    # GQA with G = 4: each q-head is gated against its own kv-head's pooled keys
    inp = make_inputs([1024, 700], hq=8, hkv=2, d=32, block=64, topk=4, dtype="bf16", seed=11)
    res = oracle_mod.all_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk)
    np.testing.assert_array_equal(res["sel"], inp.targets.numpy())
    m = res["margin"]
    assert np.all(m[np.isfinite(m)] >= 0.5)


def test_sampled_rows_equal_full_rows(oracle_mod):
    inp = make_inputs([900, 500], hq=4, hkv=2, d=16, block=64, topk=3, dtype="bf16", seed=12)
    full = oracle_mod.all_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk)
    toks = sample_tokens(inp.seqlens, inp.block, 50, seed=1)
    heads = np.arange(4)
    tt, hh = np.repeat(toks, 4), np.tile(heads, len(toks))
    part = oracle_mod.rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk, tt, hh)
    np.testing.assert_array_equal(part["out"], full["out"][tt, hh])
    np.testing.assert_array_equal(part["sel"], full["sel"][tt, hh])


def test_sample_tokens_covers_block_edges():
    toks = sample_tokens([16384, 19456], 2048, 64, seed=0)
    for t in (0, 16383, 2047, 2048, 4095, 4096, 6143, 14336, 16384, 16384 + 18432,
              16384 + 19455):
        assert t in toks
    assert np.all(np.diff(toks) > 0)


@pytest.mark.slow
def test_planted_llama_shape_sampled_rows(oracle_mod):
    # the 32K Llama-shaped workload, built on the CPU: planted targets hold on a
    # sample of rows, with the promised margin
    inp = make_config("llama32k", seed=0)
    toks = sample_tokens(inp.seqlens, inp.block, 24, seed=2)
    tt, hh = np.repeat(toks, 32), np.tile(np.arange(32), len(toks))
    res = oracle_mod.rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk, tt, hh)
    np.testing.assert_array_equal(res["sel"], inp.targets.numpy()[tt, hh])
    m = res["margin"]
    assert np.all(m[np.isfinite(m)] >= 0.5)
