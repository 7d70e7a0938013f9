"""GPU parity of the decode path (gated decode / chunked-prefill continuation
against a KV cache) through the C ABI.

A new row at position p is the prefill's row p, so the fp64 oracle's row
function is the reference: selections bit-exact, outputs within 1e-4 (fp32) /
2e-2 (bf16) max-abs, lse within 1e-3. The pooled-key cache must equal the
prefill's pooling bitwise (same fp32 summation order).
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_causal_amd as moba
import oracle
from synth_inputs import cu_seqlens_of, make_inputs

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def _say(msg):
    print("\n[case] " + msg, flush=True)
    sys.stdout.flush()


def _max_blocks(seqlens, block):
    return max(1, max((s + block - 1) // block for s in seqlens))


def _tail_rows(seqlens, nnew):
    """Global token ids of each sequence's last nnew[n] tokens, and cu_q."""
    cu = cu_seqlens_of(seqlens).tolist()
    toks = []
    for n, (s, m) in enumerate(zip(seqlens, nnew)):
        toks.extend(range(cu[n] + s - m, cu[n] + s))
    cu_q = [0]
    for m in nnew:
        cu_q.append(cu_q[-1] + m)
    return np.asarray(toks, dtype=np.int64), cu_q


def _pack_prefix(x, seqlens, lens):
    """Packed tensor of the first lens[n] tokens of every sequence of x."""
    cu = cu_seqlens_of(seqlens).tolist()
    parts = [x[cu[n]:cu[n] + lens[n]] for n in range(len(seqlens))]
    return torch.cat(parts, 0).contiguous()


def test_kbar_append_equals_prefill_pool_in_two_steps():
    seqlens, block, hkv, d = [3000, 700, 5000, 0], 256, 2, 128
    _say("kbar append seqlens=%s block=%d (two growth steps)" % (seqlens, block))
    inp = make_inputs(seqlens, 4, hkv, d, block, 3, dtype="bf16", seed=31, device="cuda")
    mb = _max_blocks(seqlens, block)
    kbar = torch.full((len(seqlens) * mb, hkv, d), float("nan"), dtype=torch.float32,
                      device="cuda")
    first = [1000, 300, 2600, 0]
    k1 = _pack_prefix(inp.k, seqlens, first)
    moba.moba_kbar_append(k1, cu_seqlens_of(first), [0] * len(seqlens), block, mb, kbar)
    moba.moba_kbar_append(inp.k, inp.cu_seqlens, first, block, mb, kbar)
    ref = moba.moba_block_pool(inp.k, inp.cu_seqlens, block)
    torch.cuda.synchronize()
    gb = 0
    for n, s in enumerate(seqlens):
        nb = (s + block - 1) // block
        for j in range(s // block):                       # complete blocks only
            assert torch.equal(kbar[n * mb + j], ref[gb + j]), (n, j)
        for j in range(s // block, mb):                   # never written
            assert torch.isnan(kbar[n * mb + j]).all(), (n, j)
        gb += nb


DECODE = [
    # name, seqlens, new rows per sequence, hq, hkv, d, block, topk, dtype
    ("decode-bf16", [3000, 5000, 700], [1, 1, 1], 8, 2, 128, 256, 3, "bf16"),
    ("chunked-bf16", [3000, 5000, 700], [300, 1, 700], 8, 2, 128, 256, 3, "bf16"),
    ("chunked-fp32-d64", [2048, 1500], [200, 64], 2, 1, 64, 256, 3, "f32"),
    ("fine-blocks-bf16", [4000], [130], 4, 2, 128, 64, 12, "bf16"),
    ("own-block-only-bf16", [1000, 333], [40, 333], 8, 8, 128, 128, 1, "bf16"),
]


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_decode_matches_oracle(case):
    name, seqlens, nnew, hq, hkv, d, block, topk, dt = case
    _say("%s seqlens=%s new=%s hq=%d hkv=%d d=%d block=%d topk=%d %s"
         % (name, seqlens, nnew, hq, hkv, d, block, topk, dt))
    inp = make_inputs(seqlens, hq, hkv, d, block, topk, dtype=dt, seed=41, device="cuda")
    toks, cu_q = _tail_rows(seqlens, nnew)
    q_new = inp.q[torch.as_tensor(toks, device="cuda")].contiguous()
    mb = _max_blocks(seqlens, block)
    kbar = torch.zeros(len(seqlens) * mb, hkv, d, dtype=torch.float32, device="cuda")
    moba.moba_kbar_append(inp.k, inp.cu_seqlens, [0] * len(seqlens), block, mb, kbar)
    out, sel, lse = moba.moba_decode(q_new, inp.k, inp.v, cu_q, inp.cu_seqlens, block, topk,
                                     kbar, mb, return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    T_new = len(toks)
    tt, hh = np.repeat(toks, hq), np.tile(np.arange(hq), T_new)
    ref = oracle.rows(inp.q, inp.k, inp.v, inp.cu_seqlens, block, topk, tt, hh)
    np.testing.assert_array_equal(sel.cpu().numpy().reshape(T_new * hq, -1), ref["sel"])
    err = np.abs(out.float().cpu().numpy().reshape(-1, d) - ref["out"]).max()
    assert err <= TOL[inp.q.dtype], "max-abs error %.3g" % err
    lerr = np.abs(lse.cpu().numpy().reshape(-1) - ref["lse"]).max()
    assert lerr <= 1e-3, "lse error %.3g" % lerr
    # and the prefill of the whole sequences keeps the same blocks for these rows
    if topk > 1:
        _, psel = moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, block, topk,
                                    return_sel=True)
        torch.cuda.synchronize()
        assert torch.equal(psel[torch.as_tensor(toks, device="cuda")], sel)


def test_decode_steps_track_the_prefill():
    """Token-by-token growth: every step appends one token, pools what it
    completed, and decodes the new row; the rows equal the prefill's."""
    seqlens, hq, hkv, d, block, topk = [600, 900], 4, 2, 128, 128, 3
    _say("decode steps seqlens=%s block=%d" % (seqlens, block))
    inp = make_inputs(seqlens, hq, hkv, d, block, topk, dtype="bf16", seed=51, device="cuda")
    full, psel = moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, block, topk,
                                   return_sel=True)
    mb = _max_blocks(seqlens, block)
    kbar = torch.zeros(len(seqlens) * mb, hkv, d, dtype=torch.float32, device="cuda")
    start = [500, 800]                                    # cached before the steps
    lens = list(start)
    kc = _pack_prefix(inp.k, seqlens, lens)
    moba.moba_kbar_append(kc, cu_seqlens_of(lens), [0, 0], block, mb, kbar)
    cu = cu_seqlens_of(seqlens).tolist()
    worst = 0.0
    for step in range(100):                               # crosses block boundaries
        prev = list(lens)
        lens = [l + 1 for l in lens]
        kc = _pack_prefix(inp.k, seqlens, lens)
        vc = _pack_prefix(inp.v, seqlens, lens)
        moba.moba_kbar_append(kc, cu_seqlens_of(lens), prev, block, mb, kbar)
        toks = [cu[n] + lens[n] - 1 for n in range(len(seqlens))]
        q_new = inp.q[torch.as_tensor(toks, device="cuda")].contiguous()
        out, sel = moba.moba_decode(q_new, kc, vc, [0, 1, 2], cu_seqlens_of(lens), block, topk,
                                    kbar, mb, return_sel=True)
        ti = torch.as_tensor(toks, device="cuda")
        assert torch.equal(sel, psel[ti]), step
        worst = max(worst, (out.float() - full[ti].float()).abs().max().item())
    torch.cuda.synchronize()
    assert worst <= 2e-2, worst
