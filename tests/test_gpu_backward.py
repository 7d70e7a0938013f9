"""GPU parity of the backward (dq, dk, dv with the forward's selection held
fixed) through the C ABI, against the fp64 oracle.

Small cases compare every gradient element: max-abs error at most 1e-4 (fp32
inputs) or 2e-2 (bf16 inputs) times max(1, max |reference|) of that gradient.
The bf16 bar is the forward's, scaled by the gradient's size: the kernels
round the probabilities and dS to bf16 where they feed the matrix cores (a
relative error of 2^-9 per term) and write the gradients in bf16.

Full-size workloads run the benchmark's launch configuration and check dq on
sampled rows against the oracle, and dk, dv on every key through identities
that hold at any size: per (sequence, kv head), the dv rows sum to the sum of
the group's dO rows and the dk rows sum to zero.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_causal_amd as moba
import oracle
from synth_inputs import CONFIGS, make_config, make_grad, make_inputs, sample_tokens

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def _say(msg):
    print("\n[case] " + msg, flush=True)
    sys.stdout.flush()


def _fwd_bwd(inp, dout):
    out, sel, lse = moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk,
                                      return_sel=True, return_lse=True)
    dq, dk, dv = moba.moba_backward(inp.q, inp.k, inp.v, out, lse, dout, sel, inp.cu_seqlens,
                                    inp.block, inp.topk)
    torch.cuda.synchronize()
    return sel, dq, dk, dv


def _close(name, got, ref, tol):
    scale = max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)
    err = float(np.abs(got.float().cpu().numpy() - ref).max()) if ref.size else 0.0
    print("  %s: max-abs error %.3g (max |ref| %.3g)" % (name, err, scale), flush=True)
    assert err <= tol * scale, "%s: max-abs error %.3g > %.3g" % (name, err, tol * scale)


SMALL = [
    # name, seqlens, hq, hkv, d, block, topk, dtype
    ("fp32-d64-varlen", [300, 129, 64], 4, 2, 64, 64, 3, "f32"),
    ("gqa-d128-varlen-bf16", [700, 1500, 65, 0], 8, 2, 128, 128, 3, "bf16"),
    ("own-block-only-bf16", [900, 300], 4, 4, 128, 256, 1, "bf16"),
    ("fine-blocks-bf16", [2000], 4, 1, 128, 64, 8, "bf16"),
    ("mha-d128-fp32", [500], 2, 2, 128, 128, 2, "f32"),
    ("block512-d64-bf16", [3000, 1100], 8, 8, 64, 512, 3, "bf16"),
    ("g8-heads-bf16", [900], 16, 2, 128, 192, 3, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_backward_small_all_elements(case):
    name, seqlens, hq, hkv, d, block, topk, dt = case
    _say("%s seqlens=%s hq=%d hkv=%d d=%d block=%d topk=%d %s"
         % (name, seqlens, hq, hkv, d, block, topk, dt))
    inp = make_inputs(seqlens, hq, hkv, d, block, topk, dtype=dt, seed=61, device="cuda")
    dout = make_grad(inp.q.shape, dt, seed=62, device="cuda")
    sel, dq, dk, dv = _fwd_bwd(inp, dout)
    if topk > 1:   # the gradients below are those of this selection
        ref_fwd = oracle.all_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, block, topk)
        np.testing.assert_array_equal(sel.cpu().numpy(), ref_fwd["sel"])
    ref = oracle.backward(inp.q, inp.k, inp.v, dout, inp.cu_seqlens, block, topk)
    tol = TOL[inp.q.dtype]
    _close("dq", dq, ref["dq"], tol)
    _close("dk", dk, ref["dk"], tol)
    _close("dv", dv, ref["dv"], tol)


def test_backward_is_deterministic():
    _say("backward determinism gqa bf16")
    inp = make_inputs([3000, 900], 8, 2, 128, 256, 3, dtype="bf16", seed=71, device="cuda")
    dout = make_grad(inp.q.shape, "bf16", seed=72, device="cuda")
    _, dq1, dk1, dv1 = _fwd_bwd(inp, dout)
    _, dq2, dk2, dv2 = _fwd_bwd(inp, dout)
    assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)


def _identities(inp, dout, dk, dv):
    cu = inp.cu_seqlens.tolist()
    hkv = inp.k.shape[1]
    G = inp.q.shape[1] // hkv
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        if a == b:
            continue
        for g in range(hkv):
            dv_rows = dv[a:b, g].double()
            dk_rows = dk[a:b, g].double()
            do_sum = dout[a:b, g * G:(g + 1) * G].double().sum((0, 1))
            # 6 sigma of the bf16 roundings of every term, summed at random
            bound_v = 6 * 2.0 ** -8 * dv_rows.pow(2).sum(0).sqrt() + 1e-3
            bound_k = 6 * 2.0 ** -8 * dk_rows.pow(2).sum(0).sqrt() + 1e-3
            ev = (dv_rows.sum(0) - do_sum).abs()
            ek = dk_rows.sum(0).abs()
            assert bool((ev <= bound_v).all()), (n, g, float(ev.max()), float(do_sum.abs().max()))
            assert bool((ek <= bound_k).all()), (n, g, float(ek.max()))


FULL = ["llama32k", "1m"]


@pytest.mark.parametrize("name", FULL)
def test_backward_full_size(name):
    cfg = CONFIGS[name]
    _say("backward full-size %s %s" % (name, cfg))
    inp = make_config(name, seed=0, device="cuda")
    # a mean offset makes the dv identity a sum of same-sign terms
    dout = make_grad(inp.q.shape, cfg["dtype"], seed=3, device="cuda", mean=0.25)
    sel, dq, dk, dv = _fwd_bwd(inp, dout)
    assert torch.equal(sel.cpu(), inp.targets)
    # dq on 1,024 tokens x every q head, at least one token of every block
    toks = sample_tokens(inp.seqlens, inp.block, 1024, seed=4, every_block=True)
    hq = cfg["hq"]
    print("oracle dq rows: %d tokens x %d heads" % (len(toks), hq), flush=True)
    tt, hh = np.repeat(toks, hq), np.tile(np.arange(hq), len(toks))
    ref = oracle.dq_rows(inp.q, inp.k, inp.v, dout, inp.cu_seqlens, inp.block, inp.topk, tt, hh)
    got = dq[torch.as_tensor(tt, device="cuda"), torch.as_tensor(hh, device="cuda")]
    _close("dq sampled", got, ref, TOL[inp.q.dtype])
    _identities(inp, dout, dk, dv)
