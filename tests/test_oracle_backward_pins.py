"""Pins of the oracle's backward (CPU, no GPU): checks that come from the
mathematics, not from re-typing the oracle's formula.

- central finite differences of the (separately pinned) fp64 forward oracle;
- torch fp64 autograd through the dense masked formulation of the same
  attention (the mask taken from the forward oracle's selection);
- closed-form identities: per (sequence, kv head) the dV rows sum to the sum
  of the group's dO rows, and the dK rows sum to zero (every row's dS sums to 0).
The per-row dq entry (dq_rows, for sampled rows of large batches) must give
the rows of the full backward's dq.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import make_inputs

CASE = dict(seqlens=[150, 90], hq=4, hkv=2, d=16, block=32, topk=3)


@pytest.fixture(scope="module")
def setup(oracle_mod):
    c = CASE
    inp = make_inputs(c["seqlens"], c["hq"], c["hkv"], c["d"], c["block"], c["topk"],
                      dtype="f32", seed=7)
    g = torch.Generator().manual_seed(3)
    dout = torch.randn(inp.q.shape, generator=g, dtype=torch.float32)
    grads = oracle.backward(inp.q, inp.k, inp.v, dout, inp.cu_seqlens, c["block"], c["topk"])
    return inp, dout, grads


def _loss(q, k, v, dout, inp):
    ref = oracle.all_rows(q, k, v, inp.cu_seqlens, CASE["block"], CASE["topk"])
    return float((ref["out"] * dout.numpy().astype(np.float64)).sum()), ref


def test_finite_differences(setup):
    inp, dout, grads = setup
    _, ref = _loss(inp.q, inp.k, inp.v, dout, inp)
    # the planted margins keep the selection fixed under these small steps
    assert np.min(ref["margin"]) > 0.1
    h = 2.0 ** -10           # exact in fp32 for these magnitudes
    rng = np.random.default_rng(11)
    for name in ("q", "k", "v"):
        base = getattr(inp, name)
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in base.shape)
            xp, xm = base.clone(), base.clone()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": inp.q, "k": inp.k, "v": inp.v}
            args[name] = xp
            lp, _ = _loss(args["q"], args["k"], args["v"], dout, inp)
            args[name] = xm
            lm, _ = _loss(args["q"], args["k"], args["v"], dout, inp)
            fd = (lp - lm) / (2 * h)
            an = grads["d" + name][idx]
            assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (name, idx, fd, an)


def test_autograd_of_dense_masked_attention(setup):
    inp, dout, grads = setup
    c = CASE
    T = sum(c["seqlens"])
    G = c["hq"] // c["hkv"]
    ref = oracle.all_rows(inp.q, inp.k, inp.v, inp.cu_seqlens, c["block"], c["topk"])
    sel = ref["sel"].reshape(T, c["hq"], -1)
    cu = inp.cu_seqlens.tolist()
    mask = torch.zeros(c["hq"], T, T, dtype=torch.bool)
    for n in range(len(c["seqlens"])):
        for t in range(cu[n], cu[n + 1]):
            i = (t - cu[n]) // c["block"]
            own0 = cu[n] + i * c["block"]
            for h in range(c["hq"]):
                mask[h, t, own0:t + 1] = True
                for j in sel[t, h]:
                    if j >= 0:
                        s0 = cu[n] + int(j) * c["block"]
                        mask[h, t, s0:s0 + c["block"]] = True
    q = inp.q.double().transpose(0, 1).clone().requires_grad_(True)           # [hq, T, d]
    k = inp.k.double().transpose(0, 1).clone().requires_grad_(True)           # [hkv, T, d]
    v = inp.v.double().transpose(0, 1).clone().requires_grad_(True)
    kk = k.repeat_interleave(G, dim=0)
    vv = v.repeat_interleave(G, dim=0)
    s = torch.matmul(q, kk.transpose(1, 2)) / np.sqrt(c["d"])
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vv)
    (o * dout.double().transpose(0, 1)).sum().backward()
    np.testing.assert_allclose(q.grad.transpose(0, 1).numpy(), grads["dq"], atol=1e-10, rtol=0)
    np.testing.assert_allclose(k.grad.transpose(0, 1).numpy(), grads["dk"], atol=1e-10, rtol=0)
    np.testing.assert_allclose(v.grad.transpose(0, 1).numpy(), grads["dv"], atol=1e-10, rtol=0)


def test_identities(setup):
    inp, dout, grads = setup
    c = CASE
    cu = inp.cu_seqlens.tolist()
    G = c["hq"] // c["hkv"]
    do = dout.numpy().astype(np.float64)
    for n in range(len(c["seqlens"])):
        a, b = cu[n], cu[n + 1]
        for g in range(c["hkv"]):
            dv_sum = grads["dv"][a:b, g].sum(0)
            do_sum = do[a:b, g * G:(g + 1) * G].sum((0, 1))
            np.testing.assert_allclose(dv_sum, do_sum, atol=1e-9)
            np.testing.assert_allclose(grads["dk"][a:b, g].sum(0), 0.0, atol=1e-9)


def test_dq_rows_equals_full_backward(setup):
    inp, dout, grads = setup
    c = CASE
    rng = np.random.default_rng(5)
    T = sum(c["seqlens"])
    toks = rng.integers(0, T, 40).astype(np.int32)
    heads = rng.integers(0, c["hq"], 40).astype(np.int32)
    dq = oracle.dq_rows(inp.q, inp.k, inp.v, dout, inp.cu_seqlens, c["block"], c["topk"], toks,
                        heads)
    np.testing.assert_array_equal(dq, grads["dq"][toks, heads])
