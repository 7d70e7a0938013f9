#!/usr/bin/env python3
"""Benchmark: MoBA causal prefill forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 1m]

One step = one moba_forward call over the whole batch (pool, gate, route,
selected-block attention, self-block attention with the merge of the parts in
its epilogue), inputs resident in HBM.
Prints one JSON line: tokens/s, the roofline of the dominant kernel (timed live
with HIP events on the launch stream, and from the committed kernel trace), the
dense causal comparison from the same library, the CPU oracle timed on a bounded
sample of the same workload, and (for the 1M workload) the metric's 128K point,
the packed varlen batch, timed the same way in the same run.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoBA fwd tokens/s + MFMA util at S=128K/1M; speedup vs dense causal flash-attn"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 MFMA / vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
CONFIG_NAMES = {"tiny": "moba_fwd_tiny_2k_fp32", "llama32k": "moba_fwd_llama8b_32k",
                "varlen131k": "moba_fwd_varlen_131k", "1m": "moba_fwd_1m",
                "fine256k": "moba_fwd_fine_blocks_256k", "10m_shard": "moba_fwd_10m_head_shard",
                "10m_full": "moba_fwd_10m_full_width"}


def work_counts(seqlens, hq, hkv, d, block, topk, elem_bytes):
    """Algorithmic work per forward call, per stage (what the method must do)."""
    ks = topk - 1
    part_bytes = 2 if elem_bytes == 2 else 4   # partial outputs: fp16 for bf16 inputs
    rows_sel_pairs = 0      # sum over rows of min(ks, i) * B   (selected keys)
    self_pairs = 0          # sum over rows of own-block keys (causal)
    gate_pairs = 0          # sum over rows of past blocks i
    sel_parts = 0           # sum over rows of min(ks, i)
    nb_total = 0
    T = sum(seqlens)
    for s in seqlens:
        nb = (s + block - 1) // block
        nb_total += nb
        for i in range(nb):
            L = min(block, s - i * block)
            rows_sel_pairs += L * min(ks, i) * block
            self_pairs += L * (L + 1) // 2
            gate_pairs += L * i
            sel_parts += L * min(ks, i)
    return {
        "attn_selected_flop": 4.0 * d * hq * rows_sel_pairs,
        "attn_self_flop": 4.0 * d * hq * self_pairs,
        "gate_flop": 2.0 * d * hq * gate_pairs,
        "dense_flop": 4.0 * d * hq * sum(s * (s + 1) // 2 for s in seqlens),
        # bytes: pool reads K and writes fp32 pooled keys; gate reads Q and writes
        # the selection; the merge (self-block epilogue) reads the selected parts
        # (D values + lse) and writes out
        "pool_bytes": elem_bytes * T * hkv * d + 4.0 * nb_total * hkv * d,
        "gate_bytes": elem_bytes * T * hq * d + 4.0 * T * hq * ks,
        "merge_bytes": hq * sel_parts * (part_bytes * d + 4.0) + elem_bytes * T * hq * d,
        # route: the counting sort reads the selection (4 B per (row, slot)) for
        # the histograms and again for the scatter, and writes one 4-byte entry
        # per routed (row, slot)
        "route_bytes": 12.0 * hq * sel_parts,
    }


# the sources the attention kernels are built from (their launch code included)
ATTN_SOURCES = ("attention.hip", "moba_device.h", "moba_plan.h")


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_attention_causal_amd", "csrc")
    for f in ATTN_SOURCES:
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _profile_values(path):
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    return vals


def load_traffic(kernel_key, config):
    """HBM bytes per launch of `kernel_key` on workload `config` from the committed
    counter summary profiles/traffic_<kernel>_<config>.txt; None when there is no
    summary for this workload or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (kernel_key, config))
    if not os.path.exists(path):
        return None
    vals = _profile_values(path)
    if vals.get("source_digest") != source_digest() or vals.get("kernel") != kernel_key:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def load_trace_avg(kernel_key, config):
    """Average launch duration (ms) of `kernel_key` in the committed rocprofv3 kernel
    trace summary profiles/kernels_<workload>.md; None when there is none for this
    workload or it was taken on other attention sources."""
    path = os.path.join(ROOT, "profiles", "kernels_%s.md" % CONFIG_NAMES[config])
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if "digest: %s" % source_digest() not in text:
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 3 and cells[0] == kernel_key:
            try:
                return float(cells[2])
            except ValueError:
                return None
    return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def nproc():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(inp, hq, budget_s, seed):
    """The oracle, untuned, on a bounded sample of the workload's rows."""
    import numpy as np
    import oracle
    from synth_inputs import sample_tokens
    # every core this process may run on, unless OMP_NUM_THREADS sets the CPU share
    # (a machine shared by several GPUs may give each one a share of its cores so)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or nproc()
    kf = oracle._f32(inp.k)
    vf = oracle._f32(inp.v)

    def run(ntok, sseed):
        toks = sample_tokens(inp.seqlens, inp.block, ntok, seed=sseed)
        toks = np.sort(np.random.default_rng(sseed).permutation(toks)[:ntok])
        tt, hh = np.repeat(toks, hq), np.tile(np.arange(hq), len(toks))
        t0 = time.perf_counter()
        oracle.rows(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.block, inp.topk, tt, hh,
                    k_f32=kf, v_f32=vf, nthreads=threads)
        return len(toks), time.perf_counter() - t0

    # calibration: two small samples separate the fixed pooling cost from the per-token cost
    n0, t0 = run(8, seed + 100)
    n1, t1 = run(64, seed + 101)
    per_tok = max(t1 - t0, 1e-6) / max(n1 - n0, 1)
    ntok = int(max(8, min(8192, (budget_s - t0) / per_tok)))
    n, t = run(ntok, seed + 200)
    T = int(sum(inp.seqlens))
    return {"value": n / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d sampled tokens x %d q-heads of the workload (oracle fp64, pools every "
                      "block, then gate + select + attend per row); %.1f s wall" % (n, hq, t),
            "nproc": nproc(), "cpu_model": cpu_model(),
            "full_sequence_s_extrapolated": T / (n / t),
            "extrapolation": "all %d tokens at the sampled rate (linear in tokens; the "
                             "sample's rows attend as many keys on average as the workload's)"
                             % T}


def bench_decode(moba, torch, q, k, v, block, topk, steps, nseq=16):
    """Gated decode against a KV cache: the resident K/V re-read as nseq
    sequences of equal length (a multiple of the block), one new row per
    sequence (its last token), pooled keys cached beforehand. Times one decode
    call (gate, attention parts, merge) and counts the algorithmic bytes: for
    every (row, kv-head), the K and V rows of the union of keys its q-heads
    attend (own block up to the row, plus each kept block once), the pooled keys
    the gate scores, and the q and out rows."""
    import numpy as np
    T, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    L = (T // nseq) // block * block
    if L < block:
        return None
    dev = q.device
    elem = q.element_size()
    lens = [L] * nseq
    cu_k = [i * L for i in range(nseq + 1)]
    cu_q = list(range(nseq + 1))
    toks = torch.tensor([i * L + L - 1 for i in range(nseq)], device=dev)
    q_new = q[toks].contiguous()
    kc, vc = k[:nseq * L], v[:nseq * L]
    mb = L // block
    kbar = torch.zeros(nseq * mb, hkv, d, dtype=torch.float32, device=dev)
    moba.moba_kbar_append(kc, cu_k, [0] * nseq, block, mb, kbar)
    cu_q_dev = torch.tensor(cu_q, dtype=torch.int32, device=dev)
    cu_k_dev = torch.tensor(cu_k, dtype=torch.int32, device=dev)
    out = torch.empty_like(q_new)
    res = moba.moba_decode(q_new, kc, vc, cu_q, cu_k, block, topk, kbar, mb, return_sel=True,
                           cu_q_dev=cu_q_dev, cu_k_dev=cu_k_dev)
    sel = res[1].cpu().numpy()
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    for _ in range(3):
        moba.moba_decode(q_new, kc, vc, cu_q, cu_k, block, topk, kbar, mb, out=out,
                         workspace=ws, cu_q_dev=cu_q_dev, cu_k_dev=cu_k_dev)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        moba.moba_decode(q_new, kc, vc, cu_q, cu_k, block, topk, kbar, mb, out=out,
                         workspace=ws, cu_q_dev=cu_q_dev, cu_k_dev=cu_k_dev)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    p = L - 1
    own = p - (p // block) * block + 1
    i = p // block
    kv_bytes = 0
    for n in range(nseq):
        for g in range(hkv):
            blocks = set()
            for h in range(g * G, (g + 1) * G):
                blocks.update(int(j) for j in sel[n, h] if j >= 0)
            kv_bytes += (own + len(blocks) * block) * d * 2 * elem
    gate_bytes = nseq * hq * i * d * 4
    io_bytes = 2 * nseq * hq * d * elem
    total = kv_bytes + gate_bytes + io_bytes
    return {"workload": "decode_%dx%dk_last_token" % (nseq, L // 1024), "sequences": nseq,
            "cached_tokens_per_sequence": L, "new_rows_per_sequence": 1, "ms_per_step": ms,
            "tokens_per_s": nseq / (ms * 1e-3), "algorithmic_bytes": total,
            "achieved_gbs": total / (ms * 1e-3) / 1e9,
            "hbm_frac": total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bound": "hbm",
            "dense_decode_bytes": nseq * hkv * L * d * 2 * elem}


def measure_achievable(torch, dev, dtype):
    """What this machine reaches with library code, beside the datasheet peaks: dense
    matrix products (torch.mm in the workload's dtype, 8192^3 and 16384 x 16384 x
    4096, the faster counts) for the matrix cores, and a device-to-device copy of
    2 GiB (2 GiB read + 2 GiB written) for HBM. Best of several timed repetitions."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mm_tflops, mm_shape = 0.0, None
    for m, n, kk in ((8192, 8192, 8192), (16384, 16384, 4096)):
        a = torch.randn(m, kk, device=dev, dtype=torch.float32).to(dtype)
        b = torch.randn(kk, n, device=dev, dtype=torch.float32).to(dtype)
        c = torch.empty(m, n, device=dev, dtype=dtype)
        for _ in range(3):
            torch.mm(a, b, out=c)
        best = float("inf")
        for _ in range(5):
            torch.cuda.synchronize()
            e0.record()
            for _ in range(10):
                torch.mm(a, b, out=c)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 10)
        tf = 2.0 * m * n * kk / (best * 1e-3) / 1e12
        if tf > mm_tflops:
            mm_tflops, mm_shape = tf, "%dx%dx%d" % (m, n, kk)
        del a, b, c
    nbytes = 2 << 30
    src = torch.empty(nbytes // 4, device=dev, dtype=torch.float32).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(5):
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / 5)
    copy_gbs = 2.0 * nbytes / (best * 1e-3) / 1e9
    del src, dst
    return {"mfma_tflops": mm_tflops,
            "mfma_source": "torch.mm %s %s" % (str(dtype).replace("torch.", ""), mm_shape),
            "hbm_gbs": copy_gbs, "hbm_source": "device copy of 2 GiB (read + write)"}


def bench_backward(moba, torch, inp, cu_dev, attn_flop, peak_mfma, steps):
    """Backward (dq, dk, dv with the selection held fixed) after one forward that
    keeps sel and lse; inputs and the upstream gradient resident in HBM.
    Algorithmic work: the five products of the attention backward over the
    forward's attended pairs (S and dP recomputed, dQ, dK, dV), 2.5x the
    forward's two."""
    from synth_inputs import make_grad
    q, k, v = inp.q, inp.k, inp.v
    out, sel, lse = moba.moba_forward(q, k, v, inp.cu_seqlens, inp.block, inp.topk,
                                      return_sel=True, return_lse=True, cu_seqlens_dev=cu_dev)
    dout = make_grad(q.shape, q.dtype, seed=3, device=q.device)
    nbytes = moba.moba_backward_workspace_bytes(inp.cu_seqlens, q.shape[1], k.shape[1],
                                                q.shape[2], q.dtype, inp.block, inp.topk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def run():
        moba.moba_backward(q, k, v, out, lse, dout, sel, inp.cu_seqlens, inp.block, inp.topk,
                           dq=dq, dk=dk, dv=dv, workspace=ws, cu_seqlens_dev=cu_dev)

    run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(q.device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flop = 2.5 * attn_flop
    tf = flop / (ms * 1e-3) / 1e12
    del out, sel, lse, dout, ws, dq, dk, dv
    return {"ms": ms, "steps": steps, "tokens_per_s": q.shape[0] / (ms * 1e-3),
            "algorithmic_flop": flop, "achieved_tflops": tf, "mfma_frac": tf / peak_mfma}


def bench_10m_full(moba, torch, args):
    """A full-width 10M-token layer (32 q heads, 8 kv heads, D 128, block 2048,
    top-3) in the packed [T, H, D] layout, one moba_forward per step. One pass over
    all heads would need more memory than the GPU has, so the call gets the smallest
    workspace it accepts and runs the kv groups one after another inside the
    library (slab copies included in the timed step)."""
    from synth_inputs import make_10m_full
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] building inputs 10m_full", file=sys.stderr, flush=True)
    inp = make_10m_full(seed=args.seed, device=dev)
    q, k, v = inp.q, inp.k, inp.v
    T, hq, d = q.shape
    hkv = k.shape[1]
    cu_host = inp.cu_seqlens
    cu_dev = cu_host.to(dev)
    nbytes = moba.moba_workspace_bytes_min(cu_host, hq, hkv, d, q.dtype, inp.block, inp.topk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    def step():
        moba.moba_forward(q, k, v, cu_host, inp.block, inp.topk, out=out, workspace=ws,
                          cu_seqlens_dev=cu_dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    moba.moba_timing_enable(True)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    stages = moba.moba_timing_read()
    moba.moba_timing_enable(False)
    print("[bench] %d steps: %.3f ms/step" % (args.steps, ms), file=sys.stderr, flush=True)
    work = work_counts(inp.seqlens, hq, hkv, d, inp.block, inp.topk, 2)
    attn_flop = work["attn_selected_flop"] + work["attn_self_flop"]
    # every stage runs once per kv group in a step: rates from the per-step totals
    per_step = {name: (tot / args.steps, 1) for name, (tot, n) in stages.items() if n}
    rep = stage_report(per_step, work, PEAK_BF16_TFLOPS)
    for name, (tot, n) in stages.items():
        if n and name in rep:
            rep[name]["launches_per_step"] = n / args.steps
    if "slab_copy" in rep:
        # gather q, k, v of each kv group and scatter out: 2 x (q + k + v + out) bytes
        sb = 2.0 * T * (2 * hq + 2 * hkv) * d * 2
        gbs = sb / (rep["slab_copy"]["avg_ms"] * 1e-3) / 1e9
        rep["slab_copy"].update(bound="hbm", bytes_per_step=sb, achieved_gbs=gbs,
                                frac=gbs / PEAK_HBM_GBS)
    line = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V with planted needle blocks",
        "config": {"workload": CONFIG_NAMES["10m_full"], "seqlens": inp.seqlens, "tokens": T,
                   "q_heads": hq, "kv_heads": hkv, "head_dim": d,
                   "block_size": inp.block, "topk": inp.topk, "parallelism": "single GPU",
                   "layout": "packed [T, H, D]; kv groups one after another inside moba_forward",
                   "workspace_gb": nbytes / 1e9},
        "roofline": None, "cpu_baseline": None,
        "effective_attn_tflops": attn_flop / (ms * 1e-3) / 1e12,
        "attn_mfma_frac_of_step": attn_flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "gpu_memory_gb": torch.cuda.max_memory_allocated(dev) / 1e9,
        "stages": rep,
    }
    print(json.dumps(line), flush=True)


def stage_report(stages, work, peak_mfma):
    """Per-stage HIP-event averages with their rates against the roofline that
    bounds each stage."""
    rep_all = {}
    for name, (tot_ms, n) in stages.items():
        if n == 0:
            continue
        avg = tot_ms / n
        rep = {"avg_ms": avg, "launches": n}
        if name in ("attn_selected", "attn_self"):
            tf = work[name + "_flop"] / (avg * 1e-3) / 1e12
            rep.update(bound="mfma", achieved_tflops=tf, frac=tf / peak_mfma)
        elif name == "gate":
            gbs = work["gate_bytes"] / (avg * 1e-3) / 1e9
            tf = work["gate_flop"] / (avg * 1e-3) / 1e12
            # one bf16 matrix-core pass per score (the screened gate; flagged tiles
            # add three more): both the HBM and the matrix-core fraction
            rep.update(bound="hbm", achieved_gbs=gbs, frac=gbs / PEAK_HBM_GBS,
                       achieved_tflops=tf, mfma_frac=tf / PEAK_BF16_TFLOPS)
        elif name in ("pool", "route"):
            gbs = work[name + "_bytes"] / (avg * 1e-3) / 1e9
            rep.update(bound="hbm", achieved_gbs=gbs, frac=gbs / PEAK_HBM_GBS)
        rep_all[name] = rep
    return rep_all


def time_forward(moba, torch, inp, cu_dev, steps, warmup, timing=True):
    """Time `steps` moba_forward calls over the batch (after `warmup` untimed ones),
    inputs, output and workspace resident in HBM; with `timing`, also every stage's
    launches through the library's HIP events."""
    q, k, v = inp.q, inp.k, inp.v
    T, hq, d = q.shape
    hkv = k.shape[1]
    dev = q.device
    cu_host = inp.cu_seqlens
    nbytes = moba.moba_workspace_bytes(cu_host, hq, hkv, d, q.dtype, inp.block, inp.topk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    work = work_counts(inp.seqlens, hq, hkv, d, inp.block, inp.topk, q.element_size())

    def step():
        moba.moba_forward(q, k, v, cu_host, inp.block, inp.topk, out=out, workspace=ws,
                          cu_seqlens_dev=cu_dev)

    print("[bench] warmup %d" % warmup, file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if timing:
        moba.moba_timing_enable(True)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    stages = moba.moba_timing_read() if timing else {}
    moba.moba_timing_enable(False)
    print("[bench] %d steps: %.3f ms/step" % (steps, ms), file=sys.stderr, flush=True)
    del ws, out
    peak = PEAK_BF16_TFLOPS if q.dtype == torch.bfloat16 else PEAK_FP32_TFLOPS
    return {"ms": ms, "work": work, "stages": stage_report(stages, work, peak)}


def bench_merge(moba, torch, inp, cu_dev, steps, warmup, self_ms, work):
    """The merge of the parts runs inside the self-block kernel's epilogue, so it
    has no launch of its own to time. Its cost is measured as an increment: the
    same inputs through moba_forward with top-k 1 (own block only: the same
    self-block tiles and chunk form, no parts to merge) against the workload's
    own self-block time. The increment's algorithmic bytes are the parts it reads
    (D values at 2 or 4 bytes and one fp32 LSE per (row, selected slot)); the
    output store is common to both runs."""
    if inp.topk <= 1 or self_ms is None:
        return None
    own_only = type("OwnOnly", (), {})()
    for name in ("q", "k", "v", "cu_seqlens", "block", "seqlens"):
        setattr(own_only, name, getattr(inp, name))
    own_only.topk = 1
    fwd = time_forward(moba, torch, own_only, cu_dev, steps, warmup, True)
    st = fwd["stages"].get("attn_self")
    if st is None:
        return None
    inc = self_ms - st["avg_ms"]
    part_bytes = work["merge_bytes"] - inp.q.element_size() * inp.q.numel()
    res = {"self_ms_with_merge": self_ms, "self_ms_own_block_only": st["avg_ms"],
           "incremental_ms": inc, "parts_bytes": part_bytes,
           "method": "self-block kernel time at the workload's top-k minus at top-k 1 "
                     "(same inputs, HIP events on the launch stream)"}
    if inc > 0:
        gbs = part_bytes / (inc * 1e-3) / 1e9
        res.update(bound="hbm", achieved_gbs=gbs, frac=gbs / PEAK_HBM_GBS)
    return res


def bench_small_shapes(moba, torch, seed):
    """Short prefills (4K and 8K tokens, the Llama-3.1-8B-shaped layer), where the
    pages report MoBA slower than FlashAttention because of gating and routing,
    and the README's own comparison shape (32K tokens, 1 head, block 2048,
    top-3): MoBA forward and dense causal attention from the same library, each
    the median of 20 timed calls after 5 warm-ups, with MoBA's per-stage times."""
    from synth_inputs import make_inputs
    dev = torch.device("cuda:0")
    res = {}
    shapes = (("prefill_4k", [4096], 32, 8), ("prefill_8k", [8192], 32, 8),
              ("readme_32k_1head", [32768], 1, 1))
    for name, seqlens, hq, hkv in shapes:
        inp = make_inputs(seqlens, hq, hkv, 128, 2048, 3, dtype="bf16", seed=seed, device=dev)
        cu_dev = inp.cu_seqlens.to(dev)
        nbytes = moba.moba_workspace_bytes(inp.cu_seqlens, hq, hkv, 128, inp.q.dtype, 2048, 3)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        out = torch.empty_like(inp.q)

        def mo():
            moba.moba_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, 2048, 3, out=out,
                              workspace=ws, cu_seqlens_dev=cu_dev)

        def de():
            moba.moba_dense_causal_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, out=out,
                                           cu_seqlens_dev=cu_dev)

        def median_ms(fn, timing=False):
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            if timing:
                moba.moba_timing_enable(True)
            times = []
            for _ in range(20):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            st = moba.moba_timing_read() if timing else {}
            moba.moba_timing_enable(False)
            times.sort()
            return times[len(times) // 2], st

        mms, st = median_ms(mo, timing=True)
        dms, _ = median_ms(de)
        res[name] = {"tokens": sum(seqlens), "q_heads": hq, "kv_heads": hkv, "moba_ms": mms,
                     "dense_causal_ms": dms, "speedup_vs_dense": dms / mms,
                     "stages_ms": {k: t / n for k, (t, n) in st.items() if n}}
        del inp, ws, out
    torch.cuda.empty_cache()
    return res


def bench_second_workload(moba, torch, name, steps, warmup, seed, dense_steps):
    """Another workload timed like the headline one in the same run: tokens/s and
    every stage's rate, plus the dense causal comparison from the same library
    when dense_steps > 0. Used for the metric's second point (S = 128K: the packed
    varlen batch of 134,144 tokens) and for the 10M-token head share (no dense
    run there: it would take minutes)."""
    from synth_inputs import make_config
    dev = torch.device("cuda:0")
    print("[bench] second workload %s" % name, file=sys.stderr, flush=True)
    inp = make_config(name, seed=seed, device=dev)
    cu_dev = inp.cu_seqlens.to(dev)
    fwd = time_forward(moba, torch, inp, cu_dev, steps, warmup, True)
    ms, work = fwd["ms"], fwd["work"]
    T = inp.q.shape[0]
    out = torch.empty_like(inp.q)
    dms = None
    if dense_steps > 0:
        moba.moba_dense_causal_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, out=out,
                                       cu_seqlens_dev=cu_dev)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(dense_steps):
            moba.moba_dense_causal_forward(inp.q, inp.k, inp.v, inp.cu_seqlens, out=out,
                                           cu_seqlens_dev=cu_dev)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / dense_steps
    attn_flop = work["attn_selected_flop"] + work["attn_self_flop"]
    sel = fwd["stages"].get("attn_selected", {})
    res = {"workload": CONFIG_NAMES[name], "seqlens": inp.seqlens, "tokens": T,
           "steps": steps, "warmup": warmup, "ms_per_step": ms,
           "tokens_per_s": T / (ms * 1e-3),
           "effective_attn_tflops": attn_flop / (ms * 1e-3) / 1e12,
           "attn_selected_mfma_frac": sel.get("frac"),
           # HBM bytes per launch of the selected-block kernel on this workload
           # (profiles/traffic_attn_selected_<config>.txt; null when stale)
           "attn_selected_traffic": load_traffic("attn_selected", name),
           "dense_causal_ms": dms, "speedup_vs_dense": (dms / ms) if dms else None,
           "stages": fwd["stages"]}
    del inp, out
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="1m", choices=sorted(CONFIG_NAMES),
                    help="10m_full: a full-width 10M-token layer (kv groups one after "
                         "another inside moba_forward)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--dense-steps", type=int, default=1)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the gated-decode measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-merge", action="store_true",
                    help="skip the merge increment (an own-block-only forward at top-k 1)")
    ap.add_argument("--no-second", action="store_true",
                    help="skip the metric's 128K point (varlen 131K) timed after the 1M one")
    ap.add_argument("--no-10m", action="store_true",
                    help="skip the 10M-token head share timed after the 1M one")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-timing", action="store_true", help="no per-stage HIP events")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the library GEMM and copy that measure the box's reachable rates")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_causal_amd as moba
    from synth_inputs import CONFIGS, make_config

    if args.config == "10m_full":
        bench_10m_full(moba, torch, args)
        return
    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] building inputs %s" % args.config, file=sys.stderr, flush=True)
    inp = make_config(args.config, seed=args.seed, device=dev)
    q, k, v = inp.q, inp.k, inp.v
    T, hq, d = q.shape
    hkv = k.shape[1]
    cu_host = inp.cu_seqlens
    cu_dev = cu_host.to(dev)

    if args.copy_calibration_mib > 0:
        # one plain streaming kernel of known size: reads and writes N MiB of fp32
        src = torch.ones((args.copy_calibration_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    fwd = time_forward(moba, torch, inp, cu_dev, args.steps, args.warmup, not args.no_timing)
    ms, work, stage_rep = fwd["ms"], fwd["work"], fwd["stages"]
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = torch.empty_like(q)
    peak_mfma = PEAK_BF16_TFLOPS if q.dtype == torch.bfloat16 else PEAK_FP32_TFLOPS
    roofline = None
    if "attn_selected" in stage_rep:
        st = stage_rep["attn_selected"]
        traffic = load_traffic("attn_selected", args.config)
        trace_ms = load_trace_avg("attn_selected", args.config)
        roofline = {"kernel": "attn_selected", "bound": "mfma",
                    "achieved": round(st["achieved_tflops"], 2), "peak": peak_mfma,
                    "unit": "TFLOP/s", "frac": round(st["frac"], 4),
                    "traffic": traffic,
                    "avg_launch_ms": round(st["avg_ms"], 4),
                    "avg_launch_source": "HIP events on the launch stream, %d timed launches"
                                         % st["launches"],
                    "algorithmic_flop_per_launch": work["attn_selected_flop"],
                    "trace_avg_launch_ms": trace_ms,
                    "frac_from_trace": (round(work["attn_selected_flop"] / (trace_ms * 1e-3)
                                              / 1e12 / peak_mfma, 4) if trace_ms else None),
                    "trace_source": ("profiles/kernels_%s.md" % CONFIG_NAMES[args.config])
                                    if trace_ms else None}
    attn_flop = work["attn_selected_flop"] + work["attn_self_flop"]

    dense = None
    if not args.no_dense:
        print("[bench] dense causal comparison", file=sys.stderr, flush=True)
        dout = torch.empty_like(q)
        moba.moba_dense_causal_forward(q, k, v, cu_host, out=dout, cu_seqlens_dev=cu_dev)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.dense_steps):
            moba.moba_dense_causal_forward(q, k, v, cu_host, out=dout, cu_seqlens_dev=cu_dev)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.dense_steps
        dense = {"ms": dms, "tflops": work["dense_flop"] / (dms * 1e-3) / 1e12,
                 "mfma_frac": work["dense_flop"] / (dms * 1e-3) / 1e12 / peak_mfma}
        del dout

    achievable = None
    if not args.no_achievable:
        print("[bench] achievable rates (library GEMM, device copy)", file=sys.stderr, flush=True)
        achievable = measure_achievable(torch, dev, q.dtype)
        if roofline is not None:
            roofline["frac_of_achievable"] = round(roofline["achieved"] /
                                                   achievable["mfma_tflops"], 4)

    cpu = None
    if not args.no_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, hq, args.cpu_budget, args.seed)

    decode = None
    if not args.no_decode and inp.topk > 1:
        print("[bench] gated decode against a KV cache", file=sys.stderr, flush=True)
        decode = bench_decode(moba, torch, q, k, v, inp.block, inp.topk, steps=20)

    merge = None
    if not args.no_merge and not args.no_timing and "attn_self" in stage_rep:
        print("[bench] merge increment (own block only, top-k 1)", file=sys.stderr, flush=True)
        merge = bench_merge(moba, torch, inp, cu_dev, args.steps, args.warmup,
                            stage_rep["attn_self"]["avg_ms"], work)

    backward = None
    if not args.no_backward:
        print("[bench] backward", file=sys.stderr, flush=True)
        backward = bench_backward(moba, torch, inp, cu_dev, attn_flop, peak_mfma,
                                  steps=max(1, min(args.steps, 5)))

    small = None
    if not args.no_second and args.config == "1m":
        print("[bench] short prefills and the README's comparison shape", file=sys.stderr,
              flush=True)
        small = bench_small_shapes(moba, torch, args.seed)

    second = None
    if not args.no_second and args.config == "1m":
        second = bench_second_workload(moba, torch, "varlen131k", steps=max(args.steps, 10),
                                       warmup=max(args.warmup, 3), seed=args.seed,
                                       dense_steps=max(args.dense_steps, 3))

    ten_m = None
    if not args.no_10m and not args.no_second and args.config == "1m":
        ten_m = bench_second_workload(moba, torch, "10m_shard", steps=3, warmup=1,
                                      seed=args.seed, dense_steps=0)

    if achievable is not None:
        if decode is not None:
            decode["hbm_frac_of_achievable"] = decode["achieved_gbs"] / achievable["hbm_gbs"]
        if backward is not None:
            backward["mfma_frac_of_achievable"] = (backward["achieved_tflops"] /
                                                   achievable["mfma_tflops"])
    line = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if q.dtype == torch.bfloat16 else "f32",
        "data": "synthetic: seeded N(0,1) Q/K/V with planted needle blocks",
        "config": {"workload": CONFIG_NAMES[args.config], "seqlens": inp.seqlens,
                   "tokens": T, "q_heads": hq, "kv_heads": hkv, "head_dim": d,
                   "block_size": inp.block, "topk": inp.topk, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "achievable": achievable,
        "effective_attn_tflops": attn_flop / (ms * 1e-3) / 1e12,
        "attn_mfma_frac_of_step": attn_flop / (ms * 1e-3) / 1e12 / peak_mfma,
        "speedup_vs_dense": (dense["ms"] / ms) if dense else None,
        "dense_causal": dense,
        "decode": decode,
        "backward": backward,
        "stages": stage_rep,
        "merge": merge,
        "workload_128k": second,
        "workload_10m_head_share": ten_m,
        "small_shapes": small,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
