"""CPU checks of the C ABI: the library loads, exports every function that
include/moba.h declares, and rejects bad arguments on the host before any
launch. No call here reaches a kernel."""
import ctypes
import os
import re

import pytest
import torch

import block_sparse_attention_causal_amd as moba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moba.h")

FAKE = ctypes.c_void_p(0x10000000)   # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moba.LIB_PATH):
        from block_sparse_attention_causal_amd import build
        build.build()
    return moba._load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moba_[a-z_]+)\s*\(", text)))


def test_header_declares_the_core_calls():
    names = declared_functions()
    for n in ("moba_forward", "moba_workspace_bytes", "moba_dense_causal_forward",
              "moba_last_error", "moba_block_pool", "moba_route"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(moba.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert set(declared_functions()) == set(moba.exported_symbols())
    assert lib.moba_abi_version() == 1


def _shape(hq=32, hkv=8, d=128, dtype=1, scale=0.0):
    return moba.moba_shape_t(hq, hkv, d, dtype, scale)


def _cu(lens):
    cu = [0]
    for s in lens:
        cu.append(cu[-1] + s)
    return torch.tensor(cu, dtype=torch.int32)


def _fwd(lib, cu, shape, block, topk, ws_bytes=1 << 40, ws=FAKE):
    return lib.moba_forward(FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(cu.data_ptr()),
                            cu.numel() - 1, ctypes.byref(shape), block, topk, FAKE, ws, ws_bytes,
                            None, None, None)


@pytest.mark.parametrize("kw,block,topk,code", [
    (dict(hq=6, hkv=4), 2048, 3, moba.MOBA_ERR_INVALID_ARG),
    (dict(hq=0), 2048, 3, moba.MOBA_ERR_INVALID_ARG),
    (dict(d=96), 2048, 3, moba.MOBA_ERR_UNSUPPORTED),
    (dict(dtype=7), 2048, 3, moba.MOBA_ERR_UNSUPPORTED),
    (dict(), 100, 3, moba.MOBA_ERR_UNSUPPORTED),
    (dict(), 0, 3, moba.MOBA_ERR_INVALID_ARG),
    (dict(), 2048, 0, moba.MOBA_ERR_INVALID_ARG),
    (dict(), 2048, 18, moba.MOBA_ERR_UNSUPPORTED),
])
def test_invalid_shapes_are_rejected(lib, kw, block, topk, code):
    st = _fwd(lib, _cu([4096]), _shape(**kw), block, topk)
    assert st == code
    assert lib.moba_last_error().decode() != ""


def test_bad_cu_seqlens(lib):
    bad = torch.tensor([0, 100, 50], dtype=torch.int32)
    assert _fwd(lib, bad, _shape(), 64, 3) == moba.MOBA_ERR_INVALID_ARG
    bad0 = torch.tensor([5, 100], dtype=torch.int32)
    assert _fwd(lib, bad0, _shape(), 64, 3) == moba.MOBA_ERR_INVALID_ARG


def test_workspace_checks(lib):
    cu = _cu([4096])
    assert _fwd(lib, cu, _shape(), 2048, 3, ws_bytes=1000) == moba.MOBA_ERR_WORKSPACE
    assert _fwd(lib, cu, _shape(), 2048, 3, ws=ctypes.c_void_p(0x10000010)) == \
        moba.MOBA_ERR_INVALID_ARG
    assert _fwd(lib, cu, _shape(), 2048, 3, ws=None) == moba.MOBA_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op(lib):
    cu = torch.tensor([0, 0, 0], dtype=torch.int32)
    assert _fwd(lib, cu, _shape(), 2048, 3, ws_bytes=0, ws=None) == moba.MOBA_OK


def test_workspace_bytes_and_route_sizes(lib):
    n = moba.moba_workspace_bytes([0, 32768], 32, 8, 128, torch.bfloat16, 2048, 3)
    T, rows = 32768, 32768 * 32
    # the partial outputs dominate: topk-1 selected-block parts per row (the
    # self-block kernel merges them into out), fp16 for bf16 inputs
    assert n >= rows * 128 * 2 * 2
    assert moba.moba_workspace_bytes([0, 32768], 32, 8, 128, torch.float32, 2048, 3) >= \
        rows * 128 * 4 * 2
    nl, ne = moba.moba_route_sizes([0, 32768], 32, 8, 128, torch.bfloat16, 2048, 3)
    assert nl == 16 * 8
    assert ne == sum(2048 * 32 * min(2, i) for i in range(16))
    # block-diagonal attention needs no routing buffers
    assert moba.moba_workspace_bytes([0, T], 32, 8, 128, torch.bfloat16, 2048, 1) < n
    with pytest.raises(moba.MobaError):
        moba.moba_workspace_bytes([0, T], 32, 8, 128, torch.bfloat16, 100, 3)


def test_route_requires_topk_two(lib):
    cu = _cu([1024])
    st = lib.moba_route(FAKE, FAKE, ctypes.c_void_p(cu.data_ptr()), 1, ctypes.byref(_shape()), 64,
                        1, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == moba.MOBA_ERR_INVALID_ARG


def test_stage_names(lib):
    assert [moba.moba_stage_name(i) for i in range(len(moba.STAGES))] == list(moba.STAGES)
    assert moba.moba_stage_name(len(moba.STAGES)) == ""
    assert moba.moba_stage_name(99) == ""


def test_binding_refuses_cpu_tensors():
    q = torch.zeros(64, 2, 64)
    with pytest.raises(ValueError):
        moba.moba_forward(q, q, q, [0, 64], 64, 3)


def _attn(lib, mode, cu, shape, block, topk, ws_bytes=1 << 40, ws=FAKE):
    return lib.moba_attention_forward(mode, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(cu.data_ptr()),
                                      cu.numel() - 1, ctypes.byref(shape), block, topk, FAKE, ws,
                                      ws_bytes, None, None, None)


def test_hybrid_switch_validates_mode_and_routes_arguments(lib):
    cu = _cu([4096])
    for mode in (-1, 2, 7):
        assert _attn(lib, mode, cu, _shape(), 2048, 3) == moba.MOBA_ERR_INVALID_ARG
        assert "mode" in lib.moba_last_error().decode()
    # sparse mode checks MoBA's own arguments (block size, top-k, workspace) ...
    assert _attn(lib, moba.MOBA_MODE_SPARSE, cu, _shape(), 100, 3) == moba.MOBA_ERR_UNSUPPORTED
    assert _attn(lib, moba.MOBA_MODE_SPARSE, cu, _shape(), 2048, 3, ws_bytes=10) == \
        moba.MOBA_ERR_WORKSPACE
    # ... full mode ignores them but still validates the shape
    assert _attn(lib, moba.MOBA_MODE_FULL, cu, _shape(d=96), 0, 0, ws=None) == \
        moba.MOBA_ERR_UNSUPPORTED


def _dec(lib, cu_q, cu_k, shape, block, topk, max_blocks, ws_bytes=1 << 40, ws=FAKE, kbar=FAKE):
    return lib.moba_decode_forward(FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(cu_q.data_ptr()), FAKE,
                                   ctypes.c_void_p(cu_k.data_ptr()), cu_q.numel() - 1,
                                   ctypes.byref(shape), block, topk, kbar, max_blocks, FAKE, ws,
                                   ws_bytes, None, None, None)


def test_decode_validation(lib):
    cu_k, cu_q = _cu([5000, 3000]), _cu([1, 1])
    # cache longer than max_blocks * block_size
    assert _dec(lib, cu_q, cu_k, _shape(), 2048, 3, 2) == moba.MOBA_ERR_INVALID_ARG
    # more new rows than cached tokens
    assert _dec(lib, _cu([1, 4000]), cu_k, _shape(), 2048, 3, 3) == moba.MOBA_ERR_INVALID_ARG
    assert _dec(lib, cu_q, cu_k, _shape(), 100, 3, 64) == moba.MOBA_ERR_UNSUPPORTED
    assert _dec(lib, cu_q, cu_k, _shape(d=96), 2048, 3, 3) == moba.MOBA_ERR_UNSUPPORTED
    assert _dec(lib, cu_q, cu_k, _shape(), 2048, 3, 3, ws_bytes=16) == moba.MOBA_ERR_WORKSPACE
    assert _dec(lib, cu_q, cu_k, _shape(), 2048, 3, 3, kbar=None) == moba.MOBA_ERR_INVALID_ARG
    # no new rows is a no-op
    assert _dec(lib, _cu([0, 0]), cu_k, _shape(), 2048, 3, 3, ws=None) == moba.MOBA_OK


def test_decode_workspace_scales_with_new_rows(lib):
    shp = _shape()
    q1, q64, k = _cu([1]), _cu([64]), _cu([32768])   # kept alive across the calls
    one = lib.moba_decode_workspace_bytes(ctypes.c_void_p(q1.data_ptr()),
                                          ctypes.c_void_p(k.data_ptr()), 1, ctypes.byref(shp),
                                          2048, 3, 16)
    many = lib.moba_decode_workspace_bytes(ctypes.c_void_p(q64.data_ptr()),
                                           ctypes.c_void_p(k.data_ptr()), 1, ctypes.byref(shp),
                                           2048, 3, 16)
    # per row-head: 3 parts x 4 segments of 128 fp32 values + lse, and 2 kept ids
    assert one >= 32 * (3 * 4 * (128 * 4 + 4) + 2 * 4)
    assert many >= 64 * 32 * (3 * 4 * (128 * 4 + 4))


def test_kbar_append_validation(lib):
    cu_k = _cu([5000, 300])
    prev = torch.tensor([0, 400], dtype=torch.int32)     # 400 > 300 cached tokens
    st = lib.moba_kbar_append(FAKE, FAKE, ctypes.c_void_p(cu_k.data_ptr()), FAKE,
                              ctypes.c_void_p(prev.data_ptr()), 2, ctypes.byref(_shape()), 2048,
                              3, FAKE, None)
    assert st == moba.MOBA_ERR_INVALID_ARG
    ok = torch.tensor([5000, 300], dtype=torch.int32)    # nothing new to pool: a no-op
    st = lib.moba_kbar_append(None, None, ctypes.c_void_p(cu_k.data_ptr()), None,
                              ctypes.c_void_p(ok.data_ptr()), 2, ctypes.byref(_shape()), 2048,
                              3, None, None)
    assert st == moba.MOBA_OK


def _bwd(lib, cu, shape, block, topk, ws_bytes=1 << 40, ws=FAKE, sel=FAKE, dq=FAKE):
    return lib.moba_backward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, sel, FAKE,
                             ctypes.c_void_p(cu.data_ptr()), cu.numel() - 1, ctypes.byref(shape),
                             block, topk, dq, FAKE, FAKE, ws, ws_bytes, None)


def test_backward_validation(lib):
    cu = _cu([4096, 1000])
    assert _bwd(lib, cu, _shape(d=96), 2048, 3) == moba.MOBA_ERR_UNSUPPORTED
    assert _bwd(lib, cu, _shape(), 100, 3) == moba.MOBA_ERR_UNSUPPORTED
    assert _bwd(lib, cu, _shape(hq=6, hkv=4), 2048, 3) == moba.MOBA_ERR_INVALID_ARG
    assert _bwd(lib, cu, _shape(), 2048, 3, sel=None) == moba.MOBA_ERR_INVALID_ARG
    assert _bwd(lib, cu, _shape(), 2048, 3, dq=None) == moba.MOBA_ERR_INVALID_ARG
    assert _bwd(lib, cu, _shape(), 2048, 3, ws_bytes=1000) == moba.MOBA_ERR_WORKSPACE
    assert _bwd(lib, cu, _shape(), 2048, 3, ws=ctypes.c_void_p(0x10000010)) == \
        moba.MOBA_ERR_INVALID_ARG
    # topk == 1 needs no selection
    st = _bwd(lib, cu, _shape(), 2048, 1, sel=None, ws_bytes=0, ws=None)
    assert st == moba.MOBA_ERR_INVALID_ARG and "workspace" in lib.moba_last_error().decode()
    # an empty batch is a no-op
    assert _bwd(lib, _cu([0]), _shape(), 2048, 3, ws=None, sel=None) == moba.MOBA_OK


def test_backward_workspace_holds_dq_parts_and_delta(lib):
    shp = _shape()
    cu = _cu([32768])
    n = lib.moba_backward_workspace_bytes(ctypes.c_void_p(cu.data_ptr()), 1, ctypes.byref(shp),
                                          2048, 3)
    rows = 32768 * 32
    # fp32 dQ parts for every (row, slot) and Delta per row
    assert n >= rows * 2 * 128 * 4 + rows * 4
    assert n >= moba.moba_workspace_bytes([0, 32768], 32, 8, 128, torch.bfloat16, 2048, 3) - \
        rows * 2 * 128 * 2


def test_profiling_kernel_keys():
    from block_sparse_attention_causal_amd.profiling import kernel_key
    names = {
        "_ZN4moba6k_attnIDF16bLi128ELi1EEEvNS_8AttnArgsE": "attn_selected",
        "_ZN4moba6k_attnIDF16bLi128ELi0EEEvNS_8AttnArgsE": "attn_self",
        "_ZN4moba6k_attnIDF16bLi128ELi2EEEvNS_8AttnArgsE": "attn_dense",
        "_ZN4moba6k_gateIDF16bLi128ELi3ELi2EEEvPKT_PKiS5_S5_S5_S3_liiiiillPKhPi": "gate",
        "_ZN4moba11k_gate_fastILi128ELi2EEEvPKDF16bPKiS4_S4_S4_S2_PKfliiiiillPhPi": "gate_fast",
        "_ZN4moba11k_gate_fastILi128ELi2ELb1EEEvPKDF16bPKiS4_S4_S4_S2_PKfliiiiillPhPi": "gate_fast",
        "moba::k_gate_bound(int const*, float const*, int, float*)": "gate_bound",
        "void moba::k_bwd_dq_dma<1>(moba::BwdArgs)": "bwd_dq_selected",
        "void moba::k_bwd_dq_dma<0>(moba::BwdArgs)": "bwd_dq_self",
        "moba::k_bwd_dkdv_dma(moba::BwdArgs)": "bwd_dkdv",
        "_ZN4moba7k_attn4ILi1EEEvNS_8AttnArgsE": "attn_selected",
        "_ZN4moba7k_attn4ILi0EEEvNS_8AttnArgsE": "attn_self",
        "void moba::k_attn4<1>(moba::AttnArgs)": "attn_selected",
        "void moba::k_attn4<0>(moba::AttnArgs)": "attn_self",
        "_ZN4moba7k_attn4ILi1ELi32EEEvNS_8AttnArgsE": "attn_selected",
        "_ZN4moba7k_attn4ILi0ELi64EEEvNS_8AttnArgsE": "attn_self",
        "void moba::k_attn4<1, 32>(moba::AttnArgs)": "attn_selected",
        "void moba::k_attn4<0, 32>(moba::AttnArgs)": "attn_self",
        "void moba::k_attn4<0, 64>(moba::AttnArgs)": "attn_self",
        "_ZN4moba10k_dec_partIDF16bLi128EEEvNS_10DecodeArgsE": "decode_part",
        "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel": "copy_calibration",
    }
    for name, key in names.items():
        assert kernel_key(name) == key, name


def test_bench_work_counts_closed_forms():
    """The benchmark's algorithmic work against closed forms for one sequence of
    nb full blocks: own-block pairs nb*B(B+1)/2, selected pairs
    B^2 (ks nb - ks(ks+1)/2), gate pairs B nb(nb-1)/2 (per head)."""
    import bench
    B, nb, ks, hq, hkv, d = 2048, 512, 2, 32, 8, 128
    w = bench.work_counts([nb * B], hq, hkv, d, B, ks + 1, 2)
    self_pairs = nb * B * (B + 1) // 2
    sel_pairs = B * B * (ks * nb - ks * (ks + 1) // 2)
    gate_pairs = B * nb * (nb - 1) // 2
    assert w["attn_self_flop"] == 4.0 * d * hq * self_pairs
    assert w["attn_selected_flop"] == 4.0 * d * hq * sel_pairs
    assert w["gate_flop"] == 2.0 * d * hq * gate_pairs
    # the 1M workload's figures: 17.6 + 70.2 TFLOP of attention, 2.19 TFLOP of gate
    assert abs(w["attn_self_flop"] / 1e12 - 17.60) < 0.01
    assert abs(w["attn_selected_flop"] / 1e12 - 70.16) < 0.01
    assert abs(w["gate_flop"] / 1e12 - 2.19) < 0.01
    # route bytes: 12 per routed (row, slot); 1M: 0.803 GB
    assert w["route_bytes"] == 12.0 * hq * B * (ks * nb - ks * (ks + 1) // 2)
    assert abs(w["route_bytes"] / 1e9 - 0.803) < 0.001


def test_bench_merge_increment_bytes():
    """The merge increment's algorithmic bytes are the selected parts alone (D fp16
    values and one fp32 LSE per (row, selected slot)), closed form for one
    sequence of nb full blocks: hq B (ks nb - ks(ks+1)/2) (2 D + 4); 17.4 GB at
    1M. The own-block-only run is asked for at top-k 1 on the same inputs, and
    the rate is those bytes over the time difference."""
    import types
    import bench
    B, nb, ks, hq, hkv, d = 2048, 512, 2, 32, 8, 128
    T = nb * B
    w = bench.work_counts([T], hq, hkv, d, B, ks + 1, 2)
    # q: the workload's element count, as an expanded view of one element
    q = torch.zeros(1, dtype=torch.bfloat16).expand(T * hq * d)
    inp = types.SimpleNamespace(q=q, k=None, v=None, cu_seqlens=None, block=B, seqlens=[T],
                                topk=ks + 1)
    seen = {}

    def fake_time_forward(moba, torch_, own, cu_dev, steps, warmup, timing):
        seen["topk"], seen["block"], seen["seqlens"] = own.topk, own.block, own.seqlens
        return {"stages": {"attn_self": {"avg_ms": 18.0}}}

    real = bench.time_forward
    bench.time_forward = fake_time_forward
    try:
        m = bench.bench_merge(None, torch, inp, None, 2, 1, 20.0, w)
    finally:
        bench.time_forward = real
    assert seen == {"topk": 1, "block": B, "seqlens": [T]}
    parts = hq * B * (ks * nb - ks * (ks + 1) // 2) * (2 * d + 4)
    assert m["parts_bytes"] == parts
    assert abs(parts / 1e9 - 17.40) < 0.01
    assert abs(m["incremental_ms"] - 2.0) < 1e-12
    assert abs(m["achieved_gbs"] - parts / 2e-3 / 1e9) < 1e-6
    # no increment to measure at top-k 1
    inp.topk = 1
    assert bench.bench_merge(None, torch, inp, None, 2, 1, 20.0, w) is None


def test_bench_refuses_several_gpus():
    import subprocess
    import sys as _sys
    r = subprocess.run([_sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _write_counter_csv(path, rows):
    import csv
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_profiling_copy_calibration_sums_split_launches(tmp_path):
    """torch runs a copy whose byte offsets overflow 32 bits as several launches: the
    calibration must total them, else the scale factors come out twice too large."""
    from block_sparse_attention_causal_amd import profiling
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda"
    sel = "void moba::k_attn4<1>(moba::AttnArgs)"
    gib = 1 << 30
    fdir, wdir = str(tmp_path / "f"), str(tmp_path / "w")
    # a 4 GiB copy in two launches; FETCH_SIZE reads half the bytes, WRITE_SIZE all (KiB)
    _write_counter_csv(fdir, [(1, neg, "FETCH_SIZE", gib / 1024), (2, neg, "FETCH_SIZE", gib / 1024),
                              (3, sel, "FETCH_SIZE", 3 * gib / 1024)])
    _write_counter_csv(wdir, [(1, neg, "WRITE_SIZE", 2 * gib / 1024),
                              (2, neg, "WRITE_SIZE", 2 * gib / 1024),
                              (3, sel, "WRITE_SIZE", 5 * gib / 1024)])
    out = dict(l.split(": ", 1) for l in profiling.traffic(fdir, wdir, 4096, "attn_selected")
               .splitlines())
    assert float(out["fetch_scale"]) == 2.0 and float(out["write_scale"]) == 1.0
    assert abs(float(out["hbm_bytes_per_launch"]) / ((6 + 5) * gib) - 1) < 1e-5
    ddir = str(tmp_path / "d")
    _write_counter_csv(ddir, [(1, neg, profiling.DRAM_READ, gib / 16), (2, neg, profiling.DRAM_READ, gib / 16),
                              (1, neg, profiling.DRAM_WRITE, gib / 16), (2, neg, profiling.DRAM_WRITE, gib / 16),
                              (3, sel, profiling.DRAM_READ, 1e9 / 32), (3, sel, profiling.DRAM_WRITE, 2e9 / 32)])
    txt = profiling.dram(ddir, 4096)
    assert "copy_read_bytes: 4.29497e+09 (ratio 1.0000)" in txt
    assert "| attn_selected | 1 | 1.0000 | 2.0000 |" in txt


def _noalloc(lib, cu, shape, block, topk, ptr=FAKE):
    return lib.moba_forward_noalloc(ptr, ptr, ptr, ptr, ctypes.c_void_p(cu.data_ptr()),
                                    cu.numel() - 1, ctypes.byref(shape), block, topk, ptr, None,
                                    None, None)


def test_noalloc_refuses_batches_beyond_its_scratch(lib):
    """The no-allocation forward takes its workspace from a 256 MiB static array:
    a batch needing more is refused on the host, before any HIP call."""
    limit = 256 << 20
    big = _cu([1 << 20])                                   # the 1M-token workload
    assert moba.moba_workspace_bytes(big, 32, 8, 128, torch.bfloat16, 2048, 3) > limit
    assert _noalloc(lib, big, _shape(), 2048, 3) == moba.MOBA_ERR_WORKSPACE
    assert "scratch" in lib.moba_last_error().decode()
    small = _cu([4096, 1000])
    assert moba.moba_workspace_bytes(small, 32, 8, 128, torch.bfloat16, 2048, 3) <= limit
    # within the limit, the pointers are checked next (still no HIP call)
    assert _noalloc(lib, small, _shape(), 2048, 3, ptr=None) == moba.MOBA_ERR_INVALID_ARG
    # shape errors as moba_forward's
    assert _noalloc(lib, small, _shape(d=96), 2048, 3) == moba.MOBA_ERR_UNSUPPORTED
    assert _noalloc(lib, torch.tensor([0, 100, 50], dtype=torch.int32), _shape(), 64, 3) == \
        moba.MOBA_ERR_INVALID_ARG
    # an empty batch is a no-op
    assert _noalloc(lib, _cu([0]), _shape(), 2048, 3, ptr=None) == moba.MOBA_OK


def test_binding_argument_checks():
    """The binding's host checks that keep a call from reading or writing past a
    tensor: cu_seqlens must end at the tensors' token count, caller outputs must
    mirror their inputs, caches must hold the tokens cu_k names, the pooled-key
    cache must hold num_seqs * max_blocks blocks, and a workspace must be a byte
    buffer on the right device of the needed size."""
    q = torch.zeros(100, 4, 64)
    moba._check_cu_total(torch.tensor([0, 40, 100], dtype=torch.int32), 100)
    with pytest.raises(ValueError, match="cu_seqlens"):
        moba._check_cu_total(torch.tensor([0, 40, 120], dtype=torch.int32), 100)
    with pytest.raises(ValueError, match="cu_seqlens"):
        moba._check_cu_total(torch.tensor([0, 40], dtype=torch.int32), 100)
    moba._check_like("out", None, q)
    moba._check_like("out", torch.empty_like(q), q)
    for bad in (torch.zeros(99, 4, 64), torch.zeros(100, 4, 64, dtype=torch.bfloat16),
                torch.zeros(100, 64, 4).transpose(1, 2)):
        with pytest.raises(ValueError, match="out"):
            moba._check_like("out", bad, q)
    kc = torch.zeros(300, 2, 64)
    moba._check_kv_cache(kc, torch.tensor([0, 100, 300], dtype=torch.int32), "k_cache")
    with pytest.raises(ValueError, match="k_cache"):
        moba._check_kv_cache(kc, torch.tensor([0, 100, 301], dtype=torch.int32), "k_cache")
    moba._check_kbar_cache(torch.zeros(2 * 5, 2, 64), kc, 2, 5)
    with pytest.raises(ValueError, match="kbar_cache"):
        moba._check_kbar_cache(torch.zeros(2 * 5 - 1, 2, 64), kc, 2, 5)
    with pytest.raises(ValueError, match="kbar_cache"):
        moba._check_kbar_cache(torch.zeros(10, 2, 64, dtype=torch.float64), kc, 2, 5)
    moba._check_workspace(torch.zeros(1000, dtype=torch.uint8), q, 1000)
    with pytest.raises(ValueError, match="workspace"):
        moba._check_workspace(torch.zeros(999, dtype=torch.uint8), q, 1000)
    with pytest.raises(ValueError, match="workspace"):
        moba._check_workspace(torch.zeros(1000, dtype=torch.float32), q, 1000)


def test_workspace_bytes_min_runs_by_kv_group():
    """The smallest workspace moba_forward takes: one kv group's buffers plus the
    slabs, when that is smaller than one pass over all heads; a batch beyond the
    one-pass int32 limits (8M tokens x 32 heads with top-12: T Hq (topk-1) >= 2^31)
    still has one."""
    bf = torch.bfloat16
    full = moba.moba_workspace_bytes([0, 32768], 32, 8, 128, bf, 2048, 3)
    small = moba.moba_workspace_bytes_min([0, 32768], 32, 8, 128, bf, 2048, 3)
    assert small < full / 2
    # one kv head: nothing to split
    assert moba.moba_workspace_bytes_min([0, 32768], 4, 1, 128, bf, 2048, 3) == \
        moba.moba_workspace_bytes([0, 32768], 4, 1, 128, bf, 2048, 3)
    # own block only: no selected parts, one pass is the smaller
    assert moba.moba_workspace_bytes_min([0, 32768], 32, 8, 128, bf, 2048, 1) == \
        moba.moba_workspace_bytes([0, 32768], 32, 8, 128, bf, 2048, 1)
    T = 8 * 2 ** 20
    with pytest.raises(moba.MobaError):
        moba.moba_workspace_bytes([0, T], 32, 8, 128, bf, 512, 12)
    assert moba.moba_workspace_bytes_min([0, T], 32, 8, 128, bf, 512, 12) > 0
    # below the minimum: refused, both sizes named
    lib = moba._load()
    cu = _cu([32768])
    st = _fwd(lib, cu, _shape(), 2048, 3, ws_bytes=small - 1)
    assert st == moba.MOBA_ERR_WORKSPACE
    assert "kv group" in lib.moba_last_error().decode()
