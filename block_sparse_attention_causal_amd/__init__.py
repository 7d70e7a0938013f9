"""MoBA causal prefill forward on AMD Instinct MI355X (gfx950).

A thin ctypes binding over libmoba.so, whose C ABI is include/moba.h. This
module only marshals arguments: it allocates outputs and the workspace with
torch, passes raw device pointers and torch's current stream, and turns status
codes into exceptions. Every step of the computation runs in the library's HIP
kernels. There is no fallback: if libmoba.so is missing or a call fails, an
exception is raised.

Build the library first:  python -m block_sparse_attention_causal_amd.build
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOBA_LIB selects another build of the same sources (the host-sanitizer test's)
LIB_PATH = os.environ.get("MOBA_LIB") or os.path.join(_PKG, "libmoba.so")

MOBA_OK, MOBA_ERR_INVALID_ARG, MOBA_ERR_UNSUPPORTED, MOBA_ERR_WORKSPACE, MOBA_ERR_HIP = range(5)
MOBA_DTYPE_F32, MOBA_DTYPE_BF16 = 0, 1
_DTYPE_CODE = {torch.float32: MOBA_DTYPE_F32, torch.bfloat16: MOBA_DTYPE_BF16}
STAGES = ("pool", "gate", "route", "attn_self", "attn_selected", "merge", "attn_dense", "decode",
          "kbar_append", "backward", "slab_copy")


class MobaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("MoBA call failed with status %d: %s" % (status, message))
        self.status = status


class moba_shape_t(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmoba.so is not built (%s); run "
                          "`python -m block_sparse_attention_causal_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    shp = ctypes.POINTER(moba_shape_t)
    sig = {
        "moba_abi_version": ([], i32),
        "moba_last_error": ([], ctypes.c_char_p),
        "moba_workspace_bytes": ([p, i32, shp, i32, i32], sz),
        "moba_workspace_bytes_min": ([p, i32, shp, i32, i32], sz),
        "moba_forward": ([p, p, p, p, p, i32, shp, i32, i32, p, p, sz, p, p, p], ctypes.c_int),
        "moba_forward_noalloc": ([p, p, p, p, p, i32, shp, i32, i32, p, p, p, p], ctypes.c_int),
        "moba_dense_causal_forward": ([p, p, p, p, p, i32, shp, p, p, p], ctypes.c_int),
        "moba_attention_forward": ([i32, p, p, p, p, p, i32, shp, i32, i32, p, p, sz, p, p, p],
                                   ctypes.c_int),
        "moba_block_pool": ([p, p, p, i32, shp, i32, p, p, sz, p], ctypes.c_int),
        "moba_kbar_append": ([p, p, p, p, p, i32, shp, i32, i32, p, p], ctypes.c_int),
        "moba_decode_workspace_bytes": ([p, p, i32, shp, i32, i32, i32], sz),
        "moba_decode_forward": ([p, p, p, p, p, p, p, i32, shp, i32, i32, p, i32, p, p, sz, p, p,
                                 p], ctypes.c_int),
        "moba_backward_workspace_bytes": ([p, i32, shp, i32, i32], sz),
        "moba_backward": ([p, p, p, p, p, p, p, p, p, i32, shp, i32, i32, p, p, p, p, sz, p],
                          ctypes.c_int),
        "moba_route_sizes": ([p, i32, shp, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)],
                             ctypes.c_int),
        "moba_route": ([p, p, p, i32, shp, i32, i32, p, p, p, sz, p], ctypes.c_int),
        "moba_timing_enable": ([i32], ctypes.c_int),
        "moba_timing_read": ([p, p, i32], i32),
        "moba_stage_name": ([i32], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def exported_symbols():
    """Names the binding resolves in libmoba.so (loading fails if any is missing)."""
    _load()
    return ["moba_abi_version", "moba_last_error", "moba_workspace_bytes",
            "moba_workspace_bytes_min", "moba_forward",
            "moba_forward_noalloc", "moba_dense_causal_forward", "moba_attention_forward",
            "moba_block_pool", "moba_kbar_append", "moba_decode_workspace_bytes", "moba_decode_forward",
            "moba_backward_workspace_bytes", "moba_backward", "moba_route_sizes", "moba_route",
            "moba_timing_enable", "moba_timing_read", "moba_stage_name"]


def moba_last_error() -> str:
    return _load().moba_last_error().decode()


def _check(status: int):
    if status != MOBA_OK:
        raise MobaError(status, moba_last_error())


def _shape(hq, hkv, d, dtype, scale=0.0):
    if dtype not in _DTYPE_CODE:
        raise TypeError("dtype must be float32 or bfloat16, got %s" % dtype)
    return moba_shape_t(int(hq), int(hkv), int(d), _DTYPE_CODE[dtype], float(scale))


def _cu(cu_seqlens, device, dev_copy=None):
    """(host int32 tensor, device int32 tensor) for cu_seqlens given as list/tensor;
    a device copy the caller already holds is used as it is (no copy per call)."""
    host = torch.as_tensor(cu_seqlens, dtype=torch.int32).to("cpu").contiguous()
    dev = dev_copy if dev_copy is not None else host.to(device)
    return host, dev


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_cu_total(host, T, name="cu_seqlens"):
    """The library reads T = cu_seqlens[-1] tokens of every tensor; a tensor with fewer
    rows would be read and written out of bounds, so refuse the mismatch here."""
    if host.dim() != 1 or host.numel() < 1:
        raise ValueError("%s must be a 1-D list of num_seqs + 1 offsets" % name)
    if int(host[-1]) != int(T):
        raise ValueError("%s[-1] = %d but the tensors hold %d tokens" % (name, int(host[-1]),
                                                                          int(T)))


def _check_like(name, t, ref):
    """A caller-supplied output must be a contiguous tensor shaped, typed and placed
    like the tensor it mirrors (the library writes it in full)."""
    if t is None:
        return
    if (t.device != ref.device or t.dtype != ref.dtype or tuple(t.shape) != tuple(ref.shape)
            or not t.is_contiguous()):
        raise ValueError("%s must be a contiguous %s tensor %s on %s, got %s %s on %s"
                         % (name, ref.dtype, tuple(ref.shape), ref.device, t.dtype,
                            tuple(t.shape), t.device))


def _check_kv_cache(cache, cu_host, name):
    """A KV cache must hold at least cu_k[-1] token rows (the kernels read that many)."""
    if cache.shape[0] < int(cu_host[-1]):
        raise ValueError("%s holds %d token rows, but cu_k[-1] = %d" % (name, cache.shape[0],
                                                                        int(cu_host[-1])))


def _check_kbar_cache(kbar_cache, k_cache, nseq, max_blocks):
    """The pooled-key cache: fp32, contiguous, on the cache's device, with room for
    num_seqs * max_blocks blocks of [Hkv, D]."""
    if kbar_cache is None:
        raise ValueError("kbar_cache is required")
    need = int(nseq) * int(max_blocks) * k_cache.shape[1] * k_cache.shape[2]
    if (kbar_cache.dtype != torch.float32 or kbar_cache.device != k_cache.device
            or not kbar_cache.is_contiguous()):
        raise ValueError("kbar_cache must be a contiguous fp32 tensor on %s" % k_cache.device)
    if kbar_cache.numel() < need:
        raise ValueError("kbar_cache holds %d values, needs num_seqs * max_blocks * Hkv * D = %d"
                         % (kbar_cache.numel(), need))


def _check_qkv(q, k, v, same_len=True):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous [T, H, D]" % name)
        if t.dim() != 3:
            raise ValueError("%s must be [T, H, D]" % name)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if k.shape != v.shape or (same_len and q.shape[0] != k.shape[0]) or q.shape[2] != k.shape[2]:
        raise ValueError("inconsistent q/k/v shapes %s %s %s" % (q.shape, k.shape, v.shape))


def moba_workspace_bytes(cu_seqlens, num_q_heads, num_kv_heads, head_dim, dtype, block_size,
                         topk) -> int:
    host = torch.as_tensor(cu_seqlens, dtype=torch.int32).contiguous()
    shape = _shape(num_q_heads, num_kv_heads, head_dim, dtype)
    n = _load().moba_workspace_bytes(_ptr(host), host.numel() - 1, ctypes.byref(shape),
                                     int(block_size), int(topk))
    if n == 0 and moba_last_error():
        raise MobaError(MOBA_ERR_INVALID_ARG, moba_last_error())
    return int(n)


def _check_workspace(ws, ref, nbytes):
    """A caller-supplied workspace: a contiguous GPU byte buffer on the tensors' device,
    at least nbytes long (the library also checks the size it is told)."""
    if ws is None:
        return
    if ws.device != ref.device or ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % ref.device)
    if ws.numel() < nbytes:
        raise ValueError("workspace holds %d bytes, needs %d" % (ws.numel(), nbytes))


def moba_workspace_bytes_min(cu_seqlens, num_q_heads, num_kv_heads, head_dim, dtype,
                             block_size, topk) -> int:
    """Smallest workspace moba_forward accepts (the kv-group mode's, when smaller)."""
    host = torch.as_tensor(cu_seqlens, dtype=torch.int32).contiguous()
    shape = _shape(num_q_heads, num_kv_heads, head_dim, dtype)
    n = _load().moba_workspace_bytes_min(_ptr(host), host.numel() - 1, ctypes.byref(shape),
                                         int(block_size), int(topk))
    if n == 0 and moba_last_error():
        raise MobaError(MOBA_ERR_INVALID_ARG, moba_last_error())
    return int(n)


def _workspace(nbytes, device):
    # 256-byte aligned device buffer (the caching allocator returns 512-byte aligned blocks)
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def moba_forward(q, k, v, cu_seqlens, block_size, topk, *, out=None, workspace=None,
                 return_sel=False, return_lse=False, softmax_scale=0.0, cu_seqlens_dev=None,
                 by_kv_group=False):
    """MoBA causal prefill forward: q [T,Hq,D], k/v [T,Hkv,D] (bf16 or fp32, on the GPU).

    Returns out [T,Hq,D]; with return_sel / return_lse also the selected blocks
    [T,Hq,topk-1] (int32) and the log-sum-exp [T,Hq] (fp32). A workspace smaller
    than moba_workspace_bytes (at least moba_workspace_bytes_min) runs the kv groups
    one after another; by_kv_group=True allocates that smaller workspace (it is also
    used when one pass over all heads is beyond the library's limits).
    """
    _check_qkv(q, k, v)
    dev = q.device
    T, hq, d = q.shape
    hkv = k.shape[1]
    host, cu_dev = _cu(cu_seqlens, dev, cu_seqlens_dev)
    _check_cu_total(host, T)
    _check_like("out", out, q)
    shape = _shape(hq, hkv, d, q.dtype, softmax_scale)
    lib = _load()
    nmin = lib.moba_workspace_bytes_min(_ptr(host), host.numel() - 1, ctypes.byref(shape),
                                        int(block_size), int(topk))
    if nmin == 0 and moba_last_error():
        raise MobaError(MOBA_ERR_INVALID_ARG, moba_last_error())
    _check_workspace(workspace, q, nmin)
    if workspace is None:
        nbytes = 0 if by_kv_group else lib.moba_workspace_bytes(
            _ptr(host), host.numel() - 1, ctypes.byref(shape), int(block_size), int(topk))
        workspace = _workspace(nbytes if nbytes else nmin, dev)
    if out is None:
        out = torch.empty_like(q)
    sel = torch.empty(T, hq, max(topk - 1, 0), dtype=torch.int32, device=dev) \
        if (return_sel and topk > 1) else None
    lse = torch.empty(T, hq, dtype=torch.float32, device=dev) if return_lse else None
    _check(lib.moba_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_dev), _ptr(host),
                            host.numel() - 1, ctypes.byref(shape), int(block_size), int(topk),
                            _ptr(out), _ptr(workspace), workspace.numel(), _ptr(sel), _ptr(lse),
                            _stream(dev)))
    res = [out]
    if return_sel:
        res.append(sel if sel is not None else torch.empty(T, hq, 0, dtype=torch.int32, device=dev))
    if return_lse:
        res.append(lse)
    return res[0] if len(res) == 1 else tuple(res)


def moba_forward_noalloc(q, k, v, cu_seqlens, block_size, topk, *, out=None, return_sel=False,
                         return_lse=False, softmax_scale=0.0, cu_seqlens_dev=None):
    """moba_forward with the workspace in the library's static scratch (no device
    allocation inside the call; batches whose workspace exceeds the scratch are
    refused). Same arguments and results as moba_forward, without `workspace`."""
    _check_qkv(q, k, v)
    dev = q.device
    T, hq, d = q.shape
    hkv = k.shape[1]
    host, cu_dev = _cu(cu_seqlens, dev, cu_seqlens_dev)
    _check_cu_total(host, T)
    _check_like("out", out, q)
    shape = _shape(hq, hkv, d, q.dtype, softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    sel = torch.empty(T, hq, max(topk - 1, 0), dtype=torch.int32, device=dev) \
        if (return_sel and topk > 1) else None
    lse = torch.empty(T, hq, dtype=torch.float32, device=dev) if return_lse else None
    _check(_load().moba_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_dev), _ptr(host),
                                        host.numel() - 1, ctypes.byref(shape), int(block_size),
                                        int(topk), _ptr(out), _ptr(sel), _ptr(lse),
                                        _stream(dev)))
    res = [out]
    if return_sel:
        res.append(sel if sel is not None else torch.empty(T, hq, 0, dtype=torch.int32, device=dev))
    if return_lse:
        res.append(lse)
    return res[0] if len(res) == 1 else tuple(res)


def moba_dense_causal_forward(q, k, v, cu_seqlens, *, out=None, return_lse=False,
                              softmax_scale=0.0, cu_seqlens_dev=None):
    """Dense causal attention over packed sequences (the comparison kernel)."""
    _check_qkv(q, k, v)
    dev = q.device
    T, hq, d = q.shape
    host, cu_dev = _cu(cu_seqlens, dev, cu_seqlens_dev)
    _check_cu_total(host, T)
    _check_like("out", out, q)
    shape = _shape(hq, k.shape[1], d, q.dtype, softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty(T, hq, dtype=torch.float32, device=dev) if return_lse else None
    _check(_load().moba_dense_causal_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_dev), _ptr(host),
                                             host.numel() - 1, ctypes.byref(shape), _ptr(out),
                                             _ptr(lse), _stream(dev)))
    return (out, lse) if return_lse else out


def moba_backward_workspace_bytes(cu_seqlens, num_q_heads, num_kv_heads, head_dim, dtype,
                                  block_size, topk) -> int:
    host = torch.as_tensor(cu_seqlens, dtype=torch.int32).contiguous()
    shape = _shape(num_q_heads, num_kv_heads, head_dim, dtype)
    n = _load().moba_backward_workspace_bytes(_ptr(host), host.numel() - 1, ctypes.byref(shape),
                                              int(block_size), int(topk))
    if n == 0 and moba_last_error():
        raise MobaError(MOBA_ERR_INVALID_ARG, moba_last_error())
    return int(n)


def moba_backward(q, k, v, out, lse, dout, sel, cu_seqlens, block_size, topk, *, dq=None,
                  dk=None, dv=None, workspace=None, softmax_scale=0.0, cu_seqlens_dev=None):
    """Gradients (dq, dk, dv) of moba_forward's out for the upstream gradient
    dout, with the forward's selection sel [T,Hq,topk-1] and lse [T,Hq] held
    fixed (both from moba_forward with return_sel / return_lse)."""
    _check_qkv(q, k, v)
    for name, t in (("out", out), ("dout", dout)):
        if t is None:
            raise ValueError("%s is required" % name)
        _check_like(name, t, q)
    if (lse is None or lse.dtype != torch.float32 or not lse.is_contiguous()
            or tuple(lse.shape) != tuple(q.shape[:2]) or lse.device != q.device):
        raise ValueError("lse must be a contiguous fp32 tensor [T, Hq] on q's device")
    if topk > 1 and (sel is None or sel.dtype != torch.int32 or not sel.is_contiguous()
                     or tuple(sel.shape) != (q.shape[0], q.shape[1], topk - 1)
                     or sel.device != q.device):
        raise ValueError("sel must be the forward's int32 selection [T, Hq, topk-1] on q's "
                         "device")
    dev = q.device
    T, hq, d = q.shape
    host, cu_dev = _cu(cu_seqlens, dev, cu_seqlens_dev)
    _check_cu_total(host, T)
    _check_like("dq", dq, q)
    _check_like("dk", dk, k)
    _check_like("dv", dv, v)
    shape = _shape(hq, k.shape[1], d, q.dtype, softmax_scale)
    lib = _load()
    nbytes = lib.moba_backward_workspace_bytes(_ptr(host), host.numel() - 1,
                                               ctypes.byref(shape), int(block_size), int(topk))
    if nbytes == 0 and moba_last_error():
        raise MobaError(MOBA_ERR_INVALID_ARG, moba_last_error())
    _check_workspace(workspace, q, nbytes)
    if workspace is None:
        workspace = _workspace(nbytes, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check(lib.moba_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                             _ptr(sel) if topk > 1 else None, _ptr(cu_dev), _ptr(host),
                             host.numel() - 1, ctypes.byref(shape), int(block_size), int(topk),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                             _stream(dev)))
    return dq, dk, dv


MOBA_MODE_SPARSE, MOBA_MODE_FULL = 0, 1


def moba_attention(q, k, v, cu_seqlens, block_size, topk, *, full=False, out=None,
                   workspace=None, return_lse=False, softmax_scale=0.0, cu_seqlens_dev=None):
    """One attention layer of a hybrid stack: MoBA (full=False) or full causal
    attention (full=True) through moba_attention_forward; returns out [T,Hq,D]
    (and the log-sum-exp [T,Hq] with return_lse)."""
    _check_qkv(q, k, v)
    dev = q.device
    T, hq, d = q.shape
    host, cu_dev = _cu(cu_seqlens, dev, cu_seqlens_dev)
    _check_cu_total(host, T)
    _check_like("out", out, q)
    shape = _shape(hq, k.shape[1], d, q.dtype, softmax_scale)
    lib = _load()
    mode = MOBA_MODE_FULL if full else MOBA_MODE_SPARSE
    if not full:
        nbytes = lib.moba_workspace_bytes(_ptr(host), host.numel() - 1, ctypes.byref(shape),
                                          int(block_size), int(topk))
        if nbytes == 0 and moba_last_error():
            raise MobaError(MOBA_ERR_INVALID_ARG, moba_last_error())
        _check_workspace(workspace, q, nbytes)
        if workspace is None:
            workspace = _workspace(nbytes, dev)
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty(T, hq, dtype=torch.float32, device=dev) if return_lse else None
    _check(lib.moba_attention_forward(mode, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_dev), _ptr(host),
                                      host.numel() - 1, ctypes.byref(shape), int(block_size),
                                      int(topk), _ptr(out), _ptr(workspace),
                                      workspace.numel() if workspace is not None else 0, None,
                                      _ptr(lse), _stream(dev)))
    return (out, lse) if return_lse else out


def moba_kbar_append(k_cache, cu_k, prev_len, block_size, max_blocks, kbar_cache, *,
                     cu_k_dev=None):
    """Pool into kbar_cache [num_seqs * max_blocks, Hkv, D] (fp32) the blocks of each
    sequence that became complete when its cache grew from prev_len[n] tokens."""
    if not k_cache.is_cuda or not k_cache.is_contiguous() or k_cache.dim() != 3:
        raise ValueError("k_cache must be a contiguous GPU tensor [Tk, Hkv, D]")
    dev = k_cache.device
    hkv, d = k_cache.shape[1], k_cache.shape[2]
    host, cdev = _cu(cu_k, dev, cu_k_dev)
    prev_h = torch.as_tensor(prev_len, dtype=torch.int32).to("cpu").contiguous()
    prev_d = prev_h.to(dev)
    if prev_h.numel() != host.numel() - 1:
        raise ValueError("prev_len needs one entry per sequence")
    _check_kv_cache(k_cache, host, "k_cache")
    _check_kbar_cache(kbar_cache, k_cache, host.numel() - 1, max_blocks)
    shape = _shape(hkv, hkv, d, k_cache.dtype)
    _check(_load().moba_kbar_append(_ptr(k_cache), _ptr(cdev), _ptr(host), _ptr(prev_d),
                                    _ptr(prev_h), host.numel() - 1, ctypes.byref(shape),
                                    int(block_size), int(max_blocks), _ptr(kbar_cache),
                                    _stream(dev)))
    return kbar_cache


def moba_decode(q_new, k_cache, v_cache, cu_q, cu_k, block_size, topk, kbar_cache, max_blocks,
                *, out=None, workspace=None, return_sel=False, return_lse=False,
                softmax_scale=0.0, cu_q_dev=None, cu_k_dev=None):
    """MoBA attention of new rows q_new [Tq,Hq,D] (the last tokens of their
    sequences) against the caches k_cache / v_cache [Tk,Hkv,D]. Returns out, and
    with return_sel / return_lse the kept blocks [Tq,Hq,topk-1] and lse [Tq,Hq]."""
    _check_qkv(q_new, k_cache, v_cache, same_len=False)
    dev = q_new.device
    Tq, hq, d = q_new.shape
    hkv = k_cache.shape[1]
    qh, qd = _cu(cu_q, dev, cu_q_dev)
    kh, kd = _cu(cu_k, dev, cu_k_dev)
    shape = _shape(hq, hkv, d, q_new.dtype, softmax_scale)
    lib = _load()
    nseq = qh.numel() - 1
    if kh.numel() - 1 != nseq:
        raise ValueError("cu_q and cu_k must describe the same sequences")
    _check_cu_total(qh, Tq, "cu_q")
    _check_kv_cache(k_cache, kh, "k_cache")
    _check_kv_cache(v_cache, kh, "v_cache")
    if topk > 1:
        _check_kbar_cache(kbar_cache, k_cache, nseq, max_blocks)
    _check_like("out", out, q_new)
    nbytes = lib.moba_decode_workspace_bytes(_ptr(qh), _ptr(kh), nseq, ctypes.byref(shape),
                                             int(block_size), int(topk), int(max_blocks))
    if nbytes == 0 and moba_last_error():
        raise MobaError(MOBA_ERR_INVALID_ARG, moba_last_error())
    _check_workspace(workspace, q_new, nbytes)
    if workspace is None:
        workspace = _workspace(nbytes, dev)
    if out is None:
        out = torch.empty_like(q_new)
    sel = torch.empty(Tq, hq, max(topk - 1, 0), dtype=torch.int32, device=dev) \
        if (return_sel and topk > 1) else None
    lse = torch.empty(Tq, hq, dtype=torch.float32, device=dev) if return_lse else None
    _check(lib.moba_decode_forward(_ptr(q_new), _ptr(k_cache), _ptr(v_cache), _ptr(qd), _ptr(qh),
                                   _ptr(kd), _ptr(kh), nseq, ctypes.byref(shape), int(block_size),
                                   int(topk), _ptr(kbar_cache), int(max_blocks), _ptr(out),
                                   _ptr(workspace), workspace.numel(), _ptr(sel), _ptr(lse),
                                   _stream(dev)))
    res = [out]
    if return_sel:
        res.append(sel if sel is not None else torch.empty(Tq, hq, 0, dtype=torch.int32,
                                                           device=dev))
    if return_lse:
        res.append(lse)
    return res[0] if len(res) == 1 else tuple(res)


def moba_block_pool(k, cu_seqlens, block_size):
    """Mean-pooled keys [NB, Hkv, D] (fp32) of k [T, Hkv, D]."""
    if not k.is_cuda or not k.is_contiguous() or k.dim() != 3:
        raise ValueError("k must be a contiguous GPU tensor [T, Hkv, D]")
    dev = k.device
    T, hkv, d = k.shape
    host, cu_dev = _cu(cu_seqlens, dev)
    _check_cu_total(host, T)
    shape = _shape(hkv, hkv, d, k.dtype)
    lib = _load()
    nbytes = lib.moba_workspace_bytes(_ptr(host), host.numel() - 1, ctypes.byref(shape),
                                      int(block_size), 1)
    if nbytes == 0 and moba_last_error():
        raise MobaError(MOBA_ERR_INVALID_ARG, moba_last_error())
    ws = _workspace(nbytes, dev)
    lens = (host[1:] - host[:-1]).tolist()
    nb = sum((s + block_size - 1) // block_size for s in lens)
    kbar = torch.empty(nb, hkv, d, dtype=torch.float32, device=dev)
    _check(lib.moba_block_pool(_ptr(k), _ptr(cu_dev), _ptr(host), host.numel() - 1,
                               ctypes.byref(shape), int(block_size), _ptr(kbar), _ptr(ws),
                               ws.numel(), _stream(dev)))
    return kbar


def moba_route_sizes(cu_seqlens, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk):
    host = torch.as_tensor(cu_seqlens, dtype=torch.int32).contiguous()
    shape = _shape(num_q_heads, num_kv_heads, head_dim, dtype)
    nl, ne = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_load().moba_route_sizes(_ptr(host), host.numel() - 1, ctypes.byref(shape),
                                    int(block_size), int(topk), ctypes.byref(nl),
                                    ctypes.byref(ne)))
    return int(nl.value), int(ne.value)


def moba_route(sel, cu_seqlens, num_kv_heads, head_dim, dtype, block_size, topk):
    """Routing lists of a selection map sel [T, Hq, topk-1] (int32, on the GPU).

    Returns (list_offsets [num_lists+1], entries [num_entries]), both int32 on the GPU.
    """
    if not sel.is_cuda or sel.dtype != torch.int32 or not sel.is_contiguous():
        raise ValueError("sel must be a contiguous int32 GPU tensor")
    dev = sel.device
    T, hq, _ = sel.shape
    host, cu_dev = _cu(cu_seqlens, dev)
    _check_cu_total(host, T)
    if sel.dim() != 3 or sel.shape[2] != max(int(topk) - 1, 0):
        raise ValueError("sel must be [T, Hq, topk-1]")
    shape = _shape(hq, num_kv_heads, head_dim, dtype)
    lib = _load()
    nl, ne = moba_route_sizes(host, hq, num_kv_heads, head_dim, dtype, block_size, topk)
    nbytes = lib.moba_workspace_bytes(_ptr(host), host.numel() - 1, ctypes.byref(shape),
                                      int(block_size), int(topk))
    ws = _workspace(nbytes, dev)
    offs = torch.empty(nl + 1, dtype=torch.int32, device=dev)
    ent = torch.empty(max(ne, 1), dtype=torch.int32, device=dev)
    _check(lib.moba_route(_ptr(sel), _ptr(cu_dev), _ptr(host), host.numel() - 1,
                          ctypes.byref(shape), int(block_size), int(topk), _ptr(offs), _ptr(ent),
                          _ptr(ws), ws.numel(), _stream(dev)))
    return offs, ent[:ne]


def moba_timing_enable(enable: bool = True):
    _check(_load().moba_timing_enable(1 if enable else 0))


def moba_timing_read() -> dict:
    """{stage: (total_ms, launches)} of the timed launches since the last read."""
    n = len(STAGES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    k = _load().moba_timing_read(ms, cnt, n)
    return {STAGES[i]: (ms[i], cnt[i]) for i in range(k)}


def moba_stage_name(stage: int) -> str:
    return _load().moba_stage_name(int(stage)).decode()
