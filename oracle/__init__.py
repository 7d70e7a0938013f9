"""CPU oracle for the MoBA causal prefill forward pass and its backward.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are its only users. The GPU library never
imports, links or calls it, and it imports nothing from the GPU library.

The arithmetic lives in ``moba_oracle.c`` (plain C, fp64, OpenMP over rows);
this module builds it with gcc and marshals numpy/torch CPU arrays through
ctypes. What the C code computes, step by step, and which passage of the pages
each step follows, is written at the top of ``moba_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moba_oracle.c")
# MOBA_ORACLE_LIB selects another build of the same source (the sanitizer test's)
_LIB_PATH = os.environ.get("MOBA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile moba_oracle.c into oracle/liboracle.so (gcc -O2 -fopenmp, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.moba_oracle_num_blocks.argtypes = [p, i32, i32]
    lib.moba_oracle_num_blocks.restype = i64
    lib.moba_oracle_pool.argtypes = [p, p, i32, i32, i32, i32, p]
    lib.moba_oracle_pool.restype = ctypes.c_int
    lib.moba_oracle_rows.argtypes = [p, p, p, i64, p, p, p, i32, i32, i32, i32, i32, i32,
                                     f64, p, p, p, p, i32]
    lib.moba_oracle_rows.restype = ctypes.c_int
    lib.moba_oracle_rows_given_sel.argtypes = [p, p, p, i64, p, p, p, i32, i32, i32, i32, i32,
                                               i32, p, f64, p, p, i32]
    lib.moba_oracle_rows_given_sel.restype = ctypes.c_int
    lib.moba_oracle_causal_rows.argtypes = [p, p, p, i64, p, p, p, i32, i32, i32, i32, f64,
                                            p, p, i32]
    lib.moba_oracle_causal_rows.restype = ctypes.c_int
    lib.moba_oracle_backward.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, i32, f64, p, p,
                                         p, i32]
    lib.moba_oracle_backward.restype = ctypes.c_int
    lib.moba_oracle_dq_rows.argtypes = [p, p, p, p, i64, p, p, p, i32, i32, i32, i32, i32, i32,
                                        f64, p, i32]
    lib.moba_oracle_dq_rows.restype = ctypes.c_int
    _lib = lib
    return lib


def _f32(x) -> np.ndarray:
    """Host fp32 copy of a torch tensor or array. bf16 and fp32 values are exact in fp32."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float32).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_blocks(cu_seqlens, block: int) -> int:
    cu = _i32(cu_seqlens)
    return int(_load().moba_oracle_num_blocks(_ptr(cu), len(cu) - 1, block))


def pool(k, cu_seqlens, block: int) -> np.ndarray:
    """Mean-pooled keys Kbar [NB, Hkv, D] (fp64) of k [T, Hkv, D]."""
    kf = _f32(k)
    cu = _i32(cu_seqlens)
    T, hkv, d = kf.shape
    nb = num_blocks(cu, block)
    out = np.empty((nb, hkv, d), dtype=np.float64)
    rc = _load().moba_oracle_pool(_ptr(kf), _ptr(cu), len(cu) - 1, hkv, d, block, _ptr(out))
    if rc != 0:
        raise ValueError("moba_oracle_pool failed with code %d" % rc)
    return out


def _row_queries(q, tokens, heads):
    """q is either the full [T, Hq, D] tensor or already the [n, D] rows."""
    tokens = _i32(tokens)
    heads = _i32(heads)
    if q.ndim == 3:
        if hasattr(q, "detach"):
            import torch
            t_idx = torch.as_tensor(tokens, dtype=torch.long, device=q.device)
            h_idx = torch.as_tensor(heads, dtype=torch.long, device=q.device)
            qr = _f32(q[t_idx, h_idx])
        else:
            qr = _f32(np.asarray(q)[tokens, heads])
    else:
        qr = _f32(q)
    return qr, tokens, heads


def rows(q, k, v, cu_seqlens, block: int, topk: int, tokens, heads, scale: float = 0.0,
         k_f32=None, v_f32=None, nthreads: int = 0, num_q_heads: int | None = None) -> dict:
    """MoBA forward for the given (token, head) rows, exact in fp64.

    q: [T, Hq, D] (torch or numpy, any device) or the gathered rows [n, D]; in the
    second case num_q_heads must be given.
    k, v: [T, Hkv, D]. Pre-converted fp32 host copies can be passed as k_f32/v_f32.
    Returns dict(out [n,D] f64, lse [n] f64, sel [n, topk-1] i32, margin [n] f64).
    """
    qr, tokens, heads = _row_queries(q, tokens, heads)
    kf = _f32(k) if k_f32 is None else k_f32
    vf = _f32(v) if v_f32 is None else v_f32
    cu = _i32(cu_seqlens)
    n = len(tokens)
    T, hkv, d = kf.shape
    hq = q.shape[1] if q.ndim == 3 else int(num_q_heads)
    out = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    sel = np.empty((n, max(topk - 1, 1)), dtype=np.int32)
    margin = np.empty((n,), dtype=np.float64)
    rc = _load().moba_oracle_rows(_ptr(qr), _ptr(tokens), _ptr(heads), n, _ptr(kf), _ptr(vf),
                                  _ptr(cu), len(cu) - 1, hq, hkv, d, block, topk,
                                  float(scale), _ptr(out), _ptr(lse), _ptr(sel), _ptr(margin),
                                  int(nthreads))
    if rc != 0:
        raise ValueError("moba_oracle_rows failed with code %d" % rc)
    return {"out": out, "lse": lse, "sel": sel[:, :max(topk - 1, 0)], "margin": margin}


def rows_given_sel(q, k, v, cu_seqlens, block: int, topk: int, tokens, heads, sel,
                   scale: float = 0.0, k_f32=None, v_f32=None, nthreads: int = 0,
                   num_q_heads: int | None = None) -> dict:
    """Attention of the given rows over their own-block prefix and the past blocks
    named in sel [n, topk-1] (sequence-local ids, -1 skipped) instead of the gated
    ones, exact in fp64. Raises ValueError on an id that is not a distinct past
    block of its row. Returns dict(out [n, D], lse [n])."""
    qr, tokens, heads = _row_queries(q, tokens, heads)
    kf = _f32(k) if k_f32 is None else k_f32
    vf = _f32(v) if v_f32 is None else v_f32
    cu = _i32(cu_seqlens)
    n = len(tokens)
    T, hkv, d = kf.shape
    hq = q.shape[1] if q.ndim == 3 else int(num_q_heads)
    ks = max(topk - 1, 0)
    sl = np.ascontiguousarray(_i32(sel).reshape(n, ks) if ks > 0
                              else np.zeros((n, 1), dtype=np.int32))
    out = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().moba_oracle_rows_given_sel(_ptr(qr), _ptr(tokens), _ptr(heads), n, _ptr(kf),
                                            _ptr(vf), _ptr(cu), len(cu) - 1, hq, hkv, d, block,
                                            topk, _ptr(sl), float(scale),
                                            _ptr(out), _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("moba_oracle_rows_given_sel failed with code %d" % rc)
    return {"out": out, "lse": lse}


def causal_rows(q, k, v, cu_seqlens, tokens, heads, scale: float = 0.0, k_f32=None,
                v_f32=None, nthreads: int = 0, num_q_heads: int | None = None) -> dict:
    """Plain causal attention (keys 0..t of the row's sequence) for the given rows."""
    qr, tokens, heads = _row_queries(q, tokens, heads)
    kf = _f32(k) if k_f32 is None else k_f32
    vf = _f32(v) if v_f32 is None else v_f32
    cu = _i32(cu_seqlens)
    n = len(tokens)
    T, hkv, d = kf.shape
    hq = q.shape[1] if q.ndim == 3 else int(num_q_heads)
    out = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().moba_oracle_causal_rows(_ptr(qr), _ptr(tokens), _ptr(heads), n, _ptr(kf),
                                         _ptr(vf), _ptr(cu), len(cu) - 1, hq, hkv, d,
                                         float(scale), _ptr(out), _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("moba_oracle_causal_rows failed with code %d" % rc)
    return {"out": out, "lse": lse}


def all_rows(q, k, v, cu_seqlens, block: int, topk: int, scale: float = 0.0,
             nthreads: int = 0) -> dict:
    """Full mode: every (token, head) row; results shaped [T, Hq, ...]."""
    T, hq, d = q.shape
    tokens = np.repeat(np.arange(T, dtype=np.int32), hq)
    heads = np.tile(np.arange(hq, dtype=np.int32), T)
    res = rows(q, k, v, cu_seqlens, block, topk, tokens, heads, scale=scale, nthreads=nthreads)
    return {"out": res["out"].reshape(T, hq, d), "lse": res["lse"].reshape(T, hq),
            "sel": res["sel"].reshape(T, hq, max(topk - 1, 0)),
            "margin": res["margin"].reshape(T, hq)}


def backward(q, k, v, dout, cu_seqlens, block: int, topk: int, scale: float = 0.0,
             nthreads: int = 0) -> dict:
    """Gradients of the MoBA forward with the selection held fixed, exact in fp64.

    q, dout: [T, Hq, D]; k, v: [T, Hkv, D] (torch or numpy, any device).
    Returns dict(dq [T,Hq,D], dk [T,Hkv,D], dv [T,Hkv,D]) as fp64 numpy arrays.
    """
    qf, kf, vf, gf = _f32(q), _f32(k), _f32(v), _f32(dout)
    cu = _i32(cu_seqlens)
    T, hq, d = qf.shape
    hkv = kf.shape[1]
    dq = np.empty((T, hq, d), dtype=np.float64)
    dk = np.empty((T, hkv, d), dtype=np.float64)
    dv = np.empty((T, hkv, d), dtype=np.float64)
    rc = _load().moba_oracle_backward(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(gf), _ptr(cu),
                                      len(cu) - 1, hq, hkv, d, block, topk, float(scale),
                                      _ptr(dq), _ptr(dk), _ptr(dv), int(nthreads))
    if rc != 0:
        raise ValueError("moba_oracle_backward failed with code %d" % rc)
    return {"dq": dq, "dk": dk, "dv": dv}


def dq_rows(q, k, v, dout, cu_seqlens, block: int, topk: int, tokens, heads,
            scale: float = 0.0, k_f32=None, v_f32=None, nthreads: int = 0) -> np.ndarray:
    """dq of the given (token, head) rows only, exact in fp64 ([n, D]); q and
    dout are the full [T, Hq, D] tensors (any device), k/v as in rows()."""
    qr, tokens, heads = _row_queries(q, tokens, heads)
    gr, _, _ = _row_queries(dout, tokens, heads)
    kf = _f32(k) if k_f32 is None else k_f32
    vf = _f32(v) if v_f32 is None else v_f32
    cu = _i32(cu_seqlens)
    n = len(tokens)
    T, hkv, d = kf.shape
    dq = np.empty((n, d), dtype=np.float64)
    rc = _load().moba_oracle_dq_rows(_ptr(qr), _ptr(gr), _ptr(tokens), _ptr(heads), n, _ptr(kf),
                                     _ptr(vf), _ptr(cu), len(cu) - 1, q.shape[1], hkv, d, block,
                                     topk, float(scale), _ptr(dq), int(nthreads))
    if rc != 0:
        raise ValueError("moba_oracle_dq_rows failed with code %d" % rc)
    return dq
