"""Plain fp64 CPU oracle for decode attention (MLA absorbed form and GQA/MQA/MHA).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It never imports
the HIP library package and shares no code with it. The arithmetic lives in
``oracle.c`` (plain loops, double precision, OpenMP over query rows); this file
only compiles it with gcc and marshals numpy arrays through ctypes.

Inputs are raw bf16 bit patterns (``numpy.uint16``); each is widened to double
exactly. Outputs are float64.

Definitions followed (see ``oracle.c`` for the per-function citations):
  * "Mla Analysis" skill page, "Absorption Trick (FlashMLA)" and "Tensor Shapes":
    latent scores Qz.Z^T plus the decoupled rope part, output softmax.Z.
  * "Why MLA and MTP Fight Each Other", variant table in the introduction, and
    "MQA, GQA & MLA" lesson, Concept section: query-head groups share K/V heads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int
            lib.oracle_mla.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_double, P,
                                       ctypes.c_int64, P, P, P, I]
            lib.oracle_mla.restype = I
            lib.oracle_gqa.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_double, P,
                                       ctypes.c_int64, P, P, P, I]
            lib.oracle_gqa.restype = I
            lib.oracle_attn_generic.argtypes = [P, P, P, P, I, I, I, I, ctypes.c_double, P, P]
            lib.oracle_attn_generic.restype = I
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = I
            _lib = lib
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _bits(a) -> np.ndarray:
    """Accept numpy uint16/int16 or a torch bf16 CPU tensor; return contiguous uint16 bits."""
    if hasattr(a, "view") and hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch  # local: only when handed torch tensors
        a = a.contiguous().view(torch.int16).numpy()
    a = np.ascontiguousarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs must be raw bf16 bits (uint16), got %s" % a.dtype)
    return a


def _i32(a) -> np.ndarray:
    if hasattr(a, "numpy"):
        a = a.cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _rows(rows):
    if rows is None:
        return None
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def mla(q_lat, q_rope, cache, seqlens, scale, rows=None, threads=0, return_macs=False):
    """MLA absorbed decode in fp64.

    q_lat [b,s,h,k], q_rope [b,s,h,p], cache [b,t_max,k+p] (latent then rope
    columns), seqlens [b]. Returns out [b,s,h,k] and lse [b,s,h] (float64), or,
    with ``rows`` (flattened (b,s,h) indices), out [n,k] and lse [n].
    """
    ql, qr, c = _bits(q_lat), _bits(q_rope), _bits(cache)
    b, s, h, k = ql.shape
    p = qr.shape[3]
    t_max = c.shape[1]
    assert qr.shape == (b, s, h, p) and c.shape == (b, t_max, k + p)
    sl = _i32(seqlens)
    assert sl.shape == (b,)
    rr = _rows(rows)
    n = b * s * h if rr is None else rr.shape[0]
    out = np.empty((n, k), np.float64)
    lse = np.empty((n,), np.float64)
    macs = ctypes.c_int64(0)
    rc = _load().oracle_mla(_ptr(ql), _ptr(qr), _ptr(c), _ptr(sl), b, s, h, k, p, t_max,
                            float(scale), _ptr(rr), n, _ptr(out), _ptr(lse),
                            ctypes.byref(macs), int(threads))
    if rc != 0:
        raise ValueError("oracle_mla rejected its arguments")
    if rr is None:
        out, lse = out.reshape(b, s, h, k), lse.reshape(b, s, h)
    return (out, lse, macs.value) if return_macs else (out, lse)


def gqa(q, k_cache, v_cache, seqlens, scale, rows=None, threads=0, return_macs=False):
    """GQA/MQA/MHA decode in fp64.

    q [b,s,hq,d], k_cache and v_cache [b,t_max,hkv,d], seqlens [b]. Query head
    hh reads KV head hh // (hq/hkv). Returns out [b,s,hq,d], lse [b,s,hq]
    (or [n,d], [n] for a ``rows`` subset).
    """
    qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
    b, s, hq, d = qb.shape
    t_max, hkv = kb.shape[1], kb.shape[2]
    assert kb.shape == (b, t_max, hkv, d) and vb.shape == kb.shape
    sl = _i32(seqlens)
    rr = _rows(rows)
    n = b * s * hq if rr is None else rr.shape[0]
    out = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    macs = ctypes.c_int64(0)
    rc = _load().oracle_gqa(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(sl), b, s, hq, hkv, d, t_max,
                            float(scale), _ptr(rr), n, _ptr(out), _ptr(lse),
                            ctypes.byref(macs), int(threads))
    if rc != 0:
        raise ValueError("oracle_gqa rejected its arguments")
    if rr is None:
        out, lse = out.reshape(b, s, hq, d), lse.reshape(b, s, hq)
    return (out, lse, macs.value) if return_macs else (out, lse)


def attn_generic(Q, K, V, n_vis, scale):
    """Textbook single-head softmax attention in fp64 (float64 inputs).

    Q [nq,dk], K [t,dk], V [t,dv]; row r sees keys [0, n_vis[r]). Returns
    out [nq,dv], lse [nq] (natural log).
    """
    Q = np.ascontiguousarray(Q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    nq, dk = Q.shape
    t, dv = V.shape
    assert K.shape == (t, dk)
    nv = _i32(n_vis)
    assert nv.shape == (nq,)
    out = np.empty((nq, dv), np.float64)
    lse = np.empty((nq,), np.float64)
    rc = _load().oracle_attn_generic(_ptr(Q), _ptr(K), _ptr(V), _ptr(nv), nq, t, dk, dv,
                                     float(scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attn_generic rejected its arguments")
    return out, lse


def _wide(a) -> np.ndarray:
    """bf16 (bit patterns or a torch bf16 tensor) -> float64, exactly; float inputs pass through as float64."""
    if hasattr(a, "dtype") and str(a.dtype) in ("torch.float64", "torch.float32"):
        return a.double().numpy()
    if isinstance(a, np.ndarray) and a.dtype.kind == "f":
        return a.astype(np.float64)
    return (_bits(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def head_projection(A, B):
    """Per-head projection in fp64: C[m, hd, n] = sum_k A[m, hd, k] * B[hd, n, k].

    A [M, H, K] and B [H, N, K] as bf16 (bit patterns or torch bf16 tensors; any
    leading dims of A are flattened into M). With A = q_nope [b,s,h,d] and
    B = Wk [h,k,d] this is the query absorption Q Wk^T; with A = o_lat
    [b,s,h,k] and B = Wv^T [h,d,k] it is the output decompression O_lat Wv
    ("Mla Analysis" skill page, "Absorption Trick (FlashMLA)"). Returns
    float64 [..., H, N] with A's leading shape.
    """
    a = _wide(A)
    b = _wide(B)
    lead = a.shape[:-2]
    h, k = a.shape[-2], a.shape[-1]
    assert b.shape[0] == h and b.shape[2] == k
    a2 = a.reshape(-1, h, k)
    c = np.einsum("mhk,hnk->mhn", a2, b)
    return c.reshape(*lead, h, b.shape[1])
