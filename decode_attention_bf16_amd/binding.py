"""Thin Python binding of libdecode_attn.so (ctypes).

Argument marshalling only: checks shapes/dtypes/devices, allocates the outputs
and the workspace with torch on the input's device, and calls the C ABI on
torch's current stream. Every step of the computation runs in the library's
HIP kernels; there is no fallback path, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdecode_attn.so")
_lock = threading.Lock()
_lib = None

DA_OK = 0
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported dimensions", 3: "workspace too small",
           4: "HIP launch error"}

EXPORTED = ("da_version", "da_status_string", "mla_decode_workspace_size", "mla_decode",
            "gqa_decode_workspace_size", "gqa_decode", "mla_decode_unabsorbed_workspace_size",
            "mla_decode_unabsorbed", "mla_absorb_queries", "mla_decompress_output",
            "mla_decode_split_cache_workspace_size", "mla_decode_split_cache", "mla_decode_no_alloc")


class DecodeAttentionError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libdecode_attn.so (built in-tree by ``python -m decode_attention_bf16_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise DecodeAttentionError("load_library", -1,
                                       "%s is missing; build it with python -m decode_attention_bf16_amd.build"
                                       % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, Z, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        lib.da_version.argtypes, lib.da_version.restype = [], I
        lib.da_status_string.argtypes, lib.da_status_string.restype = [I], ctypes.c_char_p
        lib.mla_decode_workspace_size.argtypes = [I] * 7
        lib.mla_decode_workspace_size.restype = Z
        lib.mla_decode.argtypes = [P, P, P, P, I, I, I, I, I, I, F, P, P, P, Z, I, P]
        lib.mla_decode.restype = I
        lib.mla_decode_no_alloc.argtypes = [P, P, P, P, I, I, I, I, I, I, F, P, P, I, P]
        lib.mla_decode_no_alloc.restype = I
        lib.gqa_decode_workspace_size.argtypes = [I] * 8
        lib.gqa_decode_workspace_size.restype = Z
        lib.gqa_decode.argtypes = [P, P, P, P, I, I, I, I, I, I, F, P, P, P, Z, I, I, P]
        lib.gqa_decode.restype = I
        lib.mla_decode_unabsorbed_workspace_size.argtypes = [I] * 7
        lib.mla_decode_unabsorbed_workspace_size.restype = Z
        lib.mla_decode_unabsorbed.argtypes = [P, P, P, P, I, I, I, I, I, I, F, P, P, P, Z, I, P]
        lib.mla_decode_unabsorbed.restype = I
        lib.mla_absorb_queries.argtypes = [P, P, P, I, I, I, I, I, P]
        lib.mla_absorb_queries.restype = I
        lib.mla_decompress_output.argtypes = [P, P, P, I, I, I, I, I, P]
        lib.mla_decompress_output.restype = I
        lib.mla_decode_split_cache_workspace_size.argtypes = [I] * 6
        lib.mla_decode_split_cache_workspace_size.restype = Z
        lib.mla_decode_split_cache.argtypes = [P] * 9 + [I] * 5 + [F, P, P, P, Z, I, P]
        lib.mla_decode_split_cache.restype = I
        _lib = lib
        return lib


def _check(fn, rc):
    if rc != DA_OK:
        msg = load_library().da_status_string(rc).decode()
        raise DecodeAttentionError(fn, rc, msg)


def _need(t, name, dtype, ndim, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def mla_decode_workspace_size(b, s, h, k, p, t_max, num_workers=0) -> int:
    return int(load_library().mla_decode_workspace_size(b, s, h, k, p, t_max, num_workers))


def gqa_decode_workspace_size(b, s, hq, hkv, d, t_max, num_workers=0, path=0) -> int:
    return int(load_library().gqa_decode_workspace_size(b, s, hq, hkv, d, t_max, num_workers, path))


def mla_decode_unabsorbed_workspace_size(b, s, h, dqk, dv, t_max, num_workers=0) -> int:
    return int(load_library().mla_decode_unabsorbed_workspace_size(b, s, h, dqk, dv, t_max, num_workers))


def mla_decode_split_cache_workspace_size(b, s, h, o_max, n_max, num_workers=0) -> int:
    return int(load_library().mla_decode_split_cache_workspace_size(b, s, h, o_max, n_max, num_workers))


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel() * workspace.element_size(),
                                                                    nbytes))
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def mla_decode(q_lat, q_rope, cache, seqlens, scale, num_workers=0, out=None, lse=None, workspace=None,
               null_workspace=False):
    """Absorbed-latent MLA decode on the GPU.

    q_lat [b,s,h,k], q_rope [b,s,h,p], cache [b,t_max,k+p] (bf16), seqlens [b]
    (int32), all on one GPU. Returns (out_lat [b,s,h,k] bf16, lse [b,s,h] fp32).
    null_workspace=True passes no workspace: one worker per sequence, no split.
    """
    lib = load_library()
    _need(q_lat, "q_lat", torch.bfloat16, 4)
    dev = q_lat.device
    _need(q_rope, "q_rope", torch.bfloat16, 4, dev)
    _need(cache, "cache", torch.bfloat16, 3, dev)
    _need(seqlens, "seqlens", torch.int32, 1, dev)
    b, s, h, k = q_lat.shape
    p = q_rope.shape[3]
    t_max = cache.shape[1]
    if tuple(q_rope.shape) != (b, s, h, p):
        raise ValueError("q_rope shape %s does not match q_lat %s" % (tuple(q_rope.shape), tuple(q_lat.shape)))
    if tuple(cache.shape) != (b, t_max, k + p):
        raise ValueError("cache must be [b, t_max, k+p] = [%d, *, %d], got %s" % (b, k + p, tuple(cache.shape)))
    if seqlens.shape[0] != b:
        raise ValueError("seqlens must have b=%d entries" % b)
    if out is None:
        out = torch.empty((b, s, h, k), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, 4, dev)
    if lse is None:
        lse = torch.empty((b, s, h), dtype=torch.float32, device=dev)
    else:
        _need(lse, "lse", torch.float32, 3, dev)
    ws = None if null_workspace else _workspace(lib.mla_decode_workspace_size(b, s, h, k, p, t_max, num_workers),
                                                 dev, workspace)
    with torch.cuda.device(dev):
        rc = lib.mla_decode(_ptr(q_lat), _ptr(q_rope), _ptr(cache), _ptr(seqlens), b, s, h, k, p, t_max,
                            float(scale), _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws), int(num_workers), _stream(dev))
    _check("mla_decode", rc)
    return out, lse


def mla_decode_no_alloc(q_lat, q_rope, cache, seqlens, scale, out, lse, num_workers=0):
    """mla_decode through the library's allocation-free entry point: the caller passes the outputs
    (out [b,s,h,k] bf16, lse [b,s,h] fp32) and no workspace (the library's device scratch holds it)."""
    lib = load_library()
    _need(q_lat, "q_lat", torch.bfloat16, 4)
    dev = q_lat.device
    _need(q_rope, "q_rope", torch.bfloat16, 4, dev)
    _need(cache, "cache", torch.bfloat16, 3, dev)
    _need(seqlens, "seqlens", torch.int32, 1, dev)
    _need(out, "out", torch.bfloat16, 4, dev)
    _need(lse, "lse", torch.float32, 3, dev)
    b, s, h, k = q_lat.shape
    p = q_rope.shape[3]
    t_max = cache.shape[1]
    if (tuple(q_rope.shape) != (b, s, h, p) or tuple(cache.shape) != (b, t_max, k + p) or seqlens.shape[0] != b
            or tuple(out.shape) != (b, s, h, k) or tuple(lse.shape) != (b, s, h)):
        raise ValueError("mla_decode_no_alloc shapes: see mla_decode")
    with torch.cuda.device(dev):
        rc = lib.mla_decode_no_alloc(_ptr(q_lat), _ptr(q_rope), _ptr(cache), _ptr(seqlens), b, s, h, k, p, t_max,
                                     float(scale), _ptr(out), _ptr(lse), int(num_workers), _stream(dev))
    _check("mla_decode_no_alloc", rc)
    return out, lse


def gqa_decode(q, k_cache, v_cache, seqlens, scale, num_workers=0, path=0, out=None, lse=None, workspace=None,
               null_workspace=False):
    """Grouped-query decode on the GPU (MHA when hkv == hq, MQA when hkv == 1).

    q [b,s,hq,d], k_cache/v_cache [b,t_max,hkv,d] (bf16), seqlens [b] (int32).
    Returns (out [b,s,hq,d] bf16, lse [b,s,hq] fp32). path: 0 auto, 1 VALU, 2 MFMA.
    null_workspace=True passes no workspace: one worker per sequence, no split.
    """
    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(seqlens, "seqlens", torch.int32, 1, dev)
    b, s, hq, d = q.shape
    t_max, hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (b, t_max, hkv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must both be [b, t_max, hkv, d]")
    if seqlens.shape[0] != b:
        raise ValueError("seqlens must have b=%d entries" % b)
    if out is None:
        out = torch.empty((b, s, hq, d), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, 4, dev)
    if lse is None:
        lse = torch.empty((b, s, hq), dtype=torch.float32, device=dev)
    else:
        _need(lse, "lse", torch.float32, 3, dev)
    ws = None if null_workspace else _workspace(
        lib.gqa_decode_workspace_size(b, s, hq, hkv, d, t_max, num_workers, path), dev, workspace)
    with torch.cuda.device(dev):
        rc = lib.gqa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), b, s, hq, hkv, d, t_max,
                            float(scale), _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws), int(num_workers), int(path),
                            _stream(dev))
    _check("gqa_decode", rc)
    return out, lse


def mla_decode_unabsorbed(q, k_cache, v_cache, seqlens, scale, num_workers=0, out=None, lse=None, workspace=None,
                          null_workspace=False):
    """Un-absorbed MLA decode on the GPU: per-head decompressed keys and values.

    q [b,s,h,dqk], k_cache [b,t_max,h,dqk], v_cache [b,t_max,h,dv] (bf16), seqlens [b] (int32).
    Returns (out [b,s,h,dv] bf16, lse [b,s,h] fp32).
    null_workspace=True passes no workspace: one worker per sequence, no split.
    """
    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(seqlens, "seqlens", torch.int32, 1, dev)
    b, s, h, dqk = q.shape
    t_max, dv = k_cache.shape[1], v_cache.shape[3]
    if tuple(k_cache.shape) != (b, t_max, h, dqk) or tuple(v_cache.shape) != (b, t_max, h, dv):
        raise ValueError("k_cache must be [b, t_max, h, dqk] and v_cache [b, t_max, h, dv]")
    if seqlens.shape[0] != b:
        raise ValueError("seqlens must have b=%d entries" % b)
    if out is None:
        out = torch.empty((b, s, h, dv), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, 4, dev)
    if lse is None:
        lse = torch.empty((b, s, h), dtype=torch.float32, device=dev)
    else:
        _need(lse, "lse", torch.float32, 3, dev)
    ws = None if null_workspace else _workspace(
        lib.mla_decode_unabsorbed_workspace_size(b, s, h, dqk, dv, t_max, num_workers), dev, workspace)
    with torch.cuda.device(dev):
        rc = lib.mla_decode_unabsorbed(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), b, s, h, dqk, dv, t_max,
                                       float(scale), _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws), int(num_workers),
                                       _stream(dev))
    _check("mla_decode_unabsorbed", rc)
    return out, lse


def mla_absorb_queries(q_nope, w_k, out=None):
    """q_lat [b,s,h,k] = per head w_k[h] . q_nope[b,s,h,:]; q_nope [b,s,h,d], w_k [h,k,d] (bf16)."""
    lib = load_library()
    _need(q_nope, "q_nope", torch.bfloat16, 4)
    dev = q_nope.device
    _need(w_k, "w_k", torch.bfloat16, 3, dev)
    b, s, h, d = q_nope.shape
    if w_k.shape[0] != h or w_k.shape[2] != d:
        raise ValueError("w_k must be [h, k, d] = [%d, k, %d]" % (h, d))
    k = w_k.shape[1]
    if out is None:
        out = torch.empty((b, s, h, k), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, 4, dev)
    with torch.cuda.device(dev):
        rc = lib.mla_absorb_queries(_ptr(q_nope), _ptr(w_k), _ptr(out), b, s, h, d, k, _stream(dev))
    _check("mla_absorb_queries", rc)
    return out


def mla_decompress_output(o_lat, w_v_t, out=None):
    """out [b,s,h,d] = per head w_v_t[h] . o_lat[b,s,h,:]; o_lat [b,s,h,k], w_v_t [h,d,k] (bf16)."""
    lib = load_library()
    _need(o_lat, "o_lat", torch.bfloat16, 4)
    dev = o_lat.device
    _need(w_v_t, "w_v_t", torch.bfloat16, 3, dev)
    b, s, h, k = o_lat.shape
    if w_v_t.shape[0] != h or w_v_t.shape[2] != k:
        raise ValueError("w_v_t must be [h, d, k] = [%d, d, %d]" % (h, k))
    d = w_v_t.shape[1]
    if out is None:
        out = torch.empty((b, s, h, d), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, 4, dev)
    with torch.cuda.device(dev):
        rc = lib.mla_decompress_output(_ptr(o_lat), _ptr(w_v_t), _ptr(out), b, s, h, k, d, _stream(dev))
    _check("mla_decompress_output", rc)
    return out


def mla_decode_split_cache(q_nope, q_rope, w_k, w_v_t, latent, seqlens_old, k_new, v_new, seqlens_new, scale,
                           num_workers=0, out=None, lse=None, workspace=None):
    """MLA decode over a split cache: latent old rows plus decompressed new rows (see the C header).

    q_nope [b,s,h,128], q_rope [b,s,h,64], w_k [h,512,128], w_v_t [h,128,512], latent [b,o_max,576],
    k_new [b,n_max,h,192], v_new [b,n_max,h,128] (bf16); seqlens_old, seqlens_new [b] (int32).
    Returns (out [b,s,h,128] bf16, lse [b,s,h] fp32).
    """
    lib = load_library()
    _need(q_nope, "q_nope", torch.bfloat16, 4)
    dev = q_nope.device
    for t, nm, nd in ((q_rope, "q_rope", 4), (w_k, "w_k", 3), (w_v_t, "w_v_t", 3), (latent, "latent", 3),
                      (k_new, "k_new", 4), (v_new, "v_new", 4)):
        _need(t, nm, torch.bfloat16, nd, dev)
    _need(seqlens_old, "seqlens_old", torch.int32, 1, dev)
    _need(seqlens_new, "seqlens_new", torch.int32, 1, dev)
    b, s, h, _ = q_nope.shape
    o_max, n_max = latent.shape[1], k_new.shape[1]
    if (tuple(q_nope.shape) != (b, s, h, 128) or tuple(q_rope.shape) != (b, s, h, 64)
            or tuple(w_k.shape) != (h, 512, 128) or tuple(w_v_t.shape) != (h, 128, 512)
            or tuple(latent.shape) != (b, o_max, 576) or tuple(k_new.shape) != (b, n_max, h, 192)
            or tuple(v_new.shape) != (b, n_max, h, 128)):
        raise ValueError("split-cache shapes: see mla_decode_split_cache in include/decode_attn.h")
    if out is None:
        out = torch.empty((b, s, h, 128), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((b, s, h), dtype=torch.float32, device=dev)
    nbytes = lib.mla_decode_split_cache_workspace_size(b, s, h, o_max, n_max, num_workers)
    ws = _workspace(nbytes, dev, workspace)
    with torch.cuda.device(dev):
        rc = lib.mla_decode_split_cache(_ptr(q_nope), _ptr(q_rope), _ptr(w_k), _ptr(w_v_t), _ptr(latent),
                                        _ptr(seqlens_old), _ptr(k_new), _ptr(v_new), _ptr(seqlens_new), b, s, h,
                                        o_max, n_max, float(scale), _ptr(out), _ptr(lse), _ptr(ws),
                                        ws.numel() * ws.element_size(), int(num_workers), _stream(dev))
    _check("mla_decode_split_cache", rc)
    return out, lse
