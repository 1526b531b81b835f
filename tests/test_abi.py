"""The C ABI: the shared library loads, exports every function the header
declares, and rejects bad arguments with the documented status codes before
touching the GPU. Runs without a GPU (no kernel is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_attn.h")
LIB = os.path.join(ROOT, "decode_attention_bf16_amd", "libdecode_attn.so")

DA_OK, DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED, DA_ERR_WORKSPACE, DA_ERR_HIP = range(5)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    skip = {"extern", "if", "sizeof"}
    return sorted(set(n for n in names if n not in skip))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from decode_attention_bf16_amd import build
        build.build()
    L = ctypes.CDLL(LIB)
    P, I, Z, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    L.da_status_string.argtypes, L.da_status_string.restype = [I], ctypes.c_char_p
    L.mla_decode_workspace_size.argtypes, L.mla_decode_workspace_size.restype = [I] * 7, Z
    L.gqa_decode_workspace_size.argtypes, L.gqa_decode_workspace_size.restype = [I] * 8, Z
    L.mla_decode.argtypes = [P, P, P, P, I, I, I, I, I, I, F, P, P, P, Z, I, P]
    L.gqa_decode.argtypes = [P, P, P, P, I, I, I, I, I, I, F, P, P, P, Z, I, I, P]
    L.mla_decode_unabsorbed_workspace_size.argtypes = [I] * 7
    L.mla_decode_unabsorbed_workspace_size.restype = Z
    L.mla_decode_unabsorbed.argtypes = [P, P, P, P, I, I, I, I, I, I, F, P, P, P, Z, I, P]
    L.mla_absorb_queries.argtypes = [P, P, P, I, I, I, I, I, P]
    L.mla_decompress_output.argtypes = [P, P, P, I, I, I, I, I, P]
    L.mla_decode_split_cache_workspace_size.argtypes = [I] * 6
    L.mla_decode_split_cache_workspace_size.restype = Z
    L.mla_decode_split_cache.argtypes = [P] * 9 + [I] * 5 + [F, P, P, P, Z, I, P]
    return L


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for n in ("mla_decode", "gqa_decode", "mla_decode_workspace_size", "gqa_decode_workspace_size",
              "mla_decode_unabsorbed", "mla_decode_unabsorbed_workspace_size", "mla_absorb_queries",
              "mla_decompress_output", "mla_decode_split_cache", "mla_decode_split_cache_workspace_size",
              "da_status_string", "da_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.da_version() >= 100
    for code, text in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported dimensions"),
                       (3, b"workspace too small"), (4, b"HIP launch error")]:
        assert lib.da_status_string(code) == text
    assert lib.da_status_string(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails its host checks


def mla_call(lib, **kw):
    a = dict(q=FAKE, r=FAKE, c=FAKE, sl=FAKE, b=2, s=1, h=16, k=512, p=64, t=128, scale=0.1, o=FAKE, lse=FAKE,
             ws=FAKE, wsb=0, nw=0)
    a.update(kw)
    return lib.mla_decode(a["q"], a["r"], a["c"], a["sl"], a["b"], a["s"], a["h"], a["k"], a["p"], a["t"],
                          a["scale"], a["o"], a["lse"], a["ws"], a["wsb"], a["nw"], None)


def gqa_call(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sl=FAKE, b=2, s=1, hq=8, hkv=2, d=128, t=128, scale=0.1, o=FAKE, lse=FAKE,
             ws=FAKE, wsb=0, nw=0, path=0)
    a.update(kw)
    return lib.gqa_decode(a["q"], a["k"], a["v"], a["sl"], a["b"], a["s"], a["hq"], a["hkv"], a["d"], a["t"],
                          a["scale"], a["o"], a["lse"], a["ws"], a["wsb"], a["nw"], a["path"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=0), DA_ERR_INVALID_ARG),
    (dict(h=-1), DA_ERR_INVALID_ARG),
    (dict(s=200, t=128), DA_ERR_INVALID_ARG),
    (dict(nw=-3), DA_ERR_INVALID_ARG),
    (dict(q=None), DA_ERR_INVALID_ARG),
    (dict(ws=None, b=0), DA_ERR_INVALID_ARG),    # a null workspace is allowed, but checks still apply
    (dict(ws=None, q=None), DA_ERR_INVALID_ARG),
    (dict(ws=ctypes.c_void_p(0x100010)), DA_ERR_INVALID_ARG),  # workspace not 256-byte aligned
    (dict(k=96, p=64), DA_ERR_UNSUPPORTED),
    (dict(k=512, p=32), DA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), DA_ERR_INVALID_ARG),
    (dict(scale=-1.0), DA_ERR_INVALID_ARG),
    (dict(c=ctypes.c_void_p(0x100002)), DA_ERR_INVALID_ARG),  # misaligned cache
])
def test_mla_rejects(lib, kw, code):
    assert mla_call(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(hq=6, hkv=4), DA_ERR_INVALID_ARG),
    (dict(d=96), DA_ERR_UNSUPPORTED),
    (dict(hq=64, hkv=1, s=5), DA_ERR_UNSUPPORTED),      # 320 rows per KV head (at most 256 at d = 128)
    (dict(hq=64, hkv=2, s=5, d=256), DA_ERR_UNSUPPORTED),  # 160 rows per KV head (at most 128 at d = 256)
    (dict(ws=None, hq=6, hkv=4), DA_ERR_INVALID_ARG),
    (dict(hq=32, hkv=1, s=1, path=1), DA_ERR_UNSUPPORTED),  # VALU kernel takes at most 16 rows
    (dict(t=1 << 20, hkv=8, d=256), DA_ERR_UNSUPPORTED),   # 32-bit buffer offsets
    (dict(path=7), DA_ERR_INVALID_ARG),
    (dict(v=None), DA_ERR_INVALID_ARG),
    (dict(s=0), DA_ERR_INVALID_ARG),
])
def test_gqa_rejects(lib, kw, code):
    assert gqa_call(lib, **kw) == code


def test_workspace_size_zero_for_rejected_args(lib):
    assert lib.mla_decode_workspace_size(0, 1, 16, 512, 64, 128, 0) == 0
    assert lib.mla_decode_workspace_size(2, 1, 16, 100, 64, 128, 0) == 0
    assert lib.gqa_decode_workspace_size(2, 1, 6, 4, 128, 128, 0, 0) == 0
    assert lib.gqa_decode_workspace_size(2, 1, 8, 2, 128, 128, 0, 5) == 0


def test_workspace_size_explicit_workers(lib):
    # With an explicit worker count the size is a pure function of the shapes.
    b, s, h, k, p, t, w = 32, 1, 128, 512, 64, 4096, 128
    sz = lib.mla_decode_workspace_size(b, s, h, k, p, t, w)
    slots = b + w
    # per partial slot and query row: k bf16 outputs and one fp32 lse
    assert sz >= slots * s * h * (2 * k + 4)
    assert sz < slots * s * h * (2 * k + 4) + 64 * 1024
    # too-small workspace is reported as such (checked before any launch)
    assert mla_call(lib, b=b, s=s, h=h, t=t, nw=w, wsb=sz - 1, ws=ctypes.c_void_p(0x100000)) == DA_ERR_WORKSPACE


def unabs_call(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sl=FAKE, b=2, s=1, h=16, dqk=192, dv=128, t=128, scale=0.1, o=FAKE, lse=FAKE,
             ws=FAKE, wsb=0, nw=0)
    a.update(kw)
    return lib.mla_decode_unabsorbed(a["q"], a["k"], a["v"], a["sl"], a["b"], a["s"], a["h"], a["dqk"], a["dv"],
                                     a["t"], a["scale"], a["o"], a["lse"], a["ws"], a["wsb"], a["nw"], None)


@pytest.mark.parametrize("kw, code", [
    ({"dqk": 128}, 2), ({"dv": 192}, 2), ({"b": 0}, 1), ({"h": -1}, 1), ({"s": 65}, 2), ({"s": 200}, 1),
    ({"nw": -2}, 1), ({"t": 100000, "h": 128}, 2), ({"scale": float("nan")}, 1), ({"scale": 0.0}, 1),
    ({"q": None}, 1), ({"v": None}, 1), ({"o": ctypes.c_void_p(0x100008)}, 1), ({}, 3),
])
def test_unabsorbed_rejects(lib, kw, code):
    assert unabs_call(lib, **kw) == code


def test_unabsorbed_workspace_size(lib):
    assert lib.mla_decode_unabsorbed_workspace_size(2, 1, 16, 128, 128, 128, 0) == 0
    b, s, h, w = 4, 2, 8, 10
    sz = lib.mla_decode_unabsorbed_workspace_size(b, s, h, 192, 128, 512, w)
    # per partial slot and query row: 128 bf16 outputs and one fp32 lse
    assert (b + w) * s * h * (2 * 128 + 4) <= sz < (b + w) * s * h * (2 * 128 + 4) + 64 * 1024


@pytest.mark.parametrize("fn", ["mla_absorb_queries", "mla_decompress_output"])
@pytest.mark.parametrize("args, code", [
    ((None, FAKE, FAKE, 2, 1, 4, 128, 512), 1), ((FAKE, None, FAKE, 2, 1, 4, 128, 512), 1),
    ((FAKE, FAKE, None, 2, 1, 4, 128, 512), 1), ((FAKE, FAKE, FAKE, 0, 1, 4, 128, 512), 1),
    ((FAKE, FAKE, FAKE, 2, -1, 4, 128, 512), 1), ((FAKE, FAKE, FAKE, 2, 1, 0, 128, 512), 1),
    ((ctypes.c_void_p(0x100004), FAKE, FAKE, 2, 1, 4, 128, 512), 1),
    ((FAKE, FAKE, ctypes.c_void_p(0x100008), 2, 1, 4, 128, 512), 1),
])
def test_projection_rejects(lib, fn, args, code):
    assert getattr(lib, fn)(*args, None) == code


def test_projection_contracted_width_multiple_of_32(lib):
    # the contracted width is d for the queries (5th argument after b, s, h) and k for the output
    assert lib.mla_absorb_queries(FAKE, FAKE, FAKE, 2, 1, 4, 100, 512, None) == 2
    assert lib.mla_decompress_output(FAKE, FAKE, FAKE, 2, 1, 4, 500, 128, None) == 2


def test_projection_tile_span_limit(lib):
    # a 64-row tile's inputs span 64 * h * width * 2 bytes, which must stay below 2^31
    assert lib.mla_absorb_queries(FAKE, FAKE, FAKE, 2, 1, 1 << 17, 128, 512, None) == 2
    assert lib.mla_decompress_output(FAKE, FAKE, FAKE, 2, 1, 1 << 15, 512, 128, None) == 2


def split_call(lib, **kw):
    a = dict(b=2, s=2, h=8, o=256, n=64, scale=0.1, ws=FAKE, wsb=0, nw=0, qn=FAKE)
    a.update(kw)
    return lib.mla_decode_split_cache(a["qn"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["b"], a["s"], a["h"],
                                      a["o"], a["n"], a["scale"], FAKE, FAKE, a["ws"], a["wsb"], a["nw"], None)


@pytest.mark.parametrize("kw, code", [({"b": 0}, 1), ({"s": 65, "n": 100}, 2), ({"s": 80}, 1), ({"o": 0}, 1),
                                      ({"qn": None}, 1), ({"scale": -1.0}, 1), ({}, 3)])
def test_split_cache_rejects(lib, kw, code):
    assert split_call(lib, **kw) == code


def test_split_cache_workspace_covers_both_parts(lib):
    b, s, h, o, n = 2, 2, 8, 256, 64
    sz = lib.mla_decode_split_cache_workspace_size(b, s, h, o, n, 0)
    parts = (lib.mla_decode_workspace_size(b, 1, s * h, 512, 64, o, 0)
             + lib.mla_decode_unabsorbed_workspace_size(b, s, h, 192, 128, n, 0))
    assert sz >= parts + b * s * h * (2 * 512 * 2 + 192 * 2 + 2 * 128 * 2 + 8)
    assert lib.mla_decode_split_cache_workspace_size(b, 80, h, o, n, 0) == 0
