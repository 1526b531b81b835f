"""The allocation-free MLA entry point (mla_decode_no_alloc, through the C ABI) against mla_decode, the
entry point it varies: two calls in a row on one device, the second with a smaller input, each within
the oracle bar (max |dout| <= 1e-2 * max |out|, |dlse| <= 1e-3) of mla_decode's output on the same
inputs, and the small one also against the fp64 oracle. The size limit is checked on the host."""
import math

import numpy as np
import pytest
import torch

import workloads as wl

OUT_TOL = 1e-2
LSE_TOL = 1e-3


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _agree(o1, l1, o2, l2, what):
    o1, o2 = o1.float().cpu().numpy(), o2.float().cpu().numpy()
    l1, l2 = l1.cpu().numpy(), l2.cpu().numpy()
    fin = np.isfinite(l2)
    assert np.array_equal(np.isfinite(l1), fin), what + ": lse finiteness differs"
    assert np.all(o1[~fin] == 0), what
    err = np.abs(o1 - o2).max()
    assert err <= OUT_TOL * np.abs(o2).max(), "%s: max|dout| %.3e" % (what, err)
    if fin.any():
        assert np.abs(l1[fin] - l2[fin]).max() <= LSE_TOL, what


@pytest.mark.gpu
def test_no_alloc_matches_mla_decode_on_two_calls(oracle_mod):
    from decode_attention_bf16_amd import binding
    d = _dev()
    binding.load_library()
    big = wl.MLA_DSV3  # 21 MB of plan and partials in the library's scratch
    small = wl.MLAShape(b=3, s=2, h=20, k=512, p=64, t_max=300, scale=1.0 / math.sqrt(192), seed=55)
    for shape, sl in ((big, None), (small, [300, 1, 129])):
        cpu = wl.make_mla(shape, seqlens=sl)
        g = [t.to(d) for t in cpu]
        print("no-alloc b=%d s=%d h=%d t_max=%d" % (shape.b, shape.s, shape.h, shape.t_max), flush=True)
        out = torch.full((shape.b, shape.s, shape.h, shape.k), float("nan"), dtype=torch.bfloat16, device=d)
        lse = torch.full((shape.b, shape.s, shape.h), float("nan"), dtype=torch.float32, device=d)
        binding.mla_decode_no_alloc(*g, shape.scale, out, lse)
        ref_o, ref_l = binding.mla_decode(*g, shape.scale)
        torch.cuda.synchronize()
        _agree(out, lse, ref_o, ref_l, "no_alloc vs mla_decode b=%d" % shape.b)
        if shape is small:
            oo, ol = oracle_mod.mla(*cpu, shape.scale)
            o = out.float().cpu().numpy().astype(np.float64)
            assert np.abs(o - oo).max() <= OUT_TOL * np.abs(oo).max()
            fin = np.isfinite(ol)
            assert np.abs(lse.cpu().numpy()[fin] - ol[fin]).max() <= LSE_TOL


def test_no_alloc_rejects_calls_beyond_its_scratch():
    """A call whose plan and partials exceed the scratch returns DA_ERR_WORKSPACE before any launch."""
    import ctypes
    from decode_attention_bf16_amd import binding
    lib = binding.load_library()
    fake = ctypes.c_void_p(0x100000)
    # s = 64 drafts at h = 128: 8192 rows per sequence with 1 KB of partial each per slot
    rc = lib.mla_decode_no_alloc(fake, fake, fake, fake, 32, 64, 128, 512, 64, 4096, 0.1, fake, fake, 0, None)
    assert rc == 3
    assert lib.mla_decode_no_alloc(fake, fake, fake, fake, 0, 1, 128, 512, 64, 4096, 0.1, fake, fake, 0, None) == 1
