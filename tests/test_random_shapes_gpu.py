"""Seeded random shapes through both attention entry points, every output row against the fp64 oracle.

The shapes are drawn once from a fixed seed (the list is the same on every run) across the compiled sets:
head dims, group sizes, draft counts, batch sizes, ragged lengths including empty and full sequences,
and the three workspace modes (automatic worker count, a forced count, no workspace), so that each run
covers plans with one and several pieces per block, partial and unpadded row blocks and the causal mask."""
import math
import random

import pytest
import torch

import workloads as wl
from test_parity_gpu import compare, da, run_gqa, run_mla  # noqa: F401 (da: the library fixture)

pytestmark = pytest.mark.gpu


def gqa_cases(n=32, seed=20261204):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n:
        d = rng.choice([64, 128, 256])
        hkv = rng.choice([1, 2, 3, 4, 8])
        g = rng.choice([1, 2, 3, 6, 8, 16])
        s = rng.choice([1, 1, 2, 3, 4])
        if g * s > (128 if d == 256 else 256):
            continue
        b = rng.randint(1, 6)
        t = rng.randint(max(1, s), 420)
        lens = [rng.choice([0, 1, t, rng.randint(0, t)]) for _ in range(b)]
        mode = rng.choice(["auto", "forced", "null"])
        workers = rng.randint(1, 40) if mode == "forced" else 0
        cases.append((b, s, g * hkv, hkv, d, t, tuple(lens), mode, workers))
    return cases


def mla_cases(n=16, seed=20261205):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n:
        k, p = rng.choice([(512, 64), (256, 64), (128, 64), (64, 16)])
        s = rng.choice([1, 1, 2, 4])
        h = rng.choice([1, 5, 16, 40, 128])
        if s * h > 256:
            continue
        b = rng.randint(1, 4)
        t = rng.randint(max(1, s), 300)
        lens = [rng.choice([0, 1, t, rng.randint(0, t)]) for _ in range(b)]
        mode = rng.choice(["auto", "forced", "null"])
        workers = rng.randint(1, 24) if mode == "forced" else 0
        cases.append((b, s, h, k, p, t, tuple(lens), mode, workers))
    return cases


@pytest.mark.parametrize("case", gqa_cases(), ids=lambda c: "b%d_s%d_hq%d_hkv%d_d%d_t%d_%s%d" % (c[:6] + c[7:]))
def test_gqa_random_shape(da, oracle_mod, case):
    b, s, hq, hkv, d, t, lens, mode, workers = case
    shape = wl.GQAShape(b=b, s=s, hq=hq, hkv=hkv, d=d, t_max=t, scale=1.0 / math.sqrt(d), seed=500 + b * 7 + d)
    tensors = wl.make_gqa(shape, seqlens=list(lens))
    print("gqa random", case, flush=True)
    out, lse = run_gqa(da, shape, tensors, workers, 0, null_workspace=mode == "null")
    ref_o, ref_l = oracle_mod.gqa(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "gqa random %s" % (case,))


@pytest.mark.parametrize("case", mla_cases(), ids=lambda c: "b%d_s%d_h%d_k%d_p%d_t%d_%s%d" % (c[:6] + c[7:]))
def test_mla_random_shape(da, oracle_mod, case):
    b, s, h, k, p, t, lens, mode, workers = case
    shape = wl.MLAShape(b=b, s=s, h=h, k=k, p=p, t_max=t, scale=1.0 / math.sqrt(k / 4 + p), seed=600 + b * 5 + h)
    tensors = wl.make_mla(shape, seqlens=list(lens))
    print("mla random", case, flush=True)
    out, lse = run_mla(da, shape, tensors, workers, null_workspace=mode == "null")
    ref_o, ref_l = oracle_mod.mla(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "mla random %s" % (case,))
