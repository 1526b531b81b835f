"""Seeded synthetic workloads for decode attention.

This module only draws inputs; it holds none of the attention arithmetic. Both
sides of every parity check (the fp64 oracle and the HIP library) are fed from
here, and the benchmark uses the same recipe.

Recipe: a ``torch.Generator`` seeded with the workload's seed draws N(0,1)
float32 values, which are rounded to bf16 (round-to-nearest-even, torch's
``.to(torch.bfloat16)``). Draw order: for ragged workloads the sequence lengths
first (uniform integers), then the query tensors, then the cache tensors (MLA:
q_lat, q_rope, cache; GQA: q, k, v). Cache rows beyond a sequence's length are
drawn like the rest (they are never read as valid rows). The largest shapes
(caches of about 2 GB per sequence) are drawn the same way by a generator on
the GPU (``device=``), whose numbers differ from the CPU generator's for the
same seed; the oracle then reads a host copy.

Shapes follow the source pages' DeepSeek-V3-like geometry ("Mla Analysis"
skill page, "Cost Models" and "Tensor Shapes": h=128, k=512, p=64, t=4096,
b=32 for the timing table) and the 64-query/8-KV-head GQA example ("MHA vs GQA
70B" Q&A page, section 3). The pages use no public dataset.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class MLAShape:
    b: int
    s: int
    h: int
    k: int
    p: int
    t_max: int
    scale: float
    seed: int
    ragged: tuple | None = None  # (low, high) inclusive range of seqlens, or None for full length

    @property
    def rows(self) -> int:
        return self.b * self.s * self.h


@dataclass(frozen=True)
class GQAShape:
    b: int
    s: int
    hq: int
    hkv: int
    d: int
    t_max: int
    scale: float
    seed: int
    ragged: tuple | None = None

    @property
    def rows(self) -> int:
        return self.b * self.s * self.hq


# The workloads. Their names say what they are.
MLA_TINY = MLAShape(b=1, s=1, h=16, k=64, p=16, t_max=256, scale=1.0 / math.sqrt(48), seed=0)
GQA_LAYER = GQAShape(b=32, s=1, hq=64, hkv=8, d=128, t_max=4096, scale=1.0 / math.sqrt(128), seed=1)
MLA_DSV3 = MLAShape(b=32, s=1, h=128, k=512, p=64, t_max=4096, scale=1.0 / math.sqrt(192), seed=2)
MLA_MTP4 = MLAShape(b=32, s=4, h=128, k=512, p=64, t_max=4096, scale=1.0 / math.sqrt(192), seed=3)
MLA_RAGGED = MLAShape(b=64, s=1, h=128, k=512, p=64, t_max=32768, scale=1.0 / math.sqrt(192), seed=4,
                      ragged=(1024, 32768))
MTP_SWEEP = (1, 2, 4, 8, 16, 32)
# The two ends of the grouped family at the layer's head geometry ("Why MLA and MTP Fight Each Other",
# introduction table: MQA's intensity is the number of query heads, MHA's exactly one): one KV head
# shared by all 64 query heads, and 64 KV heads, one per query head (b=8 keeps its cache at 1 GiB).
GQA_MQA = GQAShape(b=32, s=1, hq=64, hkv=1, d=128, t_max=4096, scale=1.0 / math.sqrt(128), seed=8)
GQA_MHA = GQAShape(b=8, s=1, hq=64, hkv=64, d=128, t_max=4096, scale=1.0 / math.sqrt(128), seed=9)
# The layer's geometry with 4 draft tokens per sequence (the MTP step of "Why MLA and MTP Fight Each Other"
# applied to the grouped layer): 32 query rows per KV head under the drafts' causal mask.
GQA_MTP4 = GQAShape(b=32, s=4, hq=64, hkv=8, d=128, t_max=4096, scale=1.0 / math.sqrt(128), seed=10)
# The grouped geometry of the "MQA, GQA & MLA" lesson ("01 · Concept": 24 query heads in 4 groups of 6,
# head dimension 256) at that page's full context: its 16 GiB per sequence over 16 caching layers at
# 4 KiB per token per layer is 262,144 tokens. One sequence, one layer: K and V are 512 MiB each.
GQA_LONG = GQAShape(b=1, s=1, hq=24, hkv=4, d=256, t_max=262144, scale=1.0 / 16.0, seed=6)


def mla_mtp(s: int) -> MLAShape:
    """DeepSeek-V3-like shapes with s draft tokens per sequence (seed 3 for every s)."""
    return MLAShape(b=32, s=s, h=128, k=512, p=64, t_max=4096, scale=1.0 / math.sqrt(192), seed=3)


WORKLOADS = {
    "mla_tiny": MLA_TINY,
    "gqa_layer": GQA_LAYER,
    "mla_dsv3": MLA_DSV3,
    "mla_mtp4": MLA_MTP4,
    "mla_ragged": MLA_RAGGED,
    "gqa_mqa": GQA_MQA,
    "gqa_mha": GQA_MHA,
    "gqa_mtp4": GQA_MTP4,
}


def _normal_bf16(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32, device=gen.device).to(torch.bfloat16)


def _seqlens(gen: torch.Generator, b: int, t_max: int, ragged) -> torch.Tensor:
    if ragged is None:
        return torch.full((b,), t_max, dtype=torch.int32, device=gen.device)
    lo, hi = ragged
    return torch.randint(lo, hi + 1, (b,), generator=gen, dtype=torch.int64, device=gen.device).to(torch.int32)


def make_mla(shape: MLAShape, seqlens=None, device=None):
    """Return (q_lat, q_rope, cache, seqlens) as CPU tensors (bf16, bf16, bf16, int32),
    or, with ``device``, drawn by a generator on that device and left there (seqlens too)."""
    gen = torch.Generator(device=device if device is not None else "cpu").manual_seed(shape.seed)
    sl = _seqlens(gen, shape.b, shape.t_max, shape.ragged)
    if seqlens is not None:
        sl = torch.as_tensor(seqlens, dtype=torch.int32).clone().to(gen.device)
    q_lat = _normal_bf16(gen, (shape.b, shape.s, shape.h, shape.k))
    q_rope = _normal_bf16(gen, (shape.b, shape.s, shape.h, shape.p))
    cache = _normal_bf16(gen, (shape.b, shape.t_max, shape.k + shape.p))
    return q_lat, q_rope, cache, sl


def make_gqa(shape: GQAShape, seqlens=None, device=None):
    """Return (q, k, v, seqlens) as CPU tensors (bf16 x3, int32), or, with ``device``,
    drawn by a generator on that device and left there (seqlens too)."""
    gen = torch.Generator(device=device if device is not None else "cpu").manual_seed(shape.seed)
    sl = _seqlens(gen, shape.b, shape.t_max, shape.ragged)
    if seqlens is not None:
        sl = torch.as_tensor(seqlens, dtype=torch.int32).clone().to(gen.device)
    q = _normal_bf16(gen, (shape.b, shape.s, shape.hq, shape.d))
    k = _normal_bf16(gen, (shape.b, shape.t_max, shape.hkv, shape.d))
    v = _normal_bf16(gen, (shape.b, shape.t_max, shape.hkv, shape.d))
    return q, k, v, sl


def sample_rows(total_rows: int, n: int, seed: int) -> torch.Tensor:
    """A fixed, seeded sample of n distinct flattened row ids (sorted), always
    including the first and last row."""
    n = min(n, total_rows)
    gen = torch.Generator().manual_seed(1000 + seed)
    idx = torch.randperm(total_rows, generator=gen)[:n]
    idx[0] = 0
    if n > 1:
        idx[1] = total_rows - 1
    return torch.unique(idx).to(torch.int64)
