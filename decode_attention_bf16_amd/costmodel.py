"""Closed-form FLOP and HBM-byte counts for decode attention, and roofline helpers.

These are the *algorithmic* counts the benchmark credits: the work the method
must do and the bytes it must move at least once, independent of how a kernel
tiles, pads or re-reads. Formulas:

* MLA absorbed (latent) decode -- "Mla Analysis" skill page, "Cost Models",
  FlashMLA entry: FLOPs 2*b*h*s*t*(2k+p); bytes w*(b*h*s*(2k+p) + b*t*(k+p)).
  The byte term charges the queries (k+p per row), the latent outputs (k per
  row) and the latent+rope cache read once.
* Un-absorbed MLA (decompressed K/V) -- same page, FlashAttention entry:
  FLOPs 2*b*h*s*t*(2d+p); bytes w*b*h*(s+t)*(2d+p).
* Split latent + decompressed cache -- same page, MLAvar6+ entry.
* GQA/MQA/MHA decode -- arithmetic intensity depends on head counts only ("Why
  MLA and MTP Fight Each Other", introduction table): FLOPs 4*b*hq*s*t*d
  (two matmuls of 2 FLOPs per multiply-add), bytes K+V = 2*b*t*hkv*d*w plus
  the queries and outputs.
* KV bytes per token -- "MHA vs GQA 70B" Q&A page, section 3:
  2 (K and V) * layers * kv_heads * head_dim * bytes per element.
* Ridge point = dense peak FLOP/s / HBM bytes/s ("Why MLA and MTP Fight Each
  Other", section 1 table of balance points).

Softmax is not counted, following the same page's choice to leave it out as
small next to the two matmuls.
"""
from __future__ import annotations

from dataclasses import dataclass

W_BF16 = 2  # bytes per bf16 element

# MI355X published peaks used for the roofline (dense, no sparsity).
MI355X_HBM_BYTES_PER_S = 8.0e12
MI355X_BF16_FLOPS = 2.5e15
MI355X_FP32_VECTOR_FLOPS = 157.3e12


@dataclass(frozen=True)
class Cost:
    flops: float
    bytes: float

    @property
    def ai(self) -> float:
        return self.flops / self.bytes


# ---------------------------------------------------------------- MLA absorbed
def mla_absorbed(b, h, s, t, k, p, w=W_BF16) -> Cost:
    """Nominal cost of absorbed MLA decode with every sequence t long."""
    flops = 2.0 * b * h * s * t * (2 * k + p)
    byts = w * (b * h * s * (2 * k + p) + b * t * (k + p))
    return Cost(flops, byts)


def mla_absorbed_kv_only_ai(h, k, p) -> float:
    """AI at s=1 when only the latent+rope cache bytes are charged: h(2k+p)/(k+p)."""
    return h * (2 * k + p) / (k + p)


def visible_rows(seqlens, s, t_max):
    """Sum over sequences and drafts of the visible cache rows n_i = L - s + i + 1."""
    tot = 0
    for L in seqlens:
        L = max(0, min(int(L), t_max))
        for i in range(s):
            tot += max(0, L - s + i + 1)
    return tot


def mla_absorbed_ragged(seqlens, h, s, k, p, t_max, w=W_BF16, masked=False) -> Cost:
    """Cost with per-sequence lengths L_b.

    Nominal (masked=False): the closed form with t -> L_b, summed over b.
    Masked: FLOPs counted on the rows each draft actually sees.
    """
    flops = 0.0
    byts = 0.0
    for L in seqlens:
        L = max(0, min(int(L), t_max))
        flops += 2.0 * h * s * L * (2 * k + p)
        byts += w * (h * s * (2 * k + p) + L * (k + p))
    if masked:
        flops = 2.0 * h * (2 * k + p) * visible_rows(seqlens, s, t_max)
    return Cost(flops, byts)


# ------------------------------------------------------------ un-absorbed MLA
def mla_unabsorbed(b, h, s, t, d, p, w=W_BF16) -> Cost:
    flops = 2.0 * b * h * s * t * (2 * d + p)
    byts = w * b * h * (s + t) * (2 * d + p)
    return Cost(flops, byts)


def mla_split_latent(b, h, s, o, n, d, k, p, w=W_BF16) -> Cost:
    """Old tokens kept as latent (o of them), new tokens decompressed (n of them)."""
    t = o + n
    flops = 2.0 * b * h * s * t * p + 4.0 * b * h * s * n * d + 4.0 * b * h * s * o * k
    byts = w * (b * h * s * p + b * h * s * d + b * h * s * k + b * o * k + b * t * p
                + b * h * n * d + b * h * n * d + b * h * s * d + b * h * s * k)
    return Cost(flops, byts)


# -------------------------------------------------------------------- GQA
def gqa(b, s, hq, hkv, d, t, w=W_BF16) -> Cost:
    flops = 4.0 * b * hq * s * t * d
    byts = w * (2 * b * t * hkv * d + 2 * b * s * hq * d)
    return Cost(flops, byts)


def gqa_kv_only_ai(hq, hkv, s=1) -> float:
    """FLOPs / K+V bytes: 4*hq*s*d / (2*hkv*d*2) = s*hq/hkv."""
    return s * hq / hkv


def gqa_ragged(seqlens, s, hq, hkv, d, t_max, w=W_BF16, masked=False) -> Cost:
    flops = 0.0
    byts = 0.0
    for L in seqlens:
        L = max(0, min(int(L), t_max))
        flops += 4.0 * hq * s * L * d
        byts += w * (2 * L * hkv * d + 2 * s * hq * d)
    if masked:
        flops = 4.0 * hq * d * visible_rows(seqlens, s, t_max)
    return Cost(flops, byts)


# ---------------------------------------------------------- KV accounting
def kv_bytes_per_token(layers, kv_heads, head_dim, w=W_BF16) -> int:
    return 2 * layers * kv_heads * head_dim * w


def latent_bytes_per_token(layers, k, p, w=W_BF16) -> int:
    return layers * (k + p) * w


# --------------------------------------------------------------- roofline
def ridge(peak_flops, bw_bytes) -> float:
    return peak_flops / bw_bytes


def roofline_time(cost: Cost, peak_flops=MI355X_BF16_FLOPS, bw=MI355X_HBM_BYTES_PER_S) -> float:
    """Lower bound on run time: max(FLOPs/peak, bytes/bandwidth), seconds."""
    return max(cost.flops / peak_flops, cost.bytes / bw)


def roofline_bound(cost: Cost, peak_flops=MI355X_BF16_FLOPS, bw=MI355X_HBM_BYTES_PER_S) -> str:
    return "mfma" if cost.ai > ridge(peak_flops, bw) else "hbm"


def mla_ridge_crossing_s(h, k, p, t, peak_flops=MI355X_BF16_FLOPS, bw=MI355X_HBM_BYTES_PER_S,
                         w=W_BF16) -> float:
    """The (real-valued) s at which absorbed MLA's AI equals the ridge.

    AI(s) = 2hst(2k+p) / (w(hs(2k+p) + t(k+p))) = R  =>  s = R w t (k+p) / (h(2k+p)(2t - R w)).
    """
    R = ridge(peak_flops, bw)
    return R * w * t * (k + p) / (h * (2 * k + p) * (2 * t - R * w))
