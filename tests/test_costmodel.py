"""Cost-model closed forms against the numbers the source pages print.

Each fixture row in tests/golden/pages_worked_values.json carries its citation.
"""
import json
import math
import os

import pytest

from decode_attention_bf16_amd import costmodel as cm

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_values.json")))


@pytest.mark.parametrize("row", GOLDEN["kv_bytes_per_token"], ids=lambda r: r["cite"][:60])
def test_kv_bytes_per_token(row):
    got = cm.kv_bytes_per_token(row["layers"], row["kv_heads"], row["head_dim"], row["bytes_per_elem"])
    assert got == row["value"]


@pytest.mark.parametrize("row", GOLDEN["kv_cache_bytes"], ids=lambda r: r["cite"][:60])
def test_kv_cache_gib(row):
    got = cm.kv_bytes_per_token(row["layers"], row["kv_heads"], row["head_dim"]) * row["tokens"]
    assert got / 2**30 == pytest.approx(row["gib"], rel=1e-12)


@pytest.mark.parametrize("row", GOLDEN["arithmetic_intensity"], ids=lambda r: r["cite"][:60])
def test_arithmetic_intensity(row):
    f = row["form"]
    if f == "mla_absorbed":
        ai = cm.mla_absorbed(row["b"], row["h"], row["s"], row["t"], row["k"], row["p"]).ai
    elif f == "mla_kv_only":
        ai = cm.mla_absorbed_kv_only_ai(row["h"], row["k"], row["p"])
    elif f == "mla_unabsorbed":
        ai = cm.mla_unabsorbed(row["b"], row["h"], row["s"], row["t"], row["d"], row["p"]).ai
    elif f == "gqa_kv_only":
        ai = cm.gqa_kv_only_ai(row["hq"], row["hkv"])
    else:
        raise AssertionError(f)
    assert abs(ai - row["value"]) <= row["abs_tol"] + 1e-12


def test_gqa_ai_matches_kv_only_form_when_q_o_negligible():
    # Full closed form (K+V+Q+O bytes) approaches hq/hkv as t grows.
    c = cm.gqa(32, 1, 64, 8, 128, 4096)
    assert c.flops == 4 * 32 * 64 * 4096 * 128
    assert c.bytes == 2 * (2 * 32 * 4096 * 8 * 128 + 2 * 32 * 64 * 128)
    assert c.ai == pytest.approx(7.98, abs=0.01)


def test_mla_dsv3_closed_form_values():
    c = cm.mla_absorbed(32, 128, 1, 4096, 512, 64)
    assert c.flops == 36_507_222_016
    assert c.bytes == 159_907_840
    c4 = cm.mla_absorbed(32, 128, 4, 4096, 512, 64)
    assert c4.flops == 146_028_888_064
    assert c4.bytes == 186_646_528


def test_masked_flops_vs_nominal():
    # Draft i sees L - s + i + 1 rows; with s=4, L=4096 the masked count is
    # 2h(2k+p) * sum(4093..4096).
    m = cm.mla_absorbed_ragged([4096] * 32, 128, 4, 512, 64, 4096, masked=True)
    assert m.flops == 2 * 128 * 1088 * 32 * (4093 + 4094 + 4095 + 4096)
    n = cm.mla_absorbed_ragged([4096] * 32, 128, 4, 512, 64, 4096)
    assert n.flops == cm.mla_absorbed(32, 128, 4, 4096, 512, 64).flops


@pytest.mark.parametrize("row", GOLDEN["flop_ratio"], ids=lambda r: r["cite"][:60])
def test_flop_ratio_latent_vs_decompressed(row):
    r = cm.mla_absorbed(1, 1, 1, 1, row["k"], row["p"]).flops / cm.mla_unabsorbed(1, 1, 1, 1, row["d"], row["p"]).flops
    assert abs(r - row["value"]) <= row["abs_tol"]


@pytest.mark.parametrize("row", GOLDEN["ridge_points"], ids=lambda r: r["cite"][:60])
def test_ridge_points(row):
    r = cm.ridge(row["peak_tflops"] * 1e12, row["bw_tbs"] * 1e12)
    assert abs(r - row["value"]) <= row["abs_tol"]


def test_mla_near_two_times_heads():
    # The constant in front of the head count is (2k+p)/(k+p): a little under 2.
    c = cm.mla_absorbed_kv_only_ai(128, 512, 64) / 128
    assert 1.8 < c < 2.0
    assert c == pytest.approx(1088 / 576)


def test_ridge_crossing():
    s_star = cm.mla_ridge_crossing_s(128, 512, 64, 4096)
    assert 1.0 < s_star < 2.0
    # AI at s_star equals the ridge.
    R = cm.ridge(cm.MI355X_BF16_FLOPS, cm.MI355X_HBM_BYTES_PER_S)
    h, k, p, t, w = 128, 512, 64, 4096, 2
    ai = 2 * h * s_star * t * (2 * k + p) / (w * (h * s_star * (2 * k + p) + t * (k + p)))
    assert ai == pytest.approx(R, rel=1e-9)
    # H100's ridge from the pages gives a crossing near 1.32.
    s_h100 = cm.mla_ridge_crossing_s(128, 512, 64, 4096, peak_flops=989.5e12, bw=3.35e12)
    assert s_h100 == pytest.approx(1.317, abs=0.01)


def test_split_latent_interpolates():
    # With no decompressed tokens the split form's latent term (4bhsok) plus the rope term
    # equals the absorbed FLOPs; with no latent tokens it equals the decompressed FLOPs.
    b, h, s, t, d, k, p = 2, 4, 3, 64, 16, 32, 8
    lat = cm.mla_split_latent(b, h, s, o=t, n=0, d=d, k=k, p=p)
    assert lat.flops == cm.mla_absorbed(b, h, s, t, k, p).flops
    dec = cm.mla_split_latent(b, h, s, o=0, n=t, d=d, k=k, p=p)
    assert dec.flops == cm.mla_unabsorbed(b, h, s, t, d, p).flops
