"""Pins for the fp64 oracle against things it does not compute itself.

Each test checks the oracle against an independent library routine (torch's
fp64 scaled_dot_product_attention and logsumexp), a closed form, an algebraic
identity the source pages state, or an invariant of the definition. They are
chosen so that a plausible slip in the oracle (a dropped rope term, V taken from
the wrong columns, a transposed operand, a wrong KV-head map, an off-by-one in
the draft mask, a log in the wrong base) breaks at least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as wl


def bf16_to_f64(t):
    return t.to(torch.float64)


def rand_mla(b, s, h, k, p, t, seed, seqlens=None):
    shape = wl.MLAShape(b=b, s=s, h=h, k=k, p=p, t_max=t, scale=1.0 / math.sqrt(k + p), seed=seed)
    return (shape,) + wl.make_mla(shape, seqlens=seqlens)


def rand_gqa(b, s, hq, hkv, d, t, seed, seqlens=None):
    shape = wl.GQAShape(b=b, s=s, hq=hq, hkv=hkv, d=d, t_max=t, scale=1.0 / math.sqrt(d), seed=seed)
    return (shape,) + wl.make_gqa(shape, seqlens=seqlens)


def visible(L, s, i, t_max):
    L = max(0, min(int(L), t_max))
    return L - s + i + 1


def sdpa_rows(Q, K, V, n_vis, scale):
    """torch fp64 SDPA with an explicit boolean mask, plus torch.logsumexp for lse.

    Q [nq, dk], K [t, dk], V [t, dv]. Only rows with n_vis >= 1 are meaningful.
    """
    t = K.shape[0]
    mask = torch.arange(t)[None, :] < torch.as_tensor(n_vis)[:, None]
    out = F.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=mask[None], scale=scale)[0]
    scores = (Q @ K.T) * scale
    lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
    return out, lse


# ------------------------------------------------------------------ generic
def test_generic_matches_torch_sdpa(oracle_mod):
    g = torch.Generator().manual_seed(11)
    nq, t, dk, dv = 7, 50, 24, 10
    Q = torch.randn(nq, dk, generator=g, dtype=torch.float64)
    K = torch.randn(t, dk, generator=g, dtype=torch.float64)
    V = torch.randn(t, dv, generator=g, dtype=torch.float64)
    n_vis = [1, 2, 17, 33, 49, 50, 50]
    scale = 0.37
    out, lse = oracle_mod.attn_generic(Q.numpy(), K.numpy(), V.numpy(), n_vis, scale)
    ref, ref_lse = sdpa_rows(Q, K, V, n_vis, scale)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------- MLA
@pytest.mark.parametrize("s", [1, 3])
def test_mla_matches_torch_sdpa(oracle_mod, s):
    shape, ql, qr, c, sl = rand_mla(2, s, 4, 32, 8, 40, seed=5, seqlens=[40, 23])
    out, lse = oracle_mod.mla(ql, qr, c, sl, shape.scale)
    for bi in range(2):
        Kf = bf16_to_f64(c[bi])            # keys: latent and rope columns
        Vf = bf16_to_f64(c[bi, :, :32])    # values: latent columns only
        for i in range(s):
            Q = torch.cat([bf16_to_f64(ql[bi, i]), bf16_to_f64(qr[bi, i])], dim=-1)
            n = visible(sl[bi], s, i, 40)
            ref, ref_lse = sdpa_rows(Q, Kf, Vf, [n] * 4, shape.scale)
            np.testing.assert_allclose(out[bi, i], ref.numpy(), atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[bi, i], ref_lse.numpy(), atol=1e-12, rtol=0)


def test_mla_is_mqa_with_wide_head(oracle_mod):
    """Absorbed MLA in decode is MQA with key width k+p and value width k."""
    shape, ql, qr, c, sl = rand_mla(1, 2, 6, 48, 16, 33, seed=6)
    out, lse = oracle_mod.mla(ql, qr, c, sl, shape.scale)
    K = bf16_to_f64(c[0]).numpy()
    V = bf16_to_f64(c[0, :, :48]).numpy()
    for i in range(2):
        Q = torch.cat([bf16_to_f64(ql[0, i]), bf16_to_f64(qr[0, i])], -1).numpy()
        n = visible(sl[0], 2, i, 33)
        o2, l2 = oracle_mod.attn_generic(Q, K, V, [n] * 6, shape.scale)
        np.testing.assert_allclose(out[0, i], o2, atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse[0, i], l2, atol=1e-13, rtol=0)


def test_absorption_identity(oracle_mod):
    """Un-absorbed attention with K_h = Z Wk, V_h = Z Wv equals the absorbed
    latent result mapped through Wv, with q_lat = Wk q_h.

    Wk, Wv and the per-head queries have small integer entries so q_lat is exact
    in bf16; the cache is ordinary bf16 noise.
    """
    h, k, p, d, dv, t, s = 16, 64, 16, 32, 24, 96, 1
    g = torch.Generator().manual_seed(21)
    Z = torch.randn(1, t, k + p, generator=g).to(torch.bfloat16)
    Wk = torch.randint(-1, 2, (h, k, d), generator=g).to(torch.float64)
    Wv = torch.randint(-1, 2, (h, k, dv), generator=g).to(torch.float64)
    Qh = torch.randint(-1, 2, (h, d), generator=g).to(torch.float64)
    q_rope = torch.randn(1, s, h, p, generator=g).to(torch.bfloat16)
    q_lat64 = torch.einsum("hkd,hd->hk", Wk, Qh)
    assert q_lat64.abs().max() <= 64  # exactly representable in bf16
    q_lat = q_lat64.to(torch.bfloat16).reshape(1, s, h, k)
    assert torch.equal(q_lat.to(torch.float64).reshape(h, k), q_lat64)
    scale = 1.0 / math.sqrt(48)
    sl = torch.tensor([t], dtype=torch.int32)
    out_lat, lse = oracle_mod.mla(q_lat, q_rope, Z, sl, scale)
    Zl = bf16_to_f64(Z[0, :, :k])
    kpe = bf16_to_f64(Z[0, :, k:])
    for hh in range(h):
        K_h = torch.cat([Zl @ Wk[hh], kpe], -1)           # decompressed keys + rope part
        V_h = Zl @ Wv[hh]                                  # decompressed values
        Q_full = torch.cat([Qh[hh], bf16_to_f64(q_rope[0, 0, hh])])[None]
        o_h, l_h = oracle_mod.attn_generic(Q_full.numpy(), K_h.numpy(), V_h.numpy(), [t], scale)
        np.testing.assert_allclose(out_lat[0, 0, hh] @ Wv[hh].numpy(), o_h[0], atol=1e-10, rtol=1e-12)
        np.testing.assert_allclose(lse[0, 0, hh], l_h[0], atol=1e-11, rtol=0)


def test_head_projection_identity_and_absorption(oracle_mod):
    """The per-head projections (query absorption, output decompression):
    identity weights reproduce their input, and absorbed attention taken through
    both projections equals un-absorbed attention on K_h = Z Wk, V_h = Z Wv
    ("Mla Analysis" skill page, "Absorption Trick (FlashMLA)"). Integer-valued
    weights and queries keep q_lat exact in bf16."""
    g = torch.Generator().manual_seed(31)
    A = torch.randn(2, 3, 4, 32, generator=g).to(torch.bfloat16)
    eye = torch.zeros(4, 40, 32)
    eye[:, :32, :] = torch.eye(32)
    C = oracle_mod.head_projection(A, eye.to(torch.bfloat16))
    np.testing.assert_array_equal(C[..., :32], bf16_to_f64(A).numpy())
    np.testing.assert_array_equal(C[..., 32:], 0.0)

    h, k, p, d, dv, t = 8, 64, 16, 32, 24, 80
    Z = torch.randn(1, t, k + p, generator=g).to(torch.bfloat16)
    Wk = torch.randint(-1, 2, (h, k, d), generator=g).to(torch.bfloat16)
    WvT = torch.randint(-1, 2, (h, dv, k), generator=g).to(torch.bfloat16)
    Qh = torch.randint(-1, 2, (1, 1, h, d), generator=g).to(torch.bfloat16)
    q_rope = torch.randn(1, 1, h, p, generator=g).to(torch.bfloat16)
    q_lat64 = oracle_mod.head_projection(Qh, Wk)                 # [1, 1, h, k]
    q_lat = torch.from_numpy(q_lat64).to(torch.bfloat16)
    assert np.array_equal(bf16_to_f64(q_lat).numpy(), q_lat64)   # exact in bf16
    scale = 1.0 / math.sqrt(48)
    out_lat, lse = oracle_mod.mla(q_lat, q_rope, Z, torch.tensor([t], dtype=torch.int32), scale)
    out = oracle_mod.head_projection(out_lat, WvT)                # [1, 1, h, dv]
    Zl, kpe = bf16_to_f64(Z[0, :, :k]), bf16_to_f64(Z[0, :, k:])
    for hh in range(h):
        K_h = torch.cat([Zl @ bf16_to_f64(Wk[hh]), kpe], -1)
        V_h = Zl @ bf16_to_f64(WvT[hh]).T
        Q_full = torch.cat([bf16_to_f64(Qh[0, 0, hh]), bf16_to_f64(q_rope[0, 0, hh])])[None]
        o_h, l_h = oracle_mod.attn_generic(Q_full.numpy(), K_h.numpy(), V_h.numpy(), [t], scale)
        np.testing.assert_allclose(out[0, 0, hh], o_h[0], atol=1e-10, rtol=1e-12)
        np.testing.assert_allclose(lse[0, 0, hh], l_h[0], atol=1e-11, rtol=0)


def test_mla_single_visible_row(oracle_mod):
    """With one visible cache row the output is that row's latent part and lse its score."""
    shape, ql, qr, c, _ = rand_mla(1, 1, 3, 16, 8, 10, seed=7)
    sl = torch.tensor([1], dtype=torch.int32)
    out, lse = oracle_mod.mla(ql, qr, c, sl, 0.5)
    np.testing.assert_array_equal(out[0, 0], np.broadcast_to(bf16_to_f64(c[0, 0, :16]).numpy(), (3, 16)))
    z0 = 0.5 * (bf16_to_f64(ql[0, 0]) @ bf16_to_f64(c[0, 0, :16]) + bf16_to_f64(qr[0, 0]) @ bf16_to_f64(c[0, 0, 16:]))
    np.testing.assert_allclose(lse[0, 0], z0.numpy(), atol=1e-13)


def test_mla_zero_query_gives_mean(oracle_mod):
    """q = 0: uniform weights, output = mean of the visible latent rows, lse = ln n."""
    shape, ql, qr, c, _ = rand_mla(2, 2, 2, 16, 8, 20, seed=8)
    ql.zero_()
    qr.zero_()
    sl = torch.tensor([20, 13], dtype=torch.int32)
    out, lse = oracle_mod.mla(ql, qr, c, sl, 0.3)
    for bi in range(2):
        for i in range(2):
            n = visible(sl[bi], 2, i, 20)
            mean = bf16_to_f64(c[bi, :n, :16]).mean(0).numpy()
            np.testing.assert_allclose(out[bi, i], np.broadcast_to(mean, (2, 16)), atol=1e-14)
            np.testing.assert_allclose(lse[bi, i], math.log(n), atol=1e-14)


def test_mla_equal_rows(oracle_mod):
    """All cache rows equal: output = that row, lse = z + ln n."""
    shape, ql, qr, c, _ = rand_mla(1, 1, 4, 16, 8, 12, seed=9)
    c[:] = c[0, 0]
    sl = torch.tensor([9], dtype=torch.int32)
    out, lse = oracle_mod.mla(ql, qr, c, sl, 0.25)
    row = bf16_to_f64(c[0, 0])
    for hh in range(4):
        z = 0.25 * (torch.cat([bf16_to_f64(ql[0, 0, hh]), bf16_to_f64(qr[0, 0, hh])]) @ row)
        np.testing.assert_allclose(out[0, 0, hh], row[:16].numpy(), atol=1e-13)
        np.testing.assert_allclose(lse[0, 0, hh], z.item() + math.log(9), atol=1e-12)


def test_mla_drafts_reduce_to_single_token(oracle_mod):
    """Draft i of an s-token call equals an s=1 call whose sequence length is L - s + i + 1."""
    s = 4
    shape, ql, qr, c, _ = rand_mla(2, s, 3, 32, 8, 30, seed=10)
    sl = torch.tensor([30, 17], dtype=torch.int32)
    out, lse = oracle_mod.mla(ql, qr, c, sl, 0.2)
    for bi in range(2):
        for i in range(s):
            n = visible(sl[bi], s, i, 30)
            o1, l1 = oracle_mod.mla(ql[bi:bi + 1, i:i + 1], qr[bi:bi + 1, i:i + 1], c[bi:bi + 1],
                                    torch.tensor([n], dtype=torch.int32), 0.2)
            np.testing.assert_array_equal(out[bi, i], o1[0, 0])
            np.testing.assert_array_equal(lse[bi, i], l1[0, 0])


def test_mla_split_and_merge(oracle_mod):
    """Attention over a partition of the visible rows, merged by log-sum-exp weights,
    equals attention over all of them (natural-log lse)."""
    shape, ql, qr, c, _ = rand_mla(1, 1, 5, 32, 8, 64, seed=12)
    full_o, full_l = oracle_mod.mla(ql, qr, c, torch.tensor([64], dtype=torch.int32), 0.2)
    K = bf16_to_f64(c[0]).numpy()
    V = bf16_to_f64(c[0, :, :32]).numpy()
    Q = torch.cat([bf16_to_f64(ql[0, 0]), bf16_to_f64(qr[0, 0])], -1).numpy()
    parts = [(0, 7), (7, 40), (40, 64)]
    outs, lses = [], []
    for a, e in parts:
        o, l = oracle_mod.attn_generic(Q, K[a:e], V[a:e], [e - a] * 5, 0.2)
        outs.append(o)
        lses.append(l)
    lses = np.stack(lses)                       # [parts, rows]
    tot = np.logaddexp.reduce(lses, axis=0)
    merged = sum(np.exp(lses[r] - tot)[:, None] * outs[r] for r in range(len(parts)))
    np.testing.assert_allclose(merged, full_o[0, 0], atol=1e-13)
    np.testing.assert_allclose(tot, full_l[0, 0], atol=1e-13)


def test_mla_row_permutation_invariance(oracle_mod):
    shape, ql, qr, c, _ = rand_mla(1, 1, 3, 16, 8, 25, seed=13)
    sl = torch.tensor([21], dtype=torch.int32)
    o1, l1 = oracle_mod.mla(ql, qr, c, sl, 0.3)
    perm = torch.randperm(21, generator=torch.Generator().manual_seed(0))
    c2 = c.clone()
    c2[0, :21] = c[0, perm]
    o2, l2 = oracle_mod.mla(ql, qr, c2, sl, 0.3)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_mla_empty_and_clamped_rows(oracle_mod):
    """Rows that see no cache row give 0 / -inf; seqlens outside [0, t_max] are clamped."""
    s = 3
    shape, ql, qr, c, _ = rand_mla(3, s, 2, 16, 8, 10, seed=14)
    sl = torch.tensor([1, -5, 99], dtype=torch.int32)
    out, lse = oracle_mod.mla(ql, qr, c, sl, 0.3)
    # b=0: L=1, s=3 -> drafts 0,1 see nothing, draft 2 sees 1 row.
    assert np.all(out[0, :2] == 0) and np.all(np.isneginf(lse[0, :2]))
    np.testing.assert_array_equal(out[0, 2], np.broadcast_to(bf16_to_f64(c[0, 0, :16]).numpy(), (2, 16)))
    # b=1: negative length clamps to 0.
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    # b=2: 99 clamps to t_max = 10.
    o_ref, l_ref = oracle_mod.mla(ql[2:], qr[2:], c[2:], torch.tensor([10], dtype=torch.int32), 0.3)
    np.testing.assert_array_equal(out[2], o_ref[0])
    np.testing.assert_array_equal(lse[2], l_ref[0])


def test_mla_rows_subset(oracle_mod):
    shape, ql, qr, c, sl = rand_mla(2, 2, 4, 16, 8, 20, seed=15, seqlens=[20, 11])
    out, lse = oracle_mod.mla(ql, qr, c, sl, 0.3)
    rows = [0, 5, 9, 15]
    o2, l2 = oracle_mod.mla(ql, qr, c, sl, 0.3, rows=rows)
    np.testing.assert_array_equal(o2, out.reshape(-1, 16)[rows])
    np.testing.assert_array_equal(l2, lse.reshape(-1)[rows])


def test_mla_mac_count_matches_closed_form(oracle_mod):
    from decode_attention_bf16_amd import costmodel as cm
    s = 3
    shape, ql, qr, c, sl = rand_mla(3, s, 4, 32, 16, 40, seed=16, seqlens=[40, 25, 2])
    _, _, macs = oracle_mod.mla(ql, qr, c, sl, 0.2, return_macs=True)
    masked = cm.mla_absorbed_ragged(sl.tolist(), 4, s, 32, 16, 40, masked=True)
    assert 2 * macs == masked.flops
    # Full-length sequences at s=1: the count equals the pages' closed form 2bhst(2k+p).
    shape, ql, qr, c, sl = rand_mla(2, 1, 4, 32, 16, 40, seed=17)
    _, _, macs = oracle_mod.mla(ql, qr, c, sl, 0.2, return_macs=True)
    assert 2 * macs == cm.mla_absorbed(2, 4, 1, 40, 32, 16).flops


def test_mla_statistics_smoke(oracle_mod):
    """Loose sanity only: with N(0,1) inputs the scaled scores have variance about
    (k+p)*scale^2, so the mean lse sits near ln n + var/2."""
    shape, ql, qr, c, sl = rand_mla(1, 1, 64, 64, 16, 512, seed=18)
    _, lse = oracle_mod.mla(ql, qr, c, sl, 1.0 / math.sqrt(80))
    assert abs(lse.mean() - (math.log(512) + 0.5)) < 0.2


def test_mla_tiny_workload_runs(oracle_mod):
    ql, qr, c, sl = wl.make_mla(wl.MLA_TINY)
    out, lse = oracle_mod.mla(ql, qr, c, sl, wl.MLA_TINY.scale)
    assert out.shape == (1, 1, 16, 64) and np.isfinite(out).all() and np.isfinite(lse).all()


# ---------------------------------------------------------------------- GQA
def test_gqa_mha_matches_torch_sdpa(oracle_mod):
    """hkv = hq is MHA: every query head has its own K/V head."""
    shape, q, k, v, sl = rand_gqa(2, 2, 4, 4, 16, 30, seed=30, seqlens=[30, 19])
    out, lse = oracle_mod.gqa(q, k, v, sl, shape.scale)
    for bi in range(2):
        for i in range(2):
            n = visible(sl[bi], 2, i, 30)
            for hh in range(4):
                ref, rl = sdpa_rows(bf16_to_f64(q[bi, i, hh])[None], bf16_to_f64(k[bi, :, hh]),
                                    bf16_to_f64(v[bi, :, hh]), [n], shape.scale)
                np.testing.assert_allclose(out[bi, i, hh], ref[0].numpy(), atol=1e-12)
                np.testing.assert_allclose(lse[bi, i, hh], rl[0].item(), atol=1e-12)


def test_gqa_mqa_matches_torch_sdpa(oracle_mod):
    """hkv = 1 is MQA: all query heads read the same K/V head."""
    shape, q, k, v, sl = rand_gqa(1, 1, 6, 1, 16, 25, seed=31)
    out, lse = oracle_mod.gqa(q, k, v, sl, shape.scale)
    ref, rl = sdpa_rows(bf16_to_f64(q[0, 0]), bf16_to_f64(k[0, :, 0]), bf16_to_f64(v[0, :, 0]), [25] * 6,
                        shape.scale)
    np.testing.assert_allclose(out[0, 0], ref.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], rl.numpy(), atol=1e-12)


def test_gqa_equals_mha_on_repeated_kv(oracle_mod):
    """GQA with groups of g equals MHA on K/V heads repeated g times each (contiguous groups)."""
    shape, q, k, v, sl = rand_gqa(2, 3, 8, 2, 16, 21, seed=32, seqlens=[21, 10])
    out, lse = oracle_mod.gqa(q, k, v, sl, shape.scale)
    k_rep = k.repeat_interleave(4, dim=2)
    v_rep = v.repeat_interleave(4, dim=2)
    out2, lse2 = oracle_mod.gqa(q, k_rep, v_rep, sl, shape.scale)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)
    # and the repeated MHA against torch SDPA for one head of the second group
    ref, rl = sdpa_rows(bf16_to_f64(q[1, 2, 5])[None], bf16_to_f64(k[1, :, 1]), bf16_to_f64(v[1, :, 1]),
                        [visible(10, 3, 2, 21)], shape.scale)
    np.testing.assert_allclose(out[1, 2, 5], ref[0].numpy(), atol=1e-12)


def test_gqa_drafts_and_empty_rows(oracle_mod):
    s = 4
    shape, q, k, v, _ = rand_gqa(2, s, 4, 2, 16, 12, seed=33)
    sl = torch.tensor([12, 2], dtype=torch.int32)
    out, lse = oracle_mod.gqa(q, k, v, sl, 0.25)
    for bi in range(2):
        for i in range(s):
            n = visible(sl[bi], s, i, 12)
            if n <= 0:
                assert np.all(out[bi, i] == 0) and np.all(np.isneginf(lse[bi, i]))
                continue
            o1, l1 = oracle_mod.gqa(q[bi:bi + 1, i:i + 1], k[bi:bi + 1], v[bi:bi + 1],
                                    torch.tensor([n], dtype=torch.int32), 0.25)
            np.testing.assert_array_equal(out[bi, i], o1[0, 0])
            np.testing.assert_array_equal(lse[bi, i], l1[0, 0])


def test_gqa_zero_query_and_mac_count(oracle_mod):
    from decode_attention_bf16_amd import costmodel as cm
    shape, q, k, v, sl = rand_gqa(2, 1, 8, 2, 16, 20, seed=34, seqlens=[20, 7])
    q.zero_()
    out, lse, macs = oracle_mod.gqa(q, k, v, sl, 0.3, return_macs=True)
    for bi, n in enumerate([20, 7]):
        for hh in range(8):
            mean = bf16_to_f64(v[bi, :n, hh // 4]).mean(0).numpy()
            np.testing.assert_allclose(out[bi, 0, hh], mean, atol=1e-14)
            np.testing.assert_allclose(lse[bi, 0, hh], math.log(n), atol=1e-14)
    assert 2 * macs == cm.gqa_ragged([20, 7], 1, 8, 2, 16, 20, masked=True).flops
