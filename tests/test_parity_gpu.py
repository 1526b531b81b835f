"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

Bar (floating point): max |out - out_ref| <= 1e-2 * max |out_ref| over the
compared rows, and |lse - lse_ref| <= 1e-3 on rows that see at least one
cache row; rows that see none must be exactly out = 0, lse = -inf.
Every test compares every output row, the full-size workloads included, in
the launch configuration the benchmark times.
The workspace is poisoned (0xFF bytes = NaN) before every call so that a read
of an unwritten partial shows up.
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 1e-3


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def da():
    dev()
    import decode_attention_bf16_amd as pkg
    from decode_attention_bf16_amd import binding
    binding.load_library()
    return binding


def poisoned(nbytes, device):
    return torch.full((max(nbytes, 256),), 0xFF, dtype=torch.uint8, device=device)


def compare(out_gpu, lse_gpu, out_ref, lse_ref, what=""):
    o = out_gpu.detach().float().cpu().numpy().astype(np.float64).reshape(out_ref.shape)
    l = lse_gpu.detach().cpu().numpy().astype(np.float64).reshape(lse_ref.shape)
    empty = np.isneginf(lse_ref)
    assert np.all(np.isneginf(l[empty])), what + ": rows with no visible cache row must have lse=-inf"
    assert np.all(o[empty] == 0), what + ": rows with no visible cache row must be 0"
    full = ~empty
    if full.any():
        ref_max = np.abs(out_ref[full]).max()
        err = np.abs(o[full] - out_ref[full]).max()
        assert np.isfinite(o[full]).all(), what + ": non-finite output"
        assert err <= OUT_TOL * ref_max, "%s: max|dout| %.3e > %.1e * %.3e" % (what, err, OUT_TOL, ref_max)
        lerr = np.abs(l[full] - lse_ref[full]).max()
        assert lerr <= LSE_TOL, "%s: max|dlse| %.3e" % (what, lerr)


def run_mla(da, shape, tensors, num_workers=0, null_workspace=False):
    ql, qr, c, sl = tensors
    d = dev()
    g = [t.to(d) for t in (ql, qr, c, sl)]
    nbytes = da.mla_decode_workspace_size(shape.b, shape.s, shape.h, shape.k, shape.p, shape.t_max, num_workers)
    ws = None if null_workspace else poisoned(nbytes, d)
    # outputs poisoned too: with no workspace every row must be written by the tile kernel itself
    out = torch.full((shape.b, shape.s, shape.h, shape.k), float("nan"), dtype=torch.bfloat16, device=d)
    lse = torch.full((shape.b, shape.s, shape.h), float("nan"), dtype=torch.float32, device=d)
    da.mla_decode(*g, shape.scale, num_workers=num_workers, workspace=ws, out=out, lse=lse,
                  null_workspace=null_workspace)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def mla_shape(b, s, h, k, p, t, seed, seqlens=None, scale=None):
    return wl.MLAShape(b=b, s=s, h=h, k=k, p=p, t_max=t, scale=scale or 1.0 / math.sqrt(192), seed=seed)


# ------------------------------------------------------------------ MLA, small shapes, full compare
@pytest.mark.parametrize("workers", [0, 1, 2, 7])
def test_mla_tiny_workload(da, oracle_mod, workers):
    shape = wl.MLA_TINY
    t = wl.make_mla(shape)
    out, lse = run_mla(da, shape, t, workers)
    ref_o, ref_l = oracle_mod.mla(*t, shape.scale)
    print("mla tiny workers=%d" % workers, flush=True)
    compare(out, lse, ref_o, ref_l, "mla_tiny w=%d" % workers)


MLA_SMALL = [
    # (b, s, h, k, p, t_max, seqlens)
    (2, 1, 128, 512, 64, 200, [200, 77]),        # partial last tile, two row blocks
    (3, 3, 20, 512, 64, 150, [150, 64, 2]),      # drafts; row block partly empty; L < s
    (2, 4, 16, 256, 64, 130, [129, 130]),
    (1, 2, 40, 128, 64, 96, [95]),
    (4, 1, 16, 64, 16, 300, [0, 1, 300, 9999]),  # empty and clamped sequences
    (2, 1, 128, 512, 64, 64, [64, 63]),          # exactly one tile
    (4, 1, 16, 512, 64, 300, [0, 1, 300, 9999]),  # one row group with rows, workers spanning sequences
    (2, 1, 16, 128, 64, 300, [65, 300]),
    (2, 2, 24, 512, 64, 300, [300, 1]),            # the repair round needed by some row groups only
]


@pytest.mark.parametrize("case", MLA_SMALL, ids=lambda c: "b%d_s%d_h%d_k%d_t%d" % (c[0], c[1], c[2], c[3], c[5]))
@pytest.mark.parametrize("workers", [0, 1, 3])
def test_mla_small(da, oracle_mod, case, workers):
    b, s, h, k, p, t, sl = case
    shape = mla_shape(b, s, h, k, p, t, seed=100 + b + s + h)
    tensors = wl.make_mla(shape, seqlens=sl)
    print("mla small", case, "workers", workers, flush=True)
    out, lse = run_mla(da, shape, tensors, workers)
    ref_o, ref_l = oracle_mod.mla(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "mla %s w=%d" % (case, workers))


def seeded_lengths(n, t_max, seed):
    g = torch.Generator().manual_seed(seed)
    sl = torch.randint(0, t_max + 1, (n,), generator=g).tolist()
    sl[0], sl[1], sl[-1] = 0, t_max, 1  # an empty, a full and a one-row sequence
    return sl


@pytest.mark.parametrize("workers", [0, 7, 1000])
def test_mla_many_sequences(da, oracle_mod, workers):
    """More sequences than the planner keeps in registers (256): its later chunks take the reload path."""
    shape = mla_shape(300, 1, 16, 64, 16, 70, seed=31)
    tensors = wl.make_mla(shape, seqlens=seeded_lengths(300, 70, 5))
    print("mla many sequences workers", workers, flush=True)
    out, lse = run_mla(da, shape, tensors, workers)
    ref_o, ref_l = oracle_mod.mla(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "mla b=300 w=%d" % workers)


@pytest.mark.parametrize("workers", [0, 3])
def test_mla_all_sequences_empty(da, workers):
    """No cache row anywhere (lengths 0 and negative): every row must be out = 0, lse = -inf."""
    shape = mla_shape(3, 2, 16, 64, 16, 40, seed=33)
    tensors = wl.make_mla(shape, seqlens=[0, -5, 0])
    out, lse = run_mla(da, shape, tensors, workers)
    assert torch.all(out.float() == 0)
    assert torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("case", [(2, 1, 128, 512, 64, 3000, [3000, 1700], 120),
                                  (3, 2, 16, 64, 16, 900, [900, 0, 33], 100),
                                  (1, 4, 32, 256, 64, 2000, [1999], 64)],
                         ids=lambda c: "b%d_s%d_k%d_w%d" % (c[0], c[1], c[3], c[7]))
def test_mla_many_segments_per_row(da, oracle_mod, case):
    """Few sequences split over many workers (more than 16 segments per
    sequence on average): the combine gives each row a block of waves."""
    b, s, h, k, p, t, sl, workers = case
    shape = mla_shape(b, s, h, k, p, t, seed=200 + b + workers)
    tensors = wl.make_mla(shape, seqlens=sl)
    out, lse = run_mla(da, shape, tensors, workers)
    ref_o, ref_l = oracle_mod.mla(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "mla many segments %s" % (case,))


@pytest.mark.parametrize("case", MLA_SMALL, ids=lambda c: "b%d_s%d_h%d_k%d_t%d" % (c[0], c[1], c[2], c[3], c[5]))
def test_mla_null_workspace(da, oracle_mod, case):
    """No workspace: one worker per sequence writes its rows directly (no split, no combine), including
    out = 0 / lse = -inf for sequences with no cache row."""
    b, s, h, k, p, t, sl = case
    shape = mla_shape(b, s, h, k, p, t, seed=100 + b + s + h)
    tensors = wl.make_mla(shape, seqlens=sl)
    print("mla null workspace", case, flush=True)
    out, lse = run_mla(da, shape, tensors, null_workspace=True)
    ref_o, ref_l = oracle_mod.mla(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "mla null workspace %s" % (case,))


def test_mla_auto_one_worker_per_sequence(da, oracle_mod):
    """b=8 sequences of s*h = 2048 rows (32 row blocks each): the automatic worker count is one per
    sequence, so the library runs the per-sequence mode (no plan arrays, no combine) even with a
    workspace; ragged, draft-shorter and empty sequences included."""
    shape = mla_shape(8, 32, 64, 512, 64, 200, seed=41)
    sl = [200, 0, 31, 32, 33, 150, 1, 199]
    assert da.mla_decode_workspace_size(8, 32, 64, 512, 64, 200) > 0
    tensors = wl.make_mla(shape, seqlens=sl)
    out, lse = run_mla(da, shape, tensors, 0)
    ref_o, ref_l = oracle_mod.mla(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "mla one worker per sequence")


def test_mla_null_workspace_all_empty(da):
    shape = mla_shape(3, 2, 16, 64, 16, 40, seed=33)
    out, lse = run_mla(da, shape, wl.make_mla(shape, seqlens=[0, -5, 0]), null_workspace=True)
    assert torch.all(out.float() == 0)
    assert torch.all(torch.isneginf(lse))


def test_mla_split_counts_agree(da):
    shape = mla_shape(4, 2, 64, 512, 64, 700, seed=7)
    tensors = wl.make_mla(shape, seqlens=[700, 511, 65, 300])
    res = [run_mla(da, shape, tensors, w) for w in (1, 2, 7, 0, 40)]
    base_o, base_l = res[0]
    for o, l in res[1:]:
        assert (o.float() - base_o.float()).abs().max().item() <= 2 ** -7 * base_o.float().abs().max().item()
        fin = torch.isfinite(base_l)
        assert torch.equal(torch.isfinite(l), fin)
        assert (l[fin] - base_l[fin]).abs().max().item() <= 1e-4


def test_mla_cache_row_permutation(da):
    shape = mla_shape(1, 1, 64, 512, 64, 320, seed=8)
    ql, qr, c, sl = wl.make_mla(shape, seqlens=[300])
    o1, l1 = run_mla(da, shape, (ql, qr, c, sl))
    perm = torch.randperm(300, generator=torch.Generator().manual_seed(3))
    c2 = c.clone()
    c2[0, :300] = c[0, perm]
    o2, l2 = run_mla(da, shape, (ql, qr, c2, sl))
    assert (o1.float() - o2.float()).abs().max().item() <= 2 ** -7 * o1.float().abs().max().item()
    assert (l1 - l2).abs().max().item() <= 1e-4


def test_mla_garbage_beyond_seqlen_is_ignored(da, oracle_mod):
    """Cache rows past a sequence's length may hold anything (here NaN/Inf)."""
    shape = mla_shape(2, 2, 32, 512, 64, 256, seed=9)
    ql, qr, c, sl = wl.make_mla(shape, seqlens=[100, 37])
    ref_o, ref_l = oracle_mod.mla(ql, qr, c, sl, shape.scale)
    c[0, 100:] = float("nan")
    c[1, 37:] = float("inf")
    out, lse = run_mla(da, shape, (ql, qr, c, sl))
    compare(out, lse, ref_o, ref_l, "garbage rows")


@pytest.mark.parametrize("workers", [1, 3])
@pytest.mark.parametrize("late_row", [40, 150, 299])
@pytest.mark.parametrize("mag", [6.0, 24.0])
def test_mla_huge_late_score(da, oracle_mod, workers, late_row, mag):
    """A cache row past a segment's first tile whose score exceeds every
    earlier one by ~40 (mag 6) or ~160 (mag 24) powers of two: the kernel's
    shared softmax reference must catch up (lazily, or by redoing the tile)
    before that tile's probabilities are accumulated."""
    shape = mla_shape(2, 2, 24, 512, 64, 300, seed=11)
    ql, qr, c, sl = wl.make_mla(shape, seqlens=[300, 300])
    big = torch.zeros(512 + 64)
    big[:64] = mag
    c[0, late_row] = big.to(torch.bfloat16)
    c[1, late_row // 2] = (-big).to(torch.bfloat16)
    c[1, (late_row + 77) % 300] = big.to(torch.bfloat16)
    ql[0, :, :, :64] = torch.ones(64).to(torch.bfloat16)
    ql[1, :, :, :64] = torch.ones(64).to(torch.bfloat16)
    ref_o, ref_l = oracle_mod.mla(ql, qr, c, sl, shape.scale)
    out, lse = run_mla(da, shape, (ql, qr, c, sl), workers)
    compare(out, lse, ref_o, ref_l, "huge late score row %d workers %d" % (late_row, workers))


@pytest.mark.parametrize("workers", [1, 2])
@pytest.mark.parametrize("pos", [(40, 57, 6.0, 4.0), (40, 57, 4.0, 6.0), (70, 90, 24.0, 12.0), (33, 34, 5.0, 5.0)])
def test_mla_score_jumps_in_both_token_halves(da, oracle_mod, workers, pos):
    """Two cache rows of one 32-token tile, one in each 16-token half, whose
    scores jump far above everything before them by different amounts (or the
    same, or in two adjacent tiles): each half's softmax reference moves in the
    same step, and the common reference must be the larger of the two
    (also: both rows in one half, and jumps in different tiles)."""
    r0, r1, m0, m1 = pos
    shape = mla_shape(2, 1, 64, 512, 64, 200, seed=13)
    ql, qr, c, sl = wl.make_mla(shape, seqlens=[200, 160])
    for bq, rows_mags in enumerate([((r0, m0), (r1, m1)), ((r1 - 10, m1), ((r0 + 100) % 160, m0))]):
        for r, mag in rows_mags:
            big = torch.zeros(512 + 64)
            big[:64] = mag
            c[bq, r] = big.to(torch.bfloat16)
        ql[bq, :, :, :64] = torch.ones(64).to(torch.bfloat16)
    ref_o, ref_l = oracle_mod.mla(ql, qr, c, sl, shape.scale)
    out, lse = run_mla(da, shape, (ql, qr, c, sl), workers)
    compare(out, lse, ref_o, ref_l, "score jumps %s workers %d" % (pos, workers))


# ------------------------------------------------------------------ MLA, full-size workloads, every row
def full_size_mla(da, oracle_mod, shape, null_workspace=False):
    tensors = wl.make_mla(shape)
    print("full-size mla b=%d s=%d t_max=%d null_workspace=%s" % (shape.b, shape.s, shape.t_max, null_workspace),
          flush=True)
    out, lse = run_mla(da, shape, tensors, 0, null_workspace=null_workspace)
    ref_o, ref_l = oracle_mod.mla(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "full mla s=%d" % shape.s)
    assert torch.isfinite(lse).all()
    return tensors, out, lse


def test_mla_dsv3_full_size(da, oracle_mod):
    full_size_mla(da, oracle_mod, wl.MLA_DSV3)


def test_mla_dsv3_full_size_null_workspace(da, oracle_mod):
    full_size_mla(da, oracle_mod, wl.MLA_DSV3, null_workspace=True)


def test_mla_mtp4_full_size(da, oracle_mod):
    full_size_mla(da, oracle_mod, wl.MLA_MTP4)


def test_mla_ragged_full_size(da, oracle_mod):
    full_size_mla(da, oracle_mod, wl.MLA_RAGGED)


def test_mla_s48_full_size(da, oracle_mod):
    """48 drafts at the DeepSeek-V3-like shapes: 96 row blocks per sequence, for which the automatic
    worker count runs the blocks in several waves over the CUs."""
    full_size_mla(da, oracle_mod, wl.mla_mtp(48))


# ------------------------------------------------------------------ GQA
def run_gqa(da, shape, tensors, num_workers=0, path=0, null_workspace=False):
    q, k, v, sl = tensors
    d = dev()
    g = [t.to(d) for t in (q, k, v, sl)]
    nbytes = da.gqa_decode_workspace_size(shape.b, shape.s, shape.hq, shape.hkv, shape.d, shape.t_max, num_workers,
                                          path)
    ws = None if null_workspace else poisoned(nbytes, d)
    out = torch.full((shape.b, shape.s, shape.hq, shape.d), float("nan"), dtype=torch.bfloat16, device=d)
    lse = torch.full((shape.b, shape.s, shape.hq), float("nan"), dtype=torch.float32, device=d)
    da.gqa_decode(*g, shape.scale, num_workers=num_workers, path=path, workspace=ws, out=out, lse=lse,
                  null_workspace=null_workspace)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


GQA_SMALL = [
    # (b, s, hq, hkv, d, t_max, seqlens)
    (2, 1, 8, 8, 128, 200, [200, 77]),      # MHA
    (2, 1, 8, 1, 128, 130, [130, 5]),       # MQA
    (3, 2, 16, 4, 64, 150, [150, 64, 1]),   # groups of 4, drafts, L < s
    (2, 1, 32, 4, 256, 96, [96, 33]),       # d = 256, group 8
    (2, 2, 16, 2, 128, 300, [0, 299]),      # group 8 x 2 drafts = 16 rows, empty sequence
    (1, 1, 6, 3, 128, 70, [70]),            # group 2
    (2, 4, 16, 2, 128, 200, [200, 131]),    # 32 rows per KV head
    (2, 8, 64, 8, 64, 100, [100, 9]),       # 64 rows per KV head, d = 64
    (3, 1, 64, 8, 128, 520, [520, 1, 257]),  # the layer's geometry, ragged
    (1, 4, 32, 4, 256, 64, [64]),            # d = 256, 32 rows
    (2, 1, 10, 5, 128, 90, [90, 40]),        # 5 KV heads: the second head block has one active wave
    (2, 2, 18, 9, 64, 80, [80, 3]),          # d = 64, 9 KV heads over two head blocks
    (2, 2, 24, 4, 256, 150, [150, 77]),      # groups of 6 at d = 256 (12 rows per KV head)
    (2, 5, 16, 2, 128, 160, [160, 77]),      # group 8 x 5 drafts = 40 rows: three row blocks
    (1, 3, 48, 4, 64, 90, [90]),             # group 12 x 3 drafts = 36 rows at d = 64
    (2, 6, 32, 4, 128, 120, [120, 5]),       # 48 rows: three full row blocks, L < s in one sequence
    (2, 1, 64, 1, 128, 200, [200, 77]),      # MQA, 64 rows: one head per block, rows over four waves
    (2, 1, 128, 1, 128, 150, [150, 3]),      # MQA, 128 rows: four waves of two row blocks
    (2, 16, 64, 8, 128, 100, [100, 40]),     # group 8 x 16 drafts = 128 rows
    (1, 4, 64, 1, 128, 90, [90]),            # 256 rows: four waves of four row blocks
    (2, 2, 48, 1, 64, 120, [120, 2]),        # MQA at d = 64: two head slots per block, one real
    (2, 4, 32, 1, 256, 100, [100, 64]),      # 128 rows at d = 256: four waves of two row blocks
    (2, 3, 24, 2, 128, 130, [130, 30]),      # 36 rows, two KV heads (one head per block)
    (2, 1, 12, 3, 128, 70, [70, 70]),        # three KV heads at d = 128 (not a multiple of four)
]


def gqa_paths(case):
    rows = case[2] // case[3] * case[1]
    return [1, 2] if rows <= 16 else [2]


@pytest.mark.parametrize("case,path", [(c, p) for c in GQA_SMALL for p in gqa_paths(c)],
                         ids=lambda x: ("b%d_s%d_hq%d_hkv%d_d%d" % x[:5]) if isinstance(x, tuple) else "path%d" % x)
@pytest.mark.parametrize("workers", [0, 1, 5])
def test_gqa_small(da, oracle_mod, case, path, workers):
    b, s, hq, hkv, d, t, sl = case
    shape = wl.GQAShape(b=b, s=s, hq=hq, hkv=hkv, d=d, t_max=t, scale=1.0 / math.sqrt(d), seed=200 + hq + d)
    tensors = wl.make_gqa(shape, seqlens=sl)
    print("gqa small", case, "path", path, "workers", workers, flush=True)
    out, lse = run_gqa(da, shape, tensors, workers, path)
    ref_o, ref_l = oracle_mod.gqa(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "gqa %s path=%d w=%d" % (case, path, workers))


@pytest.mark.parametrize("case,path", [(c, p) for c in GQA_SMALL for p in gqa_paths(c)],
                         ids=lambda x: ("b%d_s%d_hq%d_hkv%d_d%d" % x[:5]) if isinstance(x, tuple) else "path%d" % x)
def test_gqa_null_workspace(da, oracle_mod, case, path):
    """No workspace: one worker per sequence writes its rows directly, empty sequences included."""
    b, s, hq, hkv, d, t, sl = case
    shape = wl.GQAShape(b=b, s=s, hq=hq, hkv=hkv, d=d, t_max=t, scale=1.0 / math.sqrt(d), seed=200 + hq + d)
    tensors = wl.make_gqa(shape, seqlens=sl)
    print("gqa null workspace", case, "path", path, flush=True)
    out, lse = run_gqa(da, shape, tensors, 0, path, null_workspace=True)
    ref_o, ref_l = oracle_mod.gqa(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "gqa null workspace %s path=%d" % (case, path))


GQA_TOKEN_GROUPS = [
    # (b, s, hq, hkv, d, t_max): with b * hkv >= 256 the automatic choice (and always the null
    # workspace) runs one block per (sequence, KV head) whose waves split the tokens and merge in
    # LDS; the waves per block (4, 2 or 1) follow from b * hkv and d; d = 64 takes 32-token
    # stages; MQA with more than 48 rows splits them over two blocks
    (32, 1, 64, 8, 128, 300),    # the layer's geometry, ragged lengths
    (16, 3, 256, 16, 128, 90),   # group 16 x 3 drafts = 48 rows: three row blocks
    (64, 4, 16, 4, 128, 70),     # 16 rows over four drafts
    (32, 8, 64, 8, 128, 60),     # 64 rows: four row blocks
    (64, 2, 16, 4, 256, 100),    # d = 256, 8 rows
    (128, 4, 16, 2, 256, 64),    # d = 256, 32 rows: two row blocks
    (64, 2, 64, 8, 128, 80),     # 512 blocks: two waves per block
    (256, 1, 8, 4, 128, 40),     # 1024 blocks: one wave per block
    (128, 2, 16, 4, 256, 50),    # d = 256, 512 blocks: one wave per block
    (32, 1, 32, 8, 64, 300),     # d = 64, 4 rows
    (64, 4, 64, 4, 64, 70),      # d = 64, 64 rows: four row blocks
    (32, 3, 40, 8, 64, 90),      # d = 64, 15 rows
    (128, 2, 16, 4, 64, 50),     # d = 64, 512 blocks: two waves per block
    (512, 1, 16, 4, 64, 40),     # d = 64, 2048 blocks: one wave per block
    (32, 1, 64, 1, 128, 300),    # MQA, 64 rows: two blocks of 32 rows per KV head
    (16, 2, 24, 1, 64, 90),      # MQA, d = 64, 48 rows over two drafts: one block
    (8, 3, 20, 1, 128, 70),      # MQA, 60 rows over three drafts: 30 + 30
    (8, 1, 56, 1, 64, 50),       # MQA, d = 64, 56 rows: 28 + 28
]


@pytest.mark.parametrize("case", GQA_TOKEN_GROUPS, ids=lambda c: "b%d_s%d_hq%d_hkv%d_d%d_t%d" % c)
@pytest.mark.parametrize("mode", ["auto", "null_workspace", "split"])
def test_gqa_token_groups(da, oracle_mod, case, mode):
    """Lengths 0, 1, stage and tile edges and t_max among the sequences; "split" forces the
    split-KV kernel (explicit worker count) on the same inputs."""
    b, s, hq, hkv, d, t = case
    shape = wl.GQAShape(b=b, s=s, hq=hq, hkv=hkv, d=d, t_max=t, scale=1.0 / math.sqrt(d), seed=400 + b + d)
    edges = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, t - 1, t]
    sl = [x for x in edges if x <= t] + seeded_lengths(b, t, 41)
    tensors = wl.make_gqa(shape, seqlens=sl[:b])
    print("gqa token groups", case, mode, flush=True)
    out, lse = run_gqa(da, shape, tensors, 96 if mode == "split" else 0, 2, null_workspace=mode == "null_workspace")
    ref_o, ref_l = oracle_mod.gqa(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "gqa token groups %s %s" % (case, mode))


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("workers", [0, 3])
def test_gqa_many_sequences(da, oracle_mod, path, workers):
    """More sequences than the planner keeps in registers (256)."""
    shape = wl.GQAShape(b=300, s=1, hq=8, hkv=2, d=64, t_max=40, scale=0.125, seed=32)
    tensors = wl.make_gqa(shape, seqlens=seeded_lengths(300, 40, 6))
    print("gqa many sequences path", path, "workers", workers, flush=True)
    out, lse = run_gqa(da, shape, tensors, workers, path)
    ref_o, ref_l = oracle_mod.gqa(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "gqa b=300 path=%d w=%d" % (path, workers))


@pytest.mark.parametrize("path", [1, 2])
def test_gqa_all_sequences_empty(da, path):
    """No cache row anywhere: every row must be out = 0, lse = -inf."""
    shape = wl.GQAShape(b=2, s=1, hq=8, hkv=2, d=128, t_max=50, scale=0.1, seed=34)
    tensors = wl.make_gqa(shape, seqlens=[0, -1])
    out, lse = run_gqa(da, shape, tensors, 0, path)
    assert torch.all(out.float() == 0)
    assert torch.all(torch.isneginf(lse))


@pytest.fixture(scope="module")
def gqa_full_cases(oracle_mod):
    """The full-size grouped workloads with the oracle's result for every row (computed once)."""
    cache = {}

    def get(name):
        if name not in cache:
            shape = wl.WORKLOADS[name]
            tensors = wl.make_gqa(shape)
            cache.clear()  # one multi-GiB workload in memory at a time
            cache[name] = (shape, tensors) + tuple(oracle_mod.gqa(*tensors, shape.scale))
        return cache[name]
    return get


@pytest.mark.parametrize("name,path,workers", [("gqa_layer", 1, 0), ("gqa_layer", 2, 0), ("gqa_layer", 2, 128),
                                               ("gqa_mqa", 0, 0), ("gqa_mha", 1, 0), ("gqa_mha", 2, 0),
                                               ("gqa_mha", 2, 64), ("gqa_mtp4", 0, 0), ("gqa_mtp4", 0, 96)])
def test_gqa_full_size(da, gqa_full_cases, name, path, workers):
    """Every row of the full-size grouped workloads: the layer (group 8, also with 4 drafts), MQA and MHA at
    b=32/8, t=4096.
    The automatic worker count runs the layer and MHA one block per (sequence, KV head); an explicit
    worker count runs the split-KV kernel and the combine."""
    shape, tensors, ref_o, ref_l = gqa_full_cases(name)
    print("full-size %s path %d workers %d" % (name, path, workers), flush=True)
    out, lse = run_gqa(da, shape, tensors, workers, path)
    compare(out, lse, ref_o, ref_l, "%s full path=%d workers=%d" % (name, path, workers))


def test_gqa_layer_full_size_null_workspace(da, gqa_full_cases):
    shape, tensors, ref_o, ref_l = gqa_full_cases("gqa_layer")
    out, lse = run_gqa(da, shape, tensors, 0, 0, null_workspace=True)
    compare(out, lse, ref_o, ref_l, "gqa layer full, null workspace")


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("case", [(2, 1, 24, 4, 256, 4000, [4000, 2500], 60),
                                  (1, 2, 16, 2, 128, 3000, [3000], 40),
                                  (2, 1, 8, 1, 64, 2048, [2048, 0], 50)],
                         ids=lambda c: "b%d_s%d_d%d_w%d" % (c[0], c[1], c[4], c[7]))
def test_gqa_many_segments_per_row(da, oracle_mod, case, path):
    """Few sequences split over many workers: the combine's block-per-row form."""
    b, s, hq, hkv, d, t, sl, workers = case
    shape = wl.GQAShape(b=b, s=s, hq=hq, hkv=hkv, d=d, t_max=t, scale=1.0 / math.sqrt(d), seed=300 + workers)
    tensors = wl.make_gqa(shape, seqlens=sl)
    out, lse = run_gqa(da, shape, tensors, workers, path)
    ref_o, ref_l = oracle_mod.gqa(*tensors, shape.scale)
    compare(out, lse, ref_o, ref_l, "gqa many segments %s path %d" % (case, path))


# ------------------------------------------------------------------ un-absorbed MLA (per-head K and V)
def unabsorbed_inputs(b, s, h, t, seqlens, seed, device="cpu"):
    gen = torch.Generator(device=device).manual_seed(seed)
    q = torch.randn((b, s, h, 192), generator=gen, device=device).to(torch.bfloat16)
    k = torch.randn((b, t, h, 192), generator=gen, device=device).to(torch.bfloat16)
    v = torch.randn((b, t, h, 128), generator=gen, device=device).to(torch.bfloat16)
    return q, k, v, torch.tensor(seqlens, dtype=torch.int32, device=device)


def unabsorbed_reference(oracle_mod, q, k, v, sl, scale):
    """Per sequence and head: textbook attention of the s drafts over the
    visible cache rows (draft i sees L - s + i + 1 of them)."""
    b, s, h, _ = q.shape
    out = np.zeros((b, s, h, 128))
    lse = np.full((b, s, h), -np.inf)
    for bq in range(b):
        L = max(0, min(int(sl[bq]), k.shape[1]))
        n_vis = [max(0, L - s + i + 1) for i in range(s)]
        if L == 0:
            continue
        for hh in range(h):
            o, l = oracle_mod.attn_generic(q[bq, :, hh].double().numpy(), k[bq, :L, hh].double().numpy(),
                                           v[bq, :L, hh].double().numpy(), n_vis, scale)
            out[bq, :, hh], lse[bq, :, hh] = o, l
    return out, lse


UNABS_SMALL = [
    # (b, s, h, t_max, seqlens, workers)
    (2, 1, 4, 150, [150, 77], 0),
    (3, 3, 8, 100, [100, 2, 0], 0),       # drafts, L < s, an empty sequence
    (1, 16, 4, 200, [200], 3),            # 16 drafts: one 16-row block
    (2, 20, 2, 130, [130, 64], 2),        # 20 drafts: two row blocks
    (1, 40, 2, 300, [300], 5),            # 40 drafts: three row blocks
    (2, 48, 2, 260, [260, 100], 3),       # 48 drafts: three full row blocks
    (1, 56, 2, 300, [300], 4),            # 56 drafts: four row blocks
    (2, 1, 5, 1000, [1000, 999], 0),      # odd head count: the last head block has one active wave
    (2, 2, 3, 700, [700, 350], 40),       # many segments per row (block-per-row combine)
]


@pytest.mark.parametrize("null_ws", [False, True], ids=["ws", "null_ws"])
@pytest.mark.parametrize("case", UNABS_SMALL, ids=lambda c: "b%d_s%d_h%d_t%d_w%d" % (c[0], c[1], c[2], c[3], c[5]))
def test_mla_unabsorbed_small(da, oracle_mod, case, null_ws):
    b, s, h, t, sl, workers = case
    q, k, v, slt = unabsorbed_inputs(b, s, h, t, sl, seed=400 + b + s + h)
    scale = 1.0 / math.sqrt(192)
    d = dev()
    out = torch.full((b, s, h, 128), float("nan"), dtype=torch.bfloat16, device=d)
    lse = torch.full((b, s, h), float("nan"), dtype=torch.float32, device=d)
    da.mla_decode_unabsorbed(q.to(d), k.to(d), v.to(d), slt.to(d), scale, num_workers=workers, out=out, lse=lse,
                             null_workspace=null_ws)
    torch.cuda.synchronize()
    ref_o, ref_l = unabsorbed_reference(oracle_mod, q, k, v, sl, scale)
    compare(out.cpu(), lse.cpu(), ref_o, ref_l, "mla unabsorbed %s" % (case,))


def test_mla_unabsorbed_longest_sequence(da, oracle_mod):
    """One sequence whose per-head keys are just under 2^31 bytes (t_max * h * 192 * 2 < 2^31:
    2,796,202 rows at h = 2), every row, with the automatic workers and with no workspace.
    Inputs drawn on the GPU."""
    b, s, h = 1, 2, 2
    t = ((1 << 31) - 1) // (h * 192 * 2)
    q, k, v, slt = unabsorbed_inputs(b, s, h, t, [t], seed=93, device=dev())
    scale = 1.0 / math.sqrt(192)
    ref_o, ref_l = unabsorbed_reference(oracle_mod, q.cpu(), k.cpu(), v.cpu(), slt.cpu(), scale)
    for null_ws in (False, True):
        print("mla unabsorbed longest sequence t=%d null_workspace=%s" % (t, null_ws), flush=True)
        out = torch.full((b, s, h, 128), float("nan"), dtype=torch.bfloat16, device=dev())
        lse = torch.full((b, s, h), float("nan"), dtype=torch.float32, device=dev())
        da.mla_decode_unabsorbed(q, k, v, slt, scale, out=out, lse=lse, null_workspace=null_ws)
        torch.cuda.synchronize()
        compare(out.cpu(), lse.cpu(), ref_o, ref_l, "mla unabsorbed t=%d null_ws=%s" % (t, null_ws))


def test_mla_unabsorbed_full_heads(da, oracle_mod):
    """The crossover's geometry (h=128, t=4096, the automatic worker layout) at b=2 and s=4, every row."""
    b, s, h, t = 2, 4, 128, 4096
    q, k, v, slt = unabsorbed_inputs(b, s, h, t, [t, t - 1000], seed=450)
    scale = 1.0 / math.sqrt(192)
    d = dev()
    out, lse = da.mla_decode_unabsorbed(q.to(d), k.to(d), v.to(d), slt.to(d), scale)
    torch.cuda.synchronize()
    ref_o, ref_l = unabsorbed_reference(oracle_mod, q, k, v, [t, t - 1000], scale)
    compare(out.cpu(), lse.cpu(), ref_o, ref_l, "mla unabsorbed b=2 s=4 h=128 t=4096")


def test_mla_unabsorbed_matches_absorbed(da):
    """With K = [Z Wk_h | Z_rope], V = Z Wv_h from a latent cache Z and
    per-head weights, and q_lat = q_nope Wk_h^T: the un-absorbed output equals
    the absorbed latent output times Wv_h^T (GPU against GPU, up to the bf16
    rounding of the decompressed K/V, the absorbed queries and the latent
    output)."""
    b, s, h, t, kl, dn, p = 2, 2, 4, 200, 128, 128, 64
    gen = torch.Generator().manual_seed(77)
    Z = torch.randn((b, t, kl + p), generator=gen)
    Wk = torch.randn((h, dn, kl), generator=gen) / math.sqrt(kl)
    Wv = torch.randn((h, dn, kl), generator=gen) / math.sqrt(kl)
    qn = torch.randn((b, s, h, dn), generator=gen)
    qr = torch.randn((b, s, h, p), generator=gen)
    sl = torch.tensor([200, 123], dtype=torch.int32)
    scale = 1.0 / math.sqrt(dn + p)
    Zb = Z.to(torch.bfloat16).float()
    K = torch.cat([torch.einsum("btk,hdk->bthd", Zb[..., :kl], Wk), Zb[..., kl:].unsqueeze(2).expand(b, t, h, p)], -1)
    V = torch.einsum("btk,hdk->bthd", Zb[..., :kl], Wv)
    q = torch.cat([qn, qr], -1)
    q_lat = torch.einsum("bshd,hdk->bshk", qn.to(torch.bfloat16).float(), Wk)
    d = dev()
    g16 = lambda x: x.to(torch.bfloat16).contiguous().to(d)  # noqa: E731
    o_u, l_u = da.mla_decode_unabsorbed(g16(q), g16(K), g16(V), sl.to(d), scale)
    o_a, l_a = da.mla_decode(g16(q_lat), g16(qr), g16(Z), sl.to(d), scale)
    torch.cuda.synchronize()
    o_a_dec = torch.einsum("bshk,hdk->bshd", o_a.float().cpu(), Wv)
    o_u = o_u.float().cpu()
    ref_max = o_a_dec.abs().max().item()
    assert (o_u - o_a_dec).abs().max().item() <= 5e-2 * ref_max
    assert (l_u.cpu() - l_a.cpu()).abs().max().item() <= 3e-2


# ------------------------------------------------------------------ per-head projections
PROJ_CASES = [
    # (kind, b, s, h, d, k)
    ("absorb", 3, 2, 5, 128, 512),       # M = 6: one partial M tile
    ("absorb", 2, 33, 3, 128, 192),      # M = 66: a ragged second M tile, N = 192
    ("decompress", 2, 33, 3, 128, 512),  # M = 66, N = 128
    ("decompress", 1, 1, 7, 100, 256),   # N = 100: a ragged N tile
    ("absorb", 32, 4, 128, 128, 512),    # DeepSeek-V3-like, s = 4
    ("decompress", 32, 4, 128, 128, 512),
    ("absorb", 2, 3, 4, 32, 64),         # one k-step
    ("decompress", 2, 5, 3, 96, 160),    # five k-steps: the load ring wraps part-way
    ("decompress", 1, 70, 2, 64, 1024),  # 32 k-steps, four per wave in the split form
]


@pytest.mark.parametrize("case", PROJ_CASES, ids=lambda c: "%s_b%d_s%d_h%d_d%d_k%d" % c)
def test_head_projection(da, oracle_mod, case):
    kind, b, s, h, d, k = case
    gen = torch.Generator().manual_seed(500 + b + s + h + d + k)
    if kind == "absorb":
        A = torch.randn((b, s, h, d), generator=gen).to(torch.bfloat16)
        W = (torch.randn((h, k, d), generator=gen) / math.sqrt(d)).to(torch.bfloat16)
        out = da.mla_absorb_queries(A.to(dev()), W.to(dev()))
    else:
        A = torch.randn((b, s, h, k), generator=gen).to(torch.bfloat16)
        W = (torch.randn((h, d, k), generator=gen) / math.sqrt(k)).to(torch.bfloat16)
        out = da.mla_decompress_output(A.to(dev()), W.to(dev()))
    torch.cuda.synchronize()
    ref = oracle_mod.head_projection(A, W)
    got = out.float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape
    err = np.abs(got - ref).max()
    assert err <= 1e-2 * np.abs(ref).max(), "%s: max|d| %.3e vs max|ref| %.3e" % (case, err, np.abs(ref).max())


def test_absorbed_path_through_projections_matches_unabsorbed(da):
    """Q-absorption -> absorbed decode -> output decompression, all on the GPU,
    against un-absorbed decode on K = [Z Wk | Z_rope], V = Z Wv (GPU against
    GPU, up to the bf16 roundings on either path)."""
    b, s, h, t, kl, dn, p = 2, 3, 8, 256, 512, 128, 64
    gen = torch.Generator().manual_seed(78)
    Z = torch.randn((b, t, kl + p), generator=gen).to(torch.bfloat16)
    Wk = (torch.randn((h, kl, dn), generator=gen) / math.sqrt(kl)).to(torch.bfloat16)
    WvT = (torch.randn((h, dn, kl), generator=gen) / math.sqrt(kl)).to(torch.bfloat16)
    qn = torch.randn((b, s, h, dn), generator=gen).to(torch.bfloat16)
    qr = torch.randn((b, s, h, p), generator=gen).to(torch.bfloat16)
    sl = torch.tensor([256, 100], dtype=torch.int32)
    scale = 1.0 / math.sqrt(dn + p)
    Zf = Z.float()
    K = torch.cat([torch.einsum("btk,hkd->bthd", Zf[..., :kl], Wk.float()),
                   Zf[..., kl:].unsqueeze(2).expand(b, t, h, p)], -1)
    V = torch.einsum("btk,hdk->bthd", Zf[..., :kl], WvT.float())
    d = dev()
    g16 = lambda x: x.to(torch.bfloat16).contiguous().to(d)  # noqa: E731
    q_lat = da.mla_absorb_queries(g16(qn), g16(Wk))
    o_lat, l_a = da.mla_decode(q_lat, g16(qr), g16(Z), sl.to(d), scale)
    o_a = da.mla_decompress_output(o_lat, g16(WvT))
    o_u, l_u = da.mla_decode_unabsorbed(g16(torch.cat([qn.float(), qr.float()], -1)), g16(K), g16(V), sl.to(d), scale)
    torch.cuda.synchronize()
    o_a, o_u = o_a.float().cpu(), o_u.float().cpu()
    assert (o_a - o_u).abs().max().item() <= 5e-2 * o_u.abs().max().item()
    assert (l_a.cpu() - l_u.cpu()).abs().max().item() <= 3e-2


# ------------------------------------------------------------------ split latent / decompressed cache
@pytest.mark.parametrize("case", [(2, 3, 4, [100, 37], [20, 5], 128, 32, 0),
                                  (1, 1, 8, [300], [1], 320, 4, 0),
                                  (3, 2, 2, [0, 64, 500], [40, 2, 9], 512, 48, 6)],
                         ids=lambda c: "b%d_s%d_h%d_w%d" % (c[0], c[1], c[2], c[7]))
def test_mla_split_cache(da, oracle_mod, case):
    """Old rows latent (absorbed, through both projections), new rows
    decompressed (un-absorbed), merged: against the oracle's textbook attention
    over all rows, old keys and values Z Wk / Z Wv and new ones as given.
    Integer-valued weights and q_nope keep q_lat exact in bf16."""
    b, s, h, o_l, n_l, o_max, n_max, workers = case
    gen = torch.Generator().manual_seed(600 + b + s + h)
    Z = torch.randn((b, o_max, 576), generator=gen).to(torch.bfloat16)
    Wk = torch.randint(-1, 2, (h, 512, 128), generator=gen).to(torch.bfloat16)
    WvT = torch.randint(-1, 2, (h, 128, 512), generator=gen).to(torch.bfloat16)
    qn = torch.randint(-1, 2, (b, s, h, 128), generator=gen).to(torch.bfloat16)
    qr = torch.randn((b, s, h, 64), generator=gen).to(torch.bfloat16)
    kn = torch.randn((b, n_max, h, 192), generator=gen).to(torch.bfloat16)
    vn = (4.0 * torch.randn((b, n_max, h, 128), generator=gen)).to(torch.bfloat16)
    so, sn = torch.tensor(o_l, dtype=torch.int32), torch.tensor(n_l, dtype=torch.int32)
    scale = 1.0 / math.sqrt(192) / 8.0
    d = dev()
    out, lse = da.mla_decode_split_cache(qn.to(d), qr.to(d), Wk.to(d), WvT.to(d), Z.to(d), so.to(d), kn.to(d),
                                         vn.to(d), sn.to(d), scale, num_workers=workers)
    torch.cuda.synchronize()
    f64 = lambda x: x.double()  # noqa: E731
    ref_o = np.zeros((b, s, h, 128))
    ref_l = np.full((b, s, h), -np.inf)
    for bq in range(b):
        o, n = o_l[bq], n_l[bq]
        for hh in range(h):
            K_old = torch.cat([f64(Z[bq, :o, :512]) @ f64(Wk[hh]), f64(Z[bq, :o, 512:])], -1)
            V_old = f64(Z[bq, :o, :512]) @ f64(WvT[hh]).T
            K = torch.cat([K_old, f64(kn[bq, :n, hh])], 0)
            V = torch.cat([V_old, f64(vn[bq, :n, hh])], 0)
            Q = torch.cat([f64(qn[bq, :, hh]), f64(qr[bq, :, hh])], -1)
            n_vis = [o + max(0, n - s + i + 1) for i in range(s)]
            if o + n == 0:
                continue
            ro, rl = oracle_mod.attn_generic(Q.numpy(), K.numpy(), V.numpy(), n_vis, scale)
            ref_o[bq, :, hh], ref_l[bq, :, hh] = ro, rl
    compare(out.cpu(), lse.cpu(), ref_o, ref_l, "split cache %s" % (case,))


# ------------------------------------------------------------------ the longest sequences the ABI takes
def test_mla_longest_sequence(da, oracle_mod):
    """One sequence whose cache is just under 2^31 bytes, the limit of the 32-bit buffer offsets
    (t_max * (k + p) * 2 < 2^31: 1,864,135 rows, the last tile ragged), every row: split over the
    automatic worker count (one row block, so the block-per-row combine) and, with no workspace,
    walked by a single block. Inputs drawn on the GPU."""
    t = ((1 << 31) - 1) // ((512 + 64) * 2)
    shape = mla_shape(1, 2, 8, 512, 64, t, seed=91)
    tensors = wl.make_mla(shape, device=dev())
    ref_o, ref_l = oracle_mod.mla(*[x.cpu() for x in tensors], shape.scale)
    for null_ws in (False, True):
        print("mla longest sequence t=%d null_workspace=%s" % (t, null_ws), flush=True)
        out, lse = run_mla(da, shape, tensors, 0, null_workspace=null_ws)
        compare(out, lse, ref_o, ref_l, "mla t=%d null_ws=%s" % (t, null_ws))


def test_gqa_longest_sequence(da, oracle_mod):
    """One sequence whose K (and V) rows are just under 2^31 bytes (t_max * hkv * d * 2 < 2^31:
    4,194,303 rows at hkv = 2, d = 128), every row: the token-group kernel under the automatic
    split and with no workspace (one block per KV head). Inputs drawn on the GPU."""
    t = ((1 << 31) - 1) // (2 * 128 * 2)
    shape = wl.GQAShape(b=1, s=1, hq=16, hkv=2, d=128, t_max=t, scale=1.0 / math.sqrt(128), seed=92)
    tensors = wl.make_gqa(shape, device=dev())
    ref_o, ref_l = oracle_mod.gqa(*[x.cpu() for x in tensors], shape.scale)
    for null_ws in (False, True):
        print("gqa longest sequence t=%d null_workspace=%s" % (t, null_ws), flush=True)
        out, lse = run_gqa(da, shape, tensors, 0, null_workspace=null_ws)
        compare(out, lse, ref_o, ref_l, "gqa t=%d null_ws=%s" % (t, null_ws))


@pytest.fixture(scope="module")
def gqa_long_case(oracle_mod):
    """One 262,144-token sequence at 24 query / 4 KV heads, d = 256, with the
    oracle's result for all 24 query rows (computed once for both paths)."""
    shape = wl.GQA_LONG
    tensors = wl.make_gqa(shape)
    ref_o, ref_l = oracle_mod.gqa(*tensors, shape.scale)
    return shape, tensors, ref_o, ref_l


@pytest.mark.parametrize("path", [1, 2])
def test_gqa_long_context_groups_of_six(da, gqa_long_case, path):
    shape, tensors, ref_o, ref_l = gqa_long_case
    print("gqa long context (t=%d, hq=%d, hkv=%d, d=%d) path %d" % (shape.t_max, shape.hq, shape.hkv, shape.d, path),
          flush=True)
    out, lse = run_gqa(da, shape, tensors, 0, path)
    compare(out.reshape(-1, shape.d), lse.reshape(-1), ref_o.reshape(-1, shape.d), ref_l.reshape(-1),
            "gqa long path=%d" % path)


@pytest.mark.parametrize("path", [1, 2])
def test_gqa_mha_equals_repeated_kv(da, path):
    """GQA equals MHA run on K/V heads repeated per group (GPU against GPU)."""
    shape = wl.GQAShape(b=2, s=1, hq=16, hkv=2, d=128, t_max=256, scale=1.0 / math.sqrt(128), seed=5)
    q, k, v, sl = wl.make_gqa(shape, seqlens=[256, 100])
    o1, l1 = run_gqa(da, shape, (q, k, v, sl), 0, path)
    mha = wl.GQAShape(b=2, s=1, hq=16, hkv=16, d=128, t_max=256, scale=shape.scale, seed=5)
    o2, l2 = run_gqa(da, mha, (q, k.repeat_interleave(8, dim=2).contiguous(),
                               v.repeat_interleave(8, dim=2).contiguous(), sl), 0, path)
    assert (o1.float() - o2.float()).abs().max().item() <= 2 ** -7 * o1.float().abs().max().item()
    assert (l1 - l2).abs().max().item() <= 1e-4


def test_gqa_paths_agree(da):
    """The VALU and MFMA kernels agree with each other on the layer's geometry."""
    shape = wl.GQAShape(b=4, s=1, hq=64, hkv=8, d=128, t_max=1000, scale=1.0 / math.sqrt(128), seed=11)
    tensors = wl.make_gqa(shape, seqlens=[1000, 999, 64, 513])
    o1, l1 = run_gqa(da, shape, tensors, 0, 1)
    o2, l2 = run_gqa(da, shape, tensors, 0, 2)
    assert (o1.float() - o2.float()).abs().max().item() <= 2 ** -7 * o1.float().abs().max().item()
    assert (l1 - l2).abs().max().item() <= 1e-4
