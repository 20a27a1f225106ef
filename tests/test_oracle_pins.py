"""Pins of the fp64 oracle against things other than itself.

Each test checks one oracle function against a library routine (torch's
scaled-dot-product attention, elu and float8 casts), a closed form, brute
force on tiny inputs, or an invariant of the mathematics, chosen so that a
plausible slip (a dropped scale or term, a wrong sign, index or axis, a
transposed operand) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import rola as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


def _rand_head(rng, n, npad, d, pad_garbage=True):
    q = rng.standard_normal((npad, d))
    k = rng.standard_normal((npad, d))
    v = rng.standard_normal((npad, d))
    if not pad_garbage:
        q[n:] = k[n:] = v[n:] = 0.0
    return q, k, v


def _sdpa(q, k, v, scale, mask=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale)
    return o[0, 0].numpy()


# ---------------------------------------------------------------- P1
def test_p1_all_tiles_kept_and_zero_wo_is_dense_sdpa():
    """k = T and W_o = 0: the hybrid reduces to dense softmax attention over the
    valid tokens (torch SDPA, fp64).  Pad rows hold garbage that must be ignored."""
    rng = np.random.default_rng(1)
    grid, d, r = (3, 10, 10), 32, 16
    n = 300
    npad = 320
    t = npad // 64
    q, k, v = _rand_head(rng, n, npad, d)
    uq, uk = rng.standard_normal((d, r)) / 6, rng.standard_normal((d, r)) / 6
    out = R.hybrid_head(q, k, v, n, grid, uq, uk, np.zeros((d, d)), topk=t, force_diag=False,
                        scale=1 / math.sqrt(d), base=10000.0)
    ref = _sdpa(q[:n], k[:n], v[:n], 1 / math.sqrt(d))
    assert rel(out["o"][:n], ref) <= 1e-12
    assert np.all(out["o"][n:] == 0)
    assert all(len(x) == t for x in out["rows"])


def test_p1b_random_mask_matches_masked_sdpa():
    """Any tile mask: the sparse branch equals SDPA with the token-level boolean
    mask expanded from the kept-tile lists (catches gather/index slips)."""
    rng = np.random.default_rng(2)
    n, npad, d = 455, 512, 48
    t = npad // 64
    q, k, v = _rand_head(rng, n, npad, d)
    rows = [np.sort(rng.choice(t, size=rng.integers(1, t + 1), replace=False)) for _ in range(t)]
    o = R.sparse_branch(q, k, v, n, rows, scale=0.3)
    mask = np.zeros((n, n), dtype=bool)
    for a, kept in enumerate(rows):
        for b in kept:
            mask[a * 64:min(a * 64 + 64, n), b * 64:min(b * 64 + 64, n)] = True
    ref = _sdpa(q[:n], k[:n], v[:n], 0.3, mask)
    assert rel(o[:n], ref) <= 1e-12
    assert np.all(o[n:] == 0)


# ---------------------------------------------------------------- P2
def test_p2_constant_values_give_constant_output():
    """v_j = c: softmax rows sum to one, so O_s = c for any mask; with every
    RoPE angle zero the linear branch is a convex combination too, so O_l = c."""
    rng = np.random.default_rng(3)
    n, npad, d, r = 200, 256, 32, 32
    q, k, _ = _rand_head(rng, n, npad, d)
    c = rng.standard_normal(d)
    v = np.tile(c, (npad, 1))
    rows = [np.sort(rng.choice(4, size=2, replace=False)) for _ in range(4)]
    o_s = R.sparse_branch(q, k, v, n, rows, scale=0.2)
    assert np.allclose(o_s[:n], c, rtol=0, atol=1e-13)
    uq, uk = rng.standard_normal((d, r)) / 5, rng.standard_normal((d, r)) / 5
    pos0 = np.zeros((n, 3), dtype=np.int64)
    o_l = R.linear_branch(q, k, v, n, uq, uk, pos0, 10000.0)
    assert np.allclose(o_l[:n], c, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P3
def test_p3_factorised_equals_explicit_nxn():
    """The S, z factorisation of the linear branch equals its explicit N x N
    form (the 4x16x16 tiny grid, N = 1024, d = 64, r = 16)."""
    rng = np.random.default_rng(4)
    grid, n, d, r = (4, 16, 16), 1024, 64, 16
    q, k, v = _rand_head(rng, n, n, d)
    uq, uk = rng.standard_normal((d, r)) / 8, rng.standard_normal((d, r)) / 8
    pos = R.token_positions(grid, n)
    a = R.linear_branch(q, k, v, n, uq, uk, pos, 10000.0)
    b = R.linear_branch_explicit(q, k, v, n, uq, uk, pos, 10000.0)
    assert rel(a, b) <= 1e-13


def test_p3b_ragged_n_ignores_pad_keys():
    """Pad keys (j >= N) carry garbage and must not enter S or z."""
    rng = np.random.default_rng(5)
    grid, n, npad, d, r = (2, 5, 7), 70, 128, 16, 16
    q, k, v = _rand_head(rng, n, npad, d)
    uq, uk = rng.standard_normal((d, r)) / 4, rng.standard_normal((d, r)) / 4
    pos = R.token_positions(grid, n)
    a = R.linear_branch(q, k, v, n, uq, uk, pos, 10000.0)
    k2, v2 = k.copy(), v.copy()
    k2[n:] = 0.0
    v2[n:] = 0.0
    b = R.linear_branch_explicit(q, k2, v2, n, uq, uk, pos, 10000.0)
    assert rel(a[:n], b[:n]) <= 1e-13
    assert np.all(a[n:] == 0)


# ---------------------------------------------------------------- P4 RoPE
def test_p4_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(6)
    n, r = 97, 64
    pos = rng.integers(0, 50, size=(n, 3))
    fq, fk = rng.standard_normal((n, r)), rng.standard_normal((n, r))
    w0 = R.rope(fq, pos, 10000.0) @ R.rope(fk, pos, 10000.0).T
    shift = np.array([3, -7, 11])
    w1 = R.rope(fq, pos + shift, 10000.0) @ R.rope(fk, pos + shift, 10000.0).T
    assert np.max(np.abs(w0 - w1)) <= 1e-12 * np.max(np.abs(w0))


def test_p4_rope_is_orthogonal_and_identity_at_origin():
    rng = np.random.default_rng(7)
    f = rng.standard_normal((40, 32))
    pos = rng.integers(0, 80, size=(40, 3))
    g = R.rope(f, pos, 10000.0)
    assert np.allclose(np.linalg.norm(g, axis=1), np.linalg.norm(f, axis=1), rtol=1e-14)
    assert np.array_equal(R.rope(f, np.zeros_like(pos), 10000.0), f)


def test_p4_rope_pairs_rotate_like_complex_multiplication():
    """Adjacent pairs (2j, 2j+1) turn counter-clockwise: x0 + i x1 -> (x0 + i x1) e^{i psi}."""
    rng = np.random.default_rng(8)
    n, r = 25, 16
    f = rng.standard_normal((n, r))
    pos = rng.integers(0, 30, size=(n, 3))
    ang = R.rope_angles(pos, r, 10000.0)
    zc = (f[:, 0::2] + 1j * f[:, 1::2]) * np.exp(1j * ang)
    g = R.rope(f, pos, 10000.0)
    assert np.allclose(g[:, 0::2], zc.real, atol=1e-14)
    assert np.allclose(g[:, 1::2], zc.imag, atol=1e-14)


def test_p4_rope_frequencies_and_axis_split_by_hand():
    """r = 16 splits 6:6:4 over (t, h, w).  At p = (1, 1, 1) and base 10000 the
    pair frequencies are 10000^(-2m/D): t and h blocks (D = 6) give 1,
    10000^(-1/3), 10000^(-2/3); the w block (D = 4) gives 1 and 0.01."""
    ang = R.rope_angles(np.array([[1, 1, 1]]), 16, 10000.0)[0]
    c3 = 10000.0 ** (-1.0 / 3.0)  # 0.0464158883...
    expect = [1.0, c3, c3 * c3, 1.0, c3, c3 * c3, 1.0, 0.01]
    assert np.allclose(ang, expect, rtol=1e-14)
    assert abs(c3 - 0.046415888336127795) < 1e-15
    # moving along one axis only touches that axis's block of feature dims
    f = np.random.default_rng(9).standard_normal((1, 64))
    base = R.rope(f, np.array([[0, 0, 0]]), 10000.0)
    for ax, (lo, hi) in enumerate([(0, 24), (24, 48), (48, 64)]):
        p = np.zeros((1, 3), dtype=np.int64)
        p[0, ax] = 5
        g = R.rope(f, p, 10000.0)
        changed = np.nonzero(np.abs(g - base)[0] > 0)[0]
        assert changed.min() >= lo and changed.max() < hi


def test_p4_elu1_matches_torch_elu_plus_one():
    x = np.concatenate([np.random.default_rng(10).standard_normal(1000) * 4, [0.0, -0.0, 1e-300, -50.0]])
    ref = (torch.nn.functional.elu(torch.from_numpy(x)) + 1.0).numpy()
    # torch forms (e^x - 1) + 1, which rounds at the scale of 1; the oracle's e^x is exact
    assert np.allclose(R.elu1(x), ref, rtol=1e-15, atol=4e-16)
    assert np.all(R.elu1(x) > 0)


def test_wo_is_applied_on_the_right():
    """O_lW = O_l W_o with row vectors: a W_o whose only entry is W_o[0, 1] = 1
    copies column 0 of O_l into column 1 of O_lW."""
    rng = np.random.default_rng(11)
    grid, n, d, r = (1, 8, 16), 128, 16, 16
    q, k, v = _rand_head(rng, n, n, d)
    uq, uk = rng.standard_normal((d, r)) / 4, rng.standard_normal((d, r)) / 4
    wo = np.zeros((d, d))
    wo[0, 1] = 1.0
    out = R.hybrid_head(q, k, v, n, grid, uq, uk, wo, topk=1, force_diag=False, scale=0.25, base=10000.0)
    assert np.array_equal(out["o_lw"][:, 1], out["o_l"][:, 0])
    assert np.all(np.delete(out["o_lw"], 1, axis=1) == 0)
    assert np.array_equal(out["o"], out["o_s"] + out["o_lw"])


# ---------------------------------------------------------------- P5 top-k
def _brute_keep(s, k):
    t = len(s)
    keep = []
    for b in range(t):
        rank = sum(1 for c in range(t) if s[c] > s[b] or (s[c] == s[b] and c < b))
        if rank < k:
            keep.append(b)
    return keep


@pytest.mark.parametrize("seed", range(20))
def test_p5_topk_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    t = int(rng.integers(1, 40))
    s = rng.integers(-5, 6, size=t).astype(np.float64)  # many exact ties
    for k in sorted({1, int(rng.integers(1, t + 1)), t}):
        assert list(R.select_row(s, k)) == _brute_keep(s, k)


def test_p5_topk_special_cases():
    s = np.array([0.5, 2.0, 2.0, -1.0, 2.0])
    assert list(R.select_row(s, 1)) == [1]          # argmax, lowest index among ties
    assert list(R.select_row(s, 5)) == [0, 1, 2, 3, 4]
    assert list(R.select_row(s, 2, diag=3)) == [1, 2, 3]   # union with the diagonal
    assert list(R.select_row(s, 2, diag=2)) == [1, 2]      # diagonal already kept


def test_p5_duplicated_tiles_force_exact_ties():
    """Two identical key tiles get identical pooled scores; the lower index wins."""
    rng = np.random.default_rng(12)
    d = 16
    k = rng.standard_normal((4 * 64, d))
    k[128:192] = k[0:64]            # tile 2 duplicates tile 0
    q = np.tile(k[0:64].mean(axis=0) * 3, (256, 1))
    sc = R.pooled_scores(R.tile_means(q, 256), R.tile_means(k, 256))
    assert sc[0, 0] == sc[0, 2]
    top1 = R.select_row(sc[0], 1)
    assert list(top1) in ([0], [1], [3])
    if sc[0, 0] == sc[0].max():
        assert list(top1) == [0]


# ---------------------------------------------------------------- O1 positions
def test_o1_token_positions_by_hand():
    """Frame-major raster on a grid whose three extents all differ (G_t, G_h,
    G_w) = (3, 5, 7): token i sits at frame i // 35, row (i // 7) mod 5, column
    i mod 7.  Coordinates written out by hand for tokens on every boundary, so
    that swapped h and w fields, or a row taken as i // G_h, fail."""
    pos = R.token_positions((3, 5, 7), 105)
    by_hand = {
        0: (0, 0, 0), 1: (0, 0, 1), 6: (0, 0, 6),       # first row of frame 0
        7: (0, 1, 0), 10: (0, 1, 3), 13: (0, 1, 6),     # second row
        34: (0, 4, 6),                                  # last token of frame 0
        35: (1, 0, 0), 36: (1, 0, 1), 43: (1, 1, 1),    # frame 1
        69: (1, 4, 6), 70: (2, 0, 0), 104: (2, 4, 6),   # last token
    }
    for i, p in by_hand.items():
        assert tuple(int(x) for x in pos[i]) == p, f"token {i}"
    # every coordinate in range and every (t, h, w) exactly once
    assert pos[:, 0].max() == 2 and pos[:, 1].max() == 4 and pos[:, 2].max() == 6
    assert len({tuple(p) for p in pos.tolist()}) == 105


def test_o1_positions_of_the_720p_latent_grid_by_hand():
    """On the 21 x 45 x 80 latent grid one frame holds 3600 tokens; token 3600
    starts frame 1, token 80 starts row 1, token 75599 is (20, 44, 79)."""
    pos = R.token_positions((21, 45, 80), 75600)
    assert tuple(pos[3600]) == (1, 0, 0)
    assert tuple(pos[80]) == (0, 1, 0)
    assert tuple(pos[3600 + 2 * 80 + 5]) == (1, 2, 5)
    assert tuple(pos[75599]) == (20, 44, 79)


# ---------------------------------------------------------------- O3 orientation
def test_o3_pooled_scores_by_hand_are_query_rows_key_columns():
    """sigma[a, b] = qbar_a . kbar_b with query tiles as rows: a 2 x 2 case
    worked out by hand, whose transpose differs."""
    qbar = np.array([[1.0, 0.0], [0.0, 2.0]])
    kbar = np.array([[3.0, 1.0], [5.0, 7.0]])
    sc = R.pooled_scores(qbar, kbar)
    assert sc.tolist() == [[3.0, 5.0], [2.0, 14.0]]   # transposed would be [[3, 2], [5, 14]]


def test_o3_asymmetric_scores_against_explicit_loops():
    rng = np.random.default_rng(33)
    qbar, kbar = rng.standard_normal((5, 6)), rng.standard_normal((5, 6))
    sc = R.pooled_scores(qbar, kbar)
    for a in range(5):
        for b in range(5):
            assert abs(sc[a, b] - sum(qbar[a, e] * kbar[b, e] for e in range(6))) <= 1e-14
    assert np.abs(sc - sc.T).max() > 0.1   # the case is asymmetric


def test_o3_o4_top1_of_the_hybrid_follows_the_query_rows():
    """Three tiles whose rows are constant: query tile a holds basis vector e_a,
    key tile b holds e_(b+1 mod 3).  Query tile 0 then matches key tile 2,
    tile 1 key tile 0, tile 2 key tile 1; read with the grid transposed (or the
    arguments swapped) the answer would be [1], [2], [0]."""
    d, r, n = 4, 16, 192
    q = np.zeros((n, d))
    k = np.zeros((n, d))
    for a in range(3):
        q[64 * a:64 * a + 64, a] = 1.0
        k[64 * a:64 * a + 64, (a + 1) % 3] = 1.0
    v = np.random.default_rng(3).standard_normal((n, d))
    uq = uk = np.zeros((d, r))
    out = R.hybrid_head(q, k, v, n, (1, 3, 64), uq, uk, np.zeros((d, d)), topk=1, force_diag=False,
                        scale=0.5, base=10000.0)
    assert [list(x) for x in out["rows"]] == [[2], [0], [1]]
    assert out["scores"][0, 2] == 1.0 and out["scores"][2, 0] == 0.0


# ---------------------------------------------------------------- P6 pooling
def test_p6_pooling_closed_forms():
    d = 8
    row = np.arange(d, dtype=np.float64) - 3.5
    x = np.tile(row, (192, 1))
    x[170:] = 1e6  # pad rows (n = 170) must not count
    m = R.tile_means(x, 170)
    assert np.array_equal(m, np.tile(row, (3, 1)))
    y = np.zeros((128, 1))
    y[64:74, 0] = np.arange(10)  # partial tile: 10 valid rows 0..9
    assert R.tile_means(y, 74)[1, 0] == 4.5


# ---------------------------------------------------------------- P7 fp8
def test_p7_e4m3fn_decode_matches_torch_over_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = R.e4m3fn_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.nanmax(got) == 448.0 and np.nanmin(got[got > 0]) == 2.0 ** -9


def test_p7_dequantize_applies_each_tiles_scale():
    codes = np.full((128, 4), 0x38, dtype=np.uint8)  # 0x38 encodes 1.0
    x = R.dequantize_tiles(codes, np.array([0.5, 3.0]))
    assert np.all(x[:64] == 0.5) and np.all(x[64:] == 3.0)


# ---------------------------------------------------------------- P8 page arithmetic
def test_p8_sparse_compute_ratio_matches_the_page():
    g = json.load(open(os.path.join(GOLDEN, "sparsity_compute_ratio.json")))
    gt, gh, gw = g["grid"]
    t = -(-gt * gh * gw // 64)
    assert t == 512
    before = R.executed_flops(t * g["topk_before"], 128)
    after = R.executed_flops(t * g["topk_after"], 128)
    assert abs(after / before - g["compute_ratio_about"]) <= g["compute_ratio_tolerance"]
    assert abs(1 - g["topk_before"] / t - 0.90) < 0.002
    assert abs(1 - g["topk_after"] / t - 0.97) < 0.002
    assert abs(g["kept_fraction_after"] / g["kept_fraction_before"] - g["compute_ratio_about"]) < 1e-12


def test_latent_grids_follow_the_pages_frame_and_pixel_sizes():
    from workloads import WORKLOADS
    g = json.load(open(os.path.join(GOLDEN, "wan_latent_grids.json")))
    for key, name in (("480p", "wan14b_480p_bf16"), ("720p", "wan14b_720p_bf16")):
        want = (1 + (g["frames"] - 1) // 4, g[key]["height"] // 16, g[key]["width"] // 16)
        assert tuple(g[key]["grid"]) == want
        assert WORKLOADS[name].grid == want and WORKLOADS[name].N == g[key]["tokens"]


# ---------------------------------------------------------------- P9 determinism
def test_p9_oracle_is_deterministic_and_thread_independent():
    from threadpoolctl import threadpool_limits
    from workloads import make_workload, generate
    from workloads.gen import to_fp64
    w = make_workload("tiny_f32")
    inp = generate(w)
    args = (to_fp64(inp.q[0, 0]), to_fp64(inp.k[0, 0]), to_fp64(inp.v[0, 0]), w.N, w.grid,
            to_fp64(inp.uq[0]), to_fp64(inp.uk[0]), to_fp64(inp.wo[0]))
    kw = dict(topk=w.topk, force_diag=w.force_diag, scale=w.softmax_scale, base=w.rope_base)
    a = R.hybrid_head(*args, **kw)
    b = R.hybrid_head(*args, **kw)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["col_idx"], b["col_idx"])
    with threadpool_limits(limits=1):
        c = R.hybrid_head(*args, **kw)
    assert np.array_equal(a["col_idx"], c["col_idx"])
    assert rel(c["o"], a["o"]) <= 1e-14
    # the tiny workload keeps the diagonal plus the top 4: 4 or 5 tiles per row
    for i, row in enumerate(a["rows"]):
        assert i in row and len(row) in (4, 5)
