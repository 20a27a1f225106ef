"""Pins of the oracle's linear branch over the complement of the kept tiles
(O8c: for the queries of tile a, the linear sums run over the valid keys whose
tile is not in M_a).

Checked against brute force over keys on tiny inputs, the all-keys branch
(itself pinned to the explicit N x N form), a closed form, and the identity
that the complement and the kept part add up to the whole.
"""
import numpy as np
import pytest
import torch

from oracle import rola as R

BASE = 10000.0


def _head(seed, grid, npad, d, r):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2]
    q = rng.standard_normal((npad, d))
    k = rng.standard_normal((npad, d))
    v = rng.standard_normal((npad, d))
    uq = rng.standard_normal((d, r)) / np.sqrt(d)
    uk = rng.standard_normal((d, r)) / np.sqrt(d)
    return rng, n, q, k, v, uq, uk


def _features(x, u):
    """phi = elu + 1 through torch (independent of the oracle's elu1)."""
    t = torch.from_numpy(np.ascontiguousarray(x)) @ torch.from_numpy(u)
    return (torch.nn.functional.elu(t) + 1.0).numpy()


def test_brute_force_over_keys_on_a_ragged_tiny_head():
    """Python loops over every (query, key) pair, keys filtered by their tile;
    asymmetric masks, an empty row and a row naming tiles twice."""
    grid, npad, d, r = (1, 10, 15), 192, 6, 16
    _, n, q, k, v, uq, uk = _head(11, grid, npad, d, r)
    pos = R.token_positions(grid, n)
    rows = [np.array([1]), np.array([0, 0, 2]), np.array([], dtype=np.int64)]
    got = R.linear_branch_complement(q, k, v, n, uq, uk, pos, BASE, rows)
    fq, fk = _features(q[:n], uq), _features(k[:n], uk)
    rq, rk = R.rope(fq, pos, BASE), R.rope(fk, pos, BASE)
    want = np.zeros((npad, d))
    for i in range(n):
        kept = set(int(b) for b in rows[i // 64])
        num = np.zeros(d)
        den = 0.0
        for j in range(n):
            if j // 64 in kept:
                continue
            num += float(np.dot(rq[i], rk[j])) * v[j]
            den += float(np.dot(fq[i], fk[j]))
        want[i] = num / den
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    assert np.all(got[n:] == 0)


def test_rows_with_no_kept_tile_equal_the_all_keys_branch():
    grid, npad, d, r = (2, 8, 9), 192, 16, 32
    _, n, q, k, v, uq, uk = _head(12, grid, npad, d, r)
    pos = R.token_positions(grid, n)
    rows = [np.array([], dtype=np.int64)] * 3
    a = R.linear_branch_complement(q, k, v, n, uq, uk, pos, BASE, rows)
    b = R.linear_branch(q, k, v, n, uq, uk, pos, BASE)
    assert np.max(np.abs(a - b)) <= 1e-13 * np.max(np.abs(b))


def test_rows_keeping_every_tile_give_zero_and_stray_entries_are_ignored():
    grid, npad, d, r = (2, 8, 9), 192, 16, 16
    _, n, q, k, v, uq, uk = _head(13, grid, npad, d, r)
    pos = R.token_positions(grid, n)
    rows = [np.array([0, 1, 2]), np.array([-1, 0, 1, 1, 2, 7]), np.array([0, 2, 5])]
    out = R.linear_branch_complement(q, k, v, n, uq, uk, pos, BASE, rows)
    assert np.all(out[:128] == 0)
    # row 2 keeps tiles 0 and 2 only (5 is no tile): its complement is tile 1
    ref = R.linear_branch_complement(q, k, v, n, uq, uk, pos, BASE, [None, None, np.array([0, 2])], tiles=[2])
    assert np.array_equal(out[128:], ref[128:])
    assert np.any(out[128:n] != 0)


def test_constant_values_and_no_rotation_give_the_constant():
    """v_j = c and every RoPE angle zero: the weights phi_q . phi_k are positive,
    so O_l is a convex combination of copies of c on every row with keys left."""
    grid, npad, d, r = (3, 7, 9), 192, 8, 32
    rng, n, q, k, _, uq, uk = _head(14, grid, npad, d, r)
    c = rng.standard_normal(d)
    v = np.tile(c, (npad, 1))
    pos0 = np.zeros((n, 3), dtype=np.int64)
    rows = [np.array([0]), np.array([0, 1, 2]), np.array([1, 2])]
    out = R.linear_branch_complement(q, k, v, n, uq, uk, pos0, BASE, rows)
    assert np.allclose(out[:64], c, rtol=0, atol=1e-13)
    assert np.all(out[64:128] == 0)
    assert np.allclose(out[128:n], c, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", [15, 16])
def test_complement_and_kept_parts_add_up_to_all_keys(seed):
    """num_C + num_M = num_all and den_C + den_M = den_all, where M's part is
    the complement branch evaluated on the complementary mask; denominators
    from torch features."""
    grid, npad, d, r = (2, 16, 11), 384, 12, 32
    rng, n, q, k, v, uq, uk = _head(seed, grid, npad, d, r)
    t = npad // 64
    pos = R.token_positions(grid, n)
    rows = [np.sort(rng.choice(t, size=rng.integers(1, t), replace=False)) for _ in range(t)]
    other = [np.setdiff1d(np.arange(t), m) for m in rows]
    oc = R.linear_branch_complement(q, k, v, n, uq, uk, pos, BASE, rows)
    om = R.linear_branch_complement(q, k, v, n, uq, uk, pos, BASE, other)
    oa = R.linear_branch(q, k, v, n, uq, uk, pos, BASE)
    fq, fk = _features(q[:n], uq), _features(k[:n], uk)
    tile_of = np.arange(n) // 64
    lhs = np.zeros((n, d))
    den_all = fq @ fk.sum(axis=0)
    for i in range(n):
        in_m = np.isin(tile_of, rows[i // 64])
        den_c = fq[i] @ fk[~in_m].sum(axis=0)
        den_m = fq[i] @ fk[in_m].sum(axis=0)
        lhs[i] = oc[i] * den_c + om[i] * den_m
    rhs = oa[:n] * den_all[:, None]
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))


def test_hybrid_head_with_complement_keys():
    grid, npad, d, r = (2, 8, 8), 128, 16, 16
    rng, n, q, k, v, uq, uk = _head(17, grid, npad, d, r)
    wo = rng.standard_normal((d, d)) * 0.1
    out = R.hybrid_head(q, k, v, n, grid, uq, uk, wo, topk=1, force_diag=False, scale=0.25, base=BASE,
                        linear_keys="complement")
    pos = R.token_positions(grid, n)
    ol = R.linear_branch_complement(q, k, v, n, uq, uk, pos, BASE, out["rows"])
    assert np.array_equal(out["o_l"], ol)
    assert np.allclose(out["o"], out["o_s"] + ol @ wo, rtol=0, atol=1e-14)
    with pytest.raises(ValueError):
        R.hybrid_head(q, k, v, n, grid, uq, uk, wo, topk=1, force_diag=False, scale=0.25, base=BASE,
                      linear_keys="kept")


def test_a_row_with_no_kept_tile_has_zero_sparse_output():
    """The sparse branch of a row that keeps nothing is 0, and the hybrid of
    such a row is the all-keys linear branch alone."""
    grid, npad, d, r = (2, 8, 9), 192, 16, 16
    rng, n, q, k, v, uq, uk = _head(18, grid, npad, d, r)
    rows = [np.array([], dtype=np.int64), np.array([0, 2]), np.array([1])]
    o_s = R.sparse_branch(q, k, v, n, rows, scale=0.3)
    assert np.all(o_s[:64] == 0) and np.any(o_s[64:n] != 0)
    wo = rng.standard_normal((d, d)) * 0.1
    out = R.hybrid_head(q, k, v, n, grid, uq, uk, wo, topk=1, force_diag=False, scale=0.3, base=BASE,
                        kept_rows=rows, linear_keys="complement")
    full = R.linear_branch(q, k, v, n, uq, uk, R.token_positions(grid, n), BASE) @ wo
    assert np.allclose(out["o"][:64], full[:64], rtol=0, atol=1e-13)
