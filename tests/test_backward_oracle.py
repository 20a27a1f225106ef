"""Pins of the oracle's gradients of the hybrid (the mask held fixed).

Central finite differences of the already-pinned forward (every input
coordinate of a tiny head, sampled ones of a larger head), torch autograd
through scaled-dot-product attention (all tiles kept), and closed forms.
"""
import math

import numpy as np
import pytest
import torch

from oracle import rola as R

BASE = 10000.0


def _head(seed, grid, npad, d, r, wo_scale=0.3):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2]
    q, k, v = (rng.standard_normal((npad, d)) for _ in range(3))
    uq = rng.standard_normal((d, r)) / np.sqrt(d)
    uk = rng.standard_normal((d, r)) / np.sqrt(d)
    wo = rng.standard_normal((d, d)) * wo_scale
    return rng, n, q, k, v, uq, uk, wo


def _loss(q, k, v, n, grid, uq, uk, wo, rows, scale, w):
    out = R.hybrid_head(q, k, v, n, grid, uq, uk, wo, topk=1, force_diag=False, scale=scale, base=BASE,
                        kept_rows=rows)
    return float((out["o"][:n] * w[:n]).sum())


def _fd(f, x, idx, h=1e-5):
    xp, xm = x.copy(), x.copy()
    xp[idx] += h
    xm[idx] -= h
    return (f(xp) - f(xm)) / (2 * h)


def test_every_coordinate_against_central_differences():
    grid, npad, d, r = (1, 10, 15), 192, 4, 16
    rng, n, q, k, v, uq, uk, wo = _head(21, grid, npad, d, r)
    rows = [np.array([0, 2]), np.array([1]), np.array([0, 1, 2])]
    w = rng.standard_normal((npad, d))
    grads = R.hybrid_backward(q, k, v, n, grid, uq, uk, wo, rows, 0.4, BASE, w)
    for t, (x, gx) in enumerate(zip((q, k, v), grads)):
        def f(xx):
            args = [q, k, v]
            args[t] = xx
            return _loss(*args, n, grid, uq, uk, wo, rows, 0.4, w)
        num = np.zeros_like(x)
        for i in range(n):
            for e in range(d):
                num[i, e] = _fd(f, x, (i, e))
        assert np.max(np.abs(num - gx)) <= 1e-7 * max(1.0, np.max(np.abs(gx))), t
        assert np.all(gx[n:] == 0)


def test_sampled_coordinates_of_a_larger_head():
    grid, npad, d, r = (2, 9, 13), 256, 16, 32
    rng, n, q, k, v, uq, uk, wo = _head(22, grid, npad, d, r)
    t = npad // 64
    rows = [np.sort(rng.choice(t, size=2, replace=False)) for _ in range(t)]
    w = rng.standard_normal((npad, d))
    grads = R.hybrid_backward(q, k, v, n, grid, uq, uk, wo, rows, d ** -0.5, BASE, w)
    for tt, (x, gx) in enumerate(zip((q, k, v), grads)):
        def f(xx):
            args = [q, k, v]
            args[tt] = xx
            return _loss(*args, n, grid, uq, uk, wo, rows, d ** -0.5, w)
        for _ in range(12):
            idx = (int(rng.integers(0, n)), int(rng.integers(0, d)))
            assert abs(_fd(f, x, idx) - gx[idx]) <= 1e-7 * max(1.0, abs(gx[idx]))


def test_all_tiles_kept_and_zero_wo_match_autograd_of_sdpa():
    """k = T, W_o = 0: the gradients are those of dense softmax attention, taken
    by torch autograd through scaled_dot_product_attention in float64."""
    grid, npad, d, r = (2, 8, 10), 192, 16, 16
    rng, n, q, k, v, uq, uk, wo = _head(23, grid, npad, d, r)
    t = npad // 64
    rows = [np.arange(t)] * t
    g = rng.standard_normal((npad, d))
    grads = R.hybrid_backward(q, k, v, n, grid, uq, uk, np.zeros((d, d)), rows, 1 / math.sqrt(d), BASE, g)
    tq, tk, tv = (torch.tensor(x[:n], dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], scale=1 / math.sqrt(d))[0]
    o.backward(torch.tensor(g[:n]))
    for got, want in zip(grads, (tq.grad, tk.grad, tv.grad)):
        assert np.max(np.abs(got[:n] - want.numpy())) <= 1e-12 * np.max(np.abs(want.numpy()))


def test_value_gradient_of_uniform_attention_is_a_mean():
    """q = 0: every kept key gets weight 1/|J|, so dv_j = sum over the queries
    keeping j of g_i / |J_i|, and dq, dk of the sparse branch vanish when g is
    orthogonal to every v (here v = 0)."""
    n, npad, d = 150, 192, 6
    rng = np.random.default_rng(24)
    q = np.zeros((npad, d))
    k = rng.standard_normal((npad, d))
    v = np.zeros((npad, d))
    g = rng.standard_normal((npad, d))
    rows = [np.array([1]), np.array([0, 2]), np.array([2])]
    dq, dk, dv = R.sparse_backward(q, k, v, n, rows, 0.5, g)
    want = np.zeros((npad, d))
    for a, kept in enumerate(rows):
        keys = [j for b in kept for j in range(64 * b, min(64 * b + 64, n))]
        for j in keys:
            want[j] += g[64 * a:min(64 * a + 64, n)].sum(axis=0) / len(keys)
    assert np.allclose(dv, want, rtol=0, atol=1e-13)
    assert np.all(dq == 0) and np.all(dk == 0)


def test_rope_transpose_inverts_rope():
    rng = np.random.default_rng(25)
    pos = rng.integers(0, 50, size=(40, 3))
    f = rng.standard_normal((40, 32))
    back = R.rope_transpose(R.rope(f, pos, BASE), pos, BASE)
    assert np.allclose(back, f, rtol=0, atol=1e-12)
    x = np.array([-2.0, -0.1, 0.0, 0.3, 4.0])
    assert np.allclose(R.elu1_grad(x), np.where(x > 0, 1.0, np.exp(x)), rtol=0, atol=0)
