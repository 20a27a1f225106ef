"""Plain, slow fp64 CPU oracle of the RoLA-style hybrid attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this module; the product path never calls it and
shares no code with it.

What it computes (one (b, h) slice at a time, every step in float64):

* The method (SparkDiffusion news article, section 05 "RoLA"; the RoLA paper
  title on the arXiv 2609.23153 listing, "Sources"): a block-sparse softmax
  branch keeps the high-energy query-key tile interactions, and a low-rank
  linear-attention branch carrying rotary position information restores the
  global context that sparsification drops.  The branches are summed.
* Tiles are 64 tokens.  Sparsity 90% / 97% means 10% / 3% of the tiles are
  kept (same article, section 01), realised here as a fixed top-k per query-tile
  row.

The pages give the structure only.  The concrete formulation used here, and
every reading taken where the pages are silent, is listed in the design notes;
in short:

  O1 positions   p_i = (t, h, w) of token i in frame-major raster order
  O2 pooling     qbar_a, kbar_a = mean of the valid rows of tile a
  O3 scores      sigma_ab = qbar_a . kbar_b (unscaled)
  O4 selection   M_a = first k tiles b by (sigma_ab desc, b asc) [+ {a} if forced]
  O5 sparse      softmax(tau q_i . k_j) over the valid keys of the kept tiles
  O6 features    phi(x) = elu(x) + 1 applied to q U_q and k U_k
  O7 3D RoPE     r dims split 3r/8 : 3r/8 : r/4 over (t, h, w); pair m of an axis
                 block of D dims turns by p_axis * base^(-2m/D)
  O8 linear      O_l,i = sum_j (rho_i phi_q,i . rho_j phi_k,j) v_j / sum_j phi_q,i . phi_k,j
                 over all valid keys, RoPE in the numerator only
  O8c variant    the same sums over the valid keys outside the query tile's kept tiles
  O9 output      O_i = O_s,i + O_l,i W_o for valid rows, 0 for pad rows
  O11 fp8        X = E4M3FN code value * per-(tile) scale

Pins: every function here is checked in tests/test_oracle_pins.py against
library routines (torch scaled-dot-product attention, torch casts, torch elu),
closed forms, brute force and invariants.  None of the absolute output values
is pinned by the pages, which print no worked example.
"""
from __future__ import annotations

import numpy as np

TILE = 64


# ---------------------------------------------------------------- O1 positions
def token_positions(grid, n):
    """Integer (t, h, w) coordinates of tokens 0..n-1, frame-major raster."""
    gt, gh, gw = (int(g) for g in grid)
    assert gt * gh * gw == n
    pos = np.empty((n, 3), dtype=np.int64)
    for i in range(n):
        pos[i, 0] = i // (gh * gw)
        pos[i, 1] = (i // gw) % gh
        pos[i, 2] = i % gw
    return pos


# ------------------------------------------------------------------ O2 pooling
def tile_means(x, n, tile=TILE):
    """Mean of the valid rows (index < n) of each tile of x [N_pad, d]."""
    npad, d = x.shape
    t = npad // tile
    out = np.zeros((t, d), dtype=np.float64)
    for a in range(t):
        lo, hi = a * tile, min(a * tile + tile, n)
        out[a] = np.asarray(x[lo:hi], dtype=np.float64).sum(axis=0) / float(hi - lo)
    return out


# ------------------------------------------------------------------- O3 scores
def pooled_scores(qbar, kbar):
    """sigma[a, b] = qbar_a . kbar_b, no scale (top-k ignores a positive scale)."""
    return np.asarray(qbar, np.float64) @ np.asarray(kbar, np.float64).T


# ---------------------------------------------------------------- O4 selection
def select_row(scores_row, topk, diag=None):
    """Kept tiles of one row: the first `topk` indices in (score desc, index asc)
    order, plus `diag` if given; returned sorted ascending."""
    s = np.asarray(scores_row, dtype=np.float64)
    order = np.lexsort((np.arange(s.size), -s))  # primary: -score, secondary: index
    kept = set(int(b) for b in order[:topk])
    if diag is not None:
        kept.add(int(diag))
    return np.array(sorted(kept), dtype=np.int64)


def select(scores, topk, force_diag=False):
    """Kept-tile lists of every row of a [T, T] score grid."""
    return [select_row(scores[a], topk, a if force_diag else None) for a in range(scores.shape[0])]


def to_csr(rows):
    """(row_ptr, col_idx) int64 arrays of a list of sorted kept-tile lists."""
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    for a, r in enumerate(rows):
        row_ptr[a + 1] = row_ptr[a] + len(r)
    col_idx = np.concatenate([np.asarray(r, np.int64) for r in rows]) if rows else np.zeros(0, np.int64)
    return row_ptr, col_idx


def from_csr(row_ptr, col_idx):
    return [np.asarray(col_idx[row_ptr[a]:row_ptr[a + 1]], np.int64) for a in range(len(row_ptr) - 1)]


# ------------------------------------------------------------- O5 sparse branch
def sparse_tile(q, k, v, n, a, kept, scale, tile=TILE):
    """Softmax attention of the valid query rows of tile a over the valid keys of
    the kept tiles.  Returns [rows, d] for rows a*tile .. min(a*tile+tile, n).
    With no kept key the rows are 0 (a softmax over nothing adds nothing)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    qlo, qhi = a * tile, min(a * tile + tile, n)
    keys = np.array([j for b in kept for j in range(b * tile, min(b * tile + tile, n))], dtype=np.int64)
    if keys.size == 0:
        return np.zeros((qhi - qlo, q.shape[1]), dtype=np.float64)
    s = scale * (q[qlo:qhi] @ k[keys].T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return (e @ v[keys]) / e.sum(axis=1, keepdims=True)


def sparse_branch(q, k, v, n, rows, scale, tile=TILE):
    """O_s [N_pad, d]; pad rows zero."""
    out = np.zeros((q.shape[0], q.shape[1]), dtype=np.float64)
    for a, kept in enumerate(rows):
        lo, hi = a * tile, min(a * tile + tile, n)
        if hi > lo:
            out[lo:hi] = sparse_tile(q, k, v, n, a, kept, scale, tile)
    return out


# ------------------------------------------------------------ O6 feature map
def elu1(x):
    """phi(x) = elu(x) + 1: x + 1 for x > 0, exp(x) otherwise (always > 0)."""
    x = np.asarray(x, np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


# ------------------------------------------------------------------ O7 3D RoPE
def rope_split(r):
    """Feature dims per axis (t, h, w): 3r/8, 3r/8, r/4 (requires r % 16 == 0)."""
    assert r % 16 == 0, "rank must be a multiple of 16 for an even 3:3:2 split"
    return (3 * r // 8, 3 * r // 8, r // 4)


def rope_angles(pos, r, base):
    """Rotation angle of every feature pair: [n, r/2].  Pair m of the block of
    axis ax (D dims) turns by pos[:, ax] * base**(-2m/D)."""
    pos = np.asarray(pos, np.float64)
    out = []
    for ax, dim in enumerate(rope_split(r)):
        m = np.arange(dim // 2, dtype=np.float64)
        theta = np.power(float(base), -2.0 * m / dim)
        out.append(pos[:, ax:ax + 1] * theta[None, :])
    return np.concatenate(out, axis=1)


def rope(f, pos, base):
    """Rotate adjacent pairs (2j, 2j+1) of f [n, r] by the angles of rope_angles."""
    f = np.asarray(f, np.float64)
    ang = rope_angles(pos, f.shape[1], base)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = f[:, 0::2], f[:, 1::2]
    out = np.empty_like(f)
    out[:, 0::2] = x0 * c - x1 * s
    out[:, 1::2] = x0 * s + x1 * c
    return out


# ------------------------------------------------------------ O8 linear branch
def linear_state(k, v, n, uk, pos, base):
    """Factorised key/value state: S = sum_j rho_j phi(k_j U_k) v_j^T  [r, d] and
    z = sum_j phi(k_j U_k)  [r], over valid keys j < n."""
    fk = elu1(np.asarray(k[:n], np.float64) @ np.asarray(uk, np.float64))
    S = rope(fk, pos[:n], base).T @ np.asarray(v[:n], np.float64)
    z = fk.sum(axis=0)
    return S, z


def linear_readout(q, n, uq, S, z, pos, base):
    """O_l,i = (rho_i phi(q_i U_q))^T S / (phi(q_i U_q) . z) for valid rows; [n, d]."""
    fq = elu1(np.asarray(q[:n], np.float64) @ np.asarray(uq, np.float64))
    num = rope(fq, pos[:n], base) @ S
    den = fq @ z
    return num / den[:, None]


def linear_branch(q, k, v, n, uq, uk, pos, base):
    S, z = linear_state(k, v, n, uk, pos, base)
    out = np.zeros((q.shape[0], q.shape[1]), dtype=np.float64)
    out[:n] = linear_readout(q, n, uq, S, z, pos, base)
    return out


def linear_branch_explicit(q, k, v, n, uq, uk, pos, base):
    """The same branch in its explicit N x N form (small n only)."""
    fq = elu1(np.asarray(q[:n], np.float64) @ np.asarray(uq, np.float64))
    fk = elu1(np.asarray(k[:n], np.float64) @ np.asarray(uk, np.float64))
    rq, rk = rope(fq, pos[:n], base), rope(fk, pos[:n], base)
    num_w = rq @ rk.T            # [n, n] rotary-positioned weights
    den_w = fq @ fk.T            # [n, n] unrotated (positive) weights
    out = np.zeros((q.shape[0], q.shape[1]), dtype=np.float64)
    out[:n] = (num_w @ np.asarray(v[:n], np.float64)) / den_w.sum(axis=1, keepdims=True)
    return out


# -------------------------------------- O8c linear branch over the complement
def complement_keys(kept, n, t, tile=TILE):
    """Valid keys j < n whose tile is not in `kept` (a list of tile indices;
    repeats count once and indices outside [0, t) name no tile)."""
    in_kept = np.zeros(t, dtype=bool)
    for b in kept:
        if 0 <= int(b) < t:
            in_kept[int(b)] = True
    return np.nonzero(~in_kept[np.arange(n) // tile])[0]


def linear_branch_complement(q, k, v, n, uq, uk, pos, base, rows, tile=TILE, tiles=None):
    """The linear branch over the context the sparse branch leaves out (the RoLA
    section of the SparkDiffusion news article: the linear branch restores what
    sparsification discards; SLA in the 2026-05-02 survey post routes the
    non-critical weights to linear attention).  For the queries of tile a the
    sums of O8 run over complement_keys(M_a) only:
      O_l,i = sum_{j in C_a} (rho_i phi_q,i . rho_j phi_k,j) v_j / sum_{j in C_a} phi_q,i . phi_k,j.
    A tile whose kept set covers every tile has no such key: its rows are 0.
    `tiles`: compute only these query tiles (the others stay 0).  [N_pad, d]"""
    q = np.asarray(q, np.float64)
    fq = elu1(q[:n] @ np.asarray(uq, np.float64))
    fk = elu1(np.asarray(k[:n], np.float64) @ np.asarray(uk, np.float64))
    rq, rk = rope(fq, pos[:n], base), rope(fk, pos[:n], base)
    vv = np.asarray(v[:n], np.float64)
    t = q.shape[0] // tile
    out = np.zeros((q.shape[0], q.shape[1]), dtype=np.float64)
    for a in (range(len(rows)) if tiles is None else tiles):
        lo, hi = a * tile, min(a * tile + tile, n)
        c = complement_keys(rows[a], n, t, tile)
        if hi <= lo or c.size == 0:
            continue
        S = rk[c].T @ vv[c]          # [r, d] state of the complement keys
        z = fk[c].sum(axis=0)        # [r]
        out[lo:hi] = (rq[lo:hi] @ S) / (fq[lo:hi] @ z)[:, None]
    return out


# --------------------------------------------------------------- O9 the hybrid
def hybrid_head(q, k, v, n, grid, uq, uk, wo, topk, force_diag, scale, base,
                tile=TILE, kept_rows=None, linear_keys="all"):
    """Everything for one (b, h): mask, O_s, O_lW = O_l W_o and O = O_s + O_lW.

    kept_rows: use this mask instead of selecting one (e.g. to evaluate outputs
    on a given CSR).  linear_keys: "all" (O8) or "complement" (O8c)."""
    pos = token_positions(grid, n)
    scores = None
    if kept_rows is None:
        scores = pooled_scores(tile_means(q, n, tile), tile_means(k, n, tile))
        kept_rows = select(scores, topk, force_diag)
    o_s = sparse_branch(q, k, v, n, kept_rows, scale, tile)
    if linear_keys == "all":
        o_l = linear_branch(q, k, v, n, uq, uk, pos, base)
    elif linear_keys == "complement":
        o_l = linear_branch_complement(q, k, v, n, uq, uk, pos, base, kept_rows, tile)
    else:
        raise ValueError(f"linear_keys={linear_keys!r}")
    o_lw = o_l @ np.asarray(wo, np.float64)
    o_lw[n:] = 0.0
    row_ptr, col_idx = to_csr(kept_rows)
    return {"scores": scores, "rows": kept_rows, "row_ptr": row_ptr, "col_idx": col_idx,
            "o_s": o_s, "o_l": o_l, "o_lw": o_lw, "o": o_s + o_lw}


# ------------------------------------------------- backward (gradients of O)
# The mask is held fixed (the top-k selection is piecewise constant in the
# inputs and has no gradient); upstream gradient g = dL/dO on the valid rows.
def elu1_grad(x):
    """phi'(x): 1 for x > 0, exp(x) otherwise."""
    x = np.asarray(x, np.float64)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def rope_transpose(f, pos, base):
    """rho_i^T applied row-wise: each pair turned back by its angle."""
    f = np.asarray(f, np.float64)
    ang = rope_angles(pos, f.shape[1], base)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = f[:, 0::2], f[:, 1::2]
    out = np.empty_like(f)
    out[:, 0::2] = x0 * c + x1 * s
    out[:, 1::2] = -x0 * s + x1 * c
    return out


def sparse_backward(q, k, v, n, rows, scale, g, tile=TILE):
    """Gradients of O_s (O5) for upstream g [N_pad, d].  For the queries of tile
    a over the kept keys: P = softmax(scale q k^T), dP = g v^T,
    dS = P * (dP - rowsum(P * dP)), dq = scale dS k, dk += scale dS^T q,
    dv += P^T g.  Returns (dq, dk, dv), each [N_pad, d], zero on pad rows."""
    q, k, v, g = (np.asarray(x, np.float64) for x in (q, k, v, g))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for a, kept in enumerate(rows):
        lo, hi = a * tile, min(a * tile + tile, n)
        keys = np.array([j for b in kept for j in range(b * tile, min(b * tile + tile, n))], dtype=np.int64)
        if hi <= lo or keys.size == 0:
            continue
        s = scale * (q[lo:hi] @ k[keys].T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = g[lo:hi] @ v[keys].T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[lo:hi] = scale * (ds @ k[keys])
        np.add.at(dk, keys, scale * (ds.T @ q[lo:hi]))
        np.add.at(dv, keys, p.T @ g[lo:hi])
    return dq, dk, dv


def linear_backward(q, k, v, n, uq, uk, pos, base, gl):
    """Gradients of O_l (O8, all valid keys) for upstream gl = dL/dO_l [N_pad, d],
    by the chain rule through O_l = num / den, num = rho(phi(q U_q)) S,
    den = phi(q U_q) . z, S = sum_j rho_j phi(k_j U_k) v_j^T, z = sum_j phi(k_j U_k).
    Returns (dq, dk, dv), each [N_pad, d], zero on pad rows."""
    q, k, v, gl = (np.asarray(x, np.float64) for x in (q, k, v, gl))
    uq, uk = np.asarray(uq, np.float64), np.asarray(uk, np.float64)
    xq, xk = q[:n] @ uq, k[:n] @ uk
    fq, fk = elu1(xq), elu1(xk)
    rq, rk = rope(fq, pos[:n], base), rope(fk, pos[:n], base)
    S, z = rk.T @ v[:n], fk.sum(axis=0)
    den = fq @ z
    ol = (rq @ S) / den[:, None]
    gnum = gl[:n] / den[:, None]                 # dL/dnum
    gden = -(gl[:n] * ol).sum(axis=1) / den      # dL/dden
    d_rq = gnum @ S.T                            # dL/d(rho phi_q)   [n, r]
    dS = rq.T @ gnum                             # dL/dS             [r, d]
    dz = fq.T @ gden                             # dL/dz             [r]
    d_xq = (gden[:, None] * z[None, :] + rope_transpose(d_rq, pos[:n], base)) * elu1_grad(xq)
    d_rk = v[:n] @ dS.T                          # dL/d(rho phi_k)   [n, r]
    d_xk = (dz[None, :] + rope_transpose(d_rk, pos[:n], base)) * elu1_grad(xk)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dq[:n] = d_xq @ uq.T
    dk[:n] = d_xk @ uk.T
    dv[:n] = rk @ dS
    return dq, dk, dv


def hybrid_backward(q, k, v, n, grid, uq, uk, wo, rows, scale, base, g, tile=TILE):
    """Gradients of O = O_s + O_l W_o (all-keys linear branch) on a fixed mask,
    for upstream g = dL/dO [N_pad, d] (pad rows of g are ignored)."""
    g = np.asarray(g, np.float64).copy()
    g[n:] = 0.0
    pos = token_positions(grid, n)
    s_grads = sparse_backward(q, k, v, n, rows, scale, g, tile)
    l_grads = linear_backward(q, k, v, n, uq, uk, pos, base, g @ np.asarray(wo, np.float64).T)
    return tuple(a + b for a, b in zip(s_grads, l_grads))


# ----------------------------------------------------------------- O11 FP8
def e4m3fn_decode(codes):
    """Value of OCP FP8 E4M3FN byte codes: 1 sign bit, 4 exponent bits (bias 7),
    3 mantissa bits, subnormals at exponent 0, NaN at S.1111.111, no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.power(2.0, e - 7)
    sub = (m / 8.0) * 2.0 ** (1 - 7)
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def dequantize_tiles(codes, scales, tile=TILE):
    """X = value(code) * scale of its 64-token tile; codes [N_pad, d], scales [T]."""
    x = e4m3fn_decode(codes)
    return x * np.repeat(np.asarray(scales, np.float64), tile)[:, None]


# ------------------------------------------------------- work accounting
def executed_flops(nnz_tiles, d, tile=TILE):
    """Multiply-add FLOPs of the sparse branch: QK^T and PV per kept tile pair."""
    return 4.0 * tile * tile * d * nnz_tiles


def dense_equivalent_flops(n, d, heads, batch=1):
    return 4.0 * n * n * d * heads * batch
