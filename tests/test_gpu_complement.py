"""GPU parity of the complement-key variant of the linear branch (for the
queries of tile a, the linear sums run over the valid keys outside the kept
tiles of row a) against the fp64 oracle, through the C ABI.

Outputs are computed on the oracle's own mask and compared by relative L2
error over all valid rows (1e-2 bf16, 5e-2 fp8, 1e-4 float32): the hybrid O
and, through the standalone call, the branch O_lW alone.  Edge rows: no kept
tile (the complement is every key), every tile kept (O_l = 0), more than half
of the tiles kept (the kernel sums the complement's states directly instead of
subtracting the kept ones), repeated and out-of-range entries.
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_linear_select_amd import binding as B
from oracle import rola as R
from tests import helpers as Hp
from workloads import generate, make_workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

NAMES = ["tiny_f32", "bf16_ragged", "bf16_r64", "bf16_d64_r16", "bf16_aligned_diag", "f32_d128_r64",
         "bf16_dense_all_tiles", "fp8_ragged", "fp8_r64_diag", "bf16_long_rows", "fp8_long_rows",
         "bf16_many_heads", "fp8_many_heads"]


def _cfg(w):
    return dataclasses.replace(B.Config.from_workload(w), linear_keys="complement")


def _oracle(inp, b, h, rows):
    w = inp.w
    q, k, v = Hp.head_arrays(inp, b, h)
    uq, uk, wo = Hp.params(inp, h)
    return R.hybrid_head(q, k, v, w.N, w.grid, uq, uk, wo, w.topk, w.force_diag, w.softmax_scale, w.rope_base,
                         kept_rows=rows, linear_keys="complement")


def _args(d):
    return (d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"])


def _scales(d):
    return dict(q_scale=d["q_scale"], k_scale=d["k_scale"], v_scale=d["v_scale"])


@pytest.mark.parametrize("name", NAMES)
def test_complement_on_oracle_mask(name):
    print(f"\n[case {name}]", flush=True)
    inp = Hp.gen(name)
    w = inp.w
    d = Hp.to_device(inp, DEV)
    cfg = _cfg(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rows = {bh: Hp.oracle_mask_head(inp, *bh)[1] for bh in heads}
    ref = {bh: _oracle(inp, *bh, rows[bh]) for bh in heads}
    rp, ci = Hp.csr_tensors([rows[bh] for bh in heads], DEV)
    o = B.hybrid_attn(cfg, *_args(d), **_scales(d), row_ptr=rp, col_idx=ci)
    ol = B.linear_attn_complement(cfg, *_args(d), rp, ci, **_scales(d))
    o_again = B.hybrid_attn(cfg, *_args(d), **_scales(d), row_ptr=rp, col_idx=ci)
    o_own, rp_own, ci_own = B.hybrid_attn(cfg, *_args(d), **_scales(d), export_mask=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_again)
    if torch.equal(rp_own, rp) and torch.equal(ci_own[: int(rp[-1])], ci):
        assert torch.equal(o_own, o)
    on, oln = o.float().cpu().numpy(), ol.float().cpu().numpy()
    err_o, err_l = Hp.RelL2(), Hp.RelL2()
    for b, h in heads:
        err_o.add(on[b, h, :w.N], ref[(b, h)]["o"][:w.N])
        err_l.add(oln[b, h, :w.N], ref[(b, h)]["o_lw"][:w.N])
        assert np.all(on[b, h, w.N:] == 0) and np.all(oln[b, h, w.N:] == 0)
    print(f"  O rel L2 {err_o}, O_lW rel L2 {err_l}", flush=True)
    assert err_o.value <= Hp.TOL[w.dtype]
    assert err_l.value <= Hp.TOL[w.dtype]


def _edge_rows(T, rng):
    rows = [np.sort(rng.choice(T, size=min(3, T), replace=False)) for _ in range(T)]
    rows[0] = np.array([], dtype=np.int64)                          # complement = every key
    rows[1] = np.arange(T)                                          # no complement: O_l = 0
    rows[2] = np.delete(np.arange(T), T // 2)                       # one tile left, summed directly
    rows[3] = np.sort(rng.choice(T, size=T // 2 + 1, replace=False))  # just over half kept
    rows[4] = np.sort(rng.choice(T, size=T // 2, replace=False))      # exactly half: subtracted
    return rows


@pytest.mark.parametrize("name", ["tiny_f32", "bf16_ragged", "fp8_ragged", "bf16_d64_r16"])
def test_complement_edge_rows(name):
    w = Hp.CASES[name]
    inp = Hp.gen(w)
    d = Hp.to_device(inp, DEV)
    cfg = _cfg(w)
    T = w.T
    assert T >= 6
    rng = np.random.default_rng(5)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rows = {bh: _edge_rows(T, rng) for bh in heads}
    # the same mask written with repeats and entries outside [0, T), which name no tile
    stray = {}
    for bh in heads:
        r = [x.copy() for x in rows[bh]]
        r[5] = np.sort(np.concatenate([[-3, -1], r[5], r[5][:1], [T, T + 7]]))
        r[0] = np.array([-1, T])
        stray[bh] = r
    rp, ci = Hp.csr_tensors([rows[bh] for bh in heads], DEV)
    rps, cis = Hp.csr_tensors([stray[bh] for bh in heads], DEV)
    o = B.hybrid_attn(cfg, *_args(d), **_scales(d), row_ptr=rp, col_idx=ci)
    ol = B.linear_attn_complement(cfg, *_args(d), rp, ci, **_scales(d))
    ol_stray = B.linear_attn_complement(cfg, *_args(d), rps, cis, **_scales(d))
    torch.cuda.synchronize()
    assert torch.equal(ol, ol_stray)
    on, oln = o.float().cpu().numpy(), ol.float().cpu().numpy()
    err_o, err_l = Hp.RelL2(), Hp.RelL2()
    for b, h in heads:
        ref = _oracle(inp, b, h, rows[(b, h)])
        ref_l = R.linear_branch_complement(*Hp.head_arrays(inp, b, h)[:3], w.N, *Hp.params(inp, h)[:2],
                                           R.token_positions(w.grid, w.N), w.rope_base, stray[(b, h)])
        ref_lw = ref_l @ Hp.params(inp, h)[2]
        ref_lw[w.N:] = 0.0
        assert np.allclose(ref_lw, ref["o_lw"], rtol=0, atol=1e-12)
        err_o.add(on[b, h, :w.N], ref["o"][:w.N])
        err_l.add(oln[b, h, :w.N], ref["o_lw"][:w.N])
        assert np.all(oln[b, h, 64:128] == 0)  # row 1 keeps every tile
        # row 0 keeps nothing: the all-keys branch
        full = R.linear_branch(*Hp.head_arrays(inp, b, h)[:3], w.N, *Hp.params(inp, h)[:2],
                               R.token_positions(w.grid, w.N), w.rope_base) @ Hp.params(inp, h)[2]
        e0 = np.linalg.norm(oln[b, h, :64] - full[:64]) / np.linalg.norm(full[:64])
        assert e0 <= Hp.TOL[w.dtype]
    print(f"  O rel L2 {err_o}, O_lW rel L2 {err_l}", flush=True)
    assert err_o.value <= Hp.TOL[w.dtype]
    assert err_l.value <= Hp.TOL[w.dtype]


def test_complement_workspace_contents_do_not_matter(monkeypatch):
    w = Hp.CASES["bf16_ragged"]
    inp = Hp.gen(w)
    d = Hp.to_device(inp, DEV)
    cfg = _cfg(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rp, ci = Hp.csr_tensors([Hp.oracle_mask_head(inp, *bh)[1] for bh in heads], DEV)

    def run(fill):
        monkeypatch.setattr(B, "_workspace", lambda c, call, dev: torch.full(
            (max(B.workspace_size(c, call), 256),), fill, dtype=torch.uint8, device=dev))
        out = [B.hybrid_attn(cfg, *_args(d), **_scales(d), export_mask=True)[0],
               B.hybrid_attn(cfg, *_args(d), **_scales(d), row_ptr=rp, col_idx=ci),
               B.linear_attn_complement(cfg, *_args(d), rp, ci, **_scales(d))]
        torch.cuda.synchronize()
        return [t.clone() for t in out]

    for x, y in zip(run(0), run(255)):
        assert torch.equal(x, y)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["wan14b_720p_bf16", "wan14b_720p_fp8"])
def test_complement_full_size_sampled(name):
    """720P, 40 heads, in the configuration a timed hybrid call runs (selection
    inside): sampled query tiles of three heads against the oracle evaluated
    on the GPU's own mask, for O and for the branch alone."""
    w = make_workload(name)
    print(f"\n[{name}] generating", flush=True)
    inp = generate(w)
    d = Hp.to_device(inp, DEV)
    cfg = _cfg(w)
    o, rp, ci = B.hybrid_attn(cfg, *_args(d), **_scales(d), export_mask=True)
    ol = B.linear_attn_complement(cfg, *_args(d), rp, ci, **_scales(d))
    torch.cuda.synchronize()
    rows = Hp.split_csr(rp, ci, w.H, w.T)
    rng = np.random.default_rng(1)
    tiles = sorted({0, 1, w.T // 2, w.T - 1, *rng.integers(0, w.T, 2).tolist()})
    pos = R.token_positions(w.grid, w.N)
    err_o, err_l = Hp.RelL2(), Hp.RelL2()
    for h in (0, w.H // 2, w.H - 1):
        qh, kh, vh = Hp.head_arrays(inp, 0, h)
        uq, uk, wo = Hp.params(inp, h)
        ref_l = R.linear_branch_complement(qh, kh, vh, w.N, uq, uk, pos, w.rope_base, rows[h], tiles=tiles)
        for a in tiles:
            lo, hi = a * 64, min(a * 64 + 64, w.N)
            ref_s = R.sparse_tile(qh, kh, vh, w.N, a, rows[h][a], w.softmax_scale)
            ref_lw = ref_l[lo:hi] @ wo
            err_o.add(o[0, h, lo:hi].float().cpu().numpy(), ref_s + ref_lw)
            err_l.add(ol[0, h, lo:hi].float().cpu().numpy(), ref_lw)
        assert torch.all(o[0, h, w.N:] == 0)
    print(f"  sampled rel L2: O {err_o.value:.2e}, O_lW {err_l.value:.2e}", flush=True)
    assert err_o.value <= Hp.TOL[w.dtype]
    assert err_l.value <= Hp.TOL[w.dtype]
