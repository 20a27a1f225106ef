"""GPU parity of the backward pass (dQ, dK, dV on a fixed mask) against the
fp64 oracle, through the C ABI.

Each case: the oracle's own mask, a seeded upstream gradient (pad rows hold
garbage the library must ignore), and relative L2 error over the valid rows
of all heads, per gradient: the whole hybrid, the sparse branch alone (W_o = 0
makes the linear branch's gradient vanish) and the linear branch alone (the
difference of the two GPU results, whose sparse parts are computed
identically).
"""
import numpy as np
import pytest
import torch

from block_sparse_linear_select_amd import binding as B
from oracle import rola as R
from tests import helpers as Hp
from workloads.gen import to_fp64, upstream_grad

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# bf16: the recomputed probabilities, dS and the operands of every product are
# rounded to bf16 (relative 2^-9 each) and D comes from the bf16-rounded O_s;
# float32: accumulation order and the hardware exp2 only.
TOL = {"f32": 1e-4, "bf16": 1e-2}

NAMES = ["tiny_f32", "bf16_ragged", "bf16_r64", "bf16_d64_r16", "bf16_aligned_diag", "f32_d128_r64",
         "bf16_dense_all_tiles", "bf16_long_rows", "bf16_many_heads"]


def _run(cfg, d, rp, ci, g, wo=None):
    return B.hybrid_attn_backward(cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"] if wo is None else wo,
                                  rp, ci, g)


@pytest.mark.parametrize("name", NAMES)
def test_backward_on_oracle_mask(name):
    print(f"\n[case {name}]", flush=True)
    inp = Hp.gen(name)
    w = inp.w
    d = Hp.to_device(inp, DEV)
    cfg = B.Config.from_workload(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rows = {bh: Hp.oracle_mask_head(inp, *bh)[1] for bh in heads}
    rp, ci = Hp.csr_tensors([rows[bh] for bh in heads], DEV)
    g = upstream_grad(w, seed=w.seed + 7, pad_value=3.0)
    gd = g.to(DEV)
    full = _run(cfg, d, rp, ci, gd)
    sparse = _run(cfg, d, rp, ci, gd, wo=torch.zeros_like(d["wo"]))
    again = _run(cfg, d, rp, ci, gd)
    torch.cuda.synchronize()
    for x, y in zip(full, again):
        assert torch.equal(x, y)  # bitwise reproducible
    full = [t.cpu().numpy() for t in full]
    sparse = [t.cpu().numpy() for t in sparse]
    errs = {k: [Hp.RelL2() for _ in range(3)] for k in ("hybrid", "sparse", "linear")}
    for b, h in heads:
        q, k, v = Hp.head_arrays(inp, b, h)
        uq, uk, wo = Hp.params(inp, h)
        gh = to_fp64(g[b, h])
        gh[w.N:] = 0.0
        ref_s = R.sparse_backward(q, k, v, w.N, rows[(b, h)], w.softmax_scale, gh)
        pos = R.token_positions(w.grid, w.N)
        ref_l = R.linear_backward(q, k, v, w.N, uq, uk, pos, w.rope_base, gh @ wo.T)
        for t in range(3):
            errs["hybrid"][t].add(full[t][b, h, :w.N], (ref_s[t] + ref_l[t])[:w.N])
            errs["sparse"][t].add(sparse[t][b, h, :w.N], ref_s[t][:w.N])
            errs["linear"][t].add((full[t] - sparse[t])[b, h, :w.N], ref_l[t][:w.N])
            assert np.all(full[t][b, h, w.N:] == 0)
    for key, e in errs.items():
        print(f"  {key}: dQ {e[0]}  dK {e[1]}  dV {e[2]}", flush=True)
    for key, e in errs.items():
        for t in range(3):
            assert e[t].value <= TOL[w.dtype], (key, t, e[t].value)


def test_backward_workspace_contents_do_not_matter(monkeypatch):
    w = Hp.CASES["bf16_ragged"]
    inp = Hp.gen(w)
    d = Hp.to_device(inp, DEV)
    cfg = B.Config.from_workload(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rp, ci = Hp.csr_tensors([Hp.oracle_mask_head(inp, *bh)[1] for bh in heads], DEV)
    gd = upstream_grad(w, seed=5).to(DEV)

    def run(fill):
        monkeypatch.setattr(B, "_workspace", lambda c, call, dev: torch.full(
            (max(B.workspace_size(c, call), 256),), fill, dtype=torch.uint8, device=dev))
        out = _run(cfg, d, rp, ci, gd)
        torch.cuda.synchronize()
        return [t.clone() for t in out]

    for x, y in zip(run(0), run(255)):
        assert torch.equal(x, y)


def test_backward_rejects_fp8_and_the_complement_variant():
    import dataclasses
    w = Hp.CASES["fp8_ragged"]
    inp = Hp.gen(w)
    d = Hp.to_device(inp, DEV)
    cfg = B.Config.from_workload(w)
    rp = torch.zeros(cfg.B * cfg.H * cfg.T + 1, dtype=torch.int32, device=DEV)
    ci = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(B.HsaError):
        B.hybrid_attn_backward(cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], rp, ci, d["q"])
    w2 = Hp.CASES["bf16_ragged"]
    inp2 = Hp.gen(w2)
    d2 = Hp.to_device(inp2, DEV)
    cfg2 = dataclasses.replace(B.Config.from_workload(w2), linear_keys="complement")
    rp2 = torch.zeros(cfg2.B * cfg2.H * cfg2.T + 1, dtype=torch.int32, device=DEV)
    with pytest.raises(B.HsaError):
        B.hybrid_attn_backward(cfg2, d2["q"], d2["k"], d2["v"], d2["uq"], d2["uk"], d2["wo"], rp2, ci, d2["q"])


@pytest.mark.timeout(900)
def test_backward_full_size_sampled():
    """720P bf16 (40 heads, 75600 tokens) on the mask the library selects:
    dQ of sampled query tiles and dK, dV of sampled key tiles of three heads
    against the oracle, which evaluates only the rows that reach them."""
    from workloads import generate, make_workload
    w = make_workload("wan14b_720p_bf16")
    print("\n[wan14b_720p_bf16] generating", flush=True)
    inp = generate(w)
    d = Hp.to_device(inp, DEV)
    cfg = B.Config.from_workload(w)
    rp, ci = B.block_select(cfg, d["q"], d["k"])
    g = upstream_grad(w, seed=11)
    dq, dk, dv = B.hybrid_attn_backward(cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], rp, ci, g.to(DEV))
    torch.cuda.synchronize()
    rows = Hp.split_csr(rp, ci, w.H, w.T)
    rng = np.random.default_rng(3)
    tiles = sorted({0, w.T // 2, w.T - 1, *rng.integers(0, w.T, 2).tolist()})
    pos = R.token_positions(w.grid, w.N)
    errs = [Hp.RelL2() for _ in range(3)]
    for h in (0, w.H // 2, w.H - 1):
        q, k, v = Hp.head_arrays(inp, 0, h)
        uq, uk, wo = Hp.params(inp, h)
        gh = to_fp64(g[0, h])
        ref_l = R.linear_backward(q, k, v, w.N, uq, uk, pos, w.rope_base, gh @ wo.T)
        for a in tiles:
            lo, hi = 64 * a, min(64 * a + 64, w.N)
            only = [rows[h][x] if x == a else np.zeros(0, np.int64) for x in range(w.T)]
            ref_q = R.sparse_backward(q, k, v, w.N, only, w.softmax_scale, gh)[0]
            errs[0].add(dq[0, h, lo:hi].cpu().numpy(), (ref_q + ref_l[0])[lo:hi])
            keepers = [x for x in range(w.T) if a in set(rows[h][x].tolist())]
            col = [rows[h][x] if x in keepers else np.zeros(0, np.int64) for x in range(w.T)]
            _, ref_k, ref_v = R.sparse_backward(q, k, v, w.N, col, w.softmax_scale, gh)
            errs[1].add(dk[0, h, lo:hi].cpu().numpy(), (ref_k + ref_l[1])[lo:hi])
            errs[2].add(dv[0, h, lo:hi].cpu().numpy(), (ref_v + ref_l[2])[lo:hi])
        for t in (dq, dk, dv):
            assert torch.all(t[0, h, w.N:] == 0)
    print(f"  sampled rel L2: dQ {errs[0]}  dK {errs[1]}  dV {errs[2]}", flush=True)
    for e in errs:
        assert e.value <= TOL["bf16"]


@pytest.mark.parametrize("name", ["tiny_f32", "bf16_ragged", "bf16_d64_r16"])
def test_backward_edge_rows(name):
    """A row keeping no tile (its sparse gradients vanish), a row keeping every
    tile, rows with entries outside [0, T) (skipped, as the forward skips
    them), on the GPU against the oracle given the same mask without them.
    The descriptor's topk is the longest row (T), which sizes the transposed
    mask."""
    import dataclasses
    w = Hp.CASES[name]
    inp = Hp.gen(w)
    d = Hp.to_device(inp, DEV)
    T = w.T
    cfg = dataclasses.replace(B.Config.from_workload(w), topk=T)
    rng = np.random.default_rng(9)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    clean, dirty = {}, {}
    for bh in heads:
        rows = [np.sort(rng.choice(T, size=min(3, T), replace=False)) for _ in range(T)]
        rows[0] = np.zeros(0, np.int64)
        rows[1] = np.arange(T)
        clean[bh] = rows
        dr = [r.copy() for r in rows]
        dr[2] = np.concatenate([[-2], dr[2], [T, T + 3]])
        dr[0] = np.array([-1, T])
        dirty[bh] = dr
    rp, ci = Hp.csr_tensors([dirty[bh] for bh in heads], DEV)
    g = upstream_grad(w, seed=w.seed + 9)
    grads = [t.cpu().numpy() for t in _run(cfg, d, rp, ci, g.to(DEV))]
    errs = [Hp.RelL2() for _ in range(3)]
    for b, h in heads:
        q, k, v = Hp.head_arrays(inp, b, h)
        uq, uk, wo = Hp.params(inp, h)
        ref = R.hybrid_backward(q, k, v, w.N, w.grid, uq, uk, wo, clean[(b, h)], w.softmax_scale, w.rope_base,
                                to_fp64(g[b, h]))
        for t in range(3):
            errs[t].add(grads[t][b, h, :w.N], ref[t][:w.N])
    print(f"  dQ {errs[0]}  dK {errs[1]}  dV {errs[2]}", flush=True)
    for e in errs:
        assert e.value <= TOL[w.dtype]


def _same_bits(a, b):
    a, b = a.contiguous(), b.contiguous()
    if a.dtype.is_floating_point:
        it = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[a.element_size()]
        a, b = a.view(it), b.view(it)
    return torch.equal(a, b)


@pytest.mark.parametrize("name", ["tiny_f32", "bf16_ragged", "bf16_d64_r16", "bf16_aligned_diag"])
def test_training_forward_saves_the_sparse_output_and_lse(name):
    """O of the training forward is bitwise hsa_hybrid_attn's; O_s and the
    log-sum-exp it saves are bitwise hsa_sparse_attn's on the same mask."""
    print(f"\n[case {name}]", flush=True)
    inp = Hp.gen(name)
    w = inp.w
    d = Hp.to_device(inp, DEV)
    cfg = B.Config.from_workload(w)
    args = (cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"])
    o, o_s, lse, rp, ci = B.hybrid_attn_train(*args, export_mask=True)
    o_ref, rp_ref, ci_ref = B.hybrid_attn(*args, export_mask=True)
    torch.cuda.synchronize()
    assert _same_bits(o, o_ref)
    assert torch.equal(rp, rp_ref)
    n = int(rp[-1])
    assert torch.equal(ci[:n], ci_ref[:n])
    os_ref, lse_ref = B.sparse_attn(cfg, d["q"], d["k"], d["v"], rp, ci, want_lse=True)
    torch.cuda.synchronize()
    assert _same_bits(o_s, os_ref)
    assert _same_bits(lse[:, :, :w.N], lse_ref[:, :, :w.N])
    assert torch.all(o_s[:, :, w.N:] == 0)


@pytest.mark.parametrize("name", ["tiny_f32", "bf16_ragged", "bf16_d64_r16", "bf16_aligned_diag", "bf16_long_rows"])
def test_backward_on_saved_statistics_equals_the_recomputing_backward(name):
    """The backward fed the training forward's O_s and log-sum-exp gives the
    recomputing backward's gradients bit for bit."""
    print(f"\n[case {name}]", flush=True)
    inp = Hp.gen(name)
    w = inp.w
    d = Hp.to_device(inp, DEV)
    cfg = B.Config.from_workload(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rp, ci = Hp.csr_tensors([Hp.oracle_mask_head(inp, *bh)[1] for bh in heads], DEV)
    g = upstream_grad(w, seed=w.seed + 21, pad_value=3.0).to(DEV)
    _, o_s, lse = B.hybrid_attn_train(cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], row_ptr=rp, col_idx=ci)
    ref = _run(cfg, d, rp, ci, g)
    got = B.hybrid_attn_backward_saved(cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], rp, ci, o_s, lse, g)
    torch.cuda.synchronize()
    for x, y, what in zip(ref, got, ("dq", "dk", "dv")):
        assert _same_bits(x, y), what
