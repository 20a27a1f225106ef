"""Pad rows (rows N .. N_pad-1 of Q, K, V and of the upstream gradient) may
hold anything: every call reads them through views bounded at row N, so
non-finite garbage there (NaN, +-inf; the NaN byte 0x7F for E4M3FN codes)
must leave every output bit and the selected mask unchanged.

Each case runs a call twice on the GPU, once with zero pad rows and once with
garbage pad rows, and compares the two results bitwise: block selection
(mask and tile means), the sparse branch alone (output and log-sum-exp), the
linear branch alone, the complement variant, the hybrid call with its
exported mask, and the backward pass.
"""
import dataclasses

import pytest
import torch

from block_sparse_linear_select_amd import binding as B
from tests import helpers as Hp

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

NAMES = ["f32_d128_r64", "bf16_ragged", "bf16_d64_r16", "fp8_ragged", "bf16_long_rows"]


def _dirty(t: torch.Tensor, N: int) -> torch.Tensor:
    """A copy of t [B, H, N_pad, d] whose rows >= N hold garbage, cycling
    over NaN, +inf, -inf and 3e38 along the rows (fp8: the NaN codes 0x7F,
    0xFF and the largest codes +-448)."""
    out = t.clone()
    pad = out.shape[2] - N
    if t.dtype == torch.float8_e4m3fn:
        codes = torch.tensor([0x7F, 0xFF, 0x7E, 0xFE], dtype=torch.uint8)
        vals = codes[torch.arange(pad) % 4].view(1, 1, pad, 1).expand(out.shape[0], out.shape[1], pad, out.shape[3])
        out.view(torch.uint8)[:, :, N:] = vals.to(t.device)
        return out
    vals = torch.tensor([float("nan"), float("inf"), float("-inf"), 3.0e38], dtype=torch.float32)
    vals = vals[torch.arange(pad) % 4].view(1, 1, pad, 1)
    out[:, :, N:] = vals.to(t.dtype).to(t.device)
    return out


def _pair(name):
    w = Hp.CASES[name]
    assert w.N < w.N_pad, "the case must have pad rows"
    inp = Hp.gen(w)
    clean = Hp.to_device(inp, DEV)
    dirty = dict(clean)
    for key in ("q", "k", "v"):
        dirty[key] = _dirty(clean[key], w.N)
    return w, B.Config.from_workload(w), clean, dirty


def _same(a, b, what):
    torch.cuda.synchronize()
    if a.dtype.is_floating_point:
        # NaN-aware bitwise: compare the raw bits
        a = a.contiguous().view(torch.uint8 if a.element_size() == 1 else
                                {2: torch.int16, 4: torch.int32, 8: torch.int64}[a.element_size()])
        b = b.contiguous().view(a.dtype)
    assert torch.equal(a, b), what


def _same_csr(a, b, what):
    """Equal masks: row pointers, and the column indices they cover (the
    index array may be longer than the mask)."""
    _same(a[0], b[0], f"{what} row_ptr")
    n = int(a[0][-1])
    _same(a[1][:n], b[1][:n], f"{what} col_idx")


def _scales(d):
    return d["q_scale"], d["k_scale"], d["v_scale"]


@pytest.mark.parametrize("name", NAMES)
def test_forward_calls_ignore_pad_rows(name):
    print(f"\n[case {name}]", flush=True)
    w, cfg, c, g = _pair(name)
    qs, ks, vs = _scales(c)
    # selection: the mask and the exported tile means
    sel = [B.block_select(cfg, d["q"], d["k"], qs, ks, want_means=True) for d in (c, g)]
    _same_csr(sel[0][:2], sel[1][:2], "select")
    _same(sel[0][2], sel[1][2], "select qbar")
    _same(sel[0][3], sel[1][3], "select kbar")
    rp, ci = sel[0][0], sel[0][1]
    # sparse branch alone
    sp = [B.sparse_attn(cfg, d["q"], d["k"], d["v"], rp, ci, qs, ks, vs, want_lse=True) for d in (c, g)]
    _same(sp[0][0], sp[1][0], "sparse o")
    _same(sp[0][1][:, :, :w.N], sp[1][1][:, :, :w.N], "sparse lse")
    assert torch.all(sp[1][0][:, :, w.N:] == 0)
    # linear branch alone
    li = [B.linear_attn(cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], qs, ks, vs) for d in (c, g)]
    _same(li[0], li[1], "linear o")
    assert torch.all(li[1][:, :, w.N:] == 0)
    # complement variant
    cc = dataclasses.replace(cfg, linear_keys="complement")
    co = [B.linear_attn_complement(cc, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], rp, ci, qs, ks, vs)
          for d in (c, g)]
    _same(co[0], co[1], "complement o")
    # hybrid with its own mask, exported
    hy = [B.hybrid_attn(cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], qs, ks, vs, export_mask=True)
          for d in (c, g)]
    _same(hy[0][0], hy[1][0], "hybrid o")
    _same_csr(hy[0][1:], hy[1][1:], "hybrid")
    _same_csr(hy[0][1:], (rp, ci), "hybrid mask = selection mask:")
    assert torch.all(hy[1][0][:, :, w.N:] == 0)
    assert torch.isfinite(hy[1][0].float()).all()
    print("  bitwise equal: select, sparse, linear, complement, hybrid", flush=True)


@pytest.mark.parametrize("name", ["f32_d128_r64", "bf16_ragged", "bf16_d64_r16"])
def test_backward_ignores_pad_rows(name):
    print(f"\n[case {name}]", flush=True)
    from workloads.gen import upstream_grad
    w, cfg, c, g = _pair(name)
    rp, ci = B.block_select(cfg, c["q"], c["k"])
    go = upstream_grad(w, seed=w.seed + 3).to(DEV)
    go_dirty = _dirty(go, w.N)
    res = [B.hybrid_attn_backward(cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], rp, ci, gg)
           for d, gg in ((c, go), (g, go_dirty))]
    for x, y, what in zip(res[0], res[1], ("dq", "dk", "dv")):
        _same(x, y, what)
        assert torch.all(y[:, :, w.N:] == 0)
    print("  bitwise equal: dq, dk, dv", flush=True)
