"""GPU parity of the W8A8 FP8 QKV projection against the CPU oracle
(oracle/proj.py), through the C ABI.

* Row quantisation of the activations: bit-exact (codes and scales).
* Projection: the kernel decides the output codes on float32 accumulators,
  whose distance from the exact Y is bounded by the float32 summation bound
  K 2^-24 sum_k |x_k w_k| (any order) plus the rounding of the two scale
  products.  Within that bound: the scales match the oracle's, and every code
  is a nearest E4M3 code of Y / s; outside the bands around rounding
  midpoints the codes equal the oracle's.  Sampled units at the 720P shape
  use the same checks.
"""
import numpy as np
import pytest
import torch

from block_sparse_linear_select_amd import binding as B
from oracle import proj as P
from oracle.rola import e4m3fn_decode
from workloads import make_workload
from workloads.gen import generate_proj

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _codes(t):
    return t.view(torch.uint8).cpu().numpy()


def test_row_quantisation_is_bit_exact():
    rng = np.random.default_rng(11)
    x = torch.from_numpy(rng.standard_normal((301, 520)).astype(np.float32) * 3).to(torch.bfloat16)
    x[7] = 0.0
    x[8, 5] = -0.0
    x[9] = torch.from_numpy(np.float32(2.0) ** rng.integers(-30, 30, 520).astype(np.float32)).to(torch.bfloat16)
    codes, sc = B.quantize_rows_fp8(x.to(DEV))
    torch.cuda.synchronize()
    ref_c, ref_s = P.quantize_rows(x.float().numpy())
    np.testing.assert_array_equal(sc.cpu().numpy(), ref_s)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_c)


def _step(v):
    """E4M3 spacing at |v| (normal range 2^-6 .. 448; subnormal spacing 2^-9)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
    return 2.0 ** (e - 3)


def _bound(y_exact, y_abs, K):
    """Largest distance of a float32 accumulation of Y from the exact value."""
    return K * 2.0 ** -24 * y_abs + 4 * 2.0 ** -24 * np.abs(y_exact)


def _check_unit(code, s_gpu, s_ref, y_exact, y_abs, K, ref_code):
    eb = _bound(y_exact, y_abs, K)
    assert abs(float(s_gpu) - float(s_ref)) <= eb.max() / 448 + 2.0 ** -22 * abs(float(s_ref))
    v = y_exact / float(s_gpu)
    dec = e4m3fn_decode(code)
    bad = np.abs(dec - v) > _step(v) / 2 + eb / float(s_gpu) + 1e-12
    assert not bad.any(), f"{bad.sum()} codes are not a nearest code of Y / s"
    return int((code != ref_code).sum())


def _abs_product(xc, xs, wq, sw):
    """sum_k |x_k| |w_k| with scales: the summation bound's reference."""
    return (np.abs(e4m3fn_decode(xc)) * xs[:, None].astype(np.float64)) @ \
        (np.abs(e4m3fn_decode(wq)) * sw[:, None].astype(np.float64)).T


def _run(w, rows=None):
    p = generate_proj(w, rows)
    C = w.H * w.d
    x = p.x.reshape(w.B * w.N_pad, C)
    xc, xs = B.quantize_rows_fp8(x.to(DEV))
    out = B.qkv_proj_fp8(xc, xs, p.wq.to(DEV), p.sw.to(DEV), w.B, w.N_pad, w.H, w.d)
    torch.cuda.synchronize()
    return p, xc.cpu().numpy(), xs.cpu().numpy(), out


@pytest.mark.parametrize("name", ["ragged", "aligned"])
def test_projection_matches_oracle(name):
    if name == "ragged":  # N_pad = 448: 128-token blocks straddle the two batch elements
        w = make_workload("wan14b_720p_fp8", B=2, H=3, grid=(3, 10, 13), seed=51)
    else:
        w = make_workload("wan14b_720p_fp8", B=1, H=2, grid=(4, 8, 16), seed=52)
    p, xc, xs, out = _run(w)
    ref = P.qkv_proj_fp8(xc, xs, p.wq.numpy(), p.sw.numpy(), w.B, w.N_pad, w.H, w.d)
    yabs = P.split_heads(_abs_product(xc, xs, p.wq.numpy(), p.sw.numpy()), w.B, w.N_pad, w.H, w.d)
    K = w.H * w.d
    differ = total = 0
    err = num = 0.0
    for t, name_t in enumerate("qkv"):
        codes = _codes(out[t])
        scales = out[3 + t].cpu().numpy()
        rc, rs = ref[name_t]
        y = ref["y"][t]
        for b in range(w.B):
            for h in range(w.H):
                for a in range(w.T):
                    sl = slice(64 * a, 64 * a + 64)
                    differ += _check_unit(codes[b, h, sl], scales[b, h, a], rs[b, h, a], y[b, h, sl],
                                          yabs[t][b, h, sl], K, rc[b, h, sl])
                    total += 64 * w.d
        deq = e4m3fn_decode(codes) * np.repeat(scales, 64, axis=2)[..., None]
        err += float(np.sum((deq - y) ** 2))
        num += float(np.sum(y ** 2))
    print(f"  codes differing from the oracle's: {differ} of {total}; rel L2 of dequantised Y {np.sqrt(err / num):.2e}",
          flush=True)
    assert differ <= total * 1e-3
    assert np.sqrt(err / num) < 3e-2


@pytest.mark.timeout(600)
def test_projection_at_720p_sampled_units():
    w = make_workload("wan14b_720p_fp8")
    p, xc, xs, out = _run(w)
    C = w.H * w.d
    rng = np.random.default_rng(0)
    differ = 0
    for t, h, a in [(0, 0, 0), (1, w.H - 1, w.T - 1), (2, w.H // 2, w.T // 2)] + \
                   [(int(rng.integers(3)), int(rng.integers(w.H)), int(rng.integers(w.T))) for _ in range(3)]:
        rows = slice(64 * a, 64 * a + 64)
        cols = slice((t * w.H + h) * w.d, (t * w.H + h + 1) * w.d)
        y = P.project(xc[rows], xs[rows], p.wq.numpy()[cols], p.sw.numpy()[cols])
        yabs = _abs_product(xc[rows], xs[rows], p.wq.numpy()[cols], p.sw.numpy()[cols])
        rc, rs = P.quantize_e4m3(y.astype(np.float32).reshape(1, -1), axis=1)
        codes = _codes(out[t])[0, h, rows]
        s_gpu = out[3 + t].cpu().numpy()[0, h, a]
        differ += _check_unit(codes, s_gpu, rs[0], y, yabs, C, rc.reshape(64, w.d))
    print(f"  sampled units: codes differing from the oracle's {differ} of {6 * 64 * w.d}", flush=True)
    assert differ <= 6 * 64 * w.d * 1e-3
