"""Plain CPU oracle of the W8A8 FP8 QKV projection that feeds the attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this module; the product path never calls it and
shares no code with it.

The step before the attention path (SparkDiffusion news article, section 07
"from algorithmic subtraction to real GPU acceleration"; the project blog,
"A simple staging principle", item 3): the linear projections are quantised
to W8A8 FP8 E4M3, with the activation scaling and the type conversions fused
into the kernels.  The pages give no formula; the reading used here (and
listed in the design notes) is:

  P1 activations  per token row x: s_x = fp32(max|x| / 448) (1 for an all-zero
                  row); code = E4M3 round-to-nearest-even of fp32(x / s_x)
  P2 weights      the same rule per output channel (row of W, [n_out, C])
  P3 product      Y = diag(s_x) dec(X8) dec(W8)^T diag(s_w), exact in float64
  P4 layout       output column j = (t * H + h) * d + e: tensor t (q, k, v),
                  head h, dim e; token row m = b * N_pad + n
  P5 output       per (tensor, b, h, 64-token tile): s = fp32(max|Y| / 448) and
                  code = E4M3 RNE of fp32(Y / s), taken from Y rounded to fp32
                  (the precision of the kernel's accumulators)

E4M3 encoding uses torch's CPU cast (pinned against a brute-force nearest-code
search in tests/test_proj_oracle.py); decoding uses rola.e4m3fn_decode.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle.rola import e4m3fn_decode

FP8_MAX = 448.0
TILE = 64


def e4m3_encode(y32):
    """E4M3FN codes (uint8) of float32 values, round to nearest even (|y| <= 448)."""
    t = torch.from_numpy(np.ascontiguousarray(y32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_e4m3(x32, axis):
    """P1/P2: absmax scaling along `axis` of a float32 array, then E4M3 codes.
    Returns (codes uint8, scales float32 with `axis` removed)."""
    x = np.asarray(x32, dtype=np.float32)
    amax = np.abs(x).max(axis=axis)
    s = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / np.expand_dims(s, axis)).astype(np.float32)
    return e4m3_encode(y), s


def quantize_rows(x32):
    """P1: per-row quantisation of activations [M, C]."""
    return quantize_e4m3(x32, axis=1)


def project(xq, sx, wq, sw):
    """P3: Y [M, n_out] in float64 from codes and scales."""
    x = e4m3fn_decode(xq) * np.asarray(sx, np.float64)[:, None]
    w = e4m3fn_decode(wq) * np.asarray(sw, np.float64)[:, None]
    return x @ w.T


def split_heads(y, B, n_pad, H, d):
    """P4: [B * N_pad, 3 H d] -> three [B, H, N_pad, d] arrays (q, k, v)."""
    yy = np.asarray(y).reshape(B, n_pad, 3, H, d)
    return tuple(np.ascontiguousarray(yy[:, :, t].transpose(0, 2, 1, 3)) for t in range(3))


def quantize_tiles(y, tile=TILE):
    """P5: per-(b, h, 64-token tile) quantisation of a [B, H, N_pad, d] array,
    decided on its float32 rounding.  Returns (codes uint8, scales [B, H, T])."""
    y32 = np.asarray(y).astype(np.float32)
    B, H, n_pad, d = y32.shape
    t = n_pad // tile
    blocks = y32.reshape(B, H, t, tile * d)
    codes, s = quantize_e4m3(blocks, axis=3)
    return codes.reshape(B, H, n_pad, d), s


def qkv_proj_fp8(xq, sx, wq, sw, B, n_pad, H, d):
    """The whole step: returns {"y": (q, k, v) in float64, "q": (codes, scales),
    "k": ..., "v": ...}."""
    y = split_heads(project(xq, sx, wq, sw), B, n_pad, H, d)
    out = {"y": y}
    for name, yt in zip("qkv", y):
        out[name] = quantize_tiles(yt)
    return out
