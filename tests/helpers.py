"""Shared helpers of the GPU parity tests: running the fp64 oracle on the same
seeded inputs and comparing masks and outputs."""
from __future__ import annotations

import numpy as np
import torch

from oracle import rola as R
from workloads import generate, make_workload
from workloads.gen import fp8_codes, to_fp64

TIE_REL = 1e-6
TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 5e-2}

# Parity cases at sizes the oracle finishes in seconds, spanning several tiles
# and a ragged tail.
CASES = {
    "tiny_f32": make_workload("tiny_f32"),
    "bf16_ragged": make_workload("wan14b_480p_bf16", B=2, H=3, grid=(3, 10, 13), topk=3, rank=32),
    "bf16_r64": make_workload("wan14b_720p_bf16", H=2, grid=(5, 12, 20), topk=5, rank=64, seed=77),
    "bf16_d64_r16": make_workload("wan14b_480p_bf16", H=2, d=64, grid=(4, 9, 15), topk=4, rank=16, seed=5),
    "bf16_aligned_diag": make_workload("wan14b_480p_bf16", H=2, grid=(4, 8, 16), topk=2, force_diag=True,
                                       rank=32, seed=9),
    "f32_d128_r64": make_workload("tiny_f32", H=2, d=128, grid=(3, 7, 11), topk=2, rank=64, seed=11),
    "bf16_dense_all_tiles": make_workload("wan14b_480p_bf16", H=1, grid=(2, 9, 14), topk=4, rank=32, seed=13),
    # fp8 attention takes the kept tiles in pairs: odd and even kept counts
    "fp8_ragged": make_workload("wan14b_720p_fp8", B=2, H=3, grid=(3, 10, 13), topk=3, rank=32, seed=21),
    "fp8_r64_diag": make_workload("wan14b_720p_fp8", H=2, grid=(5, 12, 20), topk=4, force_diag=True,
                                  rank=64, seed=23),
    # rows of more than 64 (and 128) kept tiles: the kernels hold a row's tile
    # indices 64 at a time and reload them mid-row
    "bf16_long_rows": make_workload("wan14b_480p_bf16", H=1, grid=(3, 40, 70), topk=130, rank=32, seed=31),
    "fp8_long_rows": make_workload("wan14b_720p_fp8", H=1, grid=(3, 40, 70), topk=129, rank=32, seed=33),
    # 16 heads of 36 tiles: the streaming pass gives each block two tiles
    # (chunks of several tiles, some chunk counts not dividing T)
    "bf16_many_heads": make_workload("wan14b_480p_bf16", B=2, H=8, grid=(2, 6, 190), topk=3, force_diag=True,
                                     rank=32, seed=41),
    "fp8_many_heads": make_workload("wan14b_720p_fp8", B=2, H=8, grid=(2, 6, 190), topk=4, rank=64, seed=43),
}


def head_arrays(inp, b, h):
    """fp64 (q, k, v) of one head exactly as the kernels read them."""
    w = inp.w
    if w.dtype == "fp8":
        q = R.dequantize_tiles(fp8_codes(inp.q[b, h]), inp.q_scale[b, h].numpy())
        k = R.dequantize_tiles(fp8_codes(inp.k[b, h]), inp.k_scale[b, h].numpy())
        v = R.dequantize_tiles(fp8_codes(inp.v[b, h]), inp.v_scale[b, h].numpy())
        return q, k, v
    return to_fp64(inp.q[b, h]), to_fp64(inp.k[b, h]), to_fp64(inp.v[b, h])


def params(inp, h):
    return to_fp64(inp.uq[h]), to_fp64(inp.uk[h]), to_fp64(inp.wo[h])


def oracle_head(inp, b, h, kept_rows=None):
    w = inp.w
    q, k, v = head_arrays(inp, b, h)
    uq, uk, wo = params(inp, h)
    return R.hybrid_head(q, k, v, w.N, w.grid, uq, uk, wo, w.topk, w.force_diag, w.softmax_scale,
                         w.rope_base, kept_rows=kept_rows)


def oracle_mask_head(inp, b, h):
    """(scores, kept rows) of one head."""
    w = inp.w
    q, k, _ = head_arrays(inp, b, h)
    sc = R.pooled_scores(R.tile_means(q, w.N), R.tile_means(k, w.N))
    return sc, R.select(sc, w.topk, w.force_diag)


def csr_tensors(rows_per_head, device):
    rows = [r for head in rows_per_head for r in head]
    rp, ci = R.to_csr(rows)
    return (torch.from_numpy(rp.astype(np.int32)).to(device), torch.from_numpy(ci.astype(np.int32)).to(device))


def mask_mismatches(gpu_rows, oracle_rows, scores, topk, force_diag):
    """Rows whose GPU kept set differs from the oracle's beyond the tie window.
    Returns (n_rows_outside_window, n_rows_differing_inside_window)."""
    bad = tied = 0
    for a, (g, o) in enumerate(zip(gpu_rows, oracle_rows)):
        G, O = set(int(x) for x in g), set(int(x) for x in o)
        if G == O and list(g) == sorted(G):
            continue
        if len(g) != len(o) or list(g) != sorted(G):
            bad += 1
            continue
        s = scores[a]
        kth = np.sort(s)[::-1][topk - 1]
        ok = True
        for b in G ^ O:
            if force_diag and b == a:
                ok = False
            if abs(s[b] - kth) > TIE_REL * max(abs(s[b]), abs(kth)):
                ok = False
        if ok:
            tied += 1
        else:
            bad += 1
    return bad, tied


def split_csr(row_ptr, col_idx, n_heads, T):
    rp = row_ptr.cpu().numpy()
    ci = col_idx.cpu().numpy()
    out = []
    for hh in range(n_heads):
        out.append([ci[rp[hh * T + a]:rp[hh * T + a + 1]] for a in range(T)])
    return out


class RelL2:
    """Accumulates ||gpu - ref||^2 and ||ref||^2 over valid rows (fp64), and,
    as a diagnostic beside that pooled figure, the relative L2 error of every
    64-row tile added, so that a defect confined to one tile shows."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0
        self.n_added = 0
        self.worst = (0.0, None)  # (tile relative error, (call index, tile))

    def add(self, gpu, ref):
        gpu = np.asarray(gpu, np.float64)
        ref = np.asarray(ref, np.float64)
        d2 = (gpu - ref) ** 2
        r2 = ref ** 2
        self.num += float(np.sum(d2))
        self.den += float(np.sum(r2))
        n = gpu.shape[0]
        for t0 in range(0, n, 64):
            rn = float(np.sum(r2[t0:t0 + 64]))
            if rn > 0:
                e = (float(np.sum(d2[t0:t0 + 64])) / rn) ** 0.5
                if e > self.worst[0]:
                    self.worst = (e, (self.n_added, t0 // 64))
        self.n_added += 1

    @property
    def value(self):
        return (self.num / self.den) ** 0.5 if self.den > 0 else 0.0

    def __str__(self):
        e, where = self.worst
        return f"{self.value:.3e} (worst tile {e:.3e} at {where})"


def to_device(inp, dev):
    out = {k: getattr(inp, k).to(dev) for k in ("q", "k", "v", "uq", "uk", "wo")}
    for k in ("q_scale", "k_scale", "v_scale"):
        t = getattr(inp, k)
        out[k] = None if t is None else t.to(dev)
    return out


def gen(name_or_w):
    w = CASES[name_or_w] if isinstance(name_or_w, str) else name_or_w
    return generate(w)
