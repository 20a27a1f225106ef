"""Seeded synthetic inputs with the shapes of Wan-style video DiT attention.

The pages measure on Wan2.1/Wan2.2 checkpoints (81 frames at 480x832 or
720x1280; SparkDiffusion news article, section 07).  Those weights and prompts
are not available, so the activations are replaced by a synthetic recipe of the
same shape whose structure (smooth in space-time, with noise) makes tile-level
selection meaningful:

    s(p) = sum_m A_m * sin(omega_m . p + phase_m)        (M random 3D sinusoids)
    q_i  = s(p_i) + noise_std * n_i,    k_i = s(p_i) + noise_std * n'_i
    v_i  ~ N(0, I)
    U_q, U_k ~ N(0, 1/d)  [H, d, r];   W_o ~ N(0, 0.02^2)  [H, d, d]

with p_i the (t, h, w) latent-grid coordinate of token i in frame-major raster
order, omega_m = 2*pi*(f_t/G_t, f_h/G_h, f_w/G_w) with f ~ U(0, 2) cycles per axis
extent, phase_m ~ U(0, 2*pi) and A_m ~ N(0, I_d / M).  Rows past the last valid
token are zero.

Every (b, h) slice draws from its own PCG64 stream keyed by (seed, 0, b, h), and
every head's parameters from (seed, 1, h), so any head can be regenerated alone.
Values are drawn in float32 (signals in float64, then rounded) and finally cast
to the storage type with torch's CPU casts: bf16 round-to-nearest-even, or OCP
E4M3FN after per-(b, h, 64-token tile) absmax scaling (scale = absmax / 448,
1 for an all-zero tile).  This module only builds inputs; it holds none of the
attention arithmetic.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

FP8_MAX = 448.0  # largest finite OCP E4M3FN value


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    grid: tuple  # (G_t, G_h, G_w), frame-major raster
    topk: int
    force_diag: bool
    rank: int
    sinusoids: int
    dtype: str  # "f32" | "bf16" | "fp8"
    seed: int
    tile: int = 64
    rope_base: float = 10000.0
    noise_std: float = 0.5
    N_pad_override: Optional[int] = None

    @property
    def N(self) -> int:
        gt, gh, gw = self.grid
        return gt * gh * gw

    @property
    def N_pad(self) -> int:
        if self.N_pad_override is not None:
            return self.N_pad_override
        return ((self.N + self.tile - 1) // self.tile) * self.tile

    @property
    def T(self) -> int:
        return self.N_pad // self.tile

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def kmax(self) -> int:
        return self.topk + (1 if self.force_diag else 0)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: a tiny fp32 case, then Wan-shaped 480P/720P latent grids
# (81 frames -> 21 latent frames; 480x832 -> 30x52; 720x1280 -> 45x80).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=1, H=1, d=64, grid=(4, 16, 16), topk=4,
                         force_diag=True, rank=16, sinusoids=8, dtype="f32", seed=1001),
    "wan13b_480p_bf16": Workload("wan13b_480p_bf16", B=1, H=12, d=128, grid=(21, 30, 52),
                                 topk=52, force_diag=False, rank=32, sinusoids=8,
                                 dtype="bf16", seed=1002),
    "wan14b_480p_bf16": Workload("wan14b_480p_bf16", B=1, H=40, d=128, grid=(21, 30, 52),
                                 topk=16, force_diag=False, rank=32, sinusoids=8,
                                 dtype="bf16", seed=1003),
    "wan14b_720p_bf16": Workload("wan14b_720p_bf16", B=1, H=40, d=128, grid=(21, 45, 80),
                                 topk=36, force_diag=False, rank=64, sinusoids=16,
                                 dtype="bf16", seed=1004),
    "wan14b_720p_fp8": Workload("wan14b_720p_fp8", B=1, H=40, d=128, grid=(21, 45, 80),
                                topk=36, force_diag=False, rank=64, sinusoids=16,
                                dtype="fp8", seed=1004),
}


def make_workload(name: str, **overrides) -> Workload:
    return WORKLOADS[name].with_(**overrides) if overrides else WORKLOADS[name]


def _grid_coords(grid, n):
    gt, gh, gw = grid
    i = np.arange(n, dtype=np.int64)
    return np.stack([i // (gh * gw), (i // gw) % gh, i % gw], axis=1).astype(np.float64)


def generate_head_f32(w: Workload, b: int, h: int):
    """float32 (q, k, v) of one (b, h) slice, shape [N_pad, d], pad rows zero."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(0, b, h))))
    M, d, n = w.sinusoids, w.d, w.N
    f = rng.uniform(0.0, 2.0, size=(M, 3))
    omega = 2.0 * np.pi * f / np.asarray(w.grid, dtype=np.float64)
    phase = rng.uniform(0.0, 2.0 * np.pi, size=M)
    amp = rng.standard_normal((M, d)) / math.sqrt(M)
    pos = _grid_coords(w.grid, n)
    sig = (np.sin(pos @ omega.T + phase) @ amp).astype(np.float32)
    out = []
    for _ in range(2):
        x = np.zeros((w.N_pad, d), dtype=np.float32)
        x[:n] = sig + np.float32(w.noise_std) * rng.standard_normal((n, d), dtype=np.float32)
        out.append(x)
    v = np.zeros((w.N_pad, d), dtype=np.float32)
    v[:n] = rng.standard_normal((n, d), dtype=np.float32)
    out.append(v)
    return tuple(out)


def generate_params_f32(w: Workload, h: int):
    """float32 (U_q [d, r], U_k [d, r], W_o [d, d]) of head h."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(1, h))))
    d, r = w.d, w.rank
    uq = (rng.standard_normal((d, r)) / math.sqrt(d)).astype(np.float32)
    uk = (rng.standard_normal((d, r)) / math.sqrt(d)).astype(np.float32)
    wo = (0.02 * rng.standard_normal((d, d))).astype(np.float32)
    return uq, uk, wo


def quantize_fp8_tiles(x: torch.Tensor, tile: int):
    """Per-64-token-tile absmax E4M3FN quantisation of a float32 [..., N_pad, d]
    tensor.  Returns (codes as torch.float8_e4m3fn, scales float32 [..., T])."""
    lead = x.shape[:-2]
    npad, d = x.shape[-2:]
    t = npad // tile
    xt = x.reshape(*lead, t, tile, d)
    amax = xt.abs().amax(dim=(-2, -1))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
    y = (xt / scale[..., None, None]).clamp(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).reshape(*lead, npad, d)
    return codes, scale


@dataclass
class Inputs:
    """Host-side inputs of one workload, in the storage type the kernels read.

    q, k, v: [B, H, N_pad, d] torch CPU tensors (float32, bfloat16 or
    float8_e4m3fn); q_scale, k_scale, v_scale: float32 [B, H, T] for fp8, else
    None; uq, uk: [H, d, r]; wo: [H, d, d] (float32 for the f32 workload,
    bfloat16 otherwise).
    """
    w: Workload
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    uq: torch.Tensor
    uk: torch.Tensor
    wo: torch.Tensor
    q_scale: Optional[torch.Tensor] = None
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)


def generate(w: Workload, heads: Optional[list] = None) -> Inputs:
    """Generate a workload.  `heads` restricts generation to those head indices
    (the other heads stay zero), for CPU-side sampling of large workloads."""
    store = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[w.dtype]
    pstore = torch.float32 if w.dtype == "f32" else torch.bfloat16
    B, H, npad, d = w.B, w.H, w.N_pad, w.d
    hs = list(range(H)) if heads is None else list(heads)
    q = torch.zeros((B, H, npad, d), dtype=store)
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    scales = None
    if w.dtype == "fp8":
        scales = [torch.ones((B, H, w.T), dtype=torch.float32) for _ in range(3)]
    for b in range(B):
        for h in hs:
            xs = generate_head_f32(w, b, h)
            for i, (dst, x) in enumerate(zip((q, k, v), xs)):
                xt = torch.from_numpy(x)
                if w.dtype == "fp8":
                    codes, sc = quantize_fp8_tiles(xt, w.tile)
                    dst[b, h] = codes
                    scales[i][b, h] = sc
                else:
                    dst[b, h] = xt.to(store)
    uq = torch.zeros((H, d, w.rank), dtype=pstore)
    uk = torch.zeros_like(uq)
    wo = torch.zeros((H, d, d), dtype=pstore)
    for h in range(H):
        a, bb, c = generate_params_f32(w, h)
        uq[h] = torch.from_numpy(a).to(pstore)
        uk[h] = torch.from_numpy(bb).to(pstore)
        wo[h] = torch.from_numpy(c).to(pstore)
    out = Inputs(w, q, k, v, uq, uk, wo)
    if scales is not None:
        out.q_scale, out.k_scale, out.v_scale = scales
    return out


@dataclass
class ProjInputs:
    """Inputs of the QKV projection in front of the attention: x [B, N_pad, C]
    bfloat16 activations (C = H d, pad rows zero), wq [3 H d, C] E4M3FN codes
    of the weights (row j = output column j: tensor, head, dim), sw [3 H d]
    float32 per-output-channel scales."""
    w: Workload
    x: torch.Tensor
    wq: torch.Tensor
    sw: torch.Tensor


def generate_proj(w: Workload, rows: Optional[int] = None) -> ProjInputs:
    """Activations ~ N(0, 1) from PCG64 (seed, 2, b) per batch element and
    weights ~ N(0, 1/C) from PCG64 (seed, 3), the weights quantised per output
    channel (absmax / 448 scale, round to nearest even).  `rows` limits the
    activations drawn per batch element (the rest stay zero), for small cases."""
    C = w.H * w.d
    nout = 3 * C
    x = torch.zeros((w.B, w.N_pad, C), dtype=torch.bfloat16)
    n = w.N if rows is None else min(rows, w.N)
    for b in range(w.B):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(2, b))))
        x[b, :n] = torch.from_numpy(rng.standard_normal((n, C), dtype=np.float32)).to(torch.bfloat16)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(3,))))
    wf = torch.from_numpy(rng.standard_normal((nout, C), dtype=np.float32) / np.float32(math.sqrt(C)))
    amax = wf.abs().amax(dim=1)
    sw = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
    wq = (wf / sw[:, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return ProjInputs(w, x, wq, sw)


def next_step(inp: Inputs, eps: float, seed: int) -> Inputs:
    """Inputs of a following denoising step: q, k, v of `inp` (as the kernels
    read them, dequantised for fp8) plus eps * N(0, 1) noise from PCG64(seed),
    stored again in the workload's type (fp8: quantised again per tile).  The
    parameters are shared.  Pad rows stay zero."""
    w = inp.w
    rng = np.random.Generator(np.random.PCG64(seed))
    out = Inputs(w, None, None, None, inp.uq, inp.uk, inp.wo)
    for name in ("q", "k", "v"):
        t = getattr(inp, name)
        if w.dtype == "fp8":
            sc = getattr(inp, name + "_scale")
            x = t.to(torch.float32).reshape(w.B, w.H, w.T, w.tile, w.d) * sc[..., None, None]
            x = x.reshape(w.B, w.H, w.N_pad, w.d)
        else:
            x = t.to(torch.float32)
        x = x + eps * torch.from_numpy(rng.standard_normal(x.shape).astype(np.float32))
        x[:, :, w.N:] = 0.0
        if w.dtype == "fp8":
            codes, sc = quantize_fp8_tiles(x, w.tile)
            setattr(out, name, codes)
            setattr(out, name + "_scale", sc)
        else:
            setattr(out, name, x.to(t.dtype))
    return out


def to_fp64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a float32/bfloat16 tensor to a float64 numpy array."""
    assert t.dtype in (torch.float32, torch.bfloat16)
    return t.to(torch.float64).numpy()


def fp8_codes(t: torch.Tensor) -> np.ndarray:
    """The raw E4M3FN byte codes of a float8_e4m3fn tensor, as uint8."""
    assert t.dtype == torch.float8_e4m3fn
    return t.view(torch.uint8).numpy()


def upstream_grad(w: Workload, seed: int, pad_value: float = 0.0) -> torch.Tensor:
    """An upstream gradient dL/dO for the backward pass: N(0, 1) from
    PCG64(seed) in float32, stored in the workload's input type (bf16 RNE, or
    float32), shape [B, H, N_pad, d].  Rows past N hold `pad_value` (the
    library ignores them)."""
    assert w.dtype in ("f32", "bf16"), "the backward pass takes float32 or bf16 inputs"
    rng = np.random.Generator(np.random.PCG64(seed))
    x = torch.from_numpy(rng.standard_normal((w.B, w.H, w.N_pad, w.d)).astype(np.float32))
    x[:, :, w.N:] = pad_value
    return x.to(torch.float32 if w.dtype == "f32" else torch.bfloat16)
