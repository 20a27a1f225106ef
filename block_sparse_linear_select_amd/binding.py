"""ctypes binding of libhsa_attn.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels; PyTorch only
provides device memory and the current stream.  If the library is missing the
calls raise: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhsa_attn.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
CALL_BLOCK_SELECT, CALL_SPARSE, CALL_LINEAR, CALL_HYBRID, CALL_LINEAR_COMPLEMENT, CALL_BACKWARD = 0, 1, 2, 3, 4, 5
ERRORS = {-1: "NULL", -2: "SHAPE", -3: "DTYPE", -4: "WORKSPACE", -5: "CSR", -6: "HIP"}

EXPORTED = ["hsa_attn_workspace_size", "hsa_attn_last_error", "hsa_attn_version",
            "hsa_attn_timing_enable", "hsa_attn_timing_read", "hsa_attn_read_calibrate",
            "hsa_block_select", "hsa_sparse_attn", "hsa_linear_attn", "hsa_linear_attn_complement",
            "hsa_hybrid_attn", "hsa_hybrid_attn_noalloc", "hsa_hybrid_attn_train", "hsa_hybrid_attn_backward",
            "hsa_hybrid_attn_backward_saved",
            "hsa_quantize_rows_fp8", "hsa_qkv_proj_fp8"]
KERNEL_KINDS = ["rope", "stream", "finalize", "select", "unused4", "attend", "quant", "proj", "compl", "bwd_linear",
                "bwd_sparse"]
LINEAR_KEYS = {"all": 0, "complement": 1}


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("N_pad", ctypes.c_int32), ("d", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("grid_t", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("force_diag", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("linear_keys", ctypes.c_int32)]


class HsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"hsa_attn error {code} ({ERRORS.get(code, '?')}): {msg}")
        self.code = code


_lib = None


def lib():
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32p, f32p, f64p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        dp = ctypes.POINTER(Desc)
        L.hsa_attn_workspace_size.argtypes = [dp, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        L.hsa_attn_last_error.restype = ctypes.c_char_p
        L.hsa_attn_version.restype = ctypes.c_char_p
        L.hsa_block_select.argtypes = [dp, vp, vp, f32p, f32p, i32p, i32p, f64p, f64p, vp, sz, vp]
        L.hsa_sparse_attn.argtypes = [dp, vp, vp, vp, f32p, f32p, f32p, i32p, i32p, vp, f32p, vp, sz, vp]
        L.hsa_linear_attn.argtypes = [dp, vp, vp, vp, f32p, f32p, f32p, vp, vp, vp, vp, vp, sz, vp]
        L.hsa_linear_attn_complement.argtypes = [dp, vp, vp, vp, f32p, f32p, f32p, vp, vp, vp, i32p, i32p, vp, vp,
                                                 sz, vp]
        L.hsa_hybrid_attn_backward.argtypes = [dp, vp, vp, vp, vp, vp, vp, i32p, i32p, vp, f32p, f32p, f32p, vp,
                                               sz, vp]
        L.hsa_hybrid_attn.argtypes = [dp, vp, vp, vp, f32p, f32p, f32p, vp, vp, vp, i32p, i32p, i32p, i32p,
                                      vp, vp, sz, vp]
        L.hsa_hybrid_attn_train.argtypes = [dp, vp, vp, vp, vp, vp, vp, i32p, i32p, i32p, i32p, vp, vp, f32p,
                                            vp, sz, vp]
        L.hsa_hybrid_attn_backward_saved.argtypes = [dp, vp, vp, vp, vp, vp, vp, i32p, i32p, vp, f32p, vp, f32p,
                                                     f32p, f32p, vp, sz, vp]
        L.hsa_hybrid_attn_noalloc.argtypes = [dp, vp, vp, vp, f32p, f32p, f32p, vp, vp, vp, i32p, i32p, i32p, i32p,
                                              vp, vp]
        L.hsa_quantize_rows_fp8.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, f32p, vp]
        i32 = ctypes.c_int32
        L.hsa_qkv_proj_fp8.argtypes = [vp, f32p, vp, f32p, i32, i32, i32, i32, i32, vp, vp, vp, f32p, f32p, f32p, vp]
        L.hsa_attn_timing_enable.argtypes = [ctypes.c_int]
        L.hsa_attn_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
        L.hsa_attn_read_calibrate.argtypes = [vp, sz, vp, sz, vp]
        for name in EXPORTED:
            if name not in ("hsa_attn_last_error", "hsa_attn_version"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise HsaError(rc, lib().hsa_attn_last_error().decode())


@dataclass(frozen=True)
class Config:
    """Sizes of one call, mirroring the C descriptor."""
    B: int
    H: int
    N: int
    N_pad: int
    d: int
    grid: tuple
    topk: int
    force_diag: bool
    rank: int
    softmax_scale: float
    rope_base: float
    dtype: str  # "f32" | "bf16" | "fp8"
    linear_keys: str = "all"  # "all" | "complement" (keys outside each row's kept tiles)

    @property
    def T(self) -> int:
        return self.N_pad // 64

    @property
    def kmax(self) -> int:
        return self.topk + int(self.force_diag)

    def desc(self) -> Desc:
        ind = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}[self.dtype]
        outd = F32 if self.dtype == "f32" else BF16
        gt, gh, gw = self.grid
        return Desc(self.B, self.H, self.N, self.N_pad, self.d, 64, gt, gh, gw, self.topk,
                    int(self.force_diag), self.rank, self.softmax_scale, self.rope_base, ind, outd,
                    LINEAR_KEYS[self.linear_keys])

    @staticmethod
    def from_workload(w) -> "Config":
        return Config(w.B, w.H, w.N, w.N_pad, w.d, tuple(w.grid), w.topk, bool(w.force_diag), w.rank,
                      w.softmax_scale, w.rope_base, w.dtype)


_TORCH_IN = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def _out_dtype(cfg: Config):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, shape, dtype):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_inputs(cfg: Config, q, k, v=None, scales=()):
    shp = (cfg.B, cfg.H, cfg.N_pad, cfg.d)
    dt = _TORCH_IN[cfg.dtype]
    _need(q, "q", shp, dt)
    _need(k, "k", shp, dt)
    if v is not None:
        _need(v, "v", shp, dt)
    for name, s in scales:
        if cfg.dtype == "fp8":
            _need(s, name, (cfg.B, cfg.H, cfg.T), torch.float32)
        elif s is not None:
            raise ValueError(f"{name} is only for fp8 inputs")


def _check_params(cfg: Config, uq, uk, wo):
    pdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    _need(uq, "uq", (cfg.H, cfg.d, cfg.rank), pdt)
    _need(uk, "uk", (cfg.H, cfg.d, cfg.rank), pdt)
    _need(wo, "wo", (cfg.H, cfg.d, cfg.d), pdt)


def workspace_size(cfg: Config, call: int) -> int:
    n = ctypes.c_size_t(0)
    d = cfg.desc()
    _check(lib().hsa_attn_workspace_size(ctypes.byref(d), call, ctypes.byref(n)))
    return n.value


def _workspace(cfg: Config, call: int, device) -> torch.Tensor:
    n = workspace_size(cfg, call)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def block_select(cfg: Config, q, k, q_scale=None, k_scale=None, want_means=False):
    """Returns (row_ptr, col_idx) int32 device tensors [and float64 tile means]."""
    _check_inputs(cfg, q, k, scales=(("q_scale", q_scale), ("k_scale", k_scale)))
    rows = cfg.B * cfg.H * cfg.T
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=q.device)
    col_idx = torch.empty(rows * cfg.kmax, dtype=torch.int32, device=q.device)
    qbar = kbar = None
    if want_means:
        qbar = torch.empty((cfg.B, cfg.H, cfg.T, cfg.d), dtype=torch.float64, device=q.device)
        kbar = torch.empty_like(qbar)
    ws = _workspace(cfg, CALL_BLOCK_SELECT, q.device)
    d = cfg.desc()
    _check(lib().hsa_block_select(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(q_scale), _ptr(k_scale),
                                  _ptr(row_ptr), _ptr(col_idx), _ptr(qbar), _ptr(kbar),
                                  _ptr(ws), ws.numel(), _stream()))
    return (row_ptr, col_idx, qbar, kbar) if want_means else (row_ptr, col_idx)


def sparse_attn(cfg: Config, q, k, v, row_ptr, col_idx, q_scale=None, k_scale=None, v_scale=None,
                want_lse=False):
    _check_inputs(cfg, q, k, v, (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)))
    rows = cfg.B * cfg.H * cfg.T
    _need(row_ptr, "row_ptr", (rows + 1,), torch.int32)
    if col_idx.dtype != torch.int32 or not col_idx.is_cuda or col_idx.dim() != 1:
        raise ValueError("col_idx must be a 1-D int32 device tensor")
    o = torch.empty((cfg.B, cfg.H, cfg.N_pad, cfg.d), dtype=_out_dtype(cfg), device=q.device)
    lse = torch.empty((cfg.B, cfg.H, cfg.N_pad), dtype=torch.float32, device=q.device) if want_lse else None
    ws = _workspace(cfg, CALL_SPARSE, q.device)
    d = cfg.desc()
    _check(lib().hsa_sparse_attn(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale),
                                 _ptr(v_scale), _ptr(row_ptr), _ptr(col_idx), _ptr(o), _ptr(lse),
                                 _ptr(ws), ws.numel(), _stream()))
    return (o, lse) if want_lse else o


def linear_attn(cfg: Config, q, k, v, uq, uk, wo, q_scale=None, k_scale=None, v_scale=None):
    _check_inputs(cfg, q, k, v, (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)))
    _check_params(cfg, uq, uk, wo)
    o = torch.empty((cfg.B, cfg.H, cfg.N_pad, cfg.d), dtype=_out_dtype(cfg), device=q.device)
    ws = _workspace(cfg, CALL_LINEAR, q.device)
    d = cfg.desc()
    _check(lib().hsa_linear_attn(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale),
                                 _ptr(v_scale), _ptr(uq), _ptr(uk), _ptr(wo), _ptr(o),
                                 _ptr(ws), ws.numel(), _stream()))
    return o


def linear_attn_complement(cfg: Config, q, k, v, uq, uk, wo, row_ptr, col_idx, q_scale=None, k_scale=None,
                           v_scale=None):
    """O_l W_o with the linear sums of tile a's queries over the valid keys
    outside the tiles of CSR row a."""
    _check_inputs(cfg, q, k, v, (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)))
    _check_params(cfg, uq, uk, wo)
    _need(row_ptr, "row_ptr", (cfg.B * cfg.H * cfg.T + 1,), torch.int32)
    if col_idx.dtype != torch.int32 or not col_idx.is_cuda or col_idx.dim() != 1:
        raise ValueError("col_idx must be a 1-D int32 device tensor")
    o = torch.empty((cfg.B, cfg.H, cfg.N_pad, cfg.d), dtype=_out_dtype(cfg), device=q.device)
    ws = _workspace(cfg, CALL_LINEAR_COMPLEMENT, q.device)
    d = cfg.desc()
    _check(lib().hsa_linear_attn_complement(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale),
                                            _ptr(k_scale), _ptr(v_scale), _ptr(uq), _ptr(uk), _ptr(wo),
                                            _ptr(row_ptr), _ptr(col_idx), _ptr(o), _ptr(ws), ws.numel(),
                                            _stream()))
    return o


class HybridPlan:
    """Pre-allocated output, CSR and workspace for repeated hybrid calls."""

    def __init__(self, cfg: Config, device, export_mask=False):
        self.cfg = cfg
        rows = cfg.B * cfg.H * cfg.T
        self.o = torch.empty((cfg.B, cfg.H, cfg.N_pad, cfg.d), dtype=_out_dtype(cfg), device=device)
        self.row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=device) if export_mask else None
        self.col_idx = torch.empty(rows * cfg.kmax, dtype=torch.int32, device=device) if export_mask else None
        self.ws = _workspace(cfg, CALL_HYBRID, device)
        self.desc = cfg.desc()

    def run(self, q, k, v, uq, uk, wo, q_scale=None, k_scale=None, v_scale=None, row_ptr=None, col_idx=None,
            check=True):
        cfg = self.cfg
        if check:
            _check_inputs(cfg, q, k, v, (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)))
            _check_params(cfg, uq, uk, wo)
        rp_out = None if row_ptr is not None else self.row_ptr
        ci_out = None if row_ptr is not None else self.col_idx
        _check(lib().hsa_hybrid_attn(ctypes.byref(self.desc), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale),
                                     _ptr(k_scale), _ptr(v_scale), _ptr(uq), _ptr(uk), _ptr(wo),
                                     _ptr(row_ptr), _ptr(col_idx), _ptr(rp_out), _ptr(ci_out),
                                     _ptr(self.o), _ptr(self.ws), self.ws.numel(), _stream()))
        return self.o


def hybrid_attn(cfg: Config, q, k, v, uq, uk, wo, q_scale=None, k_scale=None, v_scale=None,
                row_ptr=None, col_idx=None, export_mask=False):
    """O = O_s + O_l W_o.  With export_mask, returns (o, row_ptr, col_idx)."""
    plan = HybridPlan(cfg, q.device, export_mask=export_mask and row_ptr is None)
    o = plan.run(q, k, v, uq, uk, wo, q_scale, k_scale, v_scale, row_ptr, col_idx)
    if export_mask and row_ptr is None:
        return o, plan.row_ptr, plan.col_idx
    return o


def hybrid_attn_noalloc(cfg: Config, q, k, v, uq, uk, wo, q_scale=None, k_scale=None, v_scale=None,
                        row_ptr=None, col_idx=None, export_mask=False):
    """hybrid_attn through the entry point that allocates nothing: its
    scratch is the library's static device array (calls that overlap on one
    GPU race on it).  With export_mask, returns (o, row_ptr, col_idx)."""
    _check_inputs(cfg, q, k, v, (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)))
    _check_params(cfg, uq, uk, wo)
    rows = cfg.B * cfg.H * cfg.T
    o = torch.empty((cfg.B, cfg.H, cfg.N_pad, cfg.d), dtype=_out_dtype(cfg), device=q.device)
    rp_out = ci_out = None
    if export_mask and row_ptr is None:
        rp_out = torch.empty(rows + 1, dtype=torch.int32, device=q.device)
        ci_out = torch.empty(rows * cfg.kmax, dtype=torch.int32, device=q.device)
    d = cfg.desc()
    _check(lib().hsa_hybrid_attn_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale),
                                         _ptr(v_scale), _ptr(uq), _ptr(uk), _ptr(wo), _ptr(row_ptr), _ptr(col_idx),
                                         _ptr(rp_out), _ptr(ci_out), _ptr(o), _stream()))
    return (o, rp_out, ci_out) if rp_out is not None else o


def hybrid_attn_backward(cfg: Config, q, k, v, uq, uk, wo, row_ptr, col_idx, d_o):
    """(dQ, dK, dV) float32 for dL/dO = d_o, on the forward's mask (held fixed)."""
    _check_inputs(cfg, q, k, v)
    _check_params(cfg, uq, uk, wo)
    _need(d_o, "d_o", (cfg.B, cfg.H, cfg.N_pad, cfg.d), _TORCH_IN[cfg.dtype])
    _need(row_ptr, "row_ptr", (cfg.B * cfg.H * cfg.T + 1,), torch.int32)
    if col_idx.dtype != torch.int32 or not col_idx.is_cuda or col_idx.dim() != 1:
        raise ValueError("col_idx must be a 1-D int32 device tensor")
    shape = (cfg.B, cfg.H, cfg.N_pad, cfg.d)
    dq, dk, dv = (torch.empty(shape, dtype=torch.float32, device=q.device) for _ in range(3))
    ws = _workspace(cfg, CALL_BACKWARD, q.device)
    d = cfg.desc()
    _check(lib().hsa_hybrid_attn_backward(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(uq), _ptr(uk), _ptr(wo),
                                          _ptr(row_ptr), _ptr(col_idx), _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv),
                                          _ptr(ws), ws.numel(), _stream()))
    return dq, dk, dv



def hybrid_attn_train(cfg: Config, q, k, v, uq, uk, wo, row_ptr=None, col_idx=None, export_mask=False):
    """hybrid_attn that also returns what the backward needs from it: (o, o_s,
    lse) with o_s the sparse branch's output alone and lse its log-sum-exp
    [B, H, N_pad] float32; with export_mask, (o, o_s, lse, row_ptr, col_idx)."""
    _check_inputs(cfg, q, k, v)
    _check_params(cfg, uq, uk, wo)
    rows = cfg.B * cfg.H * cfg.T
    shape = (cfg.B, cfg.H, cfg.N_pad, cfg.d)
    o = torch.empty(shape, dtype=_out_dtype(cfg), device=q.device)
    o_s = torch.empty(shape, dtype=_out_dtype(cfg), device=q.device)
    lse = torch.empty((cfg.B, cfg.H, cfg.N_pad), dtype=torch.float32, device=q.device)
    rp_out = ci_out = None
    if export_mask and row_ptr is None:
        rp_out = torch.empty(rows + 1, dtype=torch.int32, device=q.device)
        ci_out = torch.empty(rows * cfg.kmax, dtype=torch.int32, device=q.device)
    ws = _workspace(cfg, CALL_HYBRID, q.device)
    d = cfg.desc()
    _check(lib().hsa_hybrid_attn_train(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(uq), _ptr(uk), _ptr(wo),
                                       _ptr(row_ptr), _ptr(col_idx), _ptr(rp_out), _ptr(ci_out), _ptr(o), _ptr(o_s),
                                       _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return (o, o_s, lse, rp_out, ci_out) if rp_out is not None else (o, o_s, lse)


def hybrid_attn_backward_saved(cfg: Config, q, k, v, uq, uk, wo, row_ptr, col_idx, o_s, lse, d_o):
    """hybrid_attn_backward with the sparse branch's output and log-sum-exp
    from hybrid_attn_train instead of recomputed."""
    _check_inputs(cfg, q, k, v)
    _check_params(cfg, uq, uk, wo)
    _need(d_o, "d_o", (cfg.B, cfg.H, cfg.N_pad, cfg.d), _TORCH_IN[cfg.dtype])
    _need(o_s, "o_s", (cfg.B, cfg.H, cfg.N_pad, cfg.d), _out_dtype(cfg))
    _need(lse, "lse", (cfg.B, cfg.H, cfg.N_pad), torch.float32)
    _need(row_ptr, "row_ptr", (cfg.B * cfg.H * cfg.T + 1,), torch.int32)
    if col_idx.dtype != torch.int32 or not col_idx.is_cuda or col_idx.dim() != 1:
        raise ValueError("col_idx must be a 1-D int32 device tensor")
    shape = (cfg.B, cfg.H, cfg.N_pad, cfg.d)
    dq, dk, dv = (torch.empty(shape, dtype=torch.float32, device=q.device) for _ in range(3))
    ws = _workspace(cfg, CALL_BACKWARD, q.device)
    d = cfg.desc()
    _check(lib().hsa_hybrid_attn_backward_saved(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(uq), _ptr(uk),
                                                _ptr(wo), _ptr(row_ptr), _ptr(col_idx), _ptr(o_s), _ptr(lse),
                                                _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
                                                _stream()))
    return dq, dk, dv

def timing_enable(max_launches: int):
    """Bracket every kernel launch with HIP events on its stream (0 disables)."""
    _check(lib().hsa_attn_timing_enable(max_launches))


def timing_read() -> dict:
    """{kind: (total_ms, launches)} for the launches recorded since enabling."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(lib().hsa_attn_timing_read(ms, cnt))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_KINDS)}


READ_SINK_WORDS = 2048 * 256


def read_calibrate(buf: torch.Tensor, sink: torch.Tensor):
    """One plain streaming read of the bytes of `buf` (a multiple of 16) into
    one word per thread of `sink` (int32, at least READ_SINK_WORDS): the read
    rate of a simple kernel on this GPU, not part of the attention."""
    if not buf.is_cuda or not sink.is_cuda or sink.dtype != torch.int32:
        raise ValueError("buf must be a device tensor and sink a device int32 tensor")
    _check(lib().hsa_attn_read_calibrate(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), sink.numel(),
                                         _stream()))


def version() -> str:
    return lib().hsa_attn_version().decode()


# ------------------------------------------------------------ W8A8 projections
def quantize_rows_fp8(x: torch.Tensor):
    """Per-row E4M3 codes of a bfloat16 [M, C] device tensor: (codes uint8 [M, C], scales float32 [M])."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bfloat16 device tensor")
    M, C = x.shape
    codes = torch.empty((M, C), dtype=torch.uint8, device=x.device)
    scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().hsa_quantize_rows_fp8(_ptr(x), M, C, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def qkv_proj_fp8(x_codes, x_scales, w_codes, w_scales, B: int, N_pad: int, H: int, d: int = 128):
    """FP8 Q, K, V [B, H, N_pad, d] (as float8_e4m3fn views) and their per-tile
    scales [B, H, N_pad // 64] from quantised activations [B*N_pad, C] and
    weights [3*H*d, C]."""
    M, C = x_codes.shape
    if M != B * N_pad or tuple(w_codes.shape) != (3 * H * d, C):
        raise ValueError("shapes: x_codes [B*N_pad, C], w_codes [3*H*d, C]")
    for t, dt in ((x_codes, torch.uint8), (w_codes, torch.uint8), (x_scales, torch.float32), (w_scales, torch.float32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError("x_codes / w_codes must be uint8 and the scales float32, contiguous device tensors")
    dev = x_codes.device
    outs = [torch.empty((B, H, N_pad, d), dtype=torch.uint8, device=dev) for _ in range(3)]
    scs = [torch.empty((B, H, N_pad // 64), dtype=torch.float32, device=dev) for _ in range(3)]
    _check(lib().hsa_qkv_proj_fp8(_ptr(x_codes), _ptr(x_scales), _ptr(w_codes), _ptr(w_scales), B, N_pad, C, H, d,
                                  *[_ptr(o) for o in outs], *[_ptr(c) for c in scs], _stream()))
    return tuple(o.view(torch.float8_e4m3fn) for o in outs) + tuple(scs)
