"""The C ABI library: it loads, exports what include/hsa_attn.h declares, and
rejects bad arguments before any launch (these calls touch no GPU)."""
import ctypes
import os
import re

import pytest

from block_sparse_linear_select_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsa_attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hsa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = _declared()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(L, n), n
    assert B.version().startswith("hsa_attn")


def _cfg(**kw):
    base = dict(B=1, H=2, N=390, N_pad=448, d=128, grid=(3, 10, 13), topk=3, force_diag=False, rank=32,
                softmax_scale=128 ** -0.5, rope_base=10000.0, dtype="bf16")
    base.update(kw)
    return B.Config(**base)


def _ws(cfg, call):
    n = ctypes.c_size_t(0)
    d = cfg.desc()
    rc = B.lib().hsa_attn_workspace_size(ctypes.byref(d), call, ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("bad,code", [
    (dict(d=96), -2), (dict(N_pad=512), -2), (dict(N_pad=440), -2), (dict(grid=(3, 10, 12)), -2),
    (dict(topk=0), -2), (dict(topk=8), -2), (dict(rank=24), -2), (dict(B=0), -2),
])
def test_bad_descriptors_are_rejected(bad, code):
    rc, _ = _ws(_cfg(**bad), B.CALL_HYBRID)
    assert rc == code
    assert B.lib().hsa_attn_last_error()


def test_bad_dtype_pair_is_rejected():
    d = _cfg().desc()
    d.out_dtype = B.F32
    n = ctypes.c_size_t(0)
    assert B.lib().hsa_attn_workspace_size(ctypes.byref(d), B.CALL_HYBRID, ctypes.byref(n)) == -3


def test_workspace_grows_with_the_problem():
    sizes = []
    for grid, npad in (((3, 10, 13), 448), ((6, 10, 13), 832), ((12, 10, 13), 1600)):
        cfg = _cfg(grid=grid, N=grid[0] * grid[1] * grid[2], N_pad=npad)
        rc, n = _ws(cfg, B.CALL_HYBRID)
        assert rc == 0
        sizes.append(n)
        rc2, n2 = _ws(cfg, B.CALL_SPARSE)
        assert rc2 == 0 and n2 == 0  # bf16 sparse attention needs no scratch
        assert _ws(_cfg(dtype="f32", grid=grid, N=cfg.N, N_pad=npad), B.CALL_SPARSE) == (0, 0)
        assert _ws(cfg, B.CALL_LINEAR)[1] < n
    assert sizes == sorted(sizes) and len(set(sizes)) == 3


def test_null_and_workspace_errors_enqueue_nothing():
    L = B.lib()
    cfg = _cfg()
    d = cfg.desc()
    vp = ctypes.c_void_p
    # missing tensors
    assert L.hsa_hybrid_attn(ctypes.byref(d), None, None, None, None, None, None, None, None, None,
                             None, None, None, None, None, None, 0, None) == -1
    fake = vp(1 << 20)  # never dereferenced: validation fails first
    # workspace too small
    rc = L.hsa_hybrid_attn(ctypes.byref(d), fake, fake, fake, None, None, None, fake, fake, fake,
                           None, None, None, None, fake, fake, 16, None)
    assert rc == -4
    # misaligned workspace
    need = _ws(cfg, B.CALL_HYBRID)[1]
    rc = L.hsa_hybrid_attn(ctypes.byref(d), fake, fake, fake, None, None, None, fake, fake, fake,
                           None, None, None, None, fake, vp((1 << 20) + 8), need, None)
    assert rc == -4
    # half a CSR
    rc = L.hsa_hybrid_attn(ctypes.byref(d), fake, fake, fake, None, None, None, fake, fake, fake,
                           fake, None, None, None, fake, fake, need, None)
    assert rc == -5
    # scales with bf16 inputs
    rc = L.hsa_sparse_attn(ctypes.byref(d), fake, fake, fake, fake, None, None, fake, fake, fake, None,
                           None, 0, None)
    assert rc == -3
    # fp8 without scales
    d8 = _cfg(dtype="fp8").desc()
    rc = L.hsa_block_select(ctypes.byref(d8), fake, fake, None, None, fake, fake, None, None, fake, need, None)
    assert rc == -3
    assert b"scale" in L.hsa_attn_last_error()
    # fp8 attention needs d = 128 (selection does not)
    d8 = _cfg(dtype="fp8", d=64).desc()
    rc = L.hsa_sparse_attn(ctypes.byref(d8), fake, fake, fake, fake, fake, fake, fake, fake, fake, None,
                           fake, need, None)
    assert rc == -2 and b"128" in L.hsa_attn_last_error()


def test_complement_variant_arguments():
    L = B.lib()
    cfg = _cfg(linear_keys="complement")
    d = cfg.desc()
    # the descriptor field takes 0 or 1 only
    bad = _cfg().desc()
    bad.linear_keys = 2
    n = ctypes.c_size_t(0)
    assert L.hsa_attn_workspace_size(ctypes.byref(bad), B.CALL_HYBRID, ctypes.byref(n)) == -2
    # the hybrid workspace grows by the per-tile states (B*H*T*r*d bf16 values) and more
    rc_all, n_all = _ws(_cfg(), B.CALL_HYBRID)
    rc_c, n_c = _ws(cfg, B.CALL_HYBRID)
    assert rc_all == rc_c == 0 and n_c >= n_all + cfg.B * cfg.H * cfg.T * cfg.rank * cfg.d * 2
    # the linear call cannot take the complement (it has no mask); the masked call can, whatever the field
    assert _ws(cfg, B.CALL_LINEAR)[0] == -2 and b"complement" in L.hsa_attn_last_error()
    rc_l, n_l = _ws(cfg, B.CALL_LINEAR_COMPLEMENT)
    assert rc_l == 0 and _ws(_cfg(), B.CALL_LINEAR_COMPLEMENT) == (0, n_l) and n_l > _ws(_cfg(), B.CALL_LINEAR)[1]
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    rc = L.hsa_linear_attn(ctypes.byref(d), fake, fake, fake, None, None, None, fake, fake, fake, fake,
                           fake, 1 << 40, None)
    assert rc == -2
    # the masked call needs its CSR
    rc = L.hsa_linear_attn_complement(ctypes.byref(d), fake, fake, fake, None, None, None, fake, fake, fake,
                                      None, None, fake, fake, 1 << 40, None)
    assert rc == -5
    # at most 4096 tiles per (b, h) (selection inside the hybrid call stops at 2048)
    big = _cfg(linear_keys="complement", grid=(65, 64, 64), N=65 * 64 * 64, N_pad=65 * 64 * 64)
    assert _ws(big, B.CALL_LINEAR_COMPLEMENT)[0] == -2 and b"4096" in L.hsa_attn_last_error()
    assert _ws(_cfg(grid=(65, 64, 64), N=65 * 64 * 64, N_pad=65 * 64 * 64, topk=3), B.CALL_LINEAR)[0] == 0


def test_slices_beyond_32_bit_offsets_are_rejected():
    """One (b, h) slice is addressed with 32-bit byte offsets: N_pad * d * 4
    must stay below 2^31 for every call, also those that select nothing."""
    n = (1 << 22)  # 4,194,304 tokens: 2^22 * 128 * 4 = 2^31 bytes
    grid = (1024, 64, 64)
    for call in (B.CALL_SPARSE, B.CALL_LINEAR, B.CALL_BACKWARD):
        rc, _ = _ws(_cfg(grid=grid, N=n, N_pad=n, topk=3), call)
        assert rc == -2 and b"2^31" in B.lib().hsa_attn_last_error(), call
    rc, _ = _ws(_cfg(grid=(1023, 64, 64), N=1023 * 64 * 64, N_pad=1023 * 64 * 64, topk=3), B.CALL_LINEAR)
    assert rc == 0


def test_noalloc_rejects_a_call_beyond_its_static_scratch_before_any_launch():
    """The allocation-free hybrid call checks its workspace need against the
    static scratch before it touches the GPU: 720P FP8 (~0.5 GB with the
    transposed V tiles) is rejected, with nothing enqueued."""
    from workloads import make_workload
    cfg = B.Config.from_workload(make_workload("wan14b_720p_fp8"))
    d = cfg.desc()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced
    rc = B.lib().hsa_hybrid_attn_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                         None, None, None, None, fake, None)
    assert rc == -4 and b"static scratch" in B.lib().hsa_attn_last_error()
    n = ctypes.c_size_t(0)
    assert B.lib().hsa_attn_workspace_size(ctypes.byref(d), B.CALL_HYBRID, ctypes.byref(n)) == 0
    assert n.value > (256 << 20)


def test_training_forward_and_saved_backward_arguments():
    """The training forward and the backward on saved statistics take the
    backward's domain (float32/bf16, all-keys branch) and need o_s and lse."""
    L = B.lib()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    need = _ws(_cfg(), B.CALL_HYBRID)[1]
    d = _cfg().desc()
    # o_s and lse required
    rc = L.hsa_hybrid_attn_train(ctypes.byref(d), fake, fake, fake, fake, fake, fake, None, None, None, None,
                                 fake, None, fake, fake, need, None)
    assert rc == -1 and b"o_s" in L.hsa_attn_last_error()
    rc = L.hsa_hybrid_attn_backward_saved(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                          None, fake, fake, fake, fake, fake, need, None)
    assert rc == -1
    # FP8 inputs and the complement variant are outside the backward's domain
    d8 = _cfg(dtype="fp8").desc()
    rc = L.hsa_hybrid_attn_train(ctypes.byref(d8), fake, fake, fake, fake, fake, fake, None, None, None, None,
                                 fake, fake, fake, fake, need, None)
    assert rc == -3
    dc = _cfg(linear_keys="complement").desc()
    rc = L.hsa_hybrid_attn_train(ctypes.byref(dc), fake, fake, fake, fake, fake, fake, None, None, None, None,
                                 fake, fake, fake, fake, need, None)
    assert rc == -2
    rc = L.hsa_hybrid_attn_backward_saved(ctypes.byref(dc), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                          fake, fake, fake, fake, fake, fake, need, None)
    assert rc == -2


def test_read_calibration_arguments():
    """The read-rate calibration validates its arguments before any launch."""
    L = B.lib()
    vp = ctypes.c_void_p
    fake = vp(1 << 20)  # never dereferenced: every case below is rejected first
    assert L.hsa_attn_read_calibrate(None, 1 << 20, fake, B.READ_SINK_WORDS, None) == -1
    assert L.hsa_attn_read_calibrate(fake, 1 << 20, None, B.READ_SINK_WORDS, None) == -1
    assert L.hsa_attn_read_calibrate(fake, 0, fake, B.READ_SINK_WORDS, None) == -2
    assert L.hsa_attn_read_calibrate(fake, (1 << 20) + 8, fake, B.READ_SINK_WORDS, None) == -2
    assert L.hsa_attn_read_calibrate(fake, 1 << 20, fake, B.READ_SINK_WORDS - 1, None) == -2
    assert b"sink" in L.hsa_attn_last_error()
