"""Host-side checks of the seeded input generators (CPU only)."""
import numpy as np
import torch

from workloads import generate, make_workload
from workloads.gen import next_step


def _small(dtype):
    base = "wan14b_720p_fp8" if dtype == "fp8" else "wan14b_480p_bf16"
    return make_workload(base, B=1, H=2, grid=(2, 5, 13), topk=2, rank=32, seed=7)


def test_next_step_with_no_noise_reproduces_the_inputs():
    for dtype in ("bf16", "fp8"):
        inp = generate(_small(dtype))
        nxt = next_step(inp, eps=0.0, seed=1)
        for name in ("q", "k", "v"):
            a, b = getattr(inp, name), getattr(nxt, name)
            assert a.dtype == b.dtype and a.shape == b.shape
            assert torch.equal(a.float(), b.float())  # (fp8: -0 may come back as +0)
            if dtype == "fp8":
                assert torch.equal(getattr(inp, name + "_scale"), getattr(nxt, name + "_scale"))


def test_next_step_moves_valid_rows_only_and_is_seeded():
    w = _small("bf16")
    inp = generate(w)
    a = next_step(inp, eps=0.1, seed=3)
    b = next_step(inp, eps=0.1, seed=3)
    c = next_step(inp, eps=0.1, seed=4)
    assert torch.equal(a.q, b.q) and not torch.equal(a.q, c.q)
    assert torch.all(a.q[:, :, w.N:] == 0) and torch.all(a.v[:, :, w.N:] == 0)
    diff = (a.k.float() - inp.k.float())[:, :, : w.N]
    assert 0.05 < float(diff.std()) < 0.2  # the added noise, up to bf16 rounding
    assert a.uq is inp.uq and a.wo is inp.wo  # parameters shared between steps
