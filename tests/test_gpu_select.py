"""The selection kernel on inputs that stress its exact ranking step.

The kernel scores tile pairs on the bf16 matrix cores (hi + lo parts of the
float64 means) and re-ranks by exact float64 scores only the tiles whose
approximate score lies within the error bound of the k-th one.  These cases
force that step: exact ties between duplicated key tiles (the lower tile index
wins, reading R3 of the tie-break), and heads whose query or key tiles are all
zero, where every score ties at 0 and the k lowest tiles are kept.
"""
import numpy as np
import pytest
import torch

from block_sparse_linear_select_amd import binding as B
from oracle import rola as R
from tests import helpers as Hp
from workloads import generate, make_workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _select(inp):
    w = inp.w
    d = Hp.to_device(inp, DEV)
    rp, ci = B.block_select(B.Config.from_workload(w), d["q"], d["k"], d["q_scale"], d["k_scale"])
    torch.cuda.synchronize()
    return Hp.split_csr(rp, ci, w.B * w.H, w.T)


def _oracle_rows(inp, b, h):
    return Hp.oracle_mask_head(inp, b, h)[1]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_exact_ties_go_to_the_lower_tile(dtype):
    name = "wan14b_480p_bf16" if dtype == "bf16" else "wan14b_720p_fp8"
    w = make_workload(name, H=2, grid=(4, 16, 32), topk=2, rank=32, seed=61)
    print(f"\n[ties {dtype}: T={w.T} topk={w.topk}]", flush=True)
    inp = generate(w)
    for h in range(w.H):
        for src, copies in ((3, (11, 19, 27)), (6, (14, 22))):
            # a tile scaled up by 4 (exact) so that it and its copies lead the rows that point at it
            if inp.k_scale is not None:
                inp.k_scale[0, h, src] *= 4.0
            else:
                inp.k[0, h, 64 * src:64 * src + 64] *= 4.0
            for c in copies:  # duplicated key tiles: identical means, exactly tied scores
                inp.k[0, h, 64 * c:64 * c + 64] = inp.k[0, h, 64 * src:64 * src + 64]
                if inp.k_scale is not None:
                    inp.k_scale[0, h, c] = inp.k_scale[0, h, src]
        # query tile 0 points at key tile 3, query tile 1 at key tile 6
        inp.q[0, h, 0:64] = inp.k[0, h, 3 * 64:4 * 64]
        inp.q[0, h, 64:128] = inp.k[0, h, 6 * 64:7 * 64]
        if inp.q_scale is not None:
            inp.q_scale[0, h, 0] = inp.k_scale[0, h, 3]
            inp.q_scale[0, h, 1] = inp.k_scale[0, h, 6]
    gpu = _select(inp)
    for h in range(w.H):
        sc, ref = Hp.oracle_mask_head(inp, 0, h)
        assert sc[0, 3] == sc[0, 11] == sc[0, 19] == sc[0, 27]
        assert list(ref[0]) == [3, 11] and list(ref[1]) == [6, 14]
        assert [list(x) for x in gpu[h][:2]] == [[3, 11], [6, 14]], f"head {h}"
        bad, _ = Hp.mask_mismatches(gpu[h], ref, sc, w.topk, w.force_diag)
        assert bad == 0


def test_all_zero_query_or_key_heads_keep_the_lowest_tiles():
    w = make_workload("wan14b_480p_bf16", H=3, grid=(4, 16, 32), topk=5, rank=32, seed=62)
    print(f"\n[zero heads: T={w.T} topk={w.topk}]", flush=True)
    inp = generate(w)
    inp.q[0, 1].zero_()   # every score of head 1 is exactly 0
    inp.k[0, 2].zero_()   # and of head 2
    gpu = _select(inp)
    for h in (1, 2):
        ref = _oracle_rows(inp, 0, h)
        assert all(list(r) == list(range(w.topk)) for r in ref)
        assert all(list(r) == list(range(w.topk)) for r in gpu[h]), f"head {h}"
    sc, ref = Hp.oracle_mask_head(inp, 0, 0)
    assert Hp.mask_mismatches(gpu[0], ref, sc, w.topk, w.force_diag)[0] == 0


def test_means_exported_by_selection_match_the_oracle():
    """The query means now come from the selection kernel, the key means from
    the streaming pass: both equal the oracle's float64 means (exact sums)."""
    w = make_workload("wan14b_720p_fp8", H=2, grid=(3, 10, 13), topk=3, rank=32, seed=63)
    inp = generate(w)
    d = Hp.to_device(inp, DEV)
    rp, ci, qbar, kbar = B.block_select(B.Config.from_workload(w), d["q"], d["k"], d["q_scale"], d["k_scale"],
                                        want_means=True)
    torch.cuda.synchronize()
    for h in range(w.H):
        q, k, _ = Hp.head_arrays(inp, 0, h)
        np.testing.assert_allclose(qbar[0, h].cpu().numpy(), R.tile_means(q, w.N), rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(kbar[0, h].cpu().numpy(), R.tile_means(k, w.N), rtol=1e-15, atol=1e-15)
