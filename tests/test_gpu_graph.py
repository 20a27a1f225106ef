"""The hybrid call captured in a HIP graph (torch.cuda.CUDAGraph): every
replay must give bitwise the output and mask of the eager call.  The library
enqueues only kernel launches (no memsets, copies or host syncs), so a caller
may capture it; its workspace and outputs are the plan's fixed buffers.

Each case replays the graph several times with the program's own eager work
between the replays (the outputs overwritten with garbage, an eager call on
other inputs, a synchronisation) and checks every replay.
"""
import pytest
import torch

from block_sparse_linear_select_amd import binding as B
from tests import helpers as Hp

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _same(a, b, what):
    a = a.contiguous().view(torch.uint8)
    b = b.contiguous().view(torch.uint8)
    assert torch.equal(a, b), what


@pytest.mark.parametrize("name", ["bf16_ragged", "fp8_ragged", "bf16_aligned_diag", "tiny_f32"])
def test_hybrid_call_replays_from_a_graph(name):
    print(f"\n[case {name}]", flush=True)
    w = Hp.CASES[name]
    d = Hp.to_device(Hp.gen(w), DEV)
    other = Hp.to_device(Hp.gen(w.with_(seed=w.seed + 100)), DEV)
    cfg = B.Config.from_workload(w)
    args = lambda x: (x["q"], x["k"], x["v"], x["uq"], x["uk"], x["wo"], x["q_scale"], x["k_scale"], x["v_scale"])
    plan = B.HybridPlan(cfg, DEV, export_mask=True)
    plan.run(*args(d))
    torch.cuda.synchronize()
    o_ref, rp_ref = plan.o.clone(), plan.row_ptr.clone()
    n = int(rp_ref[-1])
    ci_ref = plan.col_idx[:n].clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(*args(d), check=False)
    side = B.HybridPlan(cfg, DEV, export_mask=True)
    for rep in range(4):
        plan.o.view(torch.uint8).fill_(0xFF)  # NaN bytes: the replay must write every element
        plan.row_ptr.fill_(-1)
        plan.col_idx.fill_(-1)
        side.run(*args(other))                # eager work of the program between replays
        g.replay()
        torch.cuda.synchronize()
        _same(plan.o, o_ref, f"replay {rep}: output")
        _same(plan.row_ptr, rp_ref, f"replay {rep}: row_ptr")
        _same(plan.col_idx[:n], ci_ref, f"replay {rep}: col_idx")
    print("  4 replays bitwise equal to the eager call", flush=True)


def test_reused_mask_call_replays_from_a_graph():
    """The call on a given CSR (mask reuse across steps) captured alone."""
    w = Hp.CASES["bf16_ragged"]
    d = Hp.to_device(Hp.gen(w), DEV)
    cfg = B.Config.from_workload(w)
    rp, ci = B.block_select(cfg, d["q"], d["k"])
    plan = B.HybridPlan(cfg, DEV)
    plan.run(d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], row_ptr=rp, col_idx=ci)
    torch.cuda.synchronize()
    o_ref = plan.o.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], row_ptr=rp, col_idx=ci, check=False)
    for rep in range(3):
        plan.o.zero_()
        g.replay()
        torch.cuda.synchronize()
        _same(plan.o, o_ref, f"replay {rep}")


@pytest.mark.parametrize("name", ["bf16_ragged", "f32_d128_r64"])
def test_training_step_replays_from_a_graph(name):
    """A training step captured whole: the forward that selects its mask and
    saves the sparse statistics, then the backward on them."""
    from workloads.gen import upstream_grad
    print(f"\n[case {name}]", flush=True)
    w = Hp.CASES[name]
    d = Hp.to_device(Hp.gen(w), DEV)
    cfg = B.Config.from_workload(w)
    go = upstream_grad(w, seed=w.seed + 3).to(DEV)
    par = (d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"])

    def step():
        o, o_s, lse, rp, ci = B.hybrid_attn_train(cfg, *par, export_mask=True)
        grads = B.hybrid_attn_backward_saved(cfg, *par, rp, ci, o_s, lse, go)
        return (o, o_s, lse, rp, ci) + tuple(grads)

    ref = [t.clone() for t in step()]
    torch.cuda.synchronize()
    n = int(ref[3][-1])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    names = ("o", "o_s", "lse", "row_ptr", "col_idx", "dq", "dk", "dv")
    for rep in range(3):
        for t in out:
            t.view(torch.uint8).fill_(0xFF)
        step()  # the program's own eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for nm, x, y in zip(names, out, ref):
            if nm == "lse":  # rows >= N are undefined
                x, y = x[:, :, : w.N], y[:, :, : w.N]
            if nm == "col_idx":
                x, y = x[:n], y[:n]
            _same(x, y, f"replay {rep}: {nm}")
    print("  3 replays bitwise equal to the eager step", flush=True)
