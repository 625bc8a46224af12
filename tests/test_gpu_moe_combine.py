"""GPU parity of the MoE TopK-Reduce + ReduceScatter: the bf16 combined
partial against the float64 oracle, the reduced row block against the oracle
and -- bit for bit -- against the fixed-order float32 reduce of the GPU's own
partial and the peer partials, and the task list in the trace."""
import numpy as np
import pytest
import torch

import oracle
from oracle import schedule as sch
import workloads
from gpu_util import Trace, assert_gate, poison, say, to_bits, to_dev

pytestmark = pytest.mark.gpu


def run(ocg, x, cfg=None):
    y = to_dev(x.y)
    w = torch.from_numpy(np.ascontiguousarray(x.w)).cuda()
    T = x.R * x.m
    peers = [None if s == x.local_rank else to_dev(x.peers[s]) for s in range(x.R)]
    part = poison((T, x.N))
    out = poison((x.m, x.N))
    ocg.moe_combine_rs(y, w, peers, x.local_rank, partial=part, out=out, config=cfg)
    torch.cuda.synchronize()
    return to_bits(part), to_bits(out)


def check(x, part, out, name):
    p_ref, o_ref = oracle.moe_combine_rs(x.y, x.w, x.topk, x.peers, x.R, x.local_rank)
    assert_gate(part, p_ref, name + " partial")
    lo = x.local_rank * x.m
    # the local partial enters the reduce rounded to bf16: half an ulp of it
    assert_gate(out, o_ref, name + " out", extra=2.0 ** -8 * np.abs(p_ref[lo:lo + x.m]))
    blocks = [part[lo:lo + x.m] if s == x.local_rank else x.peers[s][lo:lo + x.m] for s in range(x.R)]
    want = oracle.reduce_fixed_order(blocks)
    diff = int((want != out).sum())
    assert diff == 0, f"{name}: {diff} reduced elements differ from the fixed-order float32 reduce"


CASES = [
    # name, R, m, N, topk, local
    ("r4_top2", 4, 96, 72, 2, 1),
    ("r8_top2_l5", 8, 64, 264, 2, 5),
    ("r3_top1_ragged", 3, 37, 8, 1, 2),
    ("r2_top4", 2, 130, 1800, 4, 0),
    ("r1_top2", 1, 50, 40, 2, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_moe_combine_rs_small(ocg, case):
    name, R, m, N, topk, local = case
    x = workloads.make_moe_combine(R, m, N, topk, seed=500 + R + local, local_rank=local)
    say("moe_combine_rs", name)
    part, out = run(ocg, x)
    check(x, part, out, name)


def test_moe_combine_rs_trace(ocg):
    """Every task runs once, in ticket order over the rotated rows, the local
    block's rows first and counted per task."""
    x = workloads.make_moe_combine(4, 200, 136, 2, seed=520, local_rank=3)
    cfg = ocg.default_config()
    info = ocg.plan_info(ocg.OP_MOE_COMBINE_RS, x.R, x.local_rank, x.m, 0, x.N, cfg, topk=x.topk)
    cr, crl = info["slab_rows"], info["copy_rows"]
    plan = sch.combine_rs_plan(x.R, x.R * x.m, x.local_rank, cr, crl)
    assert info["n_copy_or_strips"] == len(plan) and info["n_tiles"] == sum(p[3] for p in plan)
    tr = Trace(len(plan) + 8)
    tr.attach(cfg)
    say("moe_combine_rs trace")
    part, out = run(ocg, x, cfg)
    check(x, part, out, "trace")
    recs = tr.read(len(plan))
    assert np.array_equal(recs["ticket"], np.arange(len(plan)))
    base = x.local_rank * x.m
    T = x.R * x.m
    for (_, u, rows, is_local), r in zip(plan, recs):
        assert r["kind"] == 6
        r0 = (rows[0] - base) % T
        assert (int(r["a"]), int(r["b"]), int(r["c"])) == (r0, r0 + len(rows), len(rows) if is_local else 0)


def test_moe_combine_rs_rejects_bad_shapes(ocg):
    x = workloads.make_moe_combine(2, 16, 40, 2, seed=530)
    y = to_dev(x.y)
    w = torch.from_numpy(np.ascontiguousarray(x.w)).cuda()
    peers = [None, to_dev(x.peers[1])]
    with pytest.raises(ValueError):   # T not a multiple of R
        ocg.moe_combine_rs(y[: 2 * 31], w[:31].contiguous(), peers, 0)
    w5 = torch.zeros((x.R * x.m, 5), dtype=torch.float32, device="cuda")
    y5 = torch.zeros((x.R * x.m * 5, 40), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ocg.OcgError):  # topk > 4
        ocg.moe_combine_rs(y5, w5, [None, torch.zeros((x.R * x.m, 40), dtype=torch.bfloat16, device="cuda")], 0)


def test_moe_combine_rs_full_workload(ocg):
    x = workloads.workload("moe_combine_rs").make()
    say("moe_combine_rs full workload")
    part, out = run(ocg, x)
    check(x, part, out, "moe_combine_rs")
