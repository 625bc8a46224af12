"""GPU parity of the MoE layer chain in one call (AllGather + routing +
grouped GEMM, then TopK-Reduce + ReduceScatter of its output, the second
part's tasks waiting on the flags of the grouped tiles they read): the chain
against the float64 oracle chain (oracle.ag_grouped_gemm, its output rounded
to bf16 as the op writes it, then oracle.moe_combine_rs), bit for bit
against the two calls made one after the other, and the dependency order in
the trace."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Trace, assert_gate, poison, say, to_bits, to_dev

pytestmark = pytest.mark.gpu


def inputs(x, peers, local):
    chunks = [to_dev(a) for a in x.a_chunks]
    lg = torch.from_numpy(np.ascontiguousarray(x.logits)).cuda()
    wt = to_dev(x.w)
    pp = [None if s == local else to_dev(peers[s]) for s in range(x.R)]
    return chunks, lg, wt, pp


def run_layer(ocg, x, peers, local, cfg=None):
    chunks, lg, wt, pp = inputs(x, peers, local)
    T = x.R * x.m
    outs = {"y": poison((T * x.topk, x.N)), "partial": poison((T, x.N)), "out": poison((x.m, x.N))}
    o = ocg.ag_moe_layer(chunks, lg, wt, pp, x.topk, local, config=cfg, outputs=outs)
    torch.cuda.synchronize()
    return o


def run_separate(ocg, x, peers, local):
    chunks, lg, wt, pp = inputs(x, peers, local)
    g = ocg.ag_grouped_gemm(chunks, lg, wt, x.topk, local)
    part, out = ocg.moe_combine_rs(g["out"], g["topk_w"], pp, local)
    torch.cuda.synchronize()
    return g, part, out


def check_chain(ocg, x, peers, local, name, cfg=None):
    o = run_layer(ocg, x, peers, local, cfg)
    g, part, out = run_separate(ocg, x, peers, local)
    # the chain's pieces are the separate calls' bit for bit (same tiles, same combine arithmetic)
    assert np.array_equal(to_bits(o["y"]), to_bits(g["out"])), f"{name}: grouped output differs"
    assert np.array_equal(o["perm"].cpu().numpy(), g["perm"].cpu().numpy())
    assert np.array_equal(to_bits(o["partial"]), to_bits(part)), f"{name}: combined partial differs"
    assert np.array_equal(to_bits(o["out"]), to_bits(out)), f"{name}: reduced block differs"
    # against the float64 oracle chain
    res = oracle.ag_grouped_gemm(x.a_chunks, x.logits, x.w, x.topk)
    assert np.array_equal(o["perm"].cpu().numpy(), res["perm"])
    y_bits = oracle.encode_bf16_rne(res["out"])
    p_ref, o_ref = oracle.moe_combine_rs(y_bits, res["weights"], x.topk, peers, x.R, local)
    assert_gate(to_bits(o["partial"]), p_ref, name + " partial", tight=False)
    assert_gate(to_bits(o["out"]), o_ref, name + " out", tight=False)
    return o


CASES = [
    # name, R, m, K, N, E, topk, local
    ("r4_e8_top2", 4, 64, 128, 224, 8, 2, 1),
    ("r2_e6_top2_n448", 2, 96, 256, 448, 6, 2, 0),
    ("r8_e16_top1_ragged", 8, 32, 128, 96, 16, 1, 5),
    ("r3_e12_top4", 3, 40, 192, 232, 12, 4, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_moe_layer_chain_small(ocg, case):
    name, R, m, K, N, E, topk, local = case
    x = workloads.make_moe(R, m, K, N, E, seed=600 + R + E, topk=topk, scale=0.5)
    peers = workloads.make_moe_peers(R, m, N, seed=700 + R, local_rank=local, scale=0.5)
    say("moe layer", name)
    check_chain(ocg, x, peers, local, name)


def test_moe_layer_trace_dependencies(ocg):
    """Every TopK-Reduce task starts only after every grouped tile that wrote
    one of its tokens' slot rows has finished."""
    R, m, K, N, E, topk, local = 4, 96, 128, 448, 8, 2, 2
    x = workloads.make_moe(R, m, K, N, E, seed=611, topk=topk, scale=0.5)
    peers = workloads.make_moe_peers(R, m, N, seed=711, local_rank=local, scale=0.5)
    cfg = ocg.default_config(tile=ocg.TILE_128x224)
    n = 4096
    tr = Trace(n)
    tr.attach(cfg)
    say("moe layer trace")
    o = check_chain(ocg, x, peers, local, "trace", cfg)
    recs = tr.read(n)
    tiles = recs[recs["kind"] == 4]
    comb = recs[recs["kind"] == 6]
    assert len(comb) > 0 and len(tiles) > 0
    perm = o["perm"].cpu().numpy()
    pos_of = np.empty_like(perm)
    pos_of[perm] = np.arange(perm.size)
    # t_end of the last tile covering each sorted position (over all column blocks)
    done = np.zeros(perm.size, dtype=np.uint64)
    for t in tiles:
        r0, nr = int(t["b"]), int(t["c"])
        done[r0:r0 + nr] = np.maximum(done[r0:r0 + nr], t["t_end"])
    T = R * m
    for c in comb:
        r0, r1 = int(c["a"]), int(c["b"])
        toks = [(r + local * m) % T for r in range(r0, r1)]
        need = max(int(done[pos_of[t * topk + j]]) for t in toks for j in range(topk))
        assert int(c["t_ready"]) >= need, "a TopK-Reduce task read rows before their tile finished"
        assert int(c["d"]) == (r1 - r0) * topk * -(-N // 224)


def test_moe_layer_full_share(ocg):
    w = workloads.workload("ag_moe_layer")
    p = w.params
    x = w.make()
    peers = workloads.make_moe_peers(p["R"], p["m"], p["N"], p["peer_seed"], p["local_rank"])
    say("moe layer full share")
    check_chain(ocg, x, peers, p["local_rank"], "ag_moe_layer")
