"""GPU parity at the smallest shapes the boundary accepts: one row per rank,
K = 64 (two MFMA stages), N = 8 (one 16-byte chunk of a row), one rank,
and the smallest split-K halves (K = 128, one stage pair each). Tiles are
almost all padding here, so reads and stores past the last row or column
show up. AG-GEMM in both transfer modes against the float64 oracle with the
gathered buffer bit for bit; GEMM-RS partial and reduced block against the
oracle and the reduce bit for bit against the fixed-order float32 sum."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_gate, poison, say, to_bits, to_dev

pytestmark = pytest.mark.gpu

AG_EDGES = [
    # name, R, m, K, N, local, split_k
    ("r8_m1_k64_n8", 8, 1, 64, 8, 5, 1),
    ("r1_m1_k64_n8", 1, 1, 64, 8, 0, 1),
    ("r2_m3_k64_n24", 2, 3, 64, 24, 1, 1),
    ("r3_m2_k128_n16_split", 3, 2, 128, 16, 2, 2),
    ("r2_m1_k128_n8_split", 2, 1, 128, 8, 0, 2),
]


# split K runs with inline copies only
AG_RUNS = [(c, t) for c in AG_EDGES for t in (0, 1) if c[6] == 1 or t == 0]


@pytest.mark.parametrize("case,transfer", AG_RUNS, ids=[f"{c[0]}-{('inline', 'side')[t]}" for c, t in AG_RUNS])
def test_ag_gemm_smallest_shapes(ocg, case, transfer):
    name, R, m, K, N, local, split = case
    x = workloads.make_ag_gemm(R, m, K, N, seed=900 + R * 7 + m, dist="uniform", scale=1.0)
    cfg = ocg.default_config(transfer=transfer, split_k=split)
    say("ag_gemm edge", name, "transfer", transfer)
    ag, c = poison((R * m, K)), poison((R * m, N))
    ocg.ag_gemm([to_dev(a) for a in x.a_chunks], to_dev(x.b), local, a_gathered=ag, c=c, config=cfg)
    a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
    assert np.array_equal(to_bits(ag), a_full), "gathered buffer must be a bit-exact copy"
    assert_gate(to_bits(c), want, name)
    ocg.Workspace.cached(ocg.OP_AG_GEMM, R, m, K, N, config=cfg).check()


RS_EDGES = [
    # name, R, M, K, N, local
    ("r8_one_row_each", 8, 8, 64, 8, 3),
    ("r1_m1", 1, 1, 64, 8, 0),
    ("r2_m6_n24", 2, 6, 64, 24, 1),
]


@pytest.mark.parametrize("case", RS_EDGES, ids=[c[0] for c in RS_EDGES])
def test_gemm_rs_smallest_shapes(ocg, case):
    name, R, M, K, N, local = case
    x = workloads.make_gemm_rs(R, M, K, N, seed=950 + R + local, local_rank=local, dist="uniform", scale=1.0)
    a, b = to_dev(x.a), to_dev(x.b)
    peers = [None if s == local else to_dev(x.peers[s]) for s in range(R)]
    part, out = poison((M, N)), poison((M // R, N))
    say("gemm_rs edge", name)
    ocg.gemm_rs(a, b, peers, local, partial=part, out=out)
    p_ref, o_ref = oracle.gemm_rs(x.a, x.b, x.peers, R, local)
    part_bits, out_bits = to_bits(part), to_bits(out)
    assert_gate(part_bits, p_ref, name + " partial")
    blk = M // R
    assert_gate(out_bits, o_ref, name + " out", extra=2.0 ** -8 * np.abs(p_ref[local * blk:(local + 1) * blk]))
    lo = local * blk
    blocks = [part_bits[lo:lo + blk] if s == local else x.peers[s][lo:lo + blk] for s in range(R)]
    assert np.array_equal(oracle.reduce_fixed_order(blocks), out_bits), "fixed-order reduce, bit for bit"
    ocg.Workspace.cached(ocg.OP_GEMM_RS, R, M, K, N).check()
