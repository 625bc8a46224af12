"""Seeded random shapes and configurations, every entry point against the
float64 oracle: AllGather-GEMM (every tile preset, both transfers, K-slab
widths, split K), GEMM-ReduceScatter (pull and push), the AllGather + MoE
grouped GEMM, the TopK-Reduce + ReduceScatter and the AllGather-KV
attention. The fixed cases of the other files pin known edges; these draw
the combinations nobody listed (ragged rows, columns and K, odd rank counts,
any local rank), from one generator per operation so a failure names a
reproducible case."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_gate, poison, say, to_bits, to_dev
from test_gpu_attention import check as attn_check, run as attn_run, D as ATTN_D
from test_gpu_gemm_rs import check_reduce_bits, run as rs_run, run_push
from test_gpu_moe import check as moe_check, run as moe_run
from test_gpu_moe_combine import check as comb_check, run as comb_run

pytestmark = pytest.mark.gpu

INLINE, SIDE = 0, 1
TILES = [-1, 0, 1, 2, 3, 4]


def _seed(name: str) -> int:
    return zlib.crc32(name.encode())


def _ag_cases(n=48, seed=8101):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.integers(1, 9))
        m = int(rng.integers(1, 321))
        K = 64 * int(rng.integers(1, 21))
        N = 8 * int(rng.integers(1, 91))
        local = int(rng.integers(0, R))
        tile = int(rng.choice(TILES))
        transfer = int(rng.integers(0, 2))
        kslab = int(rng.choice([0, 256, 512]))
        split = 2 if (transfer == INLINE and kslab == 0 and K % 128 == 0 and rng.random() < 0.35) else 0
        out.append((f"ag{i}_r{R}_m{m}_k{K}_n{N}_l{local}_t{tile}_x{transfer}_ks{kslab}_sk{split}",
                    R, m, K, N, local, tile, transfer, kslab, split))
    return out


AG = _ag_cases()


@pytest.mark.parametrize("case", AG, ids=[c[0] for c in AG])
def test_ag_gemm_random(ocg, case):
    name, R, m, K, N, local, tile, transfer, kslab, split = case
    cfg = ocg.default_config(tile=tile, transfer=transfer, kslab_cols=kslab, split_k=split)
    try:
        ocg.plan_ag(R, local, m, K, N, cfg, handle=ocg.handle())
    except ocg.OcgError as e:
        # combinations the header rejects (a side producer that does not fit
        # beside this tile, split K on a preset that cannot): the same shape
        # with the default transfer
        assert e.code in (ocg.ERR_UNSUPPORTED_SHAPE, ocg.ERR_INVALID_ARG)
        cfg = ocg.default_config(tile=tile)
    x = workloads.make_ag_gemm(R, m, K, N, seed=_seed(name), dist="normal", scale=0.02)
    say("ag_gemm random", name)
    chunks = [to_dev(c) for c in x.a_chunks]
    ag = poison((R * m, K))
    c = poison((R * m, N))
    ocg.ag_gemm(chunks, to_dev(x.b), local, a_gathered=ag, c=c, config=cfg)
    torch.cuda.synchronize()
    ocg.Workspace.cached(ocg.OP_AG_GEMM, R, m, K, N, config=cfg).check()
    a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
    assert np.array_equal(to_bits(ag), a_full), "gathered buffer must be a bit-exact copy"
    assert_gate(to_bits(c), want, name)


def _rs_cases(n=24, seed=8202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.integers(1, 9))
        blk = int(rng.integers(1, 260))
        K = 64 * int(rng.integers(1, 13))
        N = 8 * int(rng.integers(1, 91))
        local = int(rng.integers(0, R))
        tile = int(rng.choice(TILES))
        out.append((f"rs{i}_r{R}_blk{blk}_k{K}_n{N}_l{local}_t{tile}", R, R * blk, K, N, local, tile))
    return out


RS = _rs_cases()


@pytest.mark.parametrize("case", RS, ids=[c[0] for c in RS])
def test_gemm_rs_random(ocg, case):
    """Pull: the partial within the gate, the reduce bit for bit against the
    fixed-order float32 sum; push (where the row block is whole tiles, which
    the push transfer needs): the same reduced bits."""
    name, R, M, K, N, local, tile = case
    x = workloads.make_gemm_rs(R, M, K, N, seed=_seed(name), local_rank=local, dist="uniform",
                               scale=1.0)
    cfg = ocg.default_config(tile=tile)
    say("gemm_rs random", name)
    part, out = rs_run(ocg, x, cfg)
    ocg.Workspace.cached(ocg.OP_GEMM_RS, R, M, K, N).check()
    check_reduce_bits(x, part, out)
    p_ref, o_ref = oracle.gemm_rs(x.a, x.b, x.peers, R, local)
    blk = M // R
    assert_gate(part, p_ref, name + " partial")
    assert_gate(out, o_ref, name + " out", extra=2.0 ** -8 * np.abs(p_ref[local * blk:(local + 1) * blk]))
    info = ocg.plan_info(ocg.OP_GEMM_RS, R, local, M, K, N, cfg, handle=ocg.handle())
    if blk % info["BM"] == 0:
        say("gemm_rs random push", name)
        _, _, _, out_push = run_push(ocg, x, 40 + R, cfg)
        assert np.array_equal(out_push, out), "push and pull reduce to the same bits"


def _moe_cases(n=16, seed=8303):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.integers(1, 9))
        m = int(rng.integers(1, 200))
        K = 64 * int(rng.integers(1, 7))
        N = 8 * int(rng.integers(1, 61))
        E = int(rng.integers(1, 65))
        topk = int(rng.integers(1, min(E, 4) + 1))
        local = int(rng.integers(0, R))
        out.append((f"moe{i}_r{R}_m{m}_k{K}_n{N}_e{E}_top{topk}_l{local}", R, m, K, N, E, topk, local))
    return out


MOE = _moe_cases()


@pytest.mark.parametrize("case", MOE, ids=[c[0] for c in MOE])
def test_moe_random(ocg, case):
    name, R, m, K, N, E, topk, local = case
    x = workloads.make_moe(R, m, K, N, E, seed=_seed(name), topk=topk, scale=0.5)
    say("moe random", name)
    o = moe_run(ocg, x, local)
    moe_check(ocg, x, o, name)


def _comb_cases(n=12, seed=8404):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.integers(1, 9))
        m = int(rng.integers(1, 200))
        N = 8 * int(rng.integers(1, 121))
        topk = int(rng.integers(1, 5))
        local = int(rng.integers(0, R))
        out.append((f"comb{i}_r{R}_m{m}_n{N}_top{topk}_l{local}", R, m, N, topk, local))
    return out


COMB = _comb_cases()


@pytest.mark.parametrize("case", COMB, ids=[c[0] for c in COMB])
def test_moe_combine_rs_random(ocg, case):
    name, R, m, N, topk, local = case
    x = workloads.make_moe_combine(R, m, N, topk, seed=_seed(name), local_rank=local)
    say("moe_combine_rs random", name)
    comb_check(x, *comb_run(ocg, x), name)


def _attn_cases(n=16, seed=8505):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.integers(1, 9))
        m = int(rng.integers(1, 300))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 3, 4, 8]))
        local = int(rng.integers(0, R))
        out.append((f"attn{i}_r{R}_m{m}_hq{Hq}_hkv{Hkv}_l{local}", R, m, Hq, Hkv, local))
    return out


ATTN = _attn_cases()


@pytest.mark.parametrize("case", ATTN, ids=[c[0] for c in ATTN])
def test_ag_attention_random(ocg, case):
    name, R, m, Hq, Hkv, local = case
    x = workloads.make_attention(R, m, Hq, Hkv, ATTN_D, seed=_seed(name), local_rank=local)
    say("ag_attention random", name)
    attn_check(x, *attn_run(ocg, x), name)
