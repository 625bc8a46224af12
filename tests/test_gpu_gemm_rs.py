"""GPU parity of the fused GEMM-ReduceScatter: the bf16 partial against the
float64 oracle, the reduced row block against the oracle and -- bit for bit --
against the fixed-order float32 reduce of the GPU's own partial and the peer
partials, the notify/reduce ordering in the trace, and the peer-flag wait."""
import numpy as np
import pytest
import torch

import oracle
from oracle import schedule as sch
import workloads
from gpu_util import Trace, assert_gate, poison, say, to_bits, to_dev

pytestmark = pytest.mark.gpu


def run(ocg, x, cfg=None, workspace=None):
    a, b = to_dev(x.a), to_dev(x.b)
    peers = [None if s == x.local_rank else to_dev(x.peers[s]) for s in range(x.R)]
    part = poison((x.M, x.N))
    out = poison((x.M // x.R, x.N))
    ocg.gemm_rs(a, b, peers, x.local_rank, partial=part, out=out, config=cfg, workspace=workspace)
    torch.cuda.synchronize()
    return to_bits(part), to_bits(out)


def check_reduce_bits(x, part_bits, out_bits):
    blk = x.M // x.R
    lo = x.local_rank * blk
    blocks = [part_bits[lo:lo + blk] if s == x.local_rank else x.peers[s][lo:lo + blk] for s in range(x.R)]
    want = oracle.reduce_fixed_order(blocks)
    diff = int((want != out_bits).sum())
    assert diff == 0, f"{diff} reduced elements differ from the fixed-order float32 reduce"


SMALL = [
    # name, R, M, K, N, local, tile
    ("r4_128x128", 4, 96, 64, 40, 2, 3),
    ("r3_256x224", 3, 600, 128, 264, 1, 0),
    ("r8_l0", 8, 1024, 256, 512, 0, -1),
    ("r8_l5", 8, 1024, 256, 512, 5, -1),
    ("r2_128x256", 2, 512, 192, 264, 1, 2),
    ("r4_256x256", 4, 1024, 192, 600, 3, 4),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_gemm_rs_small_full(ocg, case):
    name, R, M, K, N, local, tile = case
    x = workloads.make_gemm_rs(R, M, K, N, seed=200 + R + local, local_rank=local, dist="uniform", scale=1.0)
    say("gemm_rs", name)
    part, out = run(ocg, x, ocg.default_config(tile=tile))
    p_ref, o_ref = oracle.gemm_rs(x.a, x.b, x.peers, R, local)
    assert_gate(part, p_ref, name + " partial")
    blk = M // R
    # the local partial enters the reduce rounded to bf16: half an ulp of it
    assert_gate(out, o_ref, name + " out", extra=2.0 ** -8 * np.abs(p_ref[local * blk:(local + 1) * blk]))
    check_reduce_bits(x, part, out)
    ocg.Workspace.cached(ocg.OP_GEMM_RS, R, M, K, N).check()


def test_gemm_rs_trace_notify_before_reduce(ocg):
    R, M, K, N, local = 4, 512, 128, 456, 1
    x = workloads.make_gemm_rs(R, M, K, N, seed=31, local_rank=local, dist="uniform", scale=1.0)
    cfg = ocg.default_config(tile=ocg.TILE_128x128)
    info = ocg.plan_info(ocg.OP_GEMM_RS, R, local, M, K, N, cfg)
    plan = sch.gemm_rs_plan(R, M, N, local, info["BM"], info["BN"], info["n_slabs_or_strip_rows"])
    tr = Trace(len(plan) + 4)
    tr.attach(cfg)
    say("gemm_rs trace")
    part, out = run(ocg, x, cfg)
    recs = tr.read(len(plan))
    assert np.array_equal(recs["ticket"], np.arange(len(plan)))
    done = {}
    for t, r in zip(plan, recs):
        if t[0] == "tile":
            assert (r["kind"], r["a"], r["b"], r["c"]) == (3, t[2], t[3], int(t[4]))
            assert int(r["queue"]) == (t[5] << 16) | t[6], "tile taken from its XCD queue"
            done[(t[2], t[3])] = int(r["t_end"])
    BM, blk = info["BM"], M // R
    lo = local * blk
    pollers = {}
    for t, r in zip(plan, recs):
        if t[0] == "reduce":
            assert (r["kind"], r["a"], r["b"], r["c"]) == (5, t[2], t[3], len(t[4]))
            assert r["flag_seen"] == r["epoch"]
            # the strip starts reducing only after every tile it reads was notified
            assert int(r["t_ready"]) >= max(done[d] for d in t[4]) - 0
            # it polled the tile flags of the row blocks whose first local row it holds,
            # and their summary words for the others
            r0, r1 = t[2], t[3]
            own = [rb for rb in range(r0 // BM, (r1 - 1) // BM + 1) if r0 <= max(rb * BM, lo) < r1]
            assert int(r["queue"]) == len(own)
            for rb in own:
                pollers[rb] = pollers.get(rb, 0) + 1
    assert pollers == {rb: 1 for rb in range(lo // BM, (lo + blk - 1) // BM + 1)}, "one poller per row block"
    check_reduce_bits(x, part, out)


def test_gemm_rs_peer_flags(ocg):
    """peer_tile_wait stand-in: flags a peer would set remotely. Signalled ->
    the call completes and matches; never signalled (host-forced, 2 ms bound)
    -> the timeout is reported and the kernel still drains."""
    R, M, K, N, local = 4, 512, 128, 256, 2
    x = workloads.make_gemm_rs(R, M, K, N, seed=41, local_rank=local, dist="uniform", scale=1.0)
    cfg = ocg.default_config(tile=ocg.TILE_128x128)
    info = ocg.plan_info(ocg.OP_GEMM_RS, R, local, M, K, N, cfg)
    local_tiles = (M // R // info["BM"]) * (-(-N // info["BN"]))
    flags = torch.zeros(R * local_tiles, dtype=torch.int32, device="cuda")
    ws = ocg.Workspace(ocg.OP_GEMM_RS, R, M, K, N)
    say("gemm_rs peer flags signalled")
    ocg.signal(flags, 7)
    cfg.peer_flags = flags.data_ptr()
    cfg.peer_flag_value = 7
    part, out = run(ocg, x, cfg, ws)
    ws.check()
    check_reduce_bits(x, part, out)
    say("gemm_rs peer flags never signalled")
    cfg.peer_flag_value = 8
    cfg.spin_timeout_us = 2000
    run(ocg, x, cfg, ws)
    with pytest.raises(ocg.OcgError) as ei:
        ws.check()
    assert ei.value.code == ocg.ERR_TIMEOUT


def test_gemm_rs_8b_share(ocg):
    x = workloads.workload("gemm_rs_8b").make()
    say("gemm_rs_8b")
    part, out = run(ocg, x)
    check_reduce_bits(x, part, out)
    blk = x.M // x.R
    # the reduced block in full against the float64 definition
    a_blk = oracle.decode_bf16(x.a[:blk])
    p_blk = a_blk @ oracle.decode_bf16(x.b)
    o_ref = p_blk + sum(oracle.decode_bf16(x.peers[s][:blk]) for s in range(1, x.R))
    assert_gate(out, o_ref, "gemm_rs_8b out", extra=2.0 ** -8 * np.abs(p_blk))
    # the whole partial (every element) against the float64 product
    p_ref = oracle.decode_bf16(x.a) @ oracle.decode_bf16(x.b)
    assert_gate(part, p_ref, "gemm_rs_8b partial")


# ---------------------------------------------------------------- push transfers

def run_push(ocg, x, flag_value, cfg=None, signal_peers=True):
    """Stand-in receive buffers and flags of every rank: rank s's buffer holds
    R slots of M/R rows; the peers' pushes into ours are placed by the
    harness (their partials' rows of our block) and their flags set with the
    peer-notify stand-in."""
    R, M, N, l = x.R, x.M, x.N, x.local_rank
    blk = M // R
    h = ocg.handle()
    info = ocg.plan_info(ocg.OP_GEMM_RS, R, l, M, x.K, N, cfg, handle=h)
    T = (blk // info["BM"]) * (-(-N // info["BN"]))
    recv = [poison((R, blk, N)) for _ in range(R)]
    flags = [torch.zeros(R * T, dtype=torch.int32, device="cuda") for _ in range(R)]
    for s in range(R):
        if s != l:
            recv[l][s].copy_(to_dev(x.peers[s][l * blk:(l + 1) * blk]))
    if signal_peers:
        for s in range(R):
            if s != l:
                ocg.signal(flags[l][s * T:(s + 1) * T], flag_value)
    out = poison((blk, N))
    ocg.gemm_rs_push(to_dev(x.a), to_dev(x.b), recv, flags, flag_value, l, out=out, config=cfg)
    torch.cuda.synchronize()
    return recv, flags, T, to_bits(out)


PUSH = [
    # name, R, M, K, N, local, tile
    ("r4_128x128", 4, 512, 128, 264, 1, 3),
    ("r4_128x224_l0", 4, 512, 192, 456, 0, 1),
    ("r8_256x224", 8, 2048, 128, 520, 5, 0),
    ("r2_256x256", 2, 512, 256, 600, 1, 4),
    ("r3_128x256", 3, 384, 64, 264, 2, 2),
]


@pytest.mark.parametrize("case", PUSH, ids=[c[0] for c in PUSH])
def test_gemm_rs_push_matches_pull(ocg, case):
    name, R, M, K, N, local, tile = case
    x = workloads.make_gemm_rs(R, M, K, N, seed=400 + R + local, local_rank=local, dist="uniform", scale=1.0)
    cfg = ocg.default_config(tile=tile)
    say("gemm_rs pull", name)
    part, out_pull = run(ocg, x, cfg)
    say("gemm_rs push", name)
    recv, flags, T, out = run_push(ocg, x, 11 + R, cfg)
    blk = M // R
    assert np.array_equal(out, out_pull), "push and pull reduce to the same bits"
    for s in range(R):
        # our partial's rows of block s landed in rank s's slot `local`
        assert np.array_equal(to_bits(recv[s][local]), part[s * blk:(s + 1) * blk])
        got = flags[s][local * T:(local + 1) * T].cpu().numpy()
        assert (got == 11 + R).all(), "every pushed tile set its flag"
    check_reduce_bits(x, part, out)
    p_ref, o_ref = oracle.gemm_rs(x.a, x.b, x.peers, R, local)
    assert_gate(out, o_ref, name + " push out", extra=2.0 ** -8 * np.abs(p_ref[local * blk:(local + 1) * blk]))


def test_gemm_rs_push_trace_and_timeout(ocg):
    R, M, K, N, local = 4, 512, 128, 456, 2
    x = workloads.make_gemm_rs(R, M, K, N, seed=43, local_rank=local, dist="uniform", scale=1.0)
    cfg = ocg.default_config(tile=ocg.TILE_128x128)
    info = ocg.plan_info(ocg.OP_GEMM_RS, R, local, M, K, N, cfg)
    plan = sch.gemm_rs_plan(R, M, N, local, info["BM"], info["BN"], info["n_slabs_or_strip_rows"], push=True)
    tr = Trace(len(plan) + 4)
    tr.attach(cfg)
    say("gemm_rs push trace")
    recv, flags, T, out = run_push(ocg, x, 5, cfg)
    recs = tr.read(len(plan))
    assert np.array_equal(recs["ticket"], np.arange(len(plan)))
    blk = M // R
    tiles = [t for t in plan if t[0] == "tile"]
    assert tiles[0][2] * info["BM"] == ((local + 1) % R) * blk, "tiles start at the block after the local one"
    assert tiles[-1][2] * info["BM"] // blk == local, "the local block comes last"
    done = {}
    for t, r in zip(plan, recs):
        if t[0] == "tile":
            assert (r["kind"], r["a"], r["b"]) == (3, t[2], t[3])
            done[(t[2], t[3])] = int(r["t_end"])
    for t, r in zip(plan, recs):
        if t[0] == "reduce":
            assert int(r["t_ready"]) >= max(done[d] for d in t[4])
    # a peer push that never lands: the reduce's bounded wait reports it
    ws = ocg.Workspace(ocg.OP_GEMM_RS, R, M, K, N)
    cfg2 = ocg.default_config(tile=ocg.TILE_128x128, spin_timeout_us=2000)
    say("gemm_rs push, peers never signal")
    blk_rows = M // R
    recv2 = [poison((R, blk_rows, N)) for _ in range(R)]
    flags2 = [torch.zeros(R * T, dtype=torch.int32, device="cuda") for _ in range(R)]
    ocg.gemm_rs_push(to_dev(x.a), to_dev(x.b), recv2, flags2, 9, local, workspace=ws, config=cfg2)
    with pytest.raises(ocg.OcgError) as ei:
        ws.check()
    assert ei.value.code == ocg.ERR_TIMEOUT


def test_gemm_rs_8b_share_push(ocg):
    x = workloads.workload("gemm_rs_8b").make()
    say("gemm_rs_8b pull")
    part, out_pull = run(ocg, x)
    say("gemm_rs_8b push")
    recv, flags, T, out = run_push(ocg, x, 77)
    assert np.array_equal(out, out_pull)
    blk = x.M // x.R
    for s in range(x.R):
        assert np.array_equal(to_bits(recv[s][x.local_rank]), part[s * blk:(s + 1) * blk])
