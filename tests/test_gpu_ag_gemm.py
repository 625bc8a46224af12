"""GPU parity of the fused AllGather-GEMM against the float64 oracle, through
the C ABI: small and ragged shapes in full, the 8B- and 70B-class shares on
sampled blocks, the gathered buffer bit for bit, the schedule trace against
the oracle's re-derivation, the measurement modes, and the timeout path."""
import numpy as np
import pytest
import torch

import oracle
from oracle import schedule as sch
import workloads
from gpu_util import Trace, assert_gate, poison, say, to_bits, to_dev

pytestmark = pytest.mark.gpu


def run(ocg, x, local=0, cfg=None):
    chunks = [to_dev(c) for c in x.a_chunks]
    b = to_dev(x.b)
    ag = poison((x.R * x.m, x.K))           # any early read of an unfilled slab shows up as NaN
    c = poison((x.R * x.m, x.N))
    ocg.ag_gemm(chunks, b, local, a_gathered=ag, c=c, config=cfg)
    torch.cuda.synchronize()
    return c, ag


SMALL = [
    # name, R, m, K, N, local, tile, dist
    ("tiny_l0", 4, 128, 256, 256, 0, -1, "uniform"),
    ("tiny_l3", 4, 128, 256, 256, 3, -1, "uniform"),
    ("ragged_128x128", 3, 100, 64, 72, 1, 3, "uniform"),
    ("ragged_r5", 5, 37, 128, 40, 4, 3, "uniform"),
    ("ragged_256x224", 3, 300, 192, 520, 2, 0, "normal"),
    ("r2_128x256", 2, 256, 512, 264, 1, 2, "uniform"),
    ("r1_128x224", 1, 200, 128, 232, 0, 1, "uniform"),
    ("r8_128x224", 8, 96, 320, 448, 6, 1, "normal"),
    ("ragged_256x256", 3, 300, 256, 600, 1, 4, "uniform"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_ag_gemm_small_full(ocg, case):
    name, R, m, K, N, local, tile, dist = case
    x = workloads.make_ag_gemm(R, m, K, N, seed=100 + R * 7 + local, dist=dist,
                               scale=1.0 if dist == "uniform" else 0.02)
    say("ag_gemm", name, R, m, K, N, local, tile)
    c, ag = run(ocg, x, local, ocg.default_config(tile=tile))
    a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
    assert np.array_equal(to_bits(ag), a_full), "gathered buffer must be a bit-exact copy"
    assert_gate(to_bits(c), want, name)
    ws = ocg.Workspace.cached(ocg.OP_AG_GEMM, R, m, K, N)
    ws.check()


def _check_trace(ocg, x, local, cfg, recs):
    info = ocg.plan_info(ocg.OP_AG_GEMM, x.R, local, x.m, x.K, x.N, cfg)
    plan = sch.ag_gemm_plan(x.R, x.m, x.K, x.N, local, info["BM"], info["BN"], info["slab_rows"],
                            info["copy_rows"], bool(cfg.swizzle), ["fused", "gemm_only", "copy_only"][cfg.mode])
    assert len(recs) == len(plan)
    assert np.array_equal(recs["ticket"], np.arange(len(plan))), "every ticket executed exactly once"
    epoch = int(recs["epoch"][0])
    assert (recs["epoch"] == epoch).all()
    publish = {}
    for t, r in zip(plan, recs):
        if isinstance(t, sch.CopyTask):
            assert (r["kind"], r["a"], r["b"], r["c"]) == (1, t.chunk, t.piece, t.slab)
            if r["d"]:
                assert t.slab not in publish, "a slab is published once"
                publish[t.slab] = int(r["t_ready"])
    for t, r in zip(plan, recs):
        if isinstance(t, sch.Tile):
            assert (r["kind"], r["a"], r["b"], r["c"]) == (2, t.rb, t.cb, len(t.deps))
            assert int(r["queue"]) == (t.queue << 16) | t.qticket, "tile taken from its XCD queue"
            if t.deps:
                assert r["flag_seen"] == epoch, "the tile saw its flag at this call's epoch"
                # consumed only after every slab it reads was published
                assert int(r["t_ready"]) >= max(publish[s] for s in t.deps)
    tgt = sch.slab_targets(x.R, x.m, info["slab_rows"], info["copy_rows"])
    if cfg.mode != 1:
        assert sorted(publish) == [s for s, n in enumerate(tgt) if n]


@pytest.mark.parametrize("local,swizzle", [(0, 1), (2, 1), (1, 0)])
def test_ag_gemm_trace_matches_schedule(ocg, local, swizzle):
    x = workloads.make_ag_gemm(4, 200, 128, 456, seed=77, dist="uniform", scale=1.0)
    cfg = ocg.default_config(tile=ocg.TILE_128x224, swizzle=swizzle)
    info = ocg.plan_info(ocg.OP_AG_GEMM, x.R, local, x.m, x.K, x.N, cfg)
    n = info["n_copy_or_strips"] + info["n_tiles"]
    tr = Trace(n + 8)
    tr.attach(cfg)
    say("ag_gemm trace", local, swizzle)
    c, ag = run(ocg, x, local, cfg)
    recs = tr.read(n)
    _check_trace(ocg, x, local, cfg, recs)
    assert_gate(to_bits(c), oracle.ag_gemm(x.a_chunks, x.b)[1], "trace case")


def test_ag_gemm_modes_and_repeated_epochs(ocg):
    x = workloads.make_ag_gemm(4, 256, 256, 448, seed=5, dist="uniform", scale=1.0)
    chunks = [to_dev(c) for c in x.a_chunks]
    a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
    ag = poison((x.R * x.m, x.K))
    say("ag_gemm copy_only")
    ocg.ag_gemm(chunks, to_dev(x.b), 1, a_gathered=ag, config=ocg.default_config(mode=ocg.MODE_COPY_ONLY))
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(ag), a_full)
    say("ag_gemm gemm_only")
    c_g, _ = ocg.ag_gemm(chunks, to_dev(x.b), 1, a_gathered=ag, config=ocg.default_config(mode=ocg.MODE_GEMM_ONLY))
    say("ag_gemm fused")
    c_f, _ = ocg.ag_gemm(chunks, to_dev(x.b), 1, a_gathered=poison((x.R * x.m, x.K)))
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(c_g), to_bits(c_f)), "same tiles, same arithmetic"
    assert_gate(to_bits(c_f), want, "fused")
    # several calls in a row on one workspace (epoch-tagged flags, no reset)
    for i in range(4):
        b2 = workloads.make_ag_gemm(4, 256, 256, 448, seed=50 + i, dist="uniform", scale=1.0).b
        say("ag_gemm repeat", i)
        c2, ag2 = ocg.ag_gemm(chunks, to_dev(b2), i % 4, a_gathered=poison((x.R * x.m, x.K)))
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(ag2), a_full)
        assert_gate(to_bits(c2), oracle.ag_gemm(x.a_chunks, b2)[1], f"repeat {i}")
    ocg.Workspace.cached(ocg.OP_AG_GEMM, 4, 256, 256, 448).check()


def test_ag_gemm_timeout_is_reported_not_hung(ocg):
    """The host forces a slab whose flag is never published and a 2 ms wait
    bound: the kernel still drains, and ocg_check reports the timeout."""
    x = workloads.make_ag_gemm(4, 128, 128, 224, seed=9, dist="uniform", scale=1.0)
    ws = ocg.Workspace(ocg.OP_AG_GEMM, 4, 128, 128, 224)
    # 128-row slabs, one per chunk here: slab 2 is rank 2's chunk (a peer of rank 0)
    cfg = ocg.default_config(fault_skip_slab=2, spin_timeout_us=2000)
    say("ag_gemm forced timeout")
    ocg.ag_gemm([to_dev(c) for c in x.a_chunks], to_dev(x.b), 0, workspace=ws, config=cfg)
    with pytest.raises(ocg.OcgError) as ei:
        ws.check()
    assert ei.value.code == ocg.ERR_TIMEOUT
    say("ag_gemm after timeout")
    c, ag = ocg.ag_gemm([to_dev(c) for c in x.a_chunks], to_dev(x.b), 0, workspace=ws,
                        a_gathered=poison((512, 128)))
    ws.check()
    assert_gate(to_bits(c), oracle.ag_gemm(x.a_chunks, x.b)[1], "after timeout")


def _sampled(ocg, name, local=0, nrows=96, ncols=96):
    w = workloads.workload(name)
    x = w.make()
    say("ag_gemm", name, "generate done")
    c, ag = run(ocg, x, local)
    a_full = np.concatenate(x.a_chunks)
    assert np.array_equal(to_bits(ag), a_full), "gathered buffer bit-exact"
    rng = np.random.default_rng(1234)
    M = x.R * x.m
    # rows from every rank chunk and both ends; columns across every column tile
    rows = np.unique(np.concatenate([rng.integers(0, M, nrows), [0, M - 1], np.arange(x.R) * x.m]))
    cols = np.unique(np.concatenate([rng.integers(0, x.N, ncols), [0, x.N - 1]]))
    cb = to_bits(c)
    assert not np.isnan(oracle.decode_bf16(cb[rows])).any()
    want = oracle.ag_gemm_block(x.a_chunks, x.b, rows, cols)
    st = assert_gate(cb[np.ix_(rows, cols)], want, name)
    # whole-matrix property at full size: ABFT column checksum of C against
    # (1^T A_full) B, both in float64 (C carries bf16 rounding: loose bound)
    csum = oracle.decode_bf16(cb).sum(axis=0)
    wsum = oracle.decode_bf16(a_full).sum(axis=0) @ oracle.decode_bf16(x.b)
    scale = np.sqrt(M) * st["rms_ref"]
    assert np.all(np.abs(csum - wsum) <= 2e-2 * np.maximum(1.0, scale) + 2.0 ** -8 * np.abs(wsum))
    return st


def test_ag_gemm_8b_share(ocg):
    _sampled(ocg, "ag_gemm_8b")


@pytest.mark.parametrize("local", [0, 5])
def test_ag_gemm_70b_share(ocg, local):
    _sampled(ocg, "ag_gemm_70b", local=local)
