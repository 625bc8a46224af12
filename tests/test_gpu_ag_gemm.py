"""GPU parity of the fused AllGather-GEMM against the float64 oracle, through
the C ABI: small and ragged shapes in full for both transfer modes (copy
tasks inline in the GEMM kernel, or a side producer kernel co-resident with
it) and several K-slab widths, the 8B- and 70B-class shares on every output
element, the gathered buffer bit for bit, the schedule trace against the
oracle's re-derivation, forced late publishes (tiles that really wait, also
inside their K loop), split K (tiles as two K halves: bit-stable across
calls, one writer per tile, within a bf16 step of whole tiles), the
measurement modes, and the timeout path."""
import numpy as np
import pytest
import torch

import oracle
from oracle import schedule as sch
import workloads
from gpu_util import Trace, assert_gate, poison, say, to_bits, to_dev

pytestmark = pytest.mark.gpu

INLINE, SIDE = 0, 1


def run(ocg, x, local=0, cfg=None):
    chunks = [to_dev(c) for c in x.a_chunks]
    b = to_dev(x.b)
    ag = poison((x.R * x.m, x.K))           # any early read of an unfilled slab shows up as NaN
    c = poison((x.R * x.m, x.N))
    ocg.ag_gemm(chunks, b, local, a_gathered=ag, c=c, config=cfg)
    torch.cuda.synchronize()
    return c, ag


SMALL = [
    # name, R, m, K, N, local, tile, dist, kslab
    ("tiny_l0", 4, 128, 256, 256, 0, -1, "uniform", 0),
    ("tiny_l3", 4, 128, 256, 256, 3, -1, "uniform", 0),
    ("ragged_128x128", 3, 100, 64, 72, 1, 3, "uniform", 0),
    ("ragged_r5", 5, 37, 128, 40, 4, 3, "uniform", 0),
    ("ragged_256x224", 3, 300, 192, 520, 2, 0, "normal", 0),
    ("r2_128x256", 2, 256, 512, 264, 1, 2, "uniform", 0),
    ("r1_128x224", 1, 200, 128, 232, 0, 1, "uniform", 0),
    ("r8_128x224", 8, 96, 320, 448, 6, 1, "normal", 0),
    ("ragged_256x256", 3, 300, 256, 600, 1, 4, "uniform", 0),
    # several K-slabs (the last one ragged in the second case)
    ("kslab4_128x224", 4, 200, 1024, 456, 1, 1, "normal", 256),
    ("kslab3_256x224", 3, 300, 1280, 520, 2, 0, "normal", 512),
    ("kslab_256x256", 2, 260, 768, 264, 0, 4, "uniform", 256),
]


@pytest.mark.parametrize("transfer", [INLINE, SIDE], ids=["inline", "side"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_ag_gemm_small_full(ocg, case, transfer):
    name, R, m, K, N, local, tile, dist, kslab = case
    x = workloads.make_ag_gemm(R, m, K, N, seed=100 + R * 7 + local, dist=dist,
                               scale=1.0 if dist == "uniform" else 0.02)
    say("ag_gemm", name, R, m, K, N, local, tile, "transfer", transfer, "kslab", kslab)
    cfg = ocg.default_config(tile=tile, transfer=transfer, kslab_cols=kslab)
    c, ag = run(ocg, x, local, cfg)
    a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
    assert np.array_equal(to_bits(ag), a_full), "gathered buffer must be a bit-exact copy"
    assert_gate(to_bits(c), want, name)
    ws = ocg.Workspace.cached(ocg.OP_AG_GEMM, R, m, K, N, config=cfg)
    ws.check()


def _check_trace(ocg, x, local, cfg, recs):
    h = ocg.handle()
    info = ocg.plan_info(ocg.OP_AG_GEMM, x.R, local, x.m, x.K, x.N, cfg, handle=h)
    ag = ocg.plan_ag(x.R, local, x.m, x.K, x.N, cfg, handle=h)
    plan = sch.ag_gemm_plan(x.R, x.m, x.K, x.N, local, info["BM"], info["BN"], info["slab_rows"],
                            info["copy_rows"], bool(cfg.swizzle), ["fused", "gemm_only", "copy_only"][cfg.mode],
                            KS=ag["kslab_cols"], xcd_remap=bool(cfg.xcd_remap), rpr=ag["rows_per_round"],
                            sk=ag["split_k"])
    nks = ag["nks"]
    assert len(recs) == len(plan)
    assert np.array_equal(recs["ticket"], np.arange(len(plan))), "every ticket executed exactly once"
    epoch = int(recs["epoch"][0])
    assert (recs["epoch"] == epoch).all()
    publish = {}
    for t, r in zip(plan, recs):
        if isinstance(t, sch.CopyTask):
            assert (r["kind"], r["a"], r["b"], r["c"], r["queue"]) == (1, t.chunk, t.piece, t.flag, t.kslab)
            # tickets below n_inline run in the GEMM kernel, the rest in the side producer
            assert bool(r["d"] & 2) == (t.ticket >= ag["n_inline"])
            if r["d"] & 1:
                assert t.flag not in publish, "a flag is published once"
                publish[t.flag] = int(r["t_ready"])
    writers = {}
    for t, r in zip(plan, recs):
        if isinstance(t, sch.Tile):
            assert (r["kind"], r["a"], r["b"], r["c"]) == (2, t.rb, t.cb, len(t.deps))
            assert int(r["queue"]) == (t.queue << 16) | t.qticket, "tile taken from its queue"
            # d: bit 0 the K part; bit 1 (split units) this half combined and wrote the tile
            assert int(r["d"]) & 1 == t.part
            writers[(t.rb, t.cb)] = writers.get((t.rb, t.cb), 0) + (1 if ag["split_k"] == 1 else int(r["d"]) >> 1)
            if t.deps:
                assert r["flag_seen"] == epoch, "the tile saw its flag at this call's epoch"
                # started on its first K-slab only after every slab it reads published it
                assert int(r["t_ready"]) >= max(publish[s * nks] for s in t.deps)
                # and finished after every K-slab of them was published
                assert int(r["t_end"]) >= max(publish[s * nks + j] for s in t.deps for j in range(nks))
    if cfg.mode != 2:
        assert len(writers) == info["n_tiles"] and set(writers.values()) == {1}, "each tile written once"
    tgt = sch.slab_targets(x.R, x.m, info["slab_rows"], info["copy_rows"])
    if cfg.mode != 1:
        assert sorted(publish) == sorted(s * nks + j for s, n in enumerate(tgt) if n for j in range(nks))
    return ag


@pytest.mark.parametrize("local,swizzle,transfer,kslab,xcd", [(0, 1, INLINE, 0, 1), (2, 1, INLINE, 0, 1),
                                                               (1, 0, INLINE, 0, 1), (0, 1, SIDE, 256, 1),
                                                               (3, 1, SIDE, 0, 1), (1, 1, INLINE, 256, 0),
                                                               (2, 0, SIDE, 512, 0)])
def test_ag_gemm_trace_matches_schedule(ocg, local, swizzle, transfer, kslab, xcd):
    x = workloads.make_ag_gemm(4, 200, 1024, 456, seed=77, dist="uniform", scale=1.0)
    cfg = ocg.default_config(tile=ocg.TILE_128x224, swizzle=swizzle, transfer=transfer, kslab_cols=kslab,
                             xcd_remap=xcd)
    info = ocg.plan_info(ocg.OP_AG_GEMM, x.R, local, x.m, x.K, x.N, cfg)
    n = info["n_copy_or_strips"] + info["n_tiles"] * ocg.plan_ag(x.R, local, x.m, x.K, x.N, cfg)["split_k"]
    tr = Trace(n + 8)
    tr.attach(cfg)
    say("ag_gemm trace", local, swizzle, transfer, kslab, xcd)
    c, ag = run(ocg, x, local, cfg)
    recs = tr.read(n)
    _check_trace(ocg, x, local, cfg, recs)
    assert_gate(to_bits(c), oracle.ag_gemm(x.a_chunks, x.b)[1], "trace case")
    assert np.array_equal(to_bits(ag), np.concatenate(x.a_chunks))


SPLIT = [
    # name, R, m, K, N, local, tile
    ("split_256x224", 3, 300, 512, 520, 2, 0),
    ("split_128x128", 5, 37, 256, 40, 4, 3),
    ("split_256x256", 2, 260, 768, 264, 0, 4),
    ("split_128x256", 2, 256, 512, 264, 1, 2),
    ("split_r1_128x224", 1, 200, 128, 232, 0, 1),
]


def _close_to(a_bits, b_bits, what):
    """Two bf16 results of one product summed in another fp32 order: equal
    but for last-bit rounding differences -- one bf16 step, or, for results
    near zero (where the fp32 sums' own rounding, ~1e-8 here, exceeds a step),
    a floor of 2^-16 of the outputs' RMS."""
    a, b = oracle.decode_bf16(a_bits), oracle.decode_bf16(b_bits)
    floor = 2.0 ** -16 * float(np.sqrt(np.mean(b.astype(np.float64) ** 2)))
    step = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + floor
    assert np.all(np.abs(a - b) <= step), f"{what}: more than one bf16 step apart"
    assert np.mean(a != b) < 0.05, f"{what}: {np.mean(a != b):.3f} of the outputs differ"


@pytest.mark.parametrize("case", SPLIT, ids=[c[0] for c in SPLIT])
def test_ag_gemm_split_k(ocg, case):
    """Every tile as two K halves (split_k = 2): the gathered buffer bit for
    bit, C within the gate of the float64 oracle, the same bits on repeated
    calls (the halves' fp32 sums add the same whichever half finishes first),
    and within a bf16 step of the unsplit kernel's C."""
    name, R, m, K, N, local, tile = case
    x = workloads.make_ag_gemm(R, m, K, N, seed=400 + R * 7 + local, dist="normal", scale=0.02)
    split = ocg.default_config(tile=tile, split_k=2)
    assert ocg.plan_ag(R, local, m, K, N, split)["split_k"] == 2
    a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
    outs = []
    for i in range(3):
        say("ag_gemm split", name, "call", i)
        c, ag = run(ocg, x, local, split)
        assert np.array_equal(to_bits(ag), a_full), "gathered buffer must be a bit-exact copy"
        outs.append(to_bits(c))
    assert_gate(outs[0], want, name)
    assert all(np.array_equal(o, outs[0]) for o in outs[1:]), "split-K output must not depend on timing"
    say("ag_gemm unsplit", name)
    c1, _ = run(ocg, x, local, ocg.default_config(tile=tile, split_k=1))
    _close_to(outs[0], to_bits(c1), name)
    ocg.Workspace.cached(ocg.OP_AG_GEMM, R, m, K, N, config=split).check()


def test_ag_gemm_split_k_back_to_back_and_trace(ocg):
    """Split calls back to back on one workspace with no host synchronisation
    (every tile's arrival count returns to zero and its flag carries the
    call's epoch), a traced call against the schedule oracle (each tile's two
    halves, exactly one of them writing the tile), and GEMM-only against
    fused (same units, same arithmetic)."""
    x = workloads.make_ag_gemm(4, 200, 1024, 456, seed=78, dist="normal", scale=0.02)
    chunks = [to_dev(a) for a in x.a_chunks]
    b = to_dev(x.b)
    cfg = ocg.default_config(tile=ocg.TILE_128x224, split_k=2)
    ws = ocg.Workspace(ocg.OP_AG_GEMM, x.R, x.m, x.K, x.N, config=cfg)
    a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
    c = poison((x.R * x.m, x.N))
    say("ag_gemm split back to back")
    for i in range(8):
        ocg.ag_gemm(chunks, b, i % 4, a_gathered=poison((x.R * x.m, x.K)), c=c, workspace=ws, config=cfg)
    ws.check()
    assert_gate(to_bits(c), want, "split back to back")
    info = ocg.plan_info(ocg.OP_AG_GEMM, x.R, 1, x.m, x.K, x.N, cfg)
    n = info["n_copy_or_strips"] + 2 * info["n_tiles"]
    tr = Trace(n + 8)
    tr.attach(cfg)
    say("ag_gemm split trace")
    ag = poison((x.R * x.m, x.K))
    c_t, _ = ocg.ag_gemm(chunks, b, 1, a_gathered=ag, workspace=ws, config=cfg)
    torch.cuda.synchronize()
    recs = tr.read(n)
    ws.check()
    assert _check_trace(ocg, x, 1, cfg, recs)["split_k"] == 2
    assert np.array_equal(to_bits(ag), a_full)
    say("ag_gemm split gemm only")
    c_g, _ = ocg.ag_gemm(chunks, b, 1, a_gathered=ag, workspace=ws,
                         config=ocg.default_config(tile=ocg.TILE_128x224, split_k=2, mode=ocg.MODE_GEMM_ONLY))
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(c_g), to_bits(c_t)), "same units, same arithmetic"


@pytest.mark.parametrize("transfer", [INLINE, SIDE], ids=["inline", "side"])
def test_ag_gemm_late_publishes_make_tiles_wait(ocg, transfer):
    """Forced late publishes (copy_delay): a copy task of K-slab j sleeps
    (j + 1) x 24 rounds of s_sleep 127 (~0.1 ms per round of K-slabs) before
    moving data, so tiles that read peer rows must wait at their start and
    again inside their K loop; buffers start poisoned with NaN, so any read
    before a publish would show in the output."""
    x = workloads.make_ag_gemm(4, 256, 1024, 448, seed=31, dist="normal", scale=0.02)
    cfg = ocg.default_config(tile=ocg.TILE_128x224, transfer=transfer, kslab_cols=256, copy_delay=24)
    info = ocg.plan_info(ocg.OP_AG_GEMM, x.R, 0, x.m, x.K, x.N, cfg)
    n = info["n_copy_or_strips"] + info["n_tiles"]
    tr = Trace(n + 8)
    tr.attach(cfg)
    say("ag_gemm late publishes", transfer)
    c, ag = run(ocg, x, 0, cfg)
    recs = tr.read(n)
    ocg.Workspace.cached(ocg.OP_AG_GEMM, x.R, x.m, x.K, x.N, config=cfg).check()
    a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
    assert np.array_equal(to_bits(ag), a_full)
    assert_gate(to_bits(c), want, "late publishes")
    ag_plan = _check_trace(ocg, x, 0, cfg, recs)
    assert ag_plan["nks"] == 4
    tiles = recs[recs["kind"] == 2]
    dep = tiles[tiles["c"] > 0]
    assert len(dep) > 0
    copies = recs[recs["kind"] == 1]
    t_first_pub = int(copies["t_ready"].min())
    # every dependent tile waited for its first K-slab: it saw it only after a publish
    assert (dep["t_ready"] >= t_first_pub).all()
    if transfer == SIDE:
        # the side producer runs beside the tiles: dependent tiles start before the
        # first publish and spin, and later K-slabs arrive while they compute
        assert (dep["t_ready"] - dep["t_start"]).max() > 2000, "tiles spun at their start (>20 us)"
        assert (dep["wait_ticks"] > 0).any(), "some tile waited inside its K loop"


def test_ag_gemm_modes_and_repeated_epochs(ocg):
    x = workloads.make_ag_gemm(4, 256, 256, 448, seed=5, dist="uniform", scale=1.0)
    chunks = [to_dev(c) for c in x.a_chunks]
    a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
    for transfer in (INLINE, SIDE):
        ag = poison((x.R * x.m, x.K))
        say("ag_gemm copy_only", transfer)
        ocg.ag_gemm(chunks, to_dev(x.b), 1, a_gathered=ag,
                    config=ocg.default_config(mode=ocg.MODE_COPY_ONLY, transfer=transfer))
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(ag), a_full)
    say("ag_gemm gemm_only")
    c_g, _ = ocg.ag_gemm(chunks, to_dev(x.b), 1, a_gathered=ag, config=ocg.default_config(mode=ocg.MODE_GEMM_ONLY))
    say("ag_gemm fused")
    c_f, _ = ocg.ag_gemm(chunks, to_dev(x.b), 1, a_gathered=poison((x.R * x.m, x.K)))
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(c_g), to_bits(c_f)), "same tiles, same arithmetic"
    assert_gate(to_bits(c_f), want, "fused")
    # several calls in a row on one workspace (epoch-tagged flags, no reset),
    # alternating the transfer modes
    for i in range(6):
        b2 = workloads.make_ag_gemm(4, 256, 256, 448, seed=50 + i, dist="uniform", scale=1.0).b
        say("ag_gemm repeat", i)
        c2, ag2 = ocg.ag_gemm(chunks, to_dev(b2), i % 4, a_gathered=poison((x.R * x.m, x.K)),
                              config=ocg.default_config(transfer=i % 2))
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(ag2), a_full)
        assert_gate(to_bits(c2), oracle.ag_gemm(x.a_chunks, b2)[1], f"repeat {i}")
    ocg.Workspace.cached(ocg.OP_AG_GEMM, 4, 256, 256, 448).check()


def test_ag_gemm_side_stream_ordering(ocg):
    """A call on a non-default stream with a fresh workspace: the clear and
    the call are ordered on that stream, and the caller's stream waits for
    the side producer (the gathered buffer is complete for the next op)."""
    x = workloads.make_ag_gemm(3, 160, 512, 256, seed=12, dist="uniform", scale=1.0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        chunks = [to_dev(c) for c in x.a_chunks]
        b = to_dev(x.b)
        ag = poison((x.R * x.m, x.K))
        say("ag_gemm on a side stream")
        c, _ = ocg.ag_gemm(chunks, b, 2, a_gathered=ag, stream=s, config=ocg.default_config(transfer=SIDE))
        snap = ag.clone()        # on s, after the call: must see every gathered row
    torch.cuda.synchronize()
    a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
    assert np.array_equal(to_bits(snap), a_full)
    assert_gate(to_bits(c), want, "side stream")


def test_ag_gemm_transfers_back_to_back(ocg):
    """Calls of both transfer modes and every measurement mode on one
    workspace, back to back on one stream with timing events between them
    and no host synchronisation (the bench's pattern): no wait times out, and
    the last call's outputs are right."""
    x = workloads.workload("ag_gemm_70b").make()
    chunks = [to_dev(a) for a in x.a_chunks]
    b = to_dev(x.b)
    ag = poison((x.R * x.m, x.K))
    c = poison((x.R * x.m, x.N))
    ws = ocg.Workspace(ocg.OP_AG_GEMM, x.R, x.m, x.K, x.N)
    s = torch.cuda.current_stream()
    D = ocg.default_config
    seq = [D(), D(transfer=SIDE), D(mode=ocg.MODE_COPY_ONLY, transfer=SIDE), D(mode=ocg.MODE_GEMM_ONLY),
           D(transfer=SIDE), D(mode=ocg.MODE_COPY_ONLY), D(), D(transfer=SIDE)] * 3
    say("ag_gemm back to back", len(seq), "calls")
    for cf in seq:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        ocg.ag_gemm(chunks, b, 0, a_gathered=ag, c=c, workspace=ws, config=cf)
        e1.record(s)
    ws.check()
    a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
    assert np.array_equal(to_bits(ag), a_full)
    assert_gate(to_bits(c), want, "back to back")


def test_ag_gemm_timeout_is_reported_not_hung(ocg):
    """The host forces a flag that is never published and a 2 ms wait
    bound: the kernel still drains, and ocg_check reports the timeout."""
    x = workloads.make_ag_gemm(4, 128, 128, 224, seed=9, dist="uniform", scale=1.0)
    for transfer in (INLINE, SIDE):
        ws = ocg.Workspace(ocg.OP_AG_GEMM, 4, 128, 128, 224)
        # 128-row slabs, one K-slab: flag 2 is rank 2's chunk (a peer of rank 0)
        cfg = ocg.default_config(fault_skip_slab=2, spin_timeout_us=2000, transfer=transfer)
        say("ag_gemm forced timeout", transfer)
        ocg.ag_gemm([to_dev(c) for c in x.a_chunks], to_dev(x.b), 0, workspace=ws, config=cfg)
        with pytest.raises(ocg.OcgError) as ei:
            ws.check()
        assert ei.value.code == ocg.ERR_TIMEOUT
        say("ag_gemm after timeout", transfer)
        c, ag = ocg.ag_gemm([to_dev(c) for c in x.a_chunks], to_dev(x.b), 0, workspace=ws,
                            a_gathered=poison((512, 128)), config=ocg.default_config(transfer=transfer))
        ws.check()
        assert_gate(to_bits(c), oracle.ag_gemm(x.a_chunks, x.b)[1], "after timeout")


def _full(ocg, name, local=0, cfg=None):
    w = workloads.workload(name)
    x = w.make()
    say("ag_gemm", name, "local", local, "generate done")
    c, ag = run(ocg, x, local, cfg)
    a_full = np.concatenate(x.a_chunks)
    assert np.array_equal(to_bits(ag), a_full), "gathered buffer bit-exact"
    cb = to_bits(c)
    say("ag_gemm", name, "oracle")
    _, want = oracle.ag_gemm(x.a_chunks, x.b)
    # the gate and the tight diagnostics on every output element
    st = assert_gate(cb, want, name)
    # whole-matrix property: ABFT column checksum of C against (1^T A_full) B
    csum = oracle.decode_bf16(cb).sum(axis=0)
    wsum = oracle.decode_bf16(a_full).sum(axis=0) @ oracle.decode_bf16(x.b)
    scale = np.sqrt(x.R * x.m) * st["rms_ref"]
    assert np.all(np.abs(csum - wsum) <= 2e-2 * np.maximum(1.0, scale) + 2.0 ** -8 * np.abs(wsum))
    return st


def test_ag_gemm_8b_share(ocg):
    _full(ocg, "ag_gemm_8b")


@pytest.mark.parametrize("local", [0, 5])
def test_ag_gemm_70b_share(ocg, local):
    """The headline configuration in the launch configuration bench.py times
    (default config)."""
    _full(ocg, "ag_gemm_70b", local=local)


def test_ag_gemm_70b_share_side(ocg):
    _full(ocg, "ag_gemm_70b", local=3, cfg=ocg.default_config(transfer=SIDE))


def test_ag_plan_on_device_matches_host_plan(ocg):
    """The host-only planning queries (no handle: a 256-CU MI355X) resolve the
    same plan as the device's handle for the configured shapes."""
    h = ocg.handle()
    for (R, m, K, N) in [(8, 1024, 8192, 3584), (8, 512, 4096, 1792), (4, 128, 256, 256)]:
        assert ocg.plan_ag(R, 0, m, K, N) == ocg.plan_ag(R, 0, m, K, N, handle=h)
        assert ocg.plan_info(ocg.OP_AG_GEMM, R, 0, m, K, N) == ocg.plan_info(ocg.OP_AG_GEMM, R, 0, m, K, N, handle=h)
