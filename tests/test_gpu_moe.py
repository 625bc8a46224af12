"""GPU parity of AllGather + MoE routing + grouped GEMM: routing outputs bit
for bit (top-k ids, expert-sorted slot list, offsets), gate weights to 1e-5,
every output row within the gate against the float64 oracle, the gathered
buffer bit for bit, and the lookup-table tiles against the oracle's list."""
import numpy as np
import pytest
import torch

import oracle
from oracle import schedule as sch
import workloads
from gpu_util import Trace, assert_gate, poison, say, to_bits, to_dev

pytestmark = pytest.mark.gpu


def run(ocg, x, local=0, cfg=None, logits=None):
    chunks = [to_dev(c) for c in x.a_chunks]
    lg = torch.from_numpy(np.ascontiguousarray(x.logits if logits is None else logits)).cuda()
    w = to_dev(x.w)
    T = x.R * x.m
    outs = dict(a_gathered=poison((T, x.K)), out=poison((T * x.topk, x.N)))
    o = ocg.ag_grouped_gemm(chunks, lg, w, x.topk, local, config=cfg, outputs=outs)
    torch.cuda.synchronize()
    # no wait of the call (routing counters, slab flags) timed out
    ocg.Workspace.cached(ocg.OP_AG_GROUPED_GEMM, x.R, x.m, x.K, x.N, x.E, x.topk).check()
    return o


def check(ocg, x, o, name, logits=None):
    lg = x.logits if logits is None else logits
    res = oracle.ag_grouped_gemm(x.a_chunks, lg, x.w, x.topk)
    assert np.array_equal(o["topk_ids"].cpu().numpy(), res["ids"]), "top-k ids"
    assert np.array_equal(o["expert_offsets"].cpu().numpy(), res["offsets"]), "expert offsets"
    assert np.array_equal(o["perm"].cpu().numpy(), res["perm"]), "expert-sorted slot list"
    w_gpu = o["topk_w"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(w_gpu - res["weights"]) <= 1e-5 * np.abs(res["weights"]) + 1e-7), "gate weights"
    assert np.array_equal(to_bits(o["a_gathered"]), res["a_full"])
    assert_gate(to_bits(o["out"]), res["out"], name)
    return res


SMALL = [
    # name, R, m, K, N, E, topk, local
    ("r2_e6", 2, 64, 128, 96, 6, 2, 0),
    ("r4_e8_l3", 4, 100, 192, 232, 8, 2, 3),
    ("r3_e5_top1", 3, 50, 64, 40, 5, 1, 1),
    ("r2_e16_top4", 2, 300, 128, 456, 16, 4, 1),
]


TILES = {"auto": -1, "128x224": 1, "256x224": 0, "288x224": 6, "320x224": 5}


@pytest.mark.parametrize("tile", list(TILES))
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_moe_small_full(ocg, case, tile):
    name, R, m, K, N, E, topk, local = case
    x = workloads.make_moe(R, m, K, N, E, seed=300 + E, topk=topk, scale=0.5)
    cfg = ocg.default_config(tile=TILES[tile])
    say("moe", name, tile)
    o = run(ocg, x, local, cfg)
    check(ocg, x, o, name)


def test_moe_rejects_other_presets(ocg):
    x = workloads.make_moe(2, 64, 128, 96, 6, seed=306, topk=2, scale=0.5)
    with pytest.raises(ocg.OcgError):
        run(ocg, x, 0, ocg.default_config(tile=ocg.TILE_128x128))


def test_moe_ties_and_empty_experts(ocg):
    """Planted exact ties (whole rows equal, pairs equal) and experts that no
    token picks: the tie rule (lower expert first) and empty groups."""
    x = workloads.make_moe(2, 96, 64, 72, 8, seed=11, topk=2, scale=0.5)
    lg = x.logits.copy()
    lg[::5] = np.float32(0.5)
    lg[1::3, 6] = lg[1::3, 2]
    lg[:, 7] = np.float32(-30.0)         # expert 7 is never chosen
    say("moe ties")
    o = run(ocg, x, 1, logits=lg)
    check(ocg, x, o, "ties", logits=lg)


def test_moe_lookup_table_tiles(ocg):
    x = workloads.make_moe(4, 128, 128, 448, 8, seed=12, topk=2, scale=0.5)
    cfg = ocg.default_config()
    info = ocg.plan_info(ocg.OP_AG_GROUPED_GEMM, 4, 0, 128, 128, 448, cfg, E=8, topk=2)
    res = oracle.ag_grouped_gemm(x.a_chunks, x.logits, x.w, 2)
    tiles = sch.moe_tiles(res["counts"], res["offsets"], res["perm"], 2, 4, 128, 448, 0, info["BM"],
                          info["BN"], info["slab_rows"])
    n = info["n_copy_or_strips"] + len(tiles)
    tr = Trace(n + 16)
    tr.attach(cfg)
    say("moe trace")
    o = run(ocg, x, 0, cfg)
    recs = tr.read(n)
    assert np.array_equal(recs["ticket"], np.arange(n))
    got = [(int(r["a"]), int(r["b"]), int(r["c"]), int(r["d"]) & 0xFFFF, int(r["d"]) >> 16)
           for r in recs[info["n_copy_or_strips"]:]]
    want = [(e, r0, nr, cb, len(deps)) for e, r0, nr, cb, deps in tiles]
    assert got == want, "grouped tiles follow the lookup table once each"
    check(ocg, x, o, "lut")


@pytest.mark.parametrize("case", [("e64_max_slots", 8, 1024, 2), ("e64_ragged_top3", 5, 1000, 3)],
                         ids=["e64_max_slots", "e64_ragged_top3"])
def test_moe_routing_limits(ocg, case):
    """The routing at its limits: 64 experts (one per lane, E + 1 offsets),
    16384 token slots (the most a call takes), more than 64 routing blocks of
    64 tokens (histograms read in several rounds), a ragged last block."""
    name, R, m, topk = case
    x = workloads.make_moe(R, m, 64, 64, 64, seed=320 + topk, topk=topk, scale=0.5)
    say("moe routing limits", name)
    o = run(ocg, x, R - 1)
    res = check(ocg, x, o, name)
    assert len(res["offsets"]) == 65


def test_moe_repeated_calls_one_workspace(ocg):
    """Calls in a row on one workspace with new logits and values each time
    and other tile presets: the routing (histograms, slot list, lookup table)
    and the slab flags start over every call."""
    for i, tile in enumerate(["128x224", "256x224", "288x224", "320x224", "128x224"]):
        x = workloads.make_moe(3, 160, 128, 232, 8, seed=330 + i, topk=2, scale=0.5)
        say("moe repeat", i, tile)
        o = run(ocg, x, i % 3, ocg.default_config(tile=TILES[tile]))
        check(ocg, x, o, f"repeat {i} {tile}")


def test_moe_full_workload(ocg):
    x = workloads.workload("ag_moe").make()
    say("moe full workload")
    o = run(ocg, x, 0)
    check(ocg, x, o, "ag_moe")


def test_moe_late_publishes_make_tiles_wait(ocg):
    """Forced late publishes (copy_delay: every copy task first sleeps ~0.1 ms):
    grouped tiles whose tokens come from peer ranks spin on the slab flags,
    see them only after a publish, and the results stay exact (buffers start
    poisoned with NaN, so a read before a publish would show)."""
    R, m, K, N, E, topk = 4, 100, 192, 232, 8, 2
    x = workloads.make_moe(R, m, K, N, E, seed=331, topk=topk, scale=0.5)
    cfg = ocg.default_config(copy_delay=24)
    info = ocg.plan_info(ocg.OP_AG_GROUPED_GEMM, R, 1, m, K, N, cfg, E=E, topk=topk)
    n_copy = info["n_copy_or_strips"]
    tr = Trace(n_copy + 4096)
    tr.attach(cfg)
    say("moe late publishes")
    o = run(ocg, x, 1, cfg)
    check(ocg, x, o, "moe late publishes")
    recs = tr.read(n_copy + 4096)
    cp = recs[:n_copy]
    assert (cp["kind"] == 1).all()
    tiles = recs[recs["kind"] == 4]
    tiles = tiles[tiles["epoch"] == cp["epoch"][0]]
    assert len(tiles) > 0
    waited = tiles[(tiles["d"] >> 16) > 0]
    assert len(waited) > 0, "some grouped tile waited on slab flags"
    first_pub = int(cp["t_ready"][cp["d"] & 1 == 1].min())
    assert (waited["t_ready"] >= first_pub).all(), "a tile passed its wait before any publish"
    spin = (waited["t_ready"].astype(np.int64) - waited["t_start"].astype(np.int64)).max()
    assert spin > 2000, f"tiles really spun (longest wait {spin / 100:.1f} us, want > 20 us)"
