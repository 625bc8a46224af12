"""GPU parity of the AllGather-KV attention: the gathered keys and values bit
for bit, the output against the float64 oracle (every element at small sizes,
sampled rows at the 16K-context GQA share), retrieval-structured inputs in
which any key / value mix-up is an O(1) error, the copy / compute modes,
repeated calls, the schedule trace and the timeout path."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Trace, assert_gate, poison, say, to_bits, to_dev

pytestmark = pytest.mark.gpu

D = 128


def run(ocg, x, cfg=None, ws=None):
    q = to_dev(x.q)
    ks = [to_dev(c) for c in x.k_chunks]
    vs = [to_dev(c) for c in x.v_chunks]
    S = x.R * x.m
    kg = poison((S, x.Hkv, D))
    vg = poison((S, x.Hkv, D))
    out = poison((x.m, x.Hq, D))
    ocg.ag_attention(q, ks, vs, x.local_rank, k_gathered=kg, v_gathered=vg, out=out, config=cfg, workspace=ws)
    torch.cuda.synchronize()
    return to_bits(out), to_bits(kg), to_bits(vg)


def check(x, out, kg, vg, name):
    kf, vf, want = oracle.ag_attention(x.q, x.k_chunks, x.v_chunks)
    assert np.array_equal(kg, kf), f"{name}: gathered keys differ"
    assert np.array_equal(vg, vf), f"{name}: gathered values differ"
    # The probabilities enter the value product rounded to bf16 (relative
    # error <= 2^-9 each): |error| <= 2^-9 * sum_j p_j |v_j| per element,
    # which is the attention of the same scores over |V| (sign bit cleared).
    _, _, absv = oracle.ag_attention(x.q, x.k_chunks, [c & np.uint16(0x7FFF) for c in x.v_chunks])
    return assert_gate(out, want, name, extra=2.0 ** -8 * absv)


CASES = [
    # name, R, m, Hq, Hkv, local
    ("r3_g4_ragged", 3, 100, 8, 2, 1),
    ("r2_mha", 2, 128, 2, 2, 0),
    ("r4_g8", 4, 64, 16, 2, 3),
    ("r2_g16", 2, 80, 16, 1, 1),
    ("r3_g3", 3, 70, 6, 2, 2),
    ("r1", 1, 96, 4, 1, 0),
    ("r8_short_chunks", 8, 32, 8, 8, 5),
    ("r2_one_token", 2, 1, 4, 4, 1),
    ("r5_two_tiles", 5, 130, 4, 1, 4),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ag_attention_small(ocg, case):
    name, R, m, Hq, Hkv, local = case
    x = workloads.make_attention(R, m, Hq, Hkv, D, seed=600 + R + m, local_rank=local)
    say("ag_attention", name)
    check(x, *run(ocg, x), name)


@pytest.mark.parametrize("case", CASES[:5], ids=[c[0] for c in CASES[:5]])
def test_ag_attention_retrieval(ocg, case):
    """Every query is 4x one gathered key of its kv head: the output is that
    key's value row (to far below a bf16 ulp), so a key read from the wrong
    chunk, row or head, or a value paired with the wrong key, is an O(1)
    error."""
    name, R, m, Hq, Hkv, local = case
    x, targets = workloads.make_attention_retrieval(R, m, Hq, Hkv, D, seed=650 + R, local_rank=local)
    say("ag_attention retrieval", name)
    out, kg, vg = run(ocg, x)
    check(x, out, kg, vg, name + " retrieval")
    v_full = oracle.decode_bf16(np.concatenate(x.v_chunks))
    picked = v_full[targets, (np.arange(Hq) // (Hq // Hkv))[None, :], :]
    got = oracle.decode_bf16(out)
    assert np.all(np.abs(got - picked) <= 2.0 ** -8 * np.abs(picked) + 1e-6), name


@pytest.mark.parametrize("opts", [dict(swizzle=0), dict(slab_rows=16, copy_rows=8), dict(grid=3),
                                  dict(slab_rows=32, grid=7, swizzle=0)],
                         ids=["natural_order", "small_slabs", "grid3", "slabs_grid7_natural"])
def test_ag_attention_configs(ocg, opts):
    x = workloads.make_attention(4, 96, 8, 2, D, seed=660, local_rank=2)
    say("ag_attention config", opts)
    check(x, *run(ocg, x, ocg.default_config(**opts)), str(opts))


def test_ag_attention_modes_and_repeated_calls(ocg):
    x = workloads.make_attention(4, 128, 8, 2, D, seed=670, local_rank=1)
    kf, vf, want = oracle.ag_attention(x.q, x.k_chunks, x.v_chunks)
    q = to_dev(x.q)
    ks = [to_dev(c) for c in x.k_chunks]
    vs = [to_dev(c) for c in x.v_chunks]
    kg, vg = poison((512, 2, D)), poison((512, 2, D))
    out_c = poison((128, 8, D))
    say("ag_attention copy_only")
    ocg.ag_attention(q, ks, vs, 1, k_gathered=kg, v_gathered=vg, out=out_c,
                     config=ocg.default_config(mode=ocg.MODE_COPY_ONLY))
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(kg), kf) and np.array_equal(to_bits(vg), vf)
    assert np.isnan(oracle.decode_bf16(to_bits(out_c))).all(), "copy-only leaves the output alone"
    say("ag_attention compute_only")
    out_g, _, _ = ocg.ag_attention(q, ks, vs, 1, k_gathered=kg, v_gathered=vg,
                                   config=ocg.default_config(mode=ocg.MODE_GEMM_ONLY))
    say("ag_attention fused")
    out_f, _, _ = ocg.ag_attention(q, ks, vs, 1, k_gathered=poison((512, 2, D)), v_gathered=poison((512, 2, D)))
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out_g), to_bits(out_f)), "same tiles, same arithmetic"
    # several calls in a row on one workspace (epoch-tagged flags, no reset),
    # each with new values and another local rank
    for i in range(4):
        y = workloads.make_attention(4, 128, 8, 2, D, seed=680 + i, local_rank=i)
        say("ag_attention repeat", i)
        check(y, *run(ocg, y), f"repeat {i}")
    ocg.Workspace.cached(ocg.OP_AG_ATTENTION, 4, 128, 8, 2).check()


def test_ag_attention_trace(ocg):
    """Every copy ticket and tile runs once; a tile waits on the slab flags
    of the R-1 peer chunks; each slab is published by exactly one task."""
    x = workloads.make_attention(3, 200, 8, 2, D, seed=690, local_rank=2)
    cfg = ocg.default_config(slab_rows=64)
    info = ocg.plan_info(ocg.OP_AG_ATTENTION, 3, 2, 200, 8, 2, cfg)
    n_copy, n_tiles, n_slabs = info["n_copy_or_strips"], info["n_tiles"], info["n_slabs_or_strip_rows"]
    assert n_slabs == 3 * 4 and n_tiles == 2 * ((4 * 200 + 255) // 256)
    tr = Trace(n_copy + n_tiles)
    tr.attach(cfg)
    say("ag_attention trace")
    check(x, *run(ocg, x, cfg), "trace")
    recs = tr.read(n_copy + n_tiles)
    assert np.array_equal(recs["ticket"], np.arange(n_copy + n_tiles))
    cp, tl = recs[:n_copy], recs[n_copy:]
    assert (cp["kind"] == 1).all() and (tl["kind"] == 7).all()
    for u, r in enumerate(cp):
        d = ocg.plan_task(ocg.OP_AG_ATTENTION, 3, 2, 200, 8, 2, u, cfg)
        assert (r["a"], r["b"] & 0xFFFF, r["b"] >> 16, r["c"]) == (d[1], d[2], d[6], d[5])
    assert sorted(cp["c"][cp["d"] == 1].tolist()) == list(range(n_slabs)), "one publish per slab"
    assert (tl["c"] == 2 * 4).all(), "each tile waits on the 4 slabs of both peer chunks"
    for v, r in enumerate(tl):
        d = ocg.plan_task(ocg.OP_AG_ATTENTION, 3, 2, 200, 8, 2, n_copy + v, cfg)
        assert (r["a"], r["b"]) == (d[1], d[2])
        assert r["flag_seen"] == r["epoch"]


def test_ag_attention_timeout_is_reported_not_hung(ocg):
    """The host forces a slab whose flag is never published and a 2 ms wait
    bound: every wave's wait ends, the kernel drains, ocg_check reports it."""
    x = workloads.make_attention(4, 64, 4, 1, D, seed=695, local_rank=0)
    ws = ocg.Workspace(ocg.OP_AG_ATTENTION, 4, 64, 4, 1)
    cfg = ocg.default_config(fault_skip_slab=2, spin_timeout_us=2000)   # slab 2 = rank 2's chunk
    say("ag_attention forced timeout")
    run(ocg, x, cfg, ws)
    with pytest.raises(ocg.OcgError) as ei:
        ws.check()
    assert ei.value.code == ocg.ERR_TIMEOUT
    say("ag_attention after timeout")
    check(x, *run(ocg, x, None, ws), "after timeout")
    ws.check()


def _full(ocg, local):
    w = workloads.workload("ag_attention")
    x = w.make()
    x.local_rank = local
    say("ag_attention full share, local", local)
    out, kg, vg = run(ocg, x)
    kf = np.concatenate(x.k_chunks)
    vf = np.concatenate(x.v_chunks)
    assert np.array_equal(kg, kf) and np.array_equal(vg, vf), "gathered keys / values bit-exact"
    assert not np.isnan(oracle.decode_bf16(out)).any()
    rng = np.random.default_rng(77)
    G = x.Hq // x.Hkv
    # rows from every tile position class: first / last query, every head,
    # random others
    rows = [(0, h) for h in range(x.Hq)] + [(x.m - 1, h) for h in range(0, x.Hq, 3)]
    rows += [(int(i), int(h)) for i, h in zip(rng.integers(0, x.m, 64), rng.integers(0, x.Hq, 64))]
    want = oracle.ag_attention_rows(x.q, kf, vf, rows)
    got = np.stack([out[i, h] for i, h in rows])
    absv = oracle.ag_attention_rows(x.q, kf, vf & np.uint16(0x7FFF), rows)
    assert_gate(got, want, f"ag_attention local {local}", extra=2.0 ** -8 * absv)
    assert G == 4


@pytest.mark.parametrize("local", [0, 5])
def test_ag_attention_16k_gqa_share(ocg, local):
    _full(ocg, local)


def test_ag_attention_16k_retrieval_all_rows(ocg):
    """Full-size share with retrieval inputs: every one of the m * Hq output
    rows must equal its target value row (a property that holds at any size,
    so all rows are checked, not a sample)."""
    w = workloads.workload("ag_attention")
    p = w.params
    x, targets = workloads.make_attention_retrieval(p["R"], p["m"], p["Hq"], p["Hkv"], D, seed=699, local_rank=3)
    say("ag_attention full share retrieval")
    out, kg, vg = run(ocg, x)
    v_full = oracle.decode_bf16(np.concatenate(x.v_chunks))
    picked = v_full[targets, (np.arange(x.Hq) // (x.Hq // x.Hkv))[None, :], :]
    got = oracle.decode_bf16(out)
    bad = np.abs(got - picked) > 2.0 ** -8 * np.abs(picked) + 1e-6
    assert not bad.any(), f"{bad.sum()} elements differ from their target value rows"


def test_ag_attention_late_publishes_make_tiles_wait(ocg):
    """Forced late publishes (copy_delay: every copy task first sleeps ~0.1 ms):
    tiles reach their peer keys before the peer chunks land, spin on the slab
    flags, see them only after a publish, and the output stays in the gate
    (gathered buffers start poisoned with NaN)."""
    x = workloads.make_attention(3, 200, 8, 2, D, seed=697, local_rank=1)
    cfg = ocg.default_config(slab_rows=64, copy_delay=24)
    info = ocg.plan_info(ocg.OP_AG_ATTENTION, 3, 1, 200, 8, 2, cfg)
    n_copy, n_tiles = info["n_copy_or_strips"], info["n_tiles"]
    tr = Trace(n_copy + n_tiles)
    tr.attach(cfg)
    say("ag_attention late publishes")
    check(x, *run(ocg, x, cfg), "late publishes")
    recs = tr.read(n_copy + n_tiles)
    cp, tl = recs[:n_copy], recs[n_copy:]
    assert (cp["kind"] == 1).all() and (tl["kind"] == 7).all()
    first_pub = int(cp["t_ready"][cp["d"] == 1].min())
    assert (tl["t_ready"] >= first_pub).all(), "a tile passed its wait before any publish"
    spin = (tl["t_ready"].astype(np.int64) - tl["t_start"].astype(np.int64)).max()
    assert spin > 2000, f"tiles really spun (longest wait {spin / 100:.1f} us, want > 20 us)"
    ocg.Workspace.cached(ocg.OP_AG_ATTENTION, 3, 200, 8, 2).check()
