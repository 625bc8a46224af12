"""Invariants of the expected schedules (oracle/schedule.py), checked by
brute-force enumeration: every tile exactly once, every gathered row copied
exactly once, every dependency published by tasks with smaller tickets, and
the rotated (swizzled) order starting at the local rank."""
import itertools

import numpy as np
import pytest

from oracle import schedule as sch
import oracle

CASES = [
    # R, m, K, N, local, BM, BN, S, CT
    (4, 128, 256, 256, 0, 128, 224, 128, 32),
    (8, 512, 4096, 1792, 0, 128, 224, 128, 32),
    (8, 1024, 8192, 3584, 0, 256, 224, 256, 16),
    (8, 1024, 8192, 3584, 3, 256, 224, 256, 16),
    (3, 100, 64, 72, 1, 64, 32, 48, 16),      # ragged: m % BM != 0, N % BN != 0
    (5, 37, 32, 40, 4, 32, 32, 32, 8),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("swizzle", [True, False])
def test_ag_gemm_plan_invariants(case, swizzle):
    R, m, K, N, local, BM, BN, S, CT = case
    M = R * m
    plan = sch.ag_gemm_plan(R, m, K, N, local, BM, BN, S, CT, swizzle)
    assert [t.ticket for t in plan] == list(range(len(plan)))
    copies = [t for t in plan if isinstance(t, sch.CopyTask)]
    tiles = [t for t in plan if isinstance(t, sch.Tile)]
    # every gathered row copied exactly once
    rows = np.zeros(M, dtype=np.int64)
    for c in copies:
        rows[c.row0:c.row1] += 1
        assert c.row0 // m == c.chunk and (c.row1 - 1) // m == c.chunk
    assert np.all(rows == 1)
    # every tile exactly once
    n_rb, n_cb = -(-M // BM), -(-N // BN)
    assert sorted((t.rb, t.cb) for t in tiles) == sorted(itertools.product(range(n_rb), range(n_cb)))
    # each slab completes by exactly its target number of copies, all with
    # tickets smaller than any tile that waits on it
    tgt = sch.slab_targets(R, m, S, CT)
    done = {}
    for c in copies:
        done.setdefault(c.slab, []).append(c.ticket)
    assert {s: len(v) for s, v in done.items()} == {s: n for s, n in enumerate(tgt) if n}
    for t in tiles:
        for s in t.deps:
            assert max(done[s]) < t.ticket
            assert s // (-(-m // S)) != local
    # swizzled: the first tile row block contains the local rank's first row,
    # and the first copies are for rank local+1
    if swizzle:
        assert tiles[0].rb * BM <= local * m < (tiles[0].rb + 1) * BM
        if R > 1:
            assert copies[0].chunk == (local + 1) % R
        assert copies[-1].chunk == local
    else:
        assert tiles[0].rb == 0 and copies[0].chunk == 0


def test_ag_gemm_plan_modes():
    args = (4, 128, 256, 256, 1, 128, 224, 128, 32)
    full = sch.ag_gemm_plan(*args)
    g = sch.ag_gemm_plan(*args, mode="gemm_only")
    c = sch.ag_gemm_plan(*args, mode="copy_only")
    assert all(isinstance(t, sch.Tile) and not t.deps for t in g)
    assert all(isinstance(t, sch.CopyTask) for t in c)
    assert len(g) + len(c) == len(full)


@pytest.mark.parametrize("R,M,N,local,BM,BN,RR", [(8, 4096, 4096, 0, 256, 256, 4), (8, 4096, 4096, 5, 256, 256, 4),
                                                  (4, 96, 40, 2, 16, 16, 5), (3, 90, 50, 1, 32, 32, 7)])
def test_gemm_rs_plan_invariants(R, M, N, local, BM, BN, RR):
    plan = sch.gemm_rs_plan(R, M, N, local, BM, BN, RR)
    assert [t[1] for t in plan] == list(range(len(plan)))
    tiles = [t for t in plan if t[0] == "tile"]
    reds = [t for t in plan if t[0] == "reduce"]
    n_rb, n_cb = -(-M // BM), -(-N // BN)
    assert sorted((t[2], t[3]) for t in tiles) == sorted(itertools.product(range(n_rb), range(n_cb)))
    blk = M // R
    assert tiles[0][4]                                 # local row block first
    assert tiles[0][2] * BM <= local * blk < (tiles[0][2] + 1) * BM
    for _, _, rb, cb, loc, _, _ in tiles:
        assert loc == (rb * BM < (local + 1) * blk and min((rb + 1) * BM, M) > local * blk)
    # reduce strips cover the local block exactly once, after the tiles they read
    rows = np.zeros(M, dtype=np.int64)
    tick = {(rb, cb): t for _, t, rb, cb, _, _, _ in tiles}
    for _, t, r0, r1, deps in reds:
        rows[r0:r1] += 1
        need = {(rb, cb) for rb in range(n_rb) for cb in range(n_cb) if rb * BM < r1 and (rb + 1) * BM > r0}
        assert set(deps) == need and all(tick[d] < t for d in deps)
    assert np.all(rows[local * blk:(local + 1) * blk] == 1) and rows.sum() == blk


def test_moe_tiles_cover_every_slot_once():
    rng = np.random.default_rng(4)
    R, m, N, E, BM, BN, S, local = 8, 64, 96, 6, 32, 32, 32, 2
    lg = rng.standard_normal((R * m, E)).astype(np.float32)
    ids, _ = oracle.route_topk(lg, 2)
    counts, offsets, perm = oracle.sort_by_expert(ids, E)
    tiles = sch.moe_tiles(counts, offsets, perm, 2, R, m, N, local, BM, BN, S)
    n_cb = -(-N // BN)
    cover = np.zeros((R * m * 2, n_cb), dtype=np.int64)
    bpr = -(-m // S)
    for e, r0, nr, cb, deps in tiles:
        assert 0 < nr <= BM and offsets[e] <= r0 and r0 + nr <= offsets[e + 1]
        cover[perm[r0:r0 + nr], cb] += 1
        toks = perm[r0:r0 + nr] // 2
        need = {(t // m) * bpr + (t % m) // S for t in toks if t // m != local}
        assert need <= set(deps)
    assert np.all(cover == 1)


@pytest.mark.parametrize("n_rb,n_cb,rb0", [(32, 16, 0), (32, 16, 4), (10, 3, 7), (1, 1, 0), (5, 9, 2), (7, 1, 6)])
def test_tile_order_groups(n_rb, n_cb, rb0):
    """Every tile once; the first GROUP tiles of a group share one column
    block and span GROUP consecutive (rotated) row blocks; the first tile is
    row block rb0."""
    order = sch.tile_order(n_rb, n_cb, rb0)
    assert sorted(order) == sorted(itertools.product(range(n_rb), range(n_cb)))
    assert order[0] == (rb0, 0)
    rot = [(rb - rb0) % n_rb for rb, _ in order]
    per = sch.GROUP * n_cb
    for v, (rb, cb) in enumerate(order):
        g = v // per
        assert g * sch.GROUP <= rot[v] < min((g + 1) * sch.GROUP, n_rb)
        if v % per:
            prev_cb = order[v - 1][1]
            assert cb == prev_cb or cb == prev_cb + 1


@pytest.mark.parametrize("n_tiles", [0, 1, 31, 32, 33, 255, 256, 257, 512, 1000, 1792])
def test_tile_queues_partition(n_tiles):
    """The queues partition the tiles; each queue holds whole batches of
    consecutive tiles in ascending order; batches go round-robin."""
    qs = sch.tile_queues(n_tiles)
    assert len(qs) == sch.XCDS
    assert sorted(v for q in qs for v in q) == list(range(n_tiles))
    for q, lst in enumerate(qs):
        assert lst == sorted(lst)
        for v in lst:
            assert (v // sch.BATCH) % sch.XCDS == q
    where = sch.queue_of(n_tiles)
    for v in range(n_tiles):
        q, t = where[v]
        assert qs[q][t] == v


def test_combine_rs_plan_covers_rows_once_local_block_first():
    """Tasks cover every token row exactly once; the local block's rows are
    exactly the rows of the first (local) tasks."""
    for R, T, local, CR, CRL in [(8, 4096, 0, 9, 2), (8, 4096, 5, 9, 2), (3, 30, 2, 7, 3), (1, 10, 0, 3, 4)]:
        plan = sch.combine_rs_plan(R, T, local, CR, CRL)
        rows = [r for p in plan for r in p[2]]
        assert sorted(rows) == list(range(T))
        blk = T // R
        n_lt = -(-blk // CRL)
        assert all(p[3] for p in plan[:n_lt]) and not any(p[3] for p in plan[n_lt:])
        assert {r for p in plan[:n_lt] for r in p[2]} == set(range(local * blk, (local + 1) * blk))
        assert all(len(p[2]) <= (CRL if p[3] else CR) for p in plan)


@pytest.mark.parametrize("R,m,Hq,Hkv,local,S,CT", [(8, 2048, 32, 8, 0, 2048, 64), (3, 200, 8, 2, 2, 64, 16),
                                                  (4, 70, 6, 2, 1, 70, 35)])
def test_attention_plan_covers_rows_and_chunks_once(R, m, Hq, Hkv, local, S, CT):
    plan = sch.attention_plan(R, m, Hq, Hkv, local, S, CT)
    copies = [t for t in plan if t[0] == "copy"]
    tiles = [t for t in plan if t[0] == "tile"]
    assert [t[1] for t in plan] == list(range(len(plan)))
    # every token row of every chunk copied once per tensor
    for tensor in (0, 1):
        rows = sorted(r for t in copies if t[3] == tensor for r in range(t[2].row0, t[2].row1))
        assert rows == list(range(R * m))
    # the slab count each slab needs is twice the AG count
    tgt = sch.slab_targets(R, m, S, CT)
    for s, n in enumerate(tgt):
        assert sum(1 for t in copies if t[2].slab == s) == 2 * n
    # every query row (i, h) in exactly one tile, with its own kv head
    G = Hq // Hkv
    seen = [r for t in tiles for r in t[4]]
    assert sorted(seen) == [(i, h) for i in range(m) for h in range(Hq)]
    for t in tiles:
        assert all(h // G == t[2] for _, h in t[4])
        assert len(t[5]) == (R - 1) * (-(-m // S)) and all(s // (-(-m // S)) != local for s in t[5])
    assert sch.attention_chunk_order(R, local)[0] == local
    assert sorted(sch.attention_chunk_order(R, local)) == list(range(R))
