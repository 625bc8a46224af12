"""Expected task lists of the persistent kernels (test infrastructure only).

This is an independent Python re-derivation, by explicit enumeration, of the
ticket -> task schedule the GPU library computes in closed form. The GPU trace
must reproduce it exactly. It follows the pages' tile-centric scheme:

  * TileLink talk summary, "Technical Deep Dive": a wait takes only a tile id;
    rank id, barrier id, tiles per rank and barriers per rank are recovered
    from it by an affine map for static workloads, and from lookup tables
    passed as parameters for dynamic (MoE) workloads;
  * same section: pull mode has two barriers (data ready at the source, then
    transfer complete); the "transfer complete" barrier is the per-slab flag
    published here by copy tasks;
  * same section: swizzling reorders tile access and communication so the
    communication lines up with compute -- here the tiles start at the local
    rank's rows and walk the other ranks in rotated order, and copies are
    issued in that same rotated order.

Schedule definition (shared contract with the device code; written here
independently):

AG-GEMM (rank count R, rows per rank m, gathered M = R*m, inner size K, tile
BM x BN, slab rows S, copy-task rows CT with S % CT == 0, K-slab columns KS):
  chunk sequence for copies: swizzled -> (l+1, l+2, ..., l+R-1, l) mod R;
  natural -> (0, 1, ..., R-1).
  The columns are cut into K-slabs of KS (the last may be shorter). When
  swizzled, the sequence is cut into phases: the peer at position q (chunk
  l+1+q) belongs to phase ((q+1)*m) // RPR -- RPR gathered rows of the
  rotated order are read per round of tiles of the persistent grid, so a
  phase holds the peers a round first reads -- and the local chunk, which no
  tile waits on, forms the last phase (natural order: one phase). Copy
  tickets run phase by phase; within a phase K-slab by K-slab; within a
  K-slab over the phase's chunks in sequence order and the pieces of each:
  piece t of chunk c in K-slab j holds rows [c*m + t*CT, c*m +
  min((t+1)*CT, m)), columns [j*KS, min((j+1)*KS, K)), slab (c, (t*CT)//S),
  and completes part of flag slab*nks + j (nks = ceil(K/KS)). With KS = K
  there is one K-slab and the flag is the slab.
  tiles follow the copies: tile v sits at slot n_copy + v. Tile order: the
  row blocks in rotated order rb0, rb0+1, ... (mod n_rb), rb0 = (l*m)//BM
  when swizzled, else 0, are cut into groups of GROUP consecutive blocks;
  the groups are taken in turn and each group is walked column block by
  column block, all of the group's row blocks for one column block before
  the next column block. A tile waits for every slab overlapping its rows
  that belongs to a chunk other than the local one (local rows are read from
  the local shard directly).
  Tiles are dealt to XCDS queues in batches of BATCH consecutive tiles, batch
  b to queue b % XCDS; a queue's tickets 0, 1, ... name its tiles in order.
  (The queue a tile sits in sets only which L2 serves it, not its result.)
  Without the XCD remap (ablation) there is one queue: tile v is ticket v of
  queue 0.
  A tile waits, for every K-slab it loads, on that K-slab's flag of each of
  its dependency slabs, before its first load of the K-slab.
  Split K (SK = 2 parts, one K-slab): tile v becomes two work units, u = 2v
  (columns [0, K/2)) and u = 2v + 1 (columns [K/2, K)), both with the tile's
  dependencies; the units take the slots n_copy + u and are what is dealt to
  the queues (batches of BATCH units). The affine map from a slot to its
  task keeps its form: tile = unit // SK, part = unit % SK.
GEMM-RS: slots [0, n_tiles) are GEMM tiles in the same order and queues,
  with rb0 = (l*M/R)//BM when swizzled -- with push transfers rb0 =
  (((l+1) mod R)*M/R)//BM, so the local block comes last; each stores its
  bf16 partial and publishes its tile flag. Slots [n_tiles, n_tiles + ceil(blk/RR)) are
  reduce tasks over RR-row strips of the local block [l*blk, (l+1)*blk),
  blk = M/R, in ascending row order; a strip waits for the flags of every
  tile of the row blocks it overlaps (and for the peers' flags of those
  tiles).
AllGather-KV attention (R ranks of m tokens, Hq query heads over Hkv kv
  heads, G = Hq/Hkv, ROWS query rows per tile): the AG copy list of one
  tensor with rows = tokens, each entry taken twice in a row -- keys, then
  values (tickets 2u and 2u+1) -- so a slab is complete after twice the AG
  count of tasks. Then the tiles: for kv head g the query rows are the pairs
  (i, h), h in [g*G, (g+1)*G), in i-major order, cut into ROWS-row blocks;
  tile v = g * n_rb + rb, in the XCD queues above. Every tile visits the
  chunks in the order local, local+1, ... (mod R) when swizzled, 0..R-1
  otherwise, and waits for all slabs of every chunk but the local one.
MoE: the AG-GEMM copy list, then one tile per (expert e, column block cb,
  row tile rt) in that nesting order; expert e's rows
  [off_e + rt*BM, min(off_e + (rt+1)*BM, off_{e+1})) of the expert-sorted slot
  list. A tile waits for every non-local slab between the slab of its first
  token and the slab of its last token (tokens ascend within an expert).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple


GROUP = 4     # row blocks per group of the tile order
BATCH = 32    # consecutive tiles per queue batch
XCDS = 8      # tile queues, one per XCD


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def tile_order(n_rb: int, n_cb: int, rb0: int) -> List[Tuple[int, int]]:
    """(rb, cb) of tiles 0, 1, ... in the grouped, rotated order."""
    rows = [(rb0 + i) % n_rb for i in range(n_rb)]
    out = []
    for g in range(0, n_rb, GROUP):
        for cb in range(n_cb):
            for rb in rows[g:g + GROUP]:
                out.append((rb, cb))
    return out


def tile_queues(n_tiles: int) -> List[List[int]]:
    """queues[q][t] = tile taken by ticket t of XCD queue q."""
    queues: List[List[int]] = [[] for _ in range(XCDS)]
    for b, start in enumerate(range(0, n_tiles, BATCH)):
        queues[b % XCDS].extend(range(start, min(start + BATCH, n_tiles)))
    return queues


def queue_of(n_tiles: int):
    """tile index -> (queue, ticket within the queue)."""
    where = {}
    for q, lst in enumerate(tile_queues(n_tiles)):
        for t, v in enumerate(lst):
            where[v] = (q, t)
    return where


@dataclass(frozen=True)
class CopyTask:
    ticket: int
    chunk: int
    piece: int
    row0: int       # first gathered row
    row1: int       # one past the last gathered row
    slab: int       # global slab id chunk*bpr + s
    kslab: int = 0  # K-slab index (columns [k0, k1))
    k0: int = 0
    k1: int = -1    # -1: every column
    flag: int = -1  # flag index slab * nks + kslab (-1: the slab)


@dataclass(frozen=True)
class Tile:
    ticket: int             # trace slot
    rb: int
    cb: int
    deps: Tuple[int, ...]   # global slab ids waited on
    queue: int = 0          # XCD queue holding the tile
    qticket: int = 0        # ticket of the tile within that queue
    part: int = 0           # K part of a split tile (0 when unsplit)


def copy_sequence(R: int, local: int, swizzle: bool) -> List[int]:
    if swizzle:
        return [(local + p) % R for p in range(1, R)] + [local]
    return list(range(R))


def copy_phases(R, m, local, swizzle, rpr=None) -> List[List[int]]:
    """The chunk sequence cut into copy phases (see the module docstring)."""
    seq = copy_sequence(R, local, swizzle)
    if not swizzle or rpr is None:
        return [seq]
    phases: dict = {}
    for q, c in enumerate(seq[:-1]):
        phases.setdefault(((q + 1) * m) // rpr, []).append(c)
    return [phases[k] for k in sorted(phases)] + [[seq[-1]]]


def copy_tasks(R, m, S, CT, local, swizzle, first_ticket=0, K=None, KS=None, rpr=None) -> List[CopyTask]:
    if S % CT:
        raise ValueError("slab rows must be a multiple of copy-task rows")
    bpr = _cdiv(m, S)
    if K is None or KS is None or KS >= K:
        kslabs = [(0, -1)]
    else:
        kslabs = [(k0, min(k0 + KS, K)) for k0 in range(0, K, KS)]
    nks = len(kslabs)
    out = []
    ticket = first_ticket
    for phase in copy_phases(R, m, local, swizzle, rpr):
        for j, (k0, k1) in enumerate(kslabs):
            for c in phase:
                t = 0
                r = 0
                while r < m:
                    r1 = min(r + CT, m)
                    slab = c * bpr + r // S
                    out.append(CopyTask(ticket, c, t, c * m + r, c * m + r1, slab, j, k0, k1, slab * nks + j))
                    ticket += 1
                    t += 1
                    r = r1
    return out


def slab_targets(R, m, S, CT) -> List[int]:
    """Number of copy tasks that complete each slab (global slab order)."""
    bpr = _cdiv(m, S)
    tgt = [0] * (R * bpr)
    for c in range(R):
        r = 0
        while r < m:
            tgt[c * bpr + r // S] += 1
            r = min(r + CT, m)
    return tgt


def ag_gemm_plan(R, m, K, N, local, BM, BN, S, CT, swizzle=True, mode="fused", KS=None, xcd_remap=True,
                 rpr=None, sk=1):
    """Full ticket list for the AG-GEMM kernel: list of CopyTask and Tile
    (one Tile per work unit: sk K parts per tile).
    rpr: gathered rows per round of tiles (copy phases); None = one round."""
    M = R * m
    n_rb, n_cb = _cdiv(M, BM), _cdiv(N, BN)
    bpr = _cdiv(m, S)
    tasks = []
    if mode in ("fused", "copy_only"):
        tasks += copy_tasks(R, m, S, CT, local, swizzle, K=K, KS=KS, rpr=rpr)
    if mode in ("fused", "gemm_only"):
        rb0 = (local * m) // BM if swizzle else 0
        base = len(tasks)
        n_units = n_rb * n_cb * sk
        where = queue_of(n_units) if xcd_remap else {u: (0, u) for u in range(n_units)}
        for v, (rb, cb) in enumerate(tile_order(n_rb, n_cb, rb0)):
            deps = set()
            if mode == "fused":
                for row in range(rb * BM, min((rb + 1) * BM, M)):
                    c = row // m
                    if c != local:
                        deps.add(c * bpr + (row % m) // S)
            for part in range(sk):
                u = v * sk + part
                tasks.append(Tile(base + u, rb, cb, tuple(sorted(deps)), *where[u], part=part))
    return tasks


def gemm_rs_plan(R, M, N, local, BM, BN, RR, swizzle=True, push=False):
    """Ticket list of the GEMM-RS kernel.

    Tiles: ("tile", slot, rb, cb, touches_local_block, queue, queue_ticket).
    Reduce strips: ("reduce", slot, row0, row1, deps) with gathered-row range
    [row0, row1) inside the local block and deps the (rb, cb) tiles waited on."""
    n_rb, n_cb = _cdiv(M, BM), _cdiv(N, BN)
    blk = M // R
    first = (local + 1) % R if push else local
    rb0 = (first * blk) // BM if swizzle else 0
    out = []
    where = queue_of(n_rb * n_cb)
    for v, (rb, cb) in enumerate(tile_order(n_rb, n_cb, rb0)):
        lo, hi = rb * BM, min((rb + 1) * BM, M)
        has_local = lo < (local + 1) * blk and hi > local * blk
        out.append(("tile", v, rb, cb, has_local, *where[v]))
    t = n_rb * n_cb
    r = local * blk
    while r < (local + 1) * blk:
        r1 = min(r + RR, (local + 1) * blk)
        deps = tuple((rb, cb) for rb in range(r // BM, (r1 - 1) // BM + 1) for cb in range(n_cb))
        out.append(("reduce", t, r, r1, deps))
        t += 1
        r = r1
    return out


def moe_tiles(counts, offsets, perm, topk, R, m, N, local, BM, BN, S):
    """MoE tile list in ticket order after the copies:
    tuples (expert, row_start, nrows, cb, deps)."""
    bpr = _cdiv(m, S)
    n_cb = _cdiv(N, BN)
    out = []
    for e in range(len(counts)):
        nrt = _cdiv(int(counts[e]), BM)
        for cb in range(n_cb):
            for rt in range(nrt):
                r0 = int(offsets[e]) + rt * BM
                r1 = min(r0 + BM, int(offsets[e + 1]))
                t_first = int(perm[r0]) // topk
                t_last = int(perm[r1 - 1]) // topk
                s_lo = (t_first // m) * bpr + (t_first % m) // S
                s_hi = (t_last // m) * bpr + (t_last % m) // S
                deps = tuple(s for s in range(s_lo, s_hi + 1) if s // bpr != local)
                out.append((e, r0, r1 - r0, cb, deps))
    return out


def combine_rs_plan(R, T, local, CR, CRL):
    """Ticket list of the TopK-Reduce + ReduceScatter kernel: tasks
    ("combine", slot, rows, is_local) over the row order rotated to start at
    the local block (row t = (r + local*T/R) mod T): first the local block's
    rows (rotated [0, T/R)) in tasks of CRL rows, which also reduce those rows
    over the ranks, then the other rows in tasks of CR rows."""
    blk = T // R
    base = local * blk
    out = []
    spans = [(r, min(r + CRL, blk), True) for r in range(0, blk, CRL)]
    spans += [(r, min(r + CR, T), False) for r in range(blk, T, CR)]
    for u, (r0, r1, is_local) in enumerate(spans):
        out.append(("combine", u, tuple((r + base) % T for r in range(r0, r1)), is_local))
    return out


ATTN_ROWS = 256   # query rows per attention tile


def attention_plan(R, m, Hq, Hkv, local, S, CT, swizzle=True, mode="fused"):
    """Ticket list of the AllGather-KV attention kernel: ("copy", slot,
    CopyTask, tensor) then ("tile", slot, g, rb, rows, deps, queue, qticket)
    with rows the (i, h) pairs of the tile and deps the slabs waited on."""
    G = Hq // Hkv
    bpr = _cdiv(m, S)
    out = []
    if mode in ("fused", "copy_only"):
        for t in copy_tasks(R, m, S, CT, local, swizzle):
            for tensor in (0, 1):
                out.append(("copy", len(out), t, tensor))
    if mode in ("fused", "gemm_only"):
        n_rb = _cdiv(G * m, ATTN_ROWS)
        where = queue_of(Hkv * n_rb)
        base = len(out)
        deps = tuple(c * bpr + s for c in range(R) if c != local for s in range(bpr)) if mode == "fused" else ()
        for g in range(Hkv):
            for rb in range(n_rb):
                rows = tuple((r // G, g * G + r % G) for r in range(rb * ATTN_ROWS, min((rb + 1) * ATTN_ROWS, G * m)))
                v = g * n_rb + rb
                out.append(("tile", base + v, g, rb, rows, deps, *where[v]))
    return out


def attention_chunk_order(R, local, swizzle=True):
    """Chunks in the order a tile's key blocks visit them."""
    return [(local + p) % R for p in range(R)] if swizzle else list(range(R))
