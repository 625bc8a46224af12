"""Plain float64 definitions of the three operations (test infrastructure only).

Sources (the pages print no formula, listing or worked example; every step
below is the plain definition of the named collective or operator):
  [TL-BG]  TileLink talk summary, section "Background": tensor parallelism
           AllGathers the activations and ReduceScatters partial results.
  [TL-KF]  same page, section "Key Findings": AllGather-GEMM and
           GEMM-ReduceScatter as the fundamental dense operations.
  [TL-TDD] same page, section "Technical Deep Dive": a GEMM-ReduceScatter is a
           GEMM that signals each finished tile, followed by a reduce over the
           ranks' partial tiles; dynamic (MoE) dependencies use lookup tables.
  [TL-EXP] same page, section "Experimental Setup & Results": the MoE layer
           chains AllGather, GroupGEMM, ReduceScatter, TopK-Reduce and a local
           scatter.

Readings where the pages are silent (each is also listed in the design doc):
  R1  the gathered rows are in ascending rank order; scheduling order never
      changes the layout;
  R2  GEMM-ReduceScatter: every partial enters the reduce as bfloat16 (what a
      rank would transmit), the sum runs in float32 in ascending rank order
      starting from rank 0's partial, with one round-to-nearest-even at the end
      (``reduce_fixed_order``); the float64 definition is ``gemm_rs``;
  R3  routing: the top-k experts of a token are the k largest float32 logits
      (softmax is strictly increasing); on equal logits the lower expert index
      ranks first; slot 0 holds the larger logit; gate weights are the softmax
      probabilities of the chosen experts (not renormalised) and are not
      applied to the GEMM output;
  R4  "sorted by expert" is stable in (expert, token, slot); token-slot order
      means output row t*topk + slot;
  R11 TopK-Reduce: a token's output is the gate-weighted sum of its top-k
      slot rows, P[t] = sum_j w[t, j] * Y[t*topk + j]; the ReduceScatter that
      follows it is the fixed-order reduce of R2 over the ranks' combined
      partials [T, N], row block l = the l-th rank's m tokens; the local
      combined partial enters that reduce as bfloat16.
  [TL-EXP] names TopK-Reduce among the MoE operators it overlaps; it prints
  neither its formula nor its precision, hence R11.
  R12 AllGather-KV attention ([TL-EXP]: the KV AllGather overlapped with the
      attention computation; no formula, mask or shape): each rank holds a
      contiguous chunk of m tokens of Q, K and V; K and V are gathered in
      rank order and rank l's queries attend, per head, over all R*m keys
      with softmax(q . k / sqrt(d)) and no mask (context-parallel attention
      read plainly: every query sees the whole gathered sequence). With
      fewer kv heads than query heads (Hq = G * Hkv), query head h reads kv
      head h // G (grouped-query attention, the layout that makes gathering
      K and V cheaper than moving Q).
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# bfloat16 codec (the oracle's own; pinned against torch's CPU cast)
# --------------------------------------------------------------------------


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bf16 value is the float32 whose upper 16 bits are the pattern and whose
    lower 16 bits are zero."""
    hi = np.asarray(bits, dtype=np.uint16).astype(np.uint32) * np.uint32(65536)
    with np.errstate(invalid="ignore"):
        return hi.view(np.float32).astype(np.float64)


def encode_bf16_rne(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits with round-to-nearest, ties to even.

    Written out on the integer representation: keep the upper 16 bits, look at
    the dropped lower 16 bits; above half -> round up, exactly half -> round up
    only if the kept pattern is odd. NaNs stay NaN (quiet bit set)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    kept = u >> np.uint64(16)
    dropped = u & np.uint64(0xFFFF)
    up = (dropped > 0x8000) | ((dropped == 0x8000) & ((kept & np.uint64(1)) == 1))
    out = (kept + up.astype(np.uint64)).astype(np.uint64)
    nan = np.isnan(x32)
    out = np.where(nan, kept | np.uint64(0x40), out)
    return (out & np.uint64(0xFFFF)).astype(np.uint16)


# --------------------------------------------------------------------------
# AllGather-GEMM  [TL-BG], [TL-KF]
# --------------------------------------------------------------------------


def _gather(a_chunks):
    """AllGather of row-sharded activations: rank r's [m, K] shard becomes row
    block r of the [R*m, K] gathered matrix (reading R1)."""
    return np.concatenate([np.asarray(c, dtype=np.uint16) for c in a_chunks], axis=0)


def ag_gemm(a_chunks, b_bits):
    """C = gather(A_0 .. A_{R-1}) x B in float64.

    Returns (a_full_bits, c): the gathered bf16 matrix (a pure copy, so the
    GPU's gathered buffer must equal it bit for bit) and the float64 product."""
    a_full = _gather(a_chunks)
    c = decode_bf16(a_full) @ decode_bf16(b_bits)
    return a_full, c


def ag_gemm_entries(a_chunks, b_bits, rows, cols):
    """Selected entries C[rows[i], cols[i]] of ``ag_gemm`` (float64 dots), for
    checks at sizes where the full product is too slow."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    m = a_chunks[0].shape[0]
    a_rows = np.stack([decode_bf16(a_chunks[int(r) // m][int(r) % m]) for r in rows])
    b_cols = decode_bf16(np.asarray(b_bits)[:, cols]).T
    return np.einsum("ik,ik->i", a_rows, b_cols)


def ag_gemm_block(a_chunks, b_bits, rows, cols):
    """The block C[rows][:, cols] of ``ag_gemm`` (float64), for sampled checks
    at full size: gathered rows times the selected columns of B."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    m = a_chunks[0].shape[0]
    a_rows = np.stack([decode_bf16(a_chunks[int(r) // m][int(r) % m]) for r in rows])
    return a_rows @ decode_bf16(np.asarray(b_bits)[:, cols])


# --------------------------------------------------------------------------
# GEMM-ReduceScatter  [TL-KF], [TL-TDD]
# --------------------------------------------------------------------------


def gemm_rs(a_bits, b_bits, peers, R, local_rank):
    """Local partial P_l = A x B, and the reduce-scattered row block
    out_l = sum over ranks s of P_s[rows l*M/R .. (l+1)*M/R), all float64.

    ``peers`` maps every rank s != local_rank to its bf16 partial [M, N].
    Returns (partial, out)."""
    a = decode_bf16(a_bits)
    b = decode_bf16(b_bits)
    M = a.shape[0]
    if M % R:
        raise ValueError("M must be a multiple of R")
    blk = M // R
    partial = a @ b
    r0 = local_rank * blk
    out = partial[r0:r0 + blk].copy()
    for s in range(R):
        if s != local_rank:
            out += decode_bf16(peers[s][r0:r0 + blk])
    return partial, out


def gemm_rs_entries(a_bits, b_bits, peers, R, local_rank, rows, cols):
    """Selected entries (rows are within the output block) of ``gemm_rs``'s
    out_l, as float64, plus the matching entries of the local partial."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    M = np.asarray(a_bits).shape[0]
    blk = M // R
    g = rows + local_rank * blk
    a_rows = decode_bf16(np.asarray(a_bits)[g])
    b_cols = decode_bf16(np.asarray(b_bits)[:, cols]).T
    part = np.einsum("ik,ik->i", a_rows, b_cols)
    out = part.copy()
    for s in range(R):
        if s != local_rank:
            out += decode_bf16(peers[s][g, cols])
    return part, out


def reduce_fixed_order(blocks_bits):
    """Reading R2 of the fixed-order reduce: given the R ranks' bf16 partial
    blocks in rank order 0..R-1, return bf16 bits of
    RNE_bf16(((P_0 + P_1) + P_2) + ... + P_{R-1}) with every addition done in
    float32 (IEEE round-to-nearest-even)."""
    acc = decode_bf16(blocks_bits[0]).astype(np.float32)
    for blk in blocks_bits[1:]:
        acc = (acc + decode_bf16(blk).astype(np.float32)).astype(np.float32)
    return encode_bf16_rne(acc)


# --------------------------------------------------------------------------
# AllGather + MoE routing + grouped GEMM  [TL-TDD], [TL-EXP]
# --------------------------------------------------------------------------


def route_topk(logits, k):
    """Top-k routing (reading R3). Returns (ids int32 [T, k], w float64 [T, k]).

    ids[t] lists the k largest float32 logits of token t, largest first, the
    lower expert index first among equal logits. w[t, j] is the softmax
    probability of expert ids[t, j] over all E logits, computed in float64."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    # a stable sort of the negated logits keeps equal logits in index order
    order = np.argsort(-lg, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    l64 = lg.astype(np.float64)
    mx = l64.max(axis=1, keepdims=True)
    p = np.exp(l64 - mx)
    p /= p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return ids, w


def sort_by_expert(ids, E):
    """Stable grouping of the token slots by expert (reading R4).

    Returns (counts int32 [E], offsets int32 [E+1], perm int32 [T*k]) where
    perm lists token-slot indices t*k + j ordered by (expert, token, slot)."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)                       # index t*k + j
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int32)   # ties keep t*k+j order
    return counts, offsets, perm


def ag_grouped_gemm(a_chunks, logits, w_bits, topk):
    """AllGather the token shards, route each token to its top-k experts and
    multiply it by each chosen expert's weight, float64.

    Returns dict with a_full (bits), ids, weights, counts, offsets, perm and
    out [T*topk, N] where out[t*topk + j] = A_full[t] x W[ids[t, j]]."""
    a_full = _gather(a_chunks)
    ids, wts = route_topk(logits, topk)
    E = np.asarray(w_bits).shape[0]
    counts, offsets, perm = sort_by_expert(ids, E)
    a = decode_bf16(a_full)
    T = a.shape[0]
    N = np.asarray(w_bits).shape[2]
    out = np.empty((T * topk, N), dtype=np.float64)
    for e in range(E):
        slots = perm[offsets[e]:offsets[e + 1]]
        if slots.size == 0:
            continue
        tokens = slots // topk
        out[slots] = a[tokens] @ decode_bf16(w_bits[e])
    return dict(a_full=a_full, ids=ids, weights=wts, counts=counts,
                offsets=offsets, perm=perm, out=out)


def ag_grouped_gemm_entries(a_chunks, ids, w_bits, slots, cols):
    """Selected entries out[slots[i], cols[i]] of ``ag_grouped_gemm`` given the
    routing ``ids`` (float64 dots)."""
    slots = np.asarray(slots, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ids = np.asarray(ids)
    topk = ids.shape[1]
    m = a_chunks[0].shape[0]
    res = np.empty(slots.shape[0], dtype=np.float64)
    for i, (s, c) in enumerate(zip(slots, cols)):
        t, j = divmod(int(s), topk)
        e = int(ids[t, j])
        arow = decode_bf16(a_chunks[t // m][t % m])
        res[i] = float(arow @ decode_bf16(w_bits[e][:, int(c)]))
    return res


# --------------------------------------------------------------------------
# MoE TopK-Reduce + ReduceScatter  [TL-EXP] (reading R11)
# --------------------------------------------------------------------------


def topk_combine(y_bits, w, topk):
    """P[t] = sum over j < topk of w[t, j] * Y[t*topk + j], float64 [T, N].

    ``y_bits``: bf16 bits [T*topk, N] in token-slot order; ``w``: gate
    weights [T, topk]."""
    y = decode_bf16(np.asarray(y_bits))
    wt = np.asarray(w, dtype=np.float64)
    T = wt.shape[0]
    if y.shape[0] != T * topk:
        raise ValueError("Y must have T*topk rows")
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(topk):
        out += wt[:, j:j + 1] * y[j::topk]
    return out


def moe_combine_rs(y_bits, w, topk, peers, R, local_rank):
    """Local combined partial P_l = topk_combine(Y, w), and
    out_l = sum over ranks s of P_s[rows l*T/R .. (l+1)*T/R), float64.

    ``peers`` maps every rank s != local_rank to its bf16 combined partial
    [T, N]. Returns (partial, out)."""
    partial = topk_combine(y_bits, w, topk)
    T = partial.shape[0]
    if T % R:
        raise ValueError("T must be a multiple of R")
    blk = T // R
    r0 = local_rank * blk
    out = partial[r0:r0 + blk].copy()
    for s in range(R):
        if s != local_rank:
            out += decode_bf16(peers[s][r0:r0 + blk])
    return partial, out


# --------------------------------------------------------------------------
# AllGather-KV attention  [TL-EXP] (reading R12)
# --------------------------------------------------------------------------


def ag_attention(q_bits, k_chunks, v_chunks):
    """Gather K and V (ascending rank order) and attend the local queries over
    them, per head, float64.

    ``q_bits``: bf16 bits [m, Hq, d] (the local queries); ``k_chunks`` /
    ``v_chunks``: R bf16 arrays [m_r, Hkv, d] with Hq a multiple of Hkv.
    Returns (k_full bits, v_full bits, out [m, Hq, d]) with
    out[i, h] = sum_j softmax_j(q[i,h] . k[j,g] / sqrt(d)) v[j,g], g = h // (Hq/Hkv)."""
    k_full = np.concatenate([np.asarray(c) for c in k_chunks], axis=0)
    v_full = np.concatenate([np.asarray(c) for c in v_chunks], axis=0)
    q = decode_bf16(np.asarray(q_bits))
    k = decode_bf16(k_full)
    v = decode_bf16(v_full)
    m, Hq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    G = Hq // Hkv
    out = np.empty((m, Hq, d), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(d)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return k_full, v_full, out


def ag_attention_rows(q_bits, k_full_bits, v_full_bits, rows):
    """out[i, h] of ag_attention for the (i, h) pairs in ``rows`` only, from
    already gathered K and V [S, Hkv, d] (float64; for sampled checks at full
    size)."""
    Hq, d = q_bits.shape[1], q_bits.shape[2]
    G = Hq // k_full_bits.shape[1]
    res = np.empty((len(rows), d), dtype=np.float64)
    for n, (i, h) in enumerate(rows):
        q = decode_bf16(np.asarray(q_bits[i, h]))
        k = decode_bf16(np.asarray(k_full_bits[:, h // G]))
        v = decode_bf16(np.asarray(v_full_bits[:, h // G]))
        s = (k @ q) / np.sqrt(d)
        p = np.exp(s - s.max())
        res[n] = (p / p.sum()) @ v
    return res
