"""Pins of the CPU oracle against things other than itself: brute force on tiny
inputs, closed forms, identities, and special cases that reduce to a library
routine. Each test names the mistake it is there to catch."""
import ast
import math
import os

import numpy as np
import pytest

import oracle
from oracle import reference as ref
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_bf16(rng, shape, lo=-2.0, hi=2.0):
    return workloads.f32_to_bf16_bits(rng.uniform(lo, hi, size=shape).astype(np.float32))


def bf16_of_ints(a):
    return workloads.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


# ---------------------------------------------------------------- bf16 codec


def test_bf16_encode_matches_torch_cast():
    """RNE encode vs torch's CPU float32->bfloat16 cast (library routine),
    including exact ties, subnormals, and large values. Catches truncation
    instead of rounding, or ties rounded away from zero."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),   # subnormals
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        # exact ties: low 16 bits == 0x8000 with odd and even kept parts
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x00008000,
                  0x7F7F8000], dtype=np.uint32).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0], dtype=np.float32),
    ])
    got = ref.encode_bf16_rne(x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_bf16_decode_exact_roundtrip():
    """decode is exact: every one of the 65536 patterns that is not NaN decodes
    to a float32 that re-encodes to itself, and matches torch's bf16->f32."""
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = ref.decode_bf16(bits)
    finite = ~np.isnan(f)
    assert np.array_equal(ref.encode_bf16_rne(f[finite].astype(np.float32)), bits[finite])
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(f[finite], t[finite])


# ---------------------------------------------------------------- AG-GEMM


def brute_gemm(a_rows, b_rows):
    """Triple loop with exactly-rounded sums (math.fsum) on Python floats."""
    M, K = len(a_rows), len(a_rows[0])
    N = len(b_rows[0])
    return [[math.fsum(a_rows[i][k] * b_rows[k][j] for k in range(K)) for j in range(N)]
            for i in range(M)]


def test_golden_hand_example():
    """Hand-worked 2-rank example (tests/golden/ag_gemm_hand.txt): integer
    inputs, product checkable by eye. Catches a transposed B or swapped
    gather order."""
    with open(os.path.join(GOLDEN, "ag_gemm_hand.txt")) as f:
        lines = [l.strip() for l in f if l.strip() and not l.startswith("#")]
    vals = {}
    for l in lines:
        k, v = l.split("=")
        vals[k.strip()] = np.array(ast.literal_eval(v.strip()), dtype=np.float32)
    a0, a1, b, c = vals["A0"], vals["A1"], vals["B"], vals["C"]
    a_full, got = oracle.ag_gemm([bf16_of_ints(a0), bf16_of_ints(a1)], bf16_of_ints(b))
    assert np.array_equal(got, c.astype(np.float64))
    assert np.array_equal(ref.decode_bf16(a_full), np.concatenate([a0, a1]).astype(np.float64))


@pytest.mark.parametrize("R,m,K,N,seed", [(2, 4, 8, 4, 0), (1, 3, 5, 2, 1), (3, 2, 7, 5, 2),
                                           (4, 1, 1, 3, 3), (2, 5, 9, 1, 4)])
def test_ag_gemm_brute_force(R, m, K, N, seed):
    """Micro shapes vs a triple loop. Catches dropped k terms and index slips."""
    rng = np.random.default_rng(seed)
    chunks = [rand_bf16(rng, (m, K)) for _ in range(R)]
    b = rand_bf16(rng, (K, N))
    a_full, c = oracle.ag_gemm(chunks, b)
    a_rows = ref.decode_bf16(np.concatenate(chunks)).tolist()
    want = brute_gemm(a_rows, ref.decode_bf16(b).tolist())
    assert np.allclose(c, np.array(want), rtol=1e-13, atol=1e-13)
    assert np.array_equal(a_full, np.concatenate(chunks))


def test_ag_gemm_gather_order_one_hot():
    """Rows of each shard are one-hot: row i of rank r selects row k(r, i) of
    B, so C's row r*m+i must equal B[k(r, i)] exactly. Catches a gather in the
    wrong (e.g. swizzled) order, or A/B transposed."""
    R, m, K, N = 4, 3, 16, 5
    rng = np.random.default_rng(11)
    b = rand_bf16(rng, (K, N))
    sel = rng.permutation(K)[:R * m].reshape(R, m)
    chunks = []
    for r in range(R):
        a = np.zeros((m, K), dtype=np.float32)
        a[np.arange(m), sel[r]] = 1.0
        chunks.append(bf16_of_ints(a))
    _, c = oracle.ag_gemm(chunks, b)
    for r in range(R):
        for i in range(m):
            assert np.array_equal(c[r * m + i], ref.decode_bf16(b[sel[r, i]]))


def test_ag_gemm_tiny_outer_product_and_concat_identity():
    """Tiny workload (R=4, [128,256] shards, [256,256] B): the oracle equals an
    outer-product k-loop (a different summation), and each row block r equals
    A_r x B computed on its own (concatenation of per-chunk GEMMs)."""
    x = workloads.workload("ag_gemm_tiny").make()
    a_full, c = oracle.ag_gemm(x.a_chunks, x.b)
    a = ref.decode_bf16(a_full)
    b = ref.decode_bf16(x.b)
    acc = np.zeros_like(c)
    for k in range(a.shape[1]):
        acc += np.outer(a[:, k], b[k])
    assert np.allclose(c, acc, rtol=1e-12, atol=1e-12)
    for r in range(x.R):
        part = np.zeros((x.m, x.N))
        ar = ref.decode_bf16(x.a_chunks[r])
        for k in range(x.K):
            part += np.outer(ar[:, k], b[k])
        assert np.allclose(c[r * x.m:(r + 1) * x.m], part, rtol=1e-12, atol=1e-12)


def test_ag_gemm_checksums():
    """ABFT identities 1^T C = (1^T A) B and C 1 = A (B 1) on a mid-size random
    case. Catches any row or column of C being wrong or missing."""
    rng = np.random.default_rng(5)
    chunks = [rand_bf16(rng, (96, 320)) for _ in range(3)]
    b = rand_bf16(rng, (320, 200))
    a_full, c = oracle.ag_gemm(chunks, b)
    a = ref.decode_bf16(a_full)
    bb = ref.decode_bf16(b)
    assert np.allclose(c.sum(axis=0), a.sum(axis=0) @ bb, rtol=1e-10, atol=1e-9)
    assert np.allclose(c.sum(axis=1), a @ bb.sum(axis=1), rtol=1e-10, atol=1e-9)


def test_ag_gemm_entries_match_full():
    rng = np.random.default_rng(6)
    chunks = [rand_bf16(rng, (8, 24)) for _ in range(3)]
    b = rand_bf16(rng, (24, 10))
    _, c = oracle.ag_gemm(chunks, b)
    rows = rng.integers(0, 24, 50)
    cols = rng.integers(0, 10, 50)
    assert np.allclose(oracle.ag_gemm_entries(chunks, b, rows, cols), c[rows, cols], rtol=1e-14)
    br, bc = rows[:7], cols[:5]
    assert np.allclose(oracle.ag_gemm_block(chunks, b, br, bc), c[np.ix_(br, bc)], rtol=1e-14)


# ---------------------------------------------------------------- GEMM-RS


def test_gemm_rs_zero_peers_and_equal_peers():
    """Zero peers -> out is the local partial's row block; every peer equal to
    Q -> out = P_blk + (R-1) Q_blk. Catches the wrong row block, or a peer
    dropped or counted twice."""
    R, M, K, N = 4, 16, 12, 6
    rng = np.random.default_rng(3)
    a = rand_bf16(rng, (M, K))
    b = rand_bf16(rng, (K, N))
    zero = np.zeros((M, N), dtype=np.uint16)
    for local in range(R):
        p, out = oracle.gemm_rs(a, b, {s: zero for s in range(R) if s != local}, R, local)
        blk = M // R
        assert np.allclose(out, p[local * blk:(local + 1) * blk], rtol=0, atol=0)
        q = rand_bf16(rng, (M, N))
        p2, out2 = oracle.gemm_rs(a, b, {s: q for s in range(R) if s != local}, R, local)
        want = p2[local * blk:(local + 1) * blk] + (R - 1) * ref.decode_bf16(q[local * blk:(local + 1) * blk])
        assert np.allclose(out2, want, rtol=1e-13, atol=1e-13)


def test_gemm_rs_allreduce_identity_brute_force():
    """Every rank s holds its own A_s; with integer inputs all partials are
    exact. Concatenating out_l over l must equal sum_s A_s B (an all-reduce),
    computed here by a triple loop."""
    R, M, K, N = 4, 8, 5, 3
    rng = np.random.default_rng(9)
    A = [bf16_of_ints(rng.integers(-4, 5, (M, K))) for _ in range(R)]
    B = bf16_of_ints(rng.integers(-4, 5, (K, N)))
    P = [np.array(brute_gemm(ref.decode_bf16(A[s]).tolist(), ref.decode_bf16(B).tolist())) for s in range(R)]
    P_bits = [bf16_of_ints(p) for p in P]      # integers |x| <= 80: exact in bf16
    total = sum(P)
    blocks = []
    for local in range(R):
        _, out = oracle.gemm_rs(A[local], B, {s: P_bits[s] for s in range(R) if s != local}, R, local)
        blocks.append(out)
    assert np.array_equal(np.concatenate(blocks), total)


def test_reduce_fixed_order_is_ascending_rank_order():
    """Partials (2^25, 1, -2^25) in rank order: ((2^25 + 1) - 2^25) is 0 in
    float32 (2^25 + 1 rounds to 2^25), while any order that adds the two
    large terms first gives 1. Pins the order of reading R2."""
    blocks = [bf16_of_ints([[2.0 ** 25]]), bf16_of_ints([[1.0]]), bf16_of_ints([[-(2.0 ** 25)]])]
    assert ref.decode_bf16(oracle.reduce_fixed_order(blocks))[0, 0] == 0.0
    assert ref.decode_bf16(oracle.reduce_fixed_order([blocks[0], blocks[2], blocks[1]]))[0, 0] == 1.0


def test_reduce_fixed_order_bounds_and_special_cases():
    """Random partials: within one bf16 rounding (+ float32 accumulation) of
    the exact float64 sum; a single partial reduces to itself; small integers
    sum exactly."""
    rng = np.random.default_rng(12)
    blocks = [rand_bf16(rng, (64, 48)) for _ in range(8)]
    got = ref.decode_bf16(oracle.reduce_fixed_order(blocks))
    exact = sum(ref.decode_bf16(b) for b in blocks)
    bound = 2.0 ** -8 * np.abs(exact) + 8 * 2.0 ** -24 * sum(np.abs(ref.decode_bf16(b)) for b in blocks)
    assert np.all(np.abs(got - exact) <= bound)
    assert np.array_equal(oracle.reduce_fixed_order([blocks[0]]), blocks[0])
    ints = [bf16_of_ints(rng.integers(-20, 21, (5, 7))) for _ in range(8)]
    assert np.array_equal(ref.decode_bf16(oracle.reduce_fixed_order(ints)),
                          sum(ref.decode_bf16(b) for b in ints))


def test_gemm_rs_entries_match_full():
    rng = np.random.default_rng(13)
    R, M, K, N = 4, 16, 9, 7
    a = rand_bf16(rng, (M, K))
    b = rand_bf16(rng, (K, N))
    peers = {s: rand_bf16(rng, (M, N)) for s in range(R) if s != 2}
    p, out = oracle.gemm_rs(a, b, peers, R, 2)
    rows = rng.integers(0, M // R, 30)
    cols = rng.integers(0, N, 30)
    part, o = oracle.gemm_rs_entries(a, b, peers, R, 2, rows, cols)
    assert np.allclose(o, out[rows, cols], rtol=1e-14)
    assert np.allclose(part, p[rows + 2 * (M // R), cols], rtol=1e-14)


# ---------------------------------------------------------------- routing


def test_route_topk_brute_force_with_ties():
    """Top-2 vs sorting each token's (-logit, index) pairs in pure Python, with
    many exact ties planted. Catches a wrong tie order or slot order."""
    rng = np.random.default_rng(21)
    T, E = 300, 12
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::3, 5] = lg[::3, 2]                     # ties between experts 2 and 5
    lg[::7] = np.float32(0.25)                  # whole rows tied
    ids, w = oracle.route_topk(lg, 2)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:2]
        assert list(ids[t]) == order
        mx = max(float(v) for v in lg[t])
        den = math.fsum(math.exp(float(v) - mx) for v in lg[t])
        for j in range(2):
            assert w[t, j] == pytest.approx(math.exp(float(lg[t, order[j]]) - mx) / den, rel=1e-14)


def test_route_top1_is_argmax():
    """k = 1 reduces to numpy.argmax (which also returns the first maximum)."""
    rng = np.random.default_rng(22)
    lg = rng.standard_normal((500, 32)).astype(np.float32)
    lg[::4, 7] = lg[::4].max(axis=1) + 0  # ties with the maximum
    ids, _ = oracle.route_topk(lg, 1)
    assert np.array_equal(ids[:, 0], np.argmax(lg, axis=1))


def test_sort_by_expert_brute_force():
    """counts/offsets/perm vs a pure-Python stable sort by (expert, slot)."""
    rng = np.random.default_rng(23)
    T, E, k = 257, 9, 2
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.route_topk(lg, k)
    counts, offsets, perm = oracle.sort_by_expert(ids, E)
    flat = ids.reshape(-1).tolist()
    want = sorted(range(T * k), key=lambda s: (flat[s], s))
    assert perm.tolist() == want
    assert counts.sum() == T * k
    assert offsets[0] == 0 and np.all(np.diff(offsets) == counts)
    for e in range(E):
        assert all(flat[s] == e for s in perm[offsets[e]:offsets[e + 1]])


# ---------------------------------------------------------------- AG + MoE


def test_ag_grouped_gemm_brute_force():
    """Micro MoE vs a triple loop per (token, slot)."""
    rng = np.random.default_rng(31)
    R, m, K, N, E = 2, 3, 6, 4, 5
    chunks = [rand_bf16(rng, (m, K)) for _ in range(R)]
    lg = rng.standard_normal((R * m, E)).astype(np.float32)
    w = np.stack([rand_bf16(rng, (K, N)) for _ in range(E)])
    res = oracle.ag_grouped_gemm(chunks, lg, w, 2)
    a = ref.decode_bf16(np.concatenate(chunks)).tolist()
    for t in range(R * m):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:2]
        for j, e in enumerate(order):
            want = brute_gemm([a[t]], ref.decode_bf16(w[e]).tolist())[0]
            assert np.allclose(res["out"][t * 2 + j], want, rtol=1e-13, atol=1e-13)


def test_ag_grouped_gemm_forced_routing_reduces_to_dense():
    """All tokens prefer experts 3 then 7: slot-0 rows are the dense
    AG-GEMM with W_3 and slot-1 rows the one with W_7."""
    rng = np.random.default_rng(32)
    R, m, K, N, E = 3, 4, 16, 8, 10
    chunks = [rand_bf16(rng, (m, K)) for _ in range(R)]
    lg = rng.standard_normal((R * m, E)).astype(np.float32)
    lg[:, 3] = 10.0
    lg[:, 7] = 9.0
    w = np.stack([rand_bf16(rng, (K, N)) for _ in range(E)])
    res = oracle.ag_grouped_gemm(chunks, lg, w, 2)
    _, c3 = oracle.ag_gemm(chunks, w[3])
    _, c7 = oracle.ag_gemm(chunks, w[7])
    assert np.array_equal(res["out"][0::2], c3)
    assert np.array_equal(res["out"][1::2], c7)
    assert res["counts"][3] == R * m and res["counts"][7] == R * m


def test_ag_grouped_gemm_equal_experts():
    """All experts equal: both slot rows of a token are the same dense row."""
    rng = np.random.default_rng(33)
    R, m, K, N, E = 2, 5, 8, 6, 4
    chunks = [rand_bf16(rng, (m, K)) for _ in range(R)]
    lg = rng.standard_normal((R * m, E)).astype(np.float32)
    w1 = rand_bf16(rng, (K, N))
    res = oracle.ag_grouped_gemm(chunks, lg, np.stack([w1] * E), 2)
    _, c = oracle.ag_gemm(chunks, w1)
    assert np.array_equal(res["out"][0::2], c)
    assert np.array_equal(res["out"][1::2], c)


def test_ag_grouped_gemm_entries_match_full():
    rng = np.random.default_rng(34)
    R, m, K, N, E = 2, 6, 8, 5, 4
    chunks = [rand_bf16(rng, (m, K)) for _ in range(R)]
    lg = rng.standard_normal((R * m, E)).astype(np.float32)
    w = np.stack([rand_bf16(rng, (K, N)) for _ in range(E)])
    res = oracle.ag_grouped_gemm(chunks, lg, w, 2)
    slots = rng.integers(0, R * m * 2, 20)
    cols = rng.integers(0, N, 20)
    got = oracle.ag_grouped_gemm_entries(chunks, res["ids"], w, slots, cols)
    assert np.allclose(got, res["out"][slots, cols], rtol=1e-14)


# ---------------------------------------------------------------- TopK-Reduce + ReduceScatter


def brute_combine(y, w, topk):
    T = len(w)
    N = len(y[0])
    return [[sum(w[t][j] * y[t * topk + j][n] for j in range(topk)) for n in range(N)] for t in range(T)]


@pytest.mark.parametrize("T,N,topk,seed", [(3, 4, 2, 0), (5, 3, 1, 1), (4, 5, 3, 2)])
def test_topk_combine_brute_force(T, N, topk, seed):
    """Triple loop over tokens, columns and slots. Catches a slot taken from
    the wrong token (row t*topk + j), a weight of the wrong slot, or a
    transposed weight matrix."""
    rng = np.random.default_rng(seed)
    y = rand_bf16(rng, (T * topk, N))
    w = rng.uniform(0, 1, (T, topk)).astype(np.float32)
    want = np.array(brute_combine(ref.decode_bf16(y).tolist(), w.astype(np.float64).tolist(), topk))
    assert np.allclose(oracle.topk_combine(y, w, topk), want, rtol=1e-13, atol=1e-13)


def test_topk_combine_special_cases():
    """topk = 1 with unit weights is the identity; a one-hot weight row picks
    exactly that slot's row; the combine is linear in the weights. Catches a
    dropped or extra slot and a scaled weight."""
    rng = np.random.default_rng(21)
    T, N = 6, 5
    y1 = rand_bf16(rng, (T, N))
    assert np.array_equal(oracle.topk_combine(y1, np.ones((T, 1), np.float32), 1), ref.decode_bf16(y1))
    y2 = rand_bf16(rng, (T * 2, N))
    onehot = np.zeros((T, 2), np.float32)
    pick = rng.integers(0, 2, T)
    onehot[np.arange(T), pick] = 1.0
    assert np.array_equal(oracle.topk_combine(y2, onehot, 2), ref.decode_bf16(y2)[np.arange(T) * 2 + pick])
    w = rng.uniform(0, 1, (T, 2)).astype(np.float32)
    assert np.allclose(oracle.topk_combine(y2, 2 * w, 2), 2 * oracle.topk_combine(y2, w, 2), rtol=1e-14, atol=0)


def test_moe_combine_rs_allreduce_identity():
    """Every rank s holds its own Y_s and w_s with small integer values, so all
    combined partials are exact. Concatenating out_l over l must equal the
    sum over s of the combined partials (an all-reduce), computed by loops."""
    R, m, N, topk = 4, 3, 5, 2
    T = R * m
    rng = np.random.default_rng(22)
    Y = [bf16_of_ints(rng.integers(-4, 5, (T * topk, N))) for _ in range(R)]
    W = [rng.integers(0, 3, (T, topk)).astype(np.float32) for _ in range(R)]
    P = [np.array(brute_combine(ref.decode_bf16(Y[s]).tolist(), W[s].tolist(), topk)) for s in range(R)]
    P_bits = [bf16_of_ints(p) for p in P]   # |x| <= 16: exact in bf16
    blocks = []
    for local in range(R):
        part, out = oracle.moe_combine_rs(Y[local], W[local], topk, {s: P_bits[s] for s in range(R) if s != local},
                                          R, local)
        assert np.array_equal(part, P[local])
        blocks.append(out)
    assert np.array_equal(np.concatenate(blocks), sum(P))


def test_moe_combine_rs_zero_peers():
    """Zero peers: out is the local combined partial's row block (catches the
    wrong block)."""
    R, m, N, topk = 4, 5, 3, 2
    rng = np.random.default_rng(23)
    y = rand_bf16(rng, (R * m * topk, N))
    w = rng.uniform(0, 1, (R * m, topk)).astype(np.float32)
    zero = np.zeros((R * m, N), dtype=np.uint16)
    for local in range(R):
        p, out = oracle.moe_combine_rs(y, w, topk, {s: zero for s in range(R) if s != local}, R, local)
        assert np.array_equal(out, p[local * m:(local + 1) * m])


# ---------------------------------------------------------------- AllGather-KV attention


def brute_attention(q, k, v):
    """Per query and head: explicit softmax over all keys, loops; query head
    h reads kv head h // (Hq / Hkv)."""
    m, H, d = len(q), len(q[0]), len(q[0][0])
    G = H // len(k[0])
    S = len(k)
    out = [[[0.0] * d for _ in range(H)] for _ in range(m)]
    for i in range(m):
        for h in range(H):
            g = h // G
            s = [sum(q[i][h][e] * k[j][g][e] for e in range(d)) / math.sqrt(d) for j in range(S)]
            mx = max(s)
            p = [math.exp(x - mx) for x in s]
            tot = sum(p)
            for e in range(d):
                out[i][h][e] = sum(p[j] * v[j][g][e] for j in range(S)) / tot
    return out


def test_ag_attention_brute_force():
    """Loops over queries, heads, keys and the head dimension on a tiny case
    with R = 3 ranks. Catches a wrong scale, a softmax over the wrong axis, a
    head mixed up, or keys gathered in the wrong order (the values would then
    be paired with the wrong keys)."""
    R, m, H, d = 3, 2, 2, 4
    rng = np.random.default_rng(30)
    q = rand_bf16(rng, (m, H, d), -1, 1)
    ks = [rand_bf16(rng, (m, H, d), -1, 1) for _ in range(R)]
    vs = [rand_bf16(rng, (m, H, d), -1, 1) for _ in range(R)]
    kf, vf, out = oracle.ag_attention(q, ks, vs)
    assert np.array_equal(kf, np.concatenate(ks)) and np.array_equal(vf, np.concatenate(vs))
    want = np.array(brute_attention(ref.decode_bf16(q).tolist(), ref.decode_bf16(kf).tolist(),
                                    ref.decode_bf16(vf).tolist()))
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)


def test_ag_attention_special_cases():
    """Equal keys -> uniform softmax -> the mean of the values; one key ->
    its value; shuffling key/value rows together leaves the output unchanged
    (attention is a set function of the key/value pairs); a key far ahead of
    the others (score gap 60) selects its value."""
    rng = np.random.default_rng(31)
    R, m, H, d = 4, 3, 2, 8
    q = rand_bf16(rng, (m, H, d), -1, 1)
    kconst = [bf16_of_ints(np.ones((m, H, d))) for _ in range(R)]
    vs = [rand_bf16(rng, (m, H, d), -1, 1) for _ in range(R)]
    _, vf, out = oracle.ag_attention(q, kconst, vs)
    assert np.allclose(out, ref.decode_bf16(vf).mean(axis=0, keepdims=True).repeat(m, 0), rtol=0, atol=1e-12)
    k1 = [rand_bf16(rng, (1, H, d), -1, 1)]
    v1 = [rand_bf16(rng, (1, H, d), -1, 1)]
    _, _, o1 = oracle.ag_attention(q, k1, v1)
    assert np.allclose(o1, np.broadcast_to(ref.decode_bf16(v1[0]), o1.shape), rtol=0, atol=1e-15)
    ks = [rand_bf16(rng, (m, H, d), -1, 1) for _ in range(R)]
    _, _, o = oracle.ag_attention(q, ks, vs)
    perm = rng.permutation(R * m)
    kf = np.concatenate(ks)[perm]
    vf = np.concatenate(vs)[perm]
    _, _, op = oracle.ag_attention(q, [kf], [vf])
    assert np.allclose(o, op, rtol=1e-12, atol=1e-13)
    # one dominant key: q = e_0 * 8, that key = e_0 * 8 * sqrt(d) (score 64 more than any other)
    qd = np.zeros((1, 1, d), np.float32); qd[0, 0, 0] = 8.0
    kd = np.zeros((5, 1, d), np.float32); kd[3, 0, 0] = 8.0 * math.sqrt(d)
    vd = rand_bf16(rng, (5, 1, d), -1, 1)
    _, _, od = oracle.ag_attention(bf16_of_ints(qd), [bf16_of_ints(kd)], [vd])
    assert np.allclose(od[0, 0], ref.decode_bf16(vd)[3, 0], rtol=0, atol=1e-20)


def test_ag_attention_grouped_heads():
    """Grouped kv heads: brute force with Hq = 6 over Hkv = 2 (G = 3; a
    head mapped to the wrong kv head fails), the result equals plain
    multi-head attention with every kv head repeated G times, and the per-row
    form used for sampled checks gives the same rows."""
    R, m, Hq, Hkv, d = 2, 3, 6, 2, 4
    rng = np.random.default_rng(32)
    q = rand_bf16(rng, (m, Hq, d), -1, 1)
    ks = [rand_bf16(rng, (m, Hkv, d), -1, 1) for _ in range(R)]
    vs = [rand_bf16(rng, (m, Hkv, d), -1, 1) for _ in range(R)]
    kf, vf, out = oracle.ag_attention(q, ks, vs)
    want = np.array(brute_attention(ref.decode_bf16(q).tolist(), ref.decode_bf16(kf).tolist(),
                                    ref.decode_bf16(vf).tolist()))
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)
    G = Hq // Hkv
    _, _, mha = oracle.ag_attention(q, [np.repeat(c, G, axis=1) for c in ks], [np.repeat(c, G, axis=1) for c in vs])
    assert np.allclose(out, mha, rtol=1e-13, atol=1e-14)
    rows = [(0, 0), (2, 5), (1, 3)]
    got = oracle.ag_attention_rows(q, kf, vf, rows)
    assert np.allclose(got, np.array([out[i, h] for i, h in rows]), rtol=1e-13, atol=1e-14)
    with pytest.raises(ValueError):
        oracle.ag_attention(rand_bf16(rng, (m, 5, d), -1, 1), ks, vs)
