"""Seeded synthetic inputs for the five tensor-parallel LLM-layer workloads.

This module is shared by the CPU oracle, the tests and the benchmark. It holds
no arithmetic of the method itself (no gather, product, reduction or routing):
it only draws random numbers and encodes them as bfloat16 bit patterns, so the
GPU path and the oracle read the very same bytes.

Recipe (the pages fix only the layer kind; shapes and seeds are the workload
definitions below):
  * generator: ``numpy.random.default_rng(seed)`` (PCG64), float64 draws;
  * float64 -> float32 by numpy's cast (round-to-nearest-even), then
    float32 -> bfloat16 by round-to-nearest-even on the low 16 bits;
  * "N(0, s)" means a normal with standard deviation s;
  * draw order: every operand in the order it is listed in the workload.

bf16 tensors are returned as ``numpy.uint16`` arrays of raw bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "AgGemmInputs", "GemmRsInputs",
    "MoeInputs", "make_ag_gemm", "make_gemm_rs", "make_moe", "make_moe_peers", "WORKLOADS",
    "workload",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as bfloat16 bits, round-to-nearest-even.

    Inputs here are finite draws, so NaN/Inf handling is only kept correct
    enough not to turn a NaN into Inf (quiet bit forced)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bits (uint16) to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw_bf16(rng: np.random.Generator, shape, dist: str, scale: float) -> np.ndarray:
    if dist == "uniform":
        v = rng.uniform(-scale, scale, size=shape)
    elif dist == "normal":
        v = rng.normal(0.0, scale, size=shape)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return f32_to_bf16_bits(v.astype(np.float32))


@dataclass
class AgGemmInputs:
    """C = gather(A_0..A_{R-1}) x B; a_chunks[r] is rank r's [m, K] shard."""
    R: int
    m: int
    K: int
    N: int
    a_chunks: List[np.ndarray]          # R x uint16 [m, K]
    b: np.ndarray                       # uint16 [K, N]
    seed: int = 0


@dataclass
class GemmRsInputs:
    """out_l = row block l of (A x B + sum of the peers' partials)."""
    R: int
    M: int
    K: int
    N: int
    local_rank: int
    a: np.ndarray                       # uint16 [M, K]
    b: np.ndarray                       # uint16 [K, N]
    peers: Dict[int, np.ndarray]        # rank s != local -> uint16 [M, N]
    seed: int = 0


@dataclass
class MoeInputs:
    """Gathered tokens routed top-k over E experts, then a per-expert GEMM."""
    R: int
    m: int
    K: int
    N: int
    E: int
    topk: int
    a_chunks: List[np.ndarray]          # R x uint16 [m, K]
    logits: np.ndarray                  # float32 [R*m, E]
    w: np.ndarray                       # uint16 [E, K, N]
    seed: int = 0


def make_ag_gemm(R: int, m: int, K: int, N: int, seed: int,
                 dist: str = "normal", scale: float = 0.02) -> AgGemmInputs:
    """Draw order: A_0 ... A_{R-1}, then B."""
    rng = np.random.default_rng(seed)
    chunks = [_draw_bf16(rng, (m, K), dist, scale) for _ in range(R)]
    b = _draw_bf16(rng, (K, N), dist, scale)
    return AgGemmInputs(R, m, K, N, chunks, b, seed)


def make_gemm_rs(R: int, M: int, K: int, N: int, seed: int, local_rank: int = 0,
                 dist: str = "normal", scale: float = 0.02,
                 peer_scale: Optional[float] = None) -> GemmRsInputs:
    """Draw order: A, B, then the peer partials P_s for s != local_rank in
    ascending s, all N(0, scale) unless ``peer_scale`` is given."""
    rng = np.random.default_rng(seed)
    a = _draw_bf16(rng, (M, K), dist, scale)
    b = _draw_bf16(rng, (K, N), dist, scale)
    ps = scale if peer_scale is None else peer_scale
    peers = {s: _draw_bf16(rng, (M, N), dist, ps) for s in range(R) if s != local_rank}
    return GemmRsInputs(R, M, K, N, local_rank, a, b, peers, seed)


def make_moe(R: int, m: int, K: int, N: int, E: int, seed: int, topk: int = 2,
             scale: float = 0.02) -> MoeInputs:
    """Draw order: A_0 ... A_{R-1} ~ N(0, scale); router logits float32
    N(0, 1) [R*m, E]; then W_0 ... W_{E-1} ~ N(0, scale) [K, N] (one expert
    at a time, so peak host memory stays near one expert's float64 draw)."""
    rng = np.random.default_rng(seed)
    chunks = [_draw_bf16(rng, (m, K), "normal", scale) for _ in range(R)]
    logits = rng.normal(0.0, 1.0, size=(R * m, E)).astype(np.float32)
    w = np.empty((E, K, N), dtype=np.uint16)
    for e in range(E):
        w[e] = _draw_bf16(rng, (K, N), "normal", scale)
    return MoeInputs(R, m, K, N, E, topk, chunks, logits, w, seed)


@dataclass
class MoeCombineInputs:
    """out_l = row block l of (TopK-Reduce of Y with gate weights w + the
    peers' combined partials)."""
    R: int
    m: int
    N: int
    topk: int
    local_rank: int
    y: np.ndarray                       # uint16 [R*m*topk, N], token-slot order
    w: np.ndarray                       # float32 [R*m, topk]
    peers: Dict[int, np.ndarray]        # rank s != local -> uint16 [R*m, N]
    seed: int = 0


def make_moe_combine(R: int, m: int, N: int, topk: int, seed: int, local_rank: int = 0,
                     scale: float = 0.02) -> MoeCombineInputs:
    """Draw order: Y ~ N(0, scale) [R*m*topk, N]; gate weights float32
    uniform [0, 0.5) [R*m, topk]; then the peer partials P_s (s != local_rank,
    ascending) ~ N(0, scale) [R*m, N]."""
    rng = np.random.default_rng(seed)
    T = R * m
    y = _draw_bf16(rng, (T * topk, N), "normal", scale)
    w = rng.uniform(0.0, 0.5, size=(T, topk)).astype(np.float32)
    peers = {s: _draw_bf16(rng, (T, N), "normal", scale) for s in range(R) if s != local_rank}
    return MoeCombineInputs(R, m, N, topk, local_rank, y, w, peers, seed)


@dataclass
class AttentionInputs:
    """Rank l's queries attend over the gathered keys / values of R ranks."""
    R: int
    m: int
    Hq: int
    Hkv: int
    d: int
    local_rank: int
    q: np.ndarray                       # uint16 [m, Hq, d], the local queries
    k_chunks: List[np.ndarray]          # R x uint16 [m, Hkv, d]
    v_chunks: List[np.ndarray]          # R x uint16 [m, Hkv, d]
    seed: int = 0


def make_attention(R: int, m: int, Hq: int, Hkv: int, d: int, seed: int, local_rank: int = 0) -> AttentionInputs:
    """Draw order: Q (local) ~ N(0, 1) [m, Hq, d]; K_0..K_{R-1}; V_0..V_{R-1}
    ([m, Hkv, d] each), all N(0, 1)."""
    rng = np.random.default_rng(seed)
    q = _draw_bf16(rng, (m, Hq, d), "normal", 1.0)
    ks = [_draw_bf16(rng, (m, Hkv, d), "normal", 1.0) for _ in range(R)]
    vs = [_draw_bf16(rng, (m, Hkv, d), "normal", 1.0) for _ in range(R)]
    return AttentionInputs(R, m, Hq, Hkv, d, local_rank, q, ks, vs, seed)


def make_attention_retrieval(R: int, m: int, Hq: int, Hkv: int, d: int, seed: int, local_rank: int = 0,
                             gain: float = 4.0):
    """Structured attention inputs in which every query picks out one key:
    K entries are +-1, V ~ N(0, 1), and query (i, h) is ``gain`` times the
    gathered key row targets[i, h] of its kv head h // (Hq / Hkv). Draw order:
    K_0..K_{R-1} signs, V_0..V_{R-1}, then the targets. Returns (inputs,
    targets [m, Hq] int64)."""
    rng = np.random.default_rng(seed)
    ks = [(rng.integers(0, 2, (m, Hkv, d)) * 2 - 1).astype(np.float32) for _ in range(R)]
    vs = [_draw_bf16(rng, (m, Hkv, d), "normal", 1.0) for _ in range(R)]
    targets = rng.integers(0, R * m, (m, Hq))
    G = Hq // Hkv
    k_full = np.concatenate(ks)
    heads = np.arange(Hq) // G
    q = gain * k_full[targets, heads[None, :], :]
    as_bits = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # exact: +-1, +-gain
    x = AttentionInputs(R, m, Hq, Hkv, d, local_rank, as_bits(q), [as_bits(c) for c in ks], vs, seed)
    return x, targets


def make_moe_peers(R: int, m: int, N: int, seed: int, local_rank: int = 0, scale: float = 0.02) -> Dict[int, np.ndarray]:
    """The other ranks' combined partials of an MoE layer (stand-ins for
    what the peers' TopK-Reduce would send): draw order P_s for s !=
    local_rank ascending, N(0, scale) [R*m, N], from their own seed."""
    rng = np.random.default_rng(seed)
    return {s: _draw_bf16(rng, (R * m, N), "normal", scale) for s in range(R) if s != local_rank}


@dataclass(frozen=True)
class Workload:
    name: str
    op: str            # "ag_gemm" | "gemm_rs" | "ag_grouped_gemm" | "moe_combine_rs" | "ag_attention"
    params: dict = field(default_factory=dict)

    def flops(self) -> float:
        p = self.params
        if self.op == "ag_gemm":
            return 2.0 * p["R"] * p["m"] * p["K"] * p["N"]
        if self.op == "gemm_rs":
            return 2.0 * p["M"] * p["K"] * p["N"]
        if self.op == "moe_combine_rs":
            return 2.0 * p["R"] * p["m"] * p["topk"] * p["N"]
        if self.op == "ag_attention":
            return 4.0 * p["m"] * p["R"] * p["m"] * p["Hq"] * p["d"]
        return 2.0 * p["R"] * p["m"] * p["topk"] * p["K"] * p["N"]

    def make(self, **over):
        p = dict(self.params)
        p.update(over)
        if self.op == "ag_gemm":
            return make_ag_gemm(p["R"], p["m"], p["K"], p["N"], p["seed"],
                                p.get("dist", "normal"), p.get("scale", 0.02))
        if self.op == "gemm_rs":
            return make_gemm_rs(p["R"], p["M"], p["K"], p["N"], p["seed"],
                                p.get("local_rank", 0))
        if self.op == "moe_combine_rs":
            return make_moe_combine(p["R"], p["m"], p["N"], p["topk"], p["seed"], p.get("local_rank", 0))
        if self.op == "ag_attention":
            return make_attention(p["R"], p["m"], p["Hq"], p["Hkv"], p["d"], p["seed"], p.get("local_rank", 0))
        return make_moe(p["R"], p["m"], p["K"], p["N"], p["E"], p["seed"], p["topk"])


# The workloads: one GPU's share of tensor-parallel (TP=8) LLM FFN layers
# (8B-class: hidden 4096, FFN 14336; 70B-class: hidden 8192, FFN 28672) plus a
# tiny case, a top-2 MoE layer with 32 experts, that layer's TopK-Reduce tail,
# and a context-parallel attention layer.
WORKLOADS = {
    "ag_gemm_tiny": Workload("ag_gemm_tiny", "ag_gemm",
                             dict(R=4, m=128, K=256, N=256, seed=0, dist="uniform", scale=1.0)),
    "ag_gemm_8b": Workload("ag_gemm_8b", "ag_gemm",
                           dict(R=8, m=512, K=4096, N=1792, seed=1)),
    "gemm_rs_8b": Workload("gemm_rs_8b", "gemm_rs",
                           dict(R=8, M=4096, K=1792, N=4096, seed=2, local_rank=0)),
    "ag_gemm_70b": Workload("ag_gemm_70b", "ag_gemm",
                            dict(R=8, m=1024, K=8192, N=3584, seed=3)),
    "ag_moe": Workload("ag_moe", "ag_grouped_gemm",
                       dict(R=8, m=512, K=4096, N=1792, E=32, topk=2, seed=4)),
    # the MoE tail: TopK-Reduce of the grouped GEMM's output rows, then the
    # ReduceScatter of the combined token rows (row block 0 kept)
    "moe_combine_rs": Workload("moe_combine_rs", "moe_combine_rs",
                               dict(R=8, m=512, N=1792, topk=2, seed=5, local_rank=0)),
    # the whole MoE layer chain: ag_moe's inputs (seed 4), then the grouped
    # output's TopK-Reduce and the ReduceScatter against the peers' combined
    # partials (seed 7)
    "ag_moe_layer": Workload("ag_moe_layer", "ag_grouped_gemm",
                             dict(R=8, m=512, K=4096, N=1792, E=32, topk=2, seed=4, peer_seed=7, local_rank=0)),
    # AllGather-KV attention: a 16384-token context over 8 ranks (2048 tokens
    # each), 32 query heads over 8 kv heads of 128 (an 8B-class GQA layer),
    # every query over the whole context
    "ag_attention": Workload("ag_attention", "ag_attention",
                             dict(R=8, m=2048, Hq=32, Hkv=8, d=128, seed=6, local_rank=0)),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]
