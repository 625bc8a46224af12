"""CPU oracle for the fused AllGather-GEMM / GEMM-ReduceScatter / AllGather +
MoE grouped-GEMM hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call, link
or execute anything in this package: only the test suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

It is a plain, slow, obviously-correct float64 restatement of what the pages
define (TileLink: Generating Efficient Compute-Communication Overlapping Kernels
using Tile-Centric Primitives, MLSys 2025 talk summary; Triton-distributed
report abstract). It shares no code with the HIP library: it has its own bf16
codec, its own routing and its own schedule re-derivation.

Parity status per function (see each docstring for the pin):
  * ag_gemm, gemm_rs, reduce_fixed_order, route_topk, sort_by_expert,
    ag_grouped_gemm, topk_combine, moe_combine_rs, ag_attention,
    ag_attention_rows, schedule re-derivations:
    pinned by the ``-m "not gpu"`` tests (brute force, closed forms,
    identities, library special cases).
"""
from .reference import (  # noqa: F401
    decode_bf16, encode_bf16_rne, ag_gemm, ag_gemm_entries, ag_gemm_block, gemm_rs,
    gemm_rs_entries, reduce_fixed_order, route_topk, sort_by_expert,
    ag_grouped_gemm, ag_grouped_gemm_entries, topk_combine, moe_combine_rs, ag_attention,
    ag_attention_rows,
)
from . import schedule  # noqa: F401
