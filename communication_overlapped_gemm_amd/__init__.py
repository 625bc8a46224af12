"""Communication-overlapped GEMM for AMD Instinct MI355X (gfx950).

Fused tile-centric AllGather-GEMM, GEMM-ReduceScatter, AllGather + MoE
grouped GEMM, MoE TopK-Reduce + ReduceScatter and AllGather-KV attention as
hand-written HIP kernels behind a C ABI (include/ocg.h). This
package is the thin Python binding: it loads libocg.so (raising if it is not
built -- there is no fallback) and marshals torch tensors to the C calls.
"""
from ._lib import (  # noqa: F401
    Config, TraceRec, OcgError, default_config, status_string, lib, LIB_PATH, EXPORTS,
    OP_AG_GEMM, OP_GEMM_RS, OP_AG_GROUPED_GEMM, OP_MOE_COMBINE_RS, OP_AG_ATTENTION, MODE_FUSED, MODE_GEMM_ONLY, MODE_COPY_ONLY,
    TRANSFER_AUTO, TRANSFER_INLINE, TRANSFER_SIDE,
    TILE_AUTO, TILE_256x224, TILE_128x224, TILE_128x256, TILE_128x128, TILE_256x256, TILE_320x224, TILE_288x224,
    OK, ERR_INVALID_ARG, ERR_UNSUPPORTED_SHAPE, ERR_WORKSPACE_TOO_SMALL, ERR_HIP, ERR_TIMEOUT, ERR_NO_DEVICE,
)
from .ops import (  # noqa: F401
    Workspace, ag_gemm, gemm_rs, ag_grouped_gemm, moe_combine_rs, ag_attention, signal, plan_info, plan_task, handle,
    plan_ag, ag_gemm_noalloc, gemm_rs_push, ag_moe_layer,
)
