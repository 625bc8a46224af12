"""The no-allocation entry point (ocg_ag_gemm_noalloc, for callers that
cannot allocate) against ocg_ag_gemm, through the C ABI: two calls in a row
on the GPU's one scratch array, the second with a smaller input, in both
transfer modes. The gathered buffer and C must be bit-identical to
ocg_ag_gemm's (same kernels, same tile arithmetic) and C within the gate of
the float64 oracle; a shape whose workspace exceeds the scratch is
rejected."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_gate, poison, say, to_bits, to_dev

pytestmark = pytest.mark.gpu

CALLS = [
    # R, m, K, N, local, transfer -- the second call of each pair is smaller
    (4, 256, 1024, 448, 1, 1),
    (3, 100, 256, 200, 2, 1),
    (8, 96, 512, 232, 5, 0),
    (2, 40, 128, 72, 0, 0),
]


def test_noalloc_matches_ag_gemm(ocg):
    for i, (R, m, K, N, local, transfer) in enumerate(CALLS):
        x = workloads.make_ag_gemm(R, m, K, N, seed=300 + i, dist="normal", scale=0.02)
        chunks = [to_dev(a) for a in x.a_chunks]
        b = to_dev(x.b)
        # split_k = 1: the same kernels on both sides (ocg_ag_gemm may split K
        # where the scratch has no room for the halves' sums)
        cfg = ocg.default_config(transfer=transfer, split_k=1)
        say("ag_gemm reference call", i, R, m, K, N, local, transfer)
        ag_ref, c_ref = poison((R * m, K)), poison((R * m, N))
        ws = ocg.Workspace(ocg.OP_AG_GEMM, R, m, K, N)
        ocg.ag_gemm(chunks, b, local, a_gathered=ag_ref, c=c_ref, workspace=ws, config=cfg)
        say("ag_gemm_noalloc call", i)
        ag, c = poison((R * m, K)), poison((R * m, N))
        ocg.ag_gemm_noalloc(chunks, b, local, ag, c, config=cfg)
        torch.cuda.synchronize()
        ws.check()
        assert np.array_equal(to_bits(ag), to_bits(ag_ref)), f"call {i}: gathered buffers differ"
        assert np.array_equal(to_bits(c), to_bits(c_ref)), f"call {i}: outputs differ"
        a_full, want = oracle.ag_gemm(x.a_chunks, x.b)
        assert np.array_equal(to_bits(ag), a_full)
        assert_gate(to_bits(c), want, f"noalloc call {i}")
        # the automatic configuration: split only where the scratch holds the sums
        say("ag_gemm_noalloc default config", i)
        ag, c = poison((R * m, K)), poison((R * m, N))
        ocg.ag_gemm_noalloc(chunks, b, local, ag, c, config=ocg.default_config(transfer=transfer))
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(ag), a_full)
        assert_gate(to_bits(c), want, f"noalloc default call {i}")


def test_noalloc_rejects_shapes_beyond_the_scratch(ocg):
    from communication_overlapped_gemm_amd import _lib
    # 16 ranks x 4096 rows x K 8192: 128 Ki flags of 8 bytes, more than the 1 MiB scratch
    R, m, K, N = 16, 4096, 8192, 256
    assert _lib.lib.ocg_workspace_bytes(None, ocg.OP_AG_GEMM, R, m, K, N, 0, 0) > (1 << 20)
    t = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    ptrs = (C.c_void_p * R)(*([t.data_ptr()] * R))
    cfg = ocg.default_config()
    rc = _lib.lib.ocg_ag_gemm_noalloc(ocg.handle(), ptrs, R, 0, m, K, t.data_ptr(), N, t.data_ptr(), t.data_ptr(),
                                      C.byref(cfg), None)
    assert rc == ocg.ERR_WORKSPACE_TOO_SMALL
