"""Torch-facing wrappers of the C ABI: validate tensors, allocate outputs with
torch, pass raw pointers and the current HIP stream. Every step of the path
runs in the HIP library; nothing here computes."""
from __future__ import annotations

import ctypes as C
from typing import Dict, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import Config, check, default_config, lib

_handles: Dict[int, C.c_void_p] = {}
_workspaces: Dict[tuple, "Workspace"] = {}


def _device_index(t: Optional[torch.Tensor] = None) -> int:
    return t.device.index if t is not None else torch.cuda.current_device()


def handle(device: Optional[int] = None) -> C.c_void_p:
    dev = torch.cuda.current_device() if device is None else device
    h = _handles.get(dev)
    if h is None:
        h = C.c_void_p()
        check(lib.ocg_create(dev, C.byref(h)), "ocg_create")
        _handles[dev] = h
    return h


def _stream(stream: Optional[torch.cuda.Stream]) -> torch.cuda.Stream:
    return stream if stream is not None else torch.cuda.current_stream()


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    return _stream(stream).cuda_stream


class Workspace:
    """Caller-owned scratch of one operation shape (flags, tickets, routing
    tables), cleared once by the library's fill kernel on `stream` (default:
    the current stream) -- the stream its calls run on. Calls that share a
    workspace must be ordered on one stream."""

    def __init__(self, op: int, R: int, m: int, K: int, N: int, E: int = 0, topk: int = 0,
                 device: Optional[int] = None, stream=None, config: Optional[Config] = None):
        dev = torch.cuda.current_device() if device is None else device
        # sized for calls with `config` (default: the default configuration)
        n = lib.ocg_workspace_bytes_for(handle(dev), op, R, m, K, N, E, topk,
                                        C.byref(config) if config is not None else None)
        if n == 0:
            raise _lib.OcgError(_lib.ERR_UNSUPPORTED_SHAPE, "ocg_workspace_bytes_for")
        self.buf = torch.empty(n, dtype=torch.uint8, device=f"cuda:{dev}")
        self.nbytes = n
        self.device = dev
        s = _stream(stream)
        cur = torch.cuda.current_stream(dev)
        if s != cur:
            # the block came from the current stream's pool: order the clear
            # after that stream's earlier work, and keep the block off the pool
            # while `s` may still use it
            s.wait_stream(cur)
            self.buf.record_stream(s)
        check(lib.ocg_workspace_init(handle(dev), self.ptr, n, s.cuda_stream), "ocg_workspace_init")

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()

    def check(self) -> None:
        """Raise if a flag wait of an earlier call timed out (synchronises)."""
        torch.cuda.synchronize(self.device)
        check(lib.ocg_check(handle(self.device), self.ptr), "ocg_check")

    @classmethod
    def cached(cls, op, R, m, K, N, E=0, topk=0, device=None, stream=None, config=None):
        """One workspace per (shape, device, stream, size the call's
        configuration needs -- an AG-GEMM plan that splits K needs room for
        the halves' sums): calls of one shape on different streams do not
        share counters."""
        dev = torch.cuda.current_device() if device is None else device
        sp = _stream_ptr(stream)
        n = lib.ocg_workspace_bytes_for(handle(dev), op, R, m, K, N, E, topk,
                                        C.byref(config) if config is not None else None)
        key = (op, R, m, K, N, E, topk, dev, sp, n)
        ws = _workspaces.get(key)
        if ws is None:
            ws = _workspaces[key] = cls(op, R, m, K, N, E, topk, dev, stream, config)
        return ws


def _check_bf16(t: torch.Tensor, name: str, shape=None) -> None:
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 CUDA tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _cfg(config: Optional[Config], **kw) -> Config:
    c = config if config is not None else default_config()
    for k, v in kw.items():
        if v is not None:
            setattr(c, k, v)
    return c


def ag_gemm(a_chunks: Sequence[torch.Tensor], b: torch.Tensor, local_rank: int = 0, *,
            a_gathered: Optional[torch.Tensor] = None, c: Optional[torch.Tensor] = None,
            workspace: Optional[Workspace] = None, config: Optional[Config] = None,
            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Fused AllGather-GEMM. Returns (c, a_gathered)."""
    R = len(a_chunks)
    m, K = a_chunks[0].shape
    N = b.shape[1]
    for r, t in enumerate(a_chunks):
        _check_bf16(t, f"a_chunks[{r}]", (m, K))
    _check_bf16(b, "b", (K, N))
    dev = b.device
    if a_gathered is None:
        a_gathered = torch.empty((R * m, K), dtype=torch.bfloat16, device=dev)
    if c is None:
        c = torch.empty((R * m, N), dtype=torch.bfloat16, device=dev)
    _check_bf16(a_gathered, "a_gathered", (R * m, K))
    _check_bf16(c, "c", (R * m, N))
    cfg = _cfg(config)
    ws = workspace or Workspace.cached(_lib.OP_AG_GEMM, R, m, K, N, device=dev.index, stream=stream, config=cfg)
    ptrs = (C.c_void_p * R)(*[t.data_ptr() for t in a_chunks])
    check(lib.ocg_ag_gemm(handle(dev.index), ptrs, R, local_rank, m, K, b.data_ptr(), N, a_gathered.data_ptr(),
                          c.data_ptr(), ws.ptr, ws.nbytes, C.byref(cfg), _stream_ptr(stream)), "ocg_ag_gemm")
    return c, a_gathered


def ag_gemm_noalloc(a_chunks: Sequence[torch.Tensor], b: torch.Tensor, local_rank: int, a_gathered: torch.Tensor,
                    c: torch.Tensor, *, config: Optional[Config] = None, stream=None) -> None:
    """Fused AllGather-GEMM through the no-allocation entry point: the caller
    passes every output; the library's per-GPU scratch stands in for the
    workspace (calls that overlap on one GPU race)."""
    R = len(a_chunks)
    m, K = a_chunks[0].shape
    N = b.shape[1]
    for r, t in enumerate(a_chunks):
        _check_bf16(t, f"a_chunks[{r}]", (m, K))
    _check_bf16(b, "b", (K, N))
    _check_bf16(a_gathered, "a_gathered", (R * m, K))
    _check_bf16(c, "c", (R * m, N))
    ptrs = (C.c_void_p * R)(*[t.data_ptr() for t in a_chunks])
    cfg = _cfg(config)
    check(lib.ocg_ag_gemm_noalloc(handle(b.device.index), ptrs, R, local_rank, m, K, b.data_ptr(), N,
                                  a_gathered.data_ptr(), c.data_ptr(), C.byref(cfg), _stream_ptr(stream)),
          "ocg_ag_gemm_noalloc")


def gemm_rs(a: torch.Tensor, b: torch.Tensor, peer_partials: Sequence[Optional[torch.Tensor]], local_rank: int = 0,
            *, partial: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            workspace: Optional[Workspace] = None, config: Optional[Config] = None,
            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Fused GEMM-ReduceScatter (one rank's share). Returns (partial, out)."""
    R = len(peer_partials)
    M, K = a.shape
    N = b.shape[1]
    _check_bf16(a, "a")
    _check_bf16(b, "b", (K, N))
    ptrs = (C.c_void_p * R)()
    for s, p in enumerate(peer_partials):
        if s == local_rank:
            continue
        _check_bf16(p, f"peer_partials[{s}]", (M, N))
        ptrs[s] = p.data_ptr()
    dev = a.device
    if partial is None:
        partial = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if out is None:
        out = torch.empty((M // R, N), dtype=torch.bfloat16, device=dev)
    _check_bf16(partial, "partial", (M, N))
    _check_bf16(out, "out", (M // R, N))
    ws = workspace or Workspace.cached(_lib.OP_GEMM_RS, R, M, K, N, device=dev.index, stream=stream)
    cfg = _cfg(config)
    check(lib.ocg_gemm_rs(handle(dev.index), a.data_ptr(), b.data_ptr(), M, K, N, R, local_rank, ptrs,
                          partial.data_ptr(), out.data_ptr(), ws.ptr, ws.nbytes, C.byref(cfg),
                          _stream_ptr(stream)), "ocg_gemm_rs")
    return partial, out


def gemm_rs_push(a: torch.Tensor, b: torch.Tensor, recv: Sequence[torch.Tensor], recv_flags: Sequence[torch.Tensor],
                 flag_value: int, local_rank: int = 0, *, out: Optional[torch.Tensor] = None,
                 workspace: Optional[Workspace] = None, config: Optional[Config] = None, stream=None) -> torch.Tensor:
    """GEMM-ReduceScatter with push transfers: recv[r] bf16 [R, M/R, N] and
    recv_flags[r] int32 [R, tiles per row block] of every rank r (stand-ins
    on one GPU). Returns out [M/R, N]."""
    R = len(recv)
    M, K = a.shape
    N = b.shape[1]
    _check_bf16(a, "a")
    _check_bf16(b, "b", (K, N))
    if len(recv_flags) != R:
        raise ValueError("one receive flag array per rank")
    for r in range(R):
        _check_bf16(recv[r], f"recv[{r}]", (R, M // R, N))
        if recv_flags[r].dtype not in (torch.int32, torch.uint32) or not recv_flags[r].is_contiguous():
            raise ValueError("recv_flags must be contiguous 32-bit tensors")
    dev = a.device
    if out is None:
        out = torch.empty((M // R, N), dtype=torch.bfloat16, device=dev)
    _check_bf16(out, "out", (M // R, N))
    ws = workspace or Workspace.cached(_lib.OP_GEMM_RS, R, M, K, N, device=dev.index, stream=stream)
    rp = (C.c_void_p * R)(*[t.data_ptr() for t in recv])
    fp = (C.c_void_p * R)(*[t.data_ptr() for t in recv_flags])
    cfg = _cfg(config)
    check(lib.ocg_gemm_rs_push(handle(dev.index), a.data_ptr(), b.data_ptr(), M, K, N, R, local_rank, rp, fp,
                               flag_value & 0xFFFFFFFF, out.data_ptr(), ws.ptr, ws.nbytes, C.byref(cfg),
                               _stream_ptr(stream)), "ocg_gemm_rs_push")
    return out


def ag_grouped_gemm(a_chunks: Sequence[torch.Tensor], logits: torch.Tensor, w: torch.Tensor, topk: int = 2,
                    local_rank: int = 0, *, workspace: Optional[Workspace] = None,
                    config: Optional[Config] = None, stream=None, outputs: Optional[dict] = None) -> dict:
    """AllGather + top-k routing + grouped GEMM. Returns a dict with out,
    a_gathered, topk_ids, topk_w, perm and expert_offsets."""
    R = len(a_chunks)
    m, K = a_chunks[0].shape
    E, K2, N = w.shape
    if K2 != K:
        raise ValueError("w must be [E, K, N]")
    for r, t in enumerate(a_chunks):
        _check_bf16(t, f"a_chunks[{r}]", (m, K))
    _check_bf16(w, "w")
    if logits.dtype != torch.float32 or not logits.is_contiguous() or tuple(logits.shape) != (R * m, E):
        raise ValueError("logits must be a contiguous float32 [R*m, E] CUDA tensor")
    dev = w.device
    T = R * m
    o = dict(outputs or {})
    o.setdefault("a_gathered", torch.empty((T, K), dtype=torch.bfloat16, device=dev))
    o.setdefault("topk_ids", torch.empty((T, topk), dtype=torch.int32, device=dev))
    o.setdefault("topk_w", torch.empty((T, topk), dtype=torch.float32, device=dev))
    o.setdefault("perm", torch.empty((T * topk,), dtype=torch.int32, device=dev))
    o.setdefault("expert_offsets", torch.empty((E + 1,), dtype=torch.int32, device=dev))
    o.setdefault("out", torch.empty((T * topk, N), dtype=torch.bfloat16, device=dev))
    ws = workspace or Workspace.cached(_lib.OP_AG_GROUPED_GEMM, R, m, K, N, E, topk, device=dev.index, stream=stream)
    ptrs = (C.c_void_p * R)(*[t.data_ptr() for t in a_chunks])
    cfg = _cfg(config)
    check(lib.ocg_ag_grouped_gemm(handle(dev.index), ptrs, R, local_rank, m, K, logits.data_ptr(), E, topk,
                                  w.data_ptr(), N, o["a_gathered"].data_ptr(), o["topk_ids"].data_ptr(),
                                  o["topk_w"].data_ptr(), o["perm"].data_ptr(), o["expert_offsets"].data_ptr(),
                                  o["out"].data_ptr(), ws.ptr, ws.nbytes, C.byref(cfg), _stream_ptr(stream)),
          "ocg_ag_grouped_gemm")
    return o


def ag_moe_layer(a_chunks: Sequence[torch.Tensor], logits: torch.Tensor, w: torch.Tensor,
                 peer_partials: Sequence[Optional[torch.Tensor]], topk: int = 2, local_rank: int = 0, *,
                 workspace: Optional[Workspace] = None, config: Optional[Config] = None, stream=None,
                 outputs: Optional[dict] = None) -> dict:
    """The MoE layer chain in one call: AllGather + routing + grouped GEMM
    (y, token-slot order) and TopK-Reduce + ReduceScatter of y (partial,
    out). Returns a dict with out, partial, y, a_gathered, topk_ids, topk_w,
    perm and expert_offsets."""
    R = len(a_chunks)
    m, K = a_chunks[0].shape
    E, K2, N = w.shape
    if K2 != K:
        raise ValueError("w must be [E, K, N]")
    for r, t in enumerate(a_chunks):
        _check_bf16(t, f"a_chunks[{r}]", (m, K))
    _check_bf16(w, "w")
    if logits.dtype != torch.float32 or not logits.is_contiguous() or tuple(logits.shape) != (R * m, E):
        raise ValueError("logits must be a contiguous float32 [R*m, E] CUDA tensor")
    if len(peer_partials) != R:
        raise ValueError("one peer partial entry per rank")
    T = R * m
    pp = (C.c_void_p * R)()
    for s_, p_ in enumerate(peer_partials):
        if s_ == local_rank:
            continue
        _check_bf16(p_, f"peer_partials[{s_}]", (T, N))
        pp[s_] = p_.data_ptr()
    dev = w.device
    o = dict(outputs or {})
    o.setdefault("a_gathered", torch.empty((T, K), dtype=torch.bfloat16, device=dev))
    o.setdefault("topk_ids", torch.empty((T, topk), dtype=torch.int32, device=dev))
    o.setdefault("topk_w", torch.empty((T, topk), dtype=torch.float32, device=dev))
    o.setdefault("perm", torch.empty((T * topk,), dtype=torch.int32, device=dev))
    o.setdefault("expert_offsets", torch.empty((E + 1,), dtype=torch.int32, device=dev))
    o.setdefault("y", torch.empty((T * topk, N), dtype=torch.bfloat16, device=dev))
    o.setdefault("partial", torch.empty((T, N), dtype=torch.bfloat16, device=dev))
    o.setdefault("out", torch.empty((m, N), dtype=torch.bfloat16, device=dev))
    ws = workspace or Workspace.cached(_lib.OP_AG_GROUPED_GEMM, R, m, K, N, E, topk, device=dev.index, stream=stream)
    ptrs = (C.c_void_p * R)(*[t.data_ptr() for t in a_chunks])
    cfg = _cfg(config)
    check(lib.ocg_ag_moe_layer(handle(dev.index), ptrs, R, local_rank, m, K, logits.data_ptr(), E, topk,
                               w.data_ptr(), N, pp, o["a_gathered"].data_ptr(), o["topk_ids"].data_ptr(),
                               o["topk_w"].data_ptr(), o["perm"].data_ptr(), o["expert_offsets"].data_ptr(),
                               o["y"].data_ptr(), o["partial"].data_ptr(), o["out"].data_ptr(), ws.ptr, ws.nbytes,
                               C.byref(cfg), _stream_ptr(stream)), "ocg_ag_moe_layer")
    return o


def moe_combine_rs(y: torch.Tensor, topk_w: torch.Tensor, peer_partials: Sequence[Optional[torch.Tensor]],
                   local_rank: int = 0, *, partial: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   workspace: Optional[Workspace] = None, config: Optional[Config] = None,
                   stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """MoE TopK-Reduce + ReduceScatter (one rank's share): y [T*topk, N] bf16
    in token-slot order, topk_w [T, topk] fp32, R = len(peer_partials) peer
    combined partials [T, N]. Returns (partial [T, N], out [T/R, N])."""
    R = len(peer_partials)
    _check_bf16(y, "y")
    if topk_w.dtype != torch.float32 or not topk_w.is_contiguous() or topk_w.dim() != 2:
        raise ValueError("topk_w must be a contiguous float32 [T, topk] CUDA tensor")
    T, topk = topk_w.shape
    N = y.shape[1]
    if tuple(y.shape) != (T * topk, N) or T % R:
        raise ValueError("y must be [T*topk, N] with T a multiple of R")
    m = T // R
    ptrs = (C.c_void_p * R)()
    for s, p in enumerate(peer_partials):
        if s == local_rank:
            continue
        _check_bf16(p, f"peer_partials[{s}]", (T, N))
        ptrs[s] = p.data_ptr()
    dev = y.device
    if partial is None:
        partial = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    if out is None:
        out = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
    _check_bf16(partial, "partial", (T, N))
    _check_bf16(out, "out", (m, N))
    ws = workspace or Workspace.cached(_lib.OP_MOE_COMBINE_RS, R, m, 0, N, 0, topk, device=dev.index, stream=stream)
    cfg = _cfg(config)
    check(lib.ocg_moe_combine_rs(handle(dev.index), y.data_ptr(), topk_w.data_ptr(), R, local_rank, m, N, topk, ptrs,
                                 partial.data_ptr(), out.data_ptr(), ws.ptr, ws.nbytes, C.byref(cfg),
                                 _stream_ptr(stream)), "ocg_moe_combine_rs")
    return partial, out


def ag_attention(q: torch.Tensor, k_chunks: Sequence[torch.Tensor], v_chunks: Sequence[torch.Tensor],
                 local_rank: int = 0, *, k_gathered: Optional[torch.Tensor] = None,
                 v_gathered: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 workspace: Optional[Workspace] = None, config: Optional[Config] = None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """AllGather-KV attention (one context-parallel rank's share): q [m, Hq, d]
    bf16, R = len(k_chunks) key / value chunks [m, Hkv, d]. Returns
    (out [m, Hq, d], k_gathered [R*m, Hkv, d], v_gathered [R*m, Hkv, d])."""
    R = len(k_chunks)
    if len(v_chunks) != R:
        raise ValueError("k_chunks and v_chunks must have one entry per rank")
    _check_bf16(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [m, Hq, d]")
    m, Hq, d = q.shape
    Hkv = k_chunks[0].shape[1]
    for r in range(R):
        _check_bf16(k_chunks[r], f"k_chunks[{r}]", (m, Hkv, d))
        _check_bf16(v_chunks[r], f"v_chunks[{r}]", (m, Hkv, d))
    dev = q.device
    if k_gathered is None:
        k_gathered = torch.empty((R * m, Hkv, d), dtype=torch.bfloat16, device=dev)
    if v_gathered is None:
        v_gathered = torch.empty((R * m, Hkv, d), dtype=torch.bfloat16, device=dev)
    if out is None:
        out = torch.empty((m, Hq, d), dtype=torch.bfloat16, device=dev)
    _check_bf16(k_gathered, "k_gathered", (R * m, Hkv, d))
    _check_bf16(v_gathered, "v_gathered", (R * m, Hkv, d))
    _check_bf16(out, "out", (m, Hq, d))
    ws = workspace or Workspace.cached(_lib.OP_AG_ATTENTION, R, m, Hq, Hkv, device=dev.index, stream=stream)
    kp = (C.c_void_p * R)(*[t.data_ptr() for t in k_chunks])
    vp = (C.c_void_p * R)(*[t.data_ptr() for t in v_chunks])
    cfg = _cfg(config)
    check(lib.ocg_ag_attention(handle(dev.index), q.data_ptr(), kp, vp, R, local_rank, m, Hq, Hkv, d,
                               k_gathered.data_ptr(), v_gathered.data_ptr(), out.data_ptr(), ws.ptr, ws.nbytes,
                               C.byref(cfg), _stream_ptr(stream)), "ocg_ag_attention")
    return out, k_gathered, v_gathered


def signal(flags: torch.Tensor, value: int, stream=None) -> None:
    """Peer-notify stand-in: write `value` into every uint32 of `flags`."""
    if flags.dtype not in (torch.int32, torch.uint32) or not flags.is_contiguous():
        raise ValueError("flags must be a contiguous 32-bit tensor")
    check(lib.ocg_signal(flags.data_ptr(), flags.numel(), value & 0xFFFFFFFF, _stream_ptr(stream)), "ocg_signal")


def plan_info(op: int, R: int, local_rank: int, m: int, K: int, N: int, config: Optional[Config] = None,
              E: int = 0, topk: int = 0, handle=None) -> dict:
    """Host-only: the resolved tile/slab/copy plan of a call (E, topk: the
    grouped GEMM's experts and picks per token). handle=None plans for a
    full 256-CU MI355X without touching a device."""
    out = _lib.I64x8()
    cfg = _cfg(config)
    check(lib.ocg_plan_info(handle, op, R, local_rank, m, K, N, E, topk, C.byref(cfg), out), "ocg_plan_info")
    keys = ["tile", "BM", "BN", "slab_rows", "copy_rows", "n_copy_or_strips", "n_tiles", "n_slabs_or_strip_rows"]
    return dict(zip(keys, list(out)))


def plan_ag(R: int, local_rank: int, m: int, K: int, N: int, config: Optional[Config] = None, handle=None) -> dict:
    """Host-only: AG-GEMM K-slab width, K-slab count, transfer mode and grids."""
    out = _lib.I64x8()
    cfg = _cfg(config)
    check(lib.ocg_plan_ag(handle, R, local_rank, m, K, N, C.byref(cfg), out), "ocg_plan_ag")
    return dict(kslab_cols=out[0], nks=out[1], transfer=out[2], gemm_grid=out[3], side_grid=out[4],
                n_inline=out[5], rows_per_round=out[6], split_k=out[7])


def plan_task(op: int, R: int, local_rank: int, m: int, K: int, N: int, ticket: int,
              config: Optional[Config] = None, handle=None) -> list:
    """Host-only: the task a ticket names (see ocg_plan_task)."""
    out = _lib.I64x8()
    cfg = _cfg(config)
    check(lib.ocg_plan_task(handle, op, R, local_rank, m, K, N, C.byref(cfg), ticket, out), "ocg_plan_task")
    return list(out)
