"""Helpers shared by the GPU parity tests: moving bf16 bit patterns to and from
the device, the tolerance gate, and reading the schedule trace."""
from __future__ import annotations

import ctypes as C
import sys

import numpy as np
import torch

from oracle import reference as ref

NAN_BF16 = 0x7FC0


def say(*a):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print(*a, file=sys.stderr, flush=True)


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def poison(shape, device="cuda") -> torch.Tensor:
    return torch.full(shape, NAN_BF16, dtype=torch.int16, device=device).view(torch.bfloat16)


def assert_gate(got_bits: np.ndarray, want: np.ndarray, what: str, tight: bool = True, extra=None) -> dict:
    """The acceptance gate |err| <= 2e-2 * max(1, |ref|) on every element, plus
    tighter diagnostics: relative Frobenius error <= 5e-3 and
    |err| <= 2^-7 |ref| + 1e-3 rms(ref) + extra (one bf16 ulp plus
    accumulation noise; ``extra`` is a per-element allowance for intermediate
    roundings a reading prescribes)."""
    got = ref.decode_bf16(got_bits)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite outputs"
    err = np.abs(got - want)
    gate = 2e-2 * np.maximum(1.0, np.abs(want))
    bad = err > gate
    assert not bad.any(), f"{what}: {bad.sum()} elements outside the gate, worst {err.max():.3e}"
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    stats = dict(max_abs=float(err.max()) if err.size else 0.0, rms_ref=rms,
                 rel_fro=float(np.linalg.norm(err) / max(np.linalg.norm(want), 1e-300)))
    if tight and want.size:
        assert stats["rel_fro"] <= 5e-3, f"{what}: relative Frobenius error {stats['rel_fro']:.3e}"
        lim = 2.0 ** -7 * np.abs(want) + 1e-3 * rms + (0.0 if extra is None else extra)
        nt = int((err > lim).sum())
        assert nt == 0, f"{what}: {nt} elements beyond one bf16 ulp + noise (worst {err.max():.3e})"
    return stats


TRACE_DTYPE = np.dtype([("ticket", "<u4"), ("kind", "<u4"), ("a", "<u4"), ("b", "<u4"), ("c", "<u4"),
                        ("d", "<u4"), ("hw", "<u4"), ("epoch", "<u4"), ("t_start", "<u8"), ("t_ready", "<u8"),
                        ("t_end", "<u8"), ("flag_seen", "<u4"), ("queue", "<u4"), ("cycles", "<u8"),
                        ("wait_ticks", "<u4"), ("pad", "<u4")])
REC = TRACE_DTYPE.itemsize
assert REC == 80


class Trace:
    def __init__(self, capacity: int):
        self.capacity = capacity
        self.buf = torch.zeros(capacity * REC, dtype=torch.uint8, device="cuda")

    def attach(self, cfg):
        cfg.trace = self.buf.data_ptr()
        cfg.trace_capacity = self.capacity
        return cfg

    def read(self, n: int) -> np.ndarray:
        torch.cuda.synchronize()
        return self.buf[: n * REC].cpu().numpy().view(TRACE_DTYPE)
