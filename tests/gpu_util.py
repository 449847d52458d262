"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from input_dependent_short_amd import binding
from input_dependent_short_amd.inputs import to_f64

TOL = {"fp32": 1e-5, "bf16": 2e-2}
GUARD = 256  # canary elements before and after every output


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def normwise_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max_i |gpu_i - ref_i| / max_i |ref_i| (0 for empty)."""
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(gpu.astype(np.float64) - ref)))
    return err / scale if scale > 0 else err


class Guarded:
    """Output buffer with NaN-poisoned body and sentinel guard bands."""

    SENTINEL = -1536.0  # exact in bf16

    def __init__(self, shape, dtype, device="cuda"):
        n = int(np.prod(shape))
        self.buf = torch.full((n + 2 * GUARD,), self.SENTINEL, dtype=dtype, device=device)
        self.buf[GUARD:GUARD + n] = float("nan")
        self.n = n
        self.t = self.buf[GUARD:GUARD + n].view(*shape)

    def check_guards(self, name: str) -> None:
        b = self.buf.float().cpu()
        assert torch.all(b[:GUARD] == self.SENTINEL), f"{name}: write before the buffer"
        assert torch.all(b[GUARD + self.n:] == self.SENTINEL), f"{name}: write after the buffer"

    def host(self) -> np.ndarray:
        return to_f64(self.t)


def dev(t: torch.Tensor | None):
    return None if t is None else t.cuda()


def run_headwise(inp: dict, residual: bool, *, guard=True):
    """Forward and backward on the GPU; returns numpy fp64 (y, dx, dw)."""
    x, w, dy = dev(inp["x"]), dev(inp["w"]), dev(inp["dy"])
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).cuda()
    y, dx, dw = Guarded(x.shape, x.dtype), Guarded(x.shape, x.dtype), Guarded(w.shape, w.dtype)
    binding.dsc_headwise_fwd(x, w, y.t, cu_seqlens=cu, residual=residual)
    binding.dsc_headwise_bwd(x, w, dy, dx.t, dw.t, cu_seqlens=cu, residual=residual)
    torch.cuda.synchronize()
    if guard:
        for name, g in (("y", y), ("dx", dx), ("dw", dw)):
            g.check_guards(name)
    return y.host(), dx.host(), dw.host()


def run_lowrank(inp: dict, W: int, residual: bool, *, guard=True, repeat_bwd: int = 1, deterministic=False):
    x, z, U, dy = dev(inp["x"]), dev(inp["z"]), dev(inp["U"]), dev(inp["dy"])
    B, T, D = x.shape
    R = z.shape[2]
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).cuda()
    y, dx, dz = Guarded(x.shape, x.dtype), Guarded(x.shape, x.dtype), Guarded(z.shape, z.dtype)
    dU = Guarded(U.shape, torch.float32)
    if deterministic:
        size, bwd = binding.dsc_lowrank_bwd_deterministic_workspace_size, binding.dsc_lowrank_bwd_deterministic
    else:
        size, bwd = binding.dsc_lowrank_bwd_workspace_size, binding.dsc_lowrank_bwd
    nws = size(x.dtype, B, T, D, W, R)
    ws = torch.full((max(nws, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda") if nws else None
    binding.dsc_lowrank_fwd(x, z, U, y.t, W=W, cu_seqlens=cu, residual=residual)
    for _ in range(repeat_bwd):
        bwd(x, z, U, dy, dx.t, dz.t, dU.t, ws, W=W, cu_seqlens=cu, residual=residual)
    torch.cuda.synchronize()
    if guard:
        for name, g in (("y", y), ("dx", dx), ("dz", dz), ("dU", dU)):
            g.check_guards(name)
    return y.host(), dx.host(), dz.host(), dU.host()


def assert_close(name: str, gpu: np.ndarray, ref: np.ndarray, tol: float) -> float:
    assert gpu.shape == ref.shape, f"{name}: shape {gpu.shape} vs {ref.shape}"
    assert not np.isnan(gpu).any(), f"{name}: unwritten (NaN) elements"
    err = normwise_err(gpu, ref)
    say(f"    {name:4s} normwise err {err:.3e} (tol {tol:.0e})")
    assert err <= tol, f"{name}: normwise error {err:.3e} > {tol:.0e}"
    return err


def run_static(inp: dict, residual: bool, *, guard=True, repeat_bwd: int = 1, deterministic=False):
    """Static conv forward and backward on the GPU; returns numpy fp64 (y, dx, dc)."""
    x, c, dy = dev(inp["x"]), dev(inp["c"]), dev(inp["dy"])
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).cuda()
    y, dx = Guarded(x.shape, x.dtype), Guarded(x.shape, x.dtype)
    dc = Guarded(c.shape, torch.float32)
    binding.dsc_static_fwd(x, c, y.t, cu_seqlens=cu, residual=residual)
    B, T, D = x.shape
    nws = binding.dsc_static_bwd_deterministic_workspace_size(x.dtype, B, T, D, c.shape[1]) if deterministic else 0
    ws = torch.full((max(nws, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda") if nws else None
    for _ in range(repeat_bwd):
        if deterministic:
            binding.dsc_static_bwd_deterministic(x, c, dy, dx.t, dc.t, ws, cu_seqlens=cu, residual=residual)
        else:
            binding.dsc_static_bwd(x, c, dy, dx.t, dc.t, cu_seqlens=cu, residual=residual)
    torch.cuda.synchronize()
    if guard:
        for name, g in (("y", y), ("dx", dx), ("dc", dc)):
            g.check_guards(name)
    return y.host(), dx.host(), dc.host()
