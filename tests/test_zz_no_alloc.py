"""The allocation-free low-rank backward (dsc_lowrank_bwd_noalloc, GPU).

It runs the same kernels as dsc_lowrank_bwd with the dz accumulator in the
library's built-in device scratch instead of a workspace.  Its outputs are
compared with dsc_lowrank_bwd's on the same inputs (dx bit for bit; dz and dU,
summed with fp32 atomics in both, within the bf16 tolerance), and with the
fp64 oracle, on two calls in a row, the second on a smaller input, so that the
scratch's leftover contents from the first call must not leak into the
second.  Then at the largest size the scratch holds (B*T*R = 4,194,304).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, assert_close, say
from input_dependent_short_amd import binding, inputs
from input_dependent_short_amd.inputs import to_f64

pytestmark = pytest.mark.gpu


def _both(inp, W, residual):
    x, z, U, dy = (inp[k].cuda() for k in ("x", "z", "U", "dy"))
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).cuda()
    B, T, D = x.shape
    R = z.shape[2]
    kw = dict(W=W, cu_seqlens=cu, residual=residual)
    outs = []
    for noalloc in (False, True):
        dx = torch.full_like(x, float("nan"))
        dz = torch.full_like(z, float("nan"))
        dU = torch.full(U.shape, float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            binding.dsc_lowrank_bwd_noalloc(x, z, U, dy, dx, dz, dU, **kw)
        else:
            nws = binding.dsc_lowrank_bwd_workspace_size(x.dtype, B, T, D, W, R)
            ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
            binding.dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, ws, **kw)
        torch.cuda.synchronize()
        outs.append((dx, dz, dU))
    return outs


def _check(inp, W, residual, oracle_too=True):
    (dx0, dz0, dU0), (dx1, dz1, dU1) = _both(inp, W, residual)
    tol = TOL["bf16"]
    assert torch.equal(dx0, dx1), "dx differs from dsc_lowrank_bwd's"
    assert_close("dz vs workspace call", to_f64(dz1), to_f64(dz0), tol)
    assert_close("dU vs workspace call", to_f64(dU1), to_f64(dU0), tol)
    if oracle_too:
        x64, z64, U64, g64 = (to_f64(inp[k]) for k in ("x", "z", "U", "dy"))
        rdx, rdz, rdU = oracle.lowrank_bwd(x64, z64, U64, g64, W, cu_seqlens=inp["cu_seqlens"],
                                           residual=residual)
        assert_close("dx", to_f64(dx1), rdx, tol)
        assert_close("dz", to_f64(dz1), rdz, tol)
        assert_close("dU", to_f64(dU1), rdU, tol)


def test_noalloc_matches_the_workspace_backward_on_two_calls():
    # first call: a larger batch with packed sequences fills the scratch with its dz sums
    _, big = inputs.small("lowrank", 3, 700, 256, 4, R=64, dtype="bf16", residual=True, varlen=True,
                          seglen_range=(20, 400), seed=71)
    say(f"[noalloc] call 1: B=3 T=700 D=256 R=64, {len(big['cu_seqlens']) - 1} sequences")
    _check(big, 4, True)
    # second call: smaller, other rank (gathered z rows); the leftover scratch must not leak in
    _, small = inputs.small("lowrank", 1, 150, 128, 4, R=20, dtype="bf16", residual=False, seed=72)
    say("[noalloc] call 2: B=1 T=150 D=128 R=20")
    _check(small, 4, False)


def test_noalloc_at_the_scratch_limit():
    """B*T*R = 4,194,304 exactly: the whole scratch is used."""
    B, T, D, R, W = 4, 16384, 64, 64, 4
    _, inp = inputs.small("lowrank", B, T, D, W, R=R, dtype="bf16", residual=False, seed=73)
    say(f"[noalloc] limit: B={B} T={T} D={D} R={R} (B*T*R = {B * T * R})")
    _check(inp, W, False, oracle_too=False)
    x, z = inp["x"].cuda(), inp["z"].cuda()
    over = torch.empty(B, T + 1, D, dtype=x.dtype, device="cuda")
    zo = torch.empty(B, T + 1, R, dtype=x.dtype, device="cuda")
    with pytest.raises(binding.DscError):
        binding.dsc_lowrank_bwd_noalloc(over, zo, inp["U"].cuda(), over.clone(), torch.empty_like(over),
                                        torch.empty_like(zo), torch.empty(R, D * W, device="cuda"), W=W)
