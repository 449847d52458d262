"""The reproducible low-rank backward, dsc_lowrank_bwd_deterministic (GPU).

Small shapes of every kernel family (matrix-core backward with two token
halves, gathered z, two rank tiles and W = 8; the generic kernels in bf16 and
fp32) against the fp64 oracle, with the outputs of two calls bitwise equal.
At the QKV ~150M (B=8 T=2048 D=2304 R=32) and MLP ~2B varlen (B=4 T=4096
D=6144 R=64) sizes: two calls bitwise equal, dx bitwise equal to the fast
backward's (same kernel), dz and dU within the rounding of a different order
of summation from the fast backward's, and sampled rows and channels against
the oracle.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, assert_close, normwise_err, run_lowrank, say
from input_dependent_short_amd import binding, inputs
from input_dependent_short_amd.inputs import to_f64

pytestmark = pytest.mark.gpu

# (dtype, B, T, D, W, R, residual, segment-length range or None)
CASES = [
    ("bf16", 3, 130, 2304, 4, 32, True, None),          # matrix cores, two token halves
    ("bf16", 3, 1000, 128, 4, 20, True, (100, 900)),    # R % 8 != 0: gathered z rows
    ("bf16", 1, 520, 6144, 4, 64, False, (1, 300)),     # two rank tiles, one token half
    ("bf16", 1, 50, 128, 8, 1, False, (1, 9)),          # W = 8
    ("bf16", 2, 31, 96, 3, 100, True, None),            # generic kernels (R > 64)
    ("bf16", 1, 64, 96, 8, 48, False, None),            # generic kernels (W > 4 with R > 32)
    ("fp32", 2, 33, 32, 3, 8, True, (1, 7)),
    ("fp32", 1, 20, 16, 4, 3, False, None),
]


def _ids():
    return [f"{c[0]}-B{c[1]}T{c[2]}D{c[3]}W{c[4]}R{c[5]}" + ("-varlen" if c[7] else "") for c in CASES]


@pytest.mark.parametrize("case", CASES, ids=_ids())
def test_deterministic_small(case):
    dt, B, T, D, W, R, res, seg = case
    wl, inp = inputs.small("lowrank", B, T, D, W, R=R, dtype=dt, residual=res, varlen=seg is not None,
                           seglen_range=seg or (1, 8), seed=zlib.crc32(repr(case).encode()) % 1000)
    say(f"[deterministic] {wl.name} residual={res} segments={inp['cu_seqlens']}")
    first = run_lowrank(inp, W, res, deterministic=True)
    again = run_lowrank(inp, W, res, deterministic=True, repeat_bwd=2)
    for name, a, b in zip(("y", "dx", "dz", "dU"), first, again):
        assert np.array_equal(a, b), f"{name} differs between two calls"
    _, dx, dz, dU = first
    cu = inp["cu_seqlens"]
    x64, z64, U64, g64 = (to_f64(inp[k]) for k in ("x", "z", "U", "dy"))
    rdx, rdz, rdU = oracle.lowrank_bwd(x64, z64, U64, g64, W, cu_seqlens=cu, residual=res)
    tol = TOL[dt]
    assert_close("dx", dx, rdx, tol)
    assert_close("dz", dz, rdz, tol)
    assert_close("dU", dU, rdU, tol)
    ws = binding.dsc_lowrank_bwd_deterministic_workspace_size(inputs.DTYPES[dt], B, T, D, W, R)
    if ws:  # the matrix-core kernel: dx comes from the same code as the fast backward's
        _, fdx, _, _ = run_lowrank(inp, W, res)
        assert np.array_equal(dx, fdx), "dx differs from the fast backward's"


def _bwd(fn, size, x, z, U, dy, W, cu, residual):
    B, T, D = x.shape
    R = z.shape[2]
    dx, dz = torch.empty_like(x), torch.empty_like(z)
    dU = torch.empty(U.shape, dtype=torch.float32, device="cuda")
    nws = size(x.dtype, B, T, D, W, R)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
    fn(x, z, U, dy, dx, dz, dU, ws if nws else None, W=W, cu_seqlens=cu, residual=residual)
    torch.cuda.synchronize()
    return dx, dz, dU


@pytest.mark.parametrize("cfg", [3, 5])
def test_deterministic_full_size(cfg):
    wl = inputs.WORKLOADS[cfg]
    say(f"[deterministic workload {cfg}] {wl.name}: B={wl.B} T={wl.T} D={wl.D} W={wl.W} R={wl.R} "
        f"varlen={wl.varlen}")
    inp = inputs.make_inputs(wl)
    x, z, U, dy = (inp[k].cuda() for k in ("x", "z", "U", "dy"))
    cu_np = inp["cu_seqlens"]
    cu = None if cu_np is None else torch.from_numpy(cu_np).cuda()
    W, R, N, D = wl.W, wl.R, wl.N, wl.D
    args = (x, z, U, dy, W, cu, wl.residual)
    det = (binding.dsc_lowrank_bwd_deterministic, binding.dsc_lowrank_bwd_deterministic_workspace_size)
    fast = (binding.dsc_lowrank_bwd, binding.dsc_lowrank_bwd_workspace_size)
    a = _bwd(*det, *args)
    b = _bwd(*det, *args)
    for name, u, v in zip(("dx", "dz", "dU"), a, b):
        assert torch.equal(u, v), f"{name} differs between two calls"
    f = _bwd(*fast, *args)
    assert torch.equal(a[0], f[0]), "dx differs from the fast backward's"
    dz_e = normwise_err(a[1].double().cpu().numpy(), f[1].double().cpu().numpy())
    dU_e = normwise_err(a[2].double().cpu().numpy(), f[2].double().cpu().numpy())
    say(f"  against the fast backward: dz {dz_e:.2e}, dU {dU_e:.2e}")
    assert dz_e <= 1e-2 and dU_e <= 1e-6
    x64, z64, U64, g64 = (to_f64(inp[k]) for k in ("x", "z", "U", "dy"))
    tol = TOL[wl.dtype]
    dz = to_f64(a[1].cpu()).reshape(N, R)
    for lo, hi in [(0, 24), (N // 2 - 7, N // 2 + 17), (N - 24, N)]:
        say(f"  rows [{lo},{hi})")
        _, rdz, _ = oracle.lowrank_bwd(x64, z64, U64, g64, W, cu_seqlens=cu_np, residual=wl.residual,
                                       rows=(lo, hi), channels=(0, 0))
        assert_close("dz", dz[lo:hi], rdz, tol)
    dU3 = a[2].cpu().double().numpy().reshape(R, D, W)
    for c0, c1 in [(0, 8), (D - 8, D)]:
        say(f"  dU channels [{c0},{c1})")
        _, _, rdU = oracle.lowrank_bwd(x64, z64, U64, g64, W, cu_seqlens=cu_np, residual=wl.residual,
                                       rows=(0, 0), channels=(c0, c1))
        assert_close("dU", dU3[:, c0:c1].reshape(R, (c1 - c0) * W), rdU, tol)
