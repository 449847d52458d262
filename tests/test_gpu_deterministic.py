"""The reproducible backward passes, dsc_lowrank_bwd_deterministic and
dsc_static_bwd_deterministic (GPU).

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
from gpu_util import TOL, assert_close, normwise_err, run_lowrank, run_static, say
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


# (dtype, B, T, D, W, residual, segment-length range or None)
STATIC_CASES = [
    ("bf16", 2, 300, 512, 4, True, None),
    ("bf16", 1, 700, 2304, 3, False, (1, 200)),
    ("bf16", 3, 45, 200, 8, True, None),      # 25 chunks: a ragged channel group
    ("fp32", 2, 130, 96, 4, True, (1, 40)),
    ("fp32", 1, 5, 16, 1, False, None),
]


@pytest.mark.parametrize("case", STATIC_CASES, ids=[f"{c[0]}-B{c[1]}T{c[2]}D{c[3]}W{c[4]}" for c in STATIC_CASES])
def test_static_deterministic_small(case):
    dt, B, T, D, W, res, seg = case
    wl, inp = inputs.small("static", B, T, D, W, dtype=dt, residual=res, varlen=seg is not None,
                           seglen_range=seg or (1, 8), seed=zlib.crc32(repr(case).encode()) % 1000)
    say(f"[deterministic static] {wl.name} residual={res}")
    first = run_static(inp, res, deterministic=True)
    again = run_static(inp, res, deterministic=True, repeat_bwd=2)
    for name, a, b in zip(("y", "dx", "dc"), first, again):
        assert np.array_equal(a, b), f"{name} differs between two calls"
    _, fdx, _ = run_static(inp, res)
    assert np.array_equal(first[1], fdx), "dx differs from the fast backward's"
    x64, c64, g64 = (to_f64(inp[k]) for k in ("x", "c", "dy"))
    rdx, rdc = oracle.static_bwd(x64, c64, g64, cu_seqlens=inp["cu_seqlens"], residual=res)
    tol = TOL[dt]
    assert_close("dx", first[1], rdx, tol)
    assert_close("dc", first[2], rdc, tol)


@pytest.mark.parametrize("shape", [(8, 2048, 2304), (4, 4096, 8192)], ids=["qkv-150m", "mlp-2b"])
def test_static_deterministic_full_size(shape):
    B, T, D = shape
    W = 4
    wl, inp = inputs.small("static", B, T, D, W, dtype="bf16", residual=True, seed=77)
    x, c, dy = (inp[k].cuda() for k in ("x", "c", "dy"))
    nws = binding.dsc_static_bwd_deterministic_workspace_size(x.dtype, B, T, D, W)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    outs = []
    for det in (True, True, False):
        dx, dc = torch.empty_like(x), torch.empty(c.shape, dtype=torch.float32, device="cuda")
        if det:
            binding.dsc_static_bwd_deterministic(x, c, dy, dx, dc, ws, residual=True)
        else:
            binding.dsc_static_bwd(x, c, dy, dx, dc, residual=True)
        torch.cuda.synchronize()
        outs.append((dx, dc))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), "two calls differ"
    assert torch.equal(outs[0][0], outs[2][0]), "dx differs from the fast backward's"
    e = normwise_err(to_f64(outs[0][1]), to_f64(outs[2][1]))
    say(f"[deterministic static] B={B} T={T} D={D}: dc against the fast backward {e:.2e}")
    assert e <= 1e-6
    c0, c1 = D - 8, D
    x64, g64 = to_f64(inp["x"][:, :, c0:c1]), to_f64(inp["dy"][:, :, c0:c1])
    _, rdc = oracle.static_bwd(x64, to_f64(inp["c"][c0:c1]), g64, residual=True, rows=(0, 0))
    assert_close("dc", to_f64(outs[0][1][c0:c1]), rdc, TOL["bf16"])
