"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small shapes are compared element by element over every output, for every
tap count W in 1..8 on each kernel family.  The five workloads run at full
size and every element of every output is compared with the oracle (the
sums over all tokens, dU, channel block by channel block); before that,
every output element is checked to have been written (outputs start as NaN)
and the guard bands around each output to be intact.  Tolerance: normwise
max-relative error max|gpu - ref| / max|ref| <= 1e-5 (fp32) or 2e-2 (bf16
inputs, fp32 accumulation).
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, assert_close, run_headwise, run_lowrank, say
from input_dependent_short_amd import binding, inputs
from input_dependent_short_amd.inputs import to_f64

pytestmark = pytest.mark.gpu

# (dtype, B, T, D, W, H, residual, segment-length range or None)
HW_CASES = [
    ("fp32", 1, 64, 64, 4, 1, False, None),
    ("fp32", 2, 37, 32, 3, 4, True, None),
    ("fp32", 1, 2, 16, 4, 2, False, None),
    ("fp32", 2, 50, 96, 8, 8, True, (1, 9)),
    ("fp32", 1, 33, 256, 4, 256, False, None),
    ("bf16", 2, 100, 128, 4, 64, True, None),
    ("bf16", 1, 77, 64, 4, 16, False, (1, 20)),
    ("bf16", 3, 19, 48, 1, 8, True, None),
    ("bf16", 2, 45, 256, 2, 1, False, None),
    ("bf16", 1, 130, 64, 5, 2, True, (1, 40)),
    ("bf16", 2, 66, 512, 7, 4, False, None),
    ("bf16", 1, 40, 1024, 4, 512, True, None),
    ("bf16", 1, 3, 40, 8, 8, True, None),
    ("bf16", 4, 65, 2304, 4, 64, True, None),
    ("bf16", 2, 300, 8192, 4, 16, True, (1, 120)),
    # W = 6 on each filter span: one filter per lane group, per chunk, and 4 per chunk
    ("bf16", 2, 90, 256, 6, 16, True, (1, 30)),
    ("bf16", 1, 70, 64, 6, 2, False, None),
    ("fp32", 1, 50, 64, 6, 4, False, (1, 12)),
    # any H with D % H == 0: groups of 3, 5, 6 and 12 channels across the
    # 16-byte chunks, and groups wider than 64 chunks (per-channel group
    # index); groups of 3, 5, 6 and 12 chunks (lane groups padded to a power
    # of two in the backward)
    ("bf16", 2, 90, 48, 4, 3, True, (1, 30)),
    ("bf16", 1, 50, 40, 8, 5, False, (1, 12)),
    ("bf16", 1, 70, 96, 4, 6, False, None),
    ("bf16", 1, 30, 96, 4, 12, True, None),
    ("bf16", 1, 20, 2048, 4, 1024, True, (1, 9)),
    ("bf16", 2, 100, 192, 4, 24, True, (1, 40)),
    ("bf16", 1, 40, 1200, 5, 40, True, None),
    ("bf16", 1, 80, 480, 3, 48, True, None),
    ("bf16", 2, 64, 768, 4, 96, False, (1, 50)),
    ("fp32", 1, 50, 60, 4, 3, True, (1, 20)),
    ("fp32", 1, 40, 96, 6, 12, False, None),
    ("fp32", 1, 30, 40, 4, 10, True, None),
]

# (dtype, B, T, D, W, R, residual, segment-length range or None)
LR_CASES = [
    ("fp32", 1, 20, 16, 4, 3, False, None),
    ("fp32", 2, 33, 32, 3, 8, True, (1, 7)),
    ("fp32", 1, 9, 8, 1, 1, False, None),
    ("bf16", 1, 64, 32, 4, 32, False, None),
    ("bf16", 2, 77, 64, 4, 64, True, None),
    ("bf16", 1, 100, 40, 4, 5, False, (1, 30)),
    ("bf16", 2, 31, 96, 3, 100, True, None),
    ("bf16", 1, 50, 128, 8, 1, False, (1, 9)),
    ("bf16", 1, 2, 32, 4, 16, False, None),
    ("bf16", 3, 130, 2304, 4, 32, False, None),
    ("bf16", 1, 200, 128, 2, 128, True, (1, 50)),
    ("bf16", 1, 520, 6144, 4, 64, False, (1, 300)),
    ("bf16", 2, 97, 200, 8, 20, True, (1, 60)),
    ("bf16", 1, 64, 96, 2, 48, False, None),
    # wide forward with R in 33..64 gathered (R % 8 != 0), several token walks per channel pair
    ("bf16", 1, 4100, 64, 3, 36, True, (1, 700)),
    # backward with the taps of a slice over two waves (33 <= R <= 64, W = 2..4):
    # gathered z rows (R % 4 != 0), a partial last slice, packed sequences,
    # several token chunks per channel group
    ("bf16", 1, 300, 96, 4, 45, True, (1, 80)),
    ("bf16", 2, 150, 64, 3, 63, False, None),
    ("bf16", 1, 700, 256, 2, 33, True, (1, 120)),
    ("bf16", 2, 333, 136, 4, 40, False, (1, 50)),
    # backward blocks of two token halves, several blocks, partial last half, R % 8 != 0
    ("bf16", 3, 1000, 128, 4, 20, True, (100, 900)),
    # W = 5, 6, 7 on every kernel family: wide forward + matrix-core backward
    # (R <= 32, whole and gathered z rows, packed sequences), wide forward +
    # vector backward (33 <= R <= 64), 32-channel matrix-core forward (R > 64),
    # and fp32
    ("bf16", 1, 150, 96, 5, 32, True, None),
    ("bf16", 2, 90, 64, 6, 12, False, (1, 40)),
    ("bf16", 1, 200, 128, 7, 24, True, (1, 60)),
    ("bf16", 1, 70, 64, 5, 40, True, None),
    ("bf16", 1, 60, 32, 6, 64, False, (1, 20)),
    ("bf16", 1, 45, 48, 7, 100, True, (1, 15)),
    ("fp32", 1, 40, 16, 5, 4, True, None),
    ("fp32", 2, 30, 8, 6, 2, False, (1, 9)),
    ("fp32", 1, 25, 12, 7, 6, True, None),
]


def _ids(cases, tag):
    return [f"{tag}-{c[0]}-B{c[1]}T{c[2]}D{c[3]}W{c[4]}{'H' if tag == 'hw' else 'R'}{c[5]}"
            f"-res{int(c[6])}-{'varlen' if c[7] else 'rows'}" for c in cases]


@pytest.mark.parametrize("case", HW_CASES, ids=_ids(HW_CASES, "hw"))
def test_headwise_small(case):
    dt, B, T, D, W, H, res, seg = case
    wl, inp = inputs.small("headwise", B, T, D, W, H=H, dtype=dt, residual=res, varlen=seg is not None,
                           seglen_range=seg or (1, 8), seed=zlib.crc32(repr(case).encode()) % 1000)
    say(f"[headwise] {wl.name} residual={res} segments={inp['cu_seqlens']}")
    y, dx, dw = run_headwise(inp, res)
    cu = inp["cu_seqlens"]
    x64, w64, g64 = to_f64(inp["x"]), to_f64(inp["w"]), to_f64(inp["dy"])
    ry = oracle.headwise_fwd(x64, w64, cu_seqlens=cu, residual=res)
    rdx, rdw = oracle.headwise_bwd(x64, w64, g64, cu_seqlens=cu, residual=res)
    tol = TOL[dt]
    assert_close("y", y, ry, tol)
    assert_close("dx", dx, rdx, tol)
    assert_close("dw", dw, rdw, tol)


@pytest.mark.parametrize("case", LR_CASES, ids=_ids(LR_CASES, "lr"))
def test_lowrank_small(case):
    dt, B, T, D, W, R, res, seg = case
    wl, inp = inputs.small("lowrank", B, T, D, W, R=R, dtype=dt, residual=res, varlen=seg is not None,
                           seglen_range=seg or (1, 8), seed=zlib.crc32(repr(case).encode()) % 1000)
    say(f"[lowrank] {wl.name} residual={res} segments={inp['cu_seqlens']}")
    y, dx, dz, dU = run_lowrank(inp, W, res, repeat_bwd=2)
    cu = inp["cu_seqlens"]
    x64, z64, U64, g64 = (to_f64(inp[k]) for k in ("x", "z", "U", "dy"))
    ry = oracle.lowrank_fwd(x64, z64, U64, W, cu_seqlens=cu, residual=res)
    rdx, rdz, rdU = oracle.lowrank_bwd(x64, z64, U64, g64, W, cu_seqlens=cu, residual=res)
    tol = TOL[dt]
    assert_close("y", y, ry, tol)
    assert_close("dx", dx, rdx, tol)
    assert_close("dz", dz, rdz, tol)
    assert_close("dU", dU, rdU, tol)


def _step_edge_cu(T: int) -> np.ndarray:
    """Sequence starts at every offset around the kernels' 16-token steps
    (first, second, third and last tokens of a step, and mid-step), with runs
    of length-1 sequences across some step edges and a ragged end."""
    offs = [0, 1, 2, 3, 7, 13, 14, 15]
    starts = {0, T}
    for j, m in enumerate(range(1, T // 16)):
        starts.add(16 * m + offs[j % len(offs)])
        if j % 5 == 0:
            starts.update({16 * m - 1, 16 * m + 1})
    return np.array(sorted(t for t in starts if 0 <= t <= T), dtype=np.int32)


@pytest.mark.parametrize("W,R", [(4, 32), (4, 64), (3, 20), (8, 8), (2, 48)])
def test_lowrank_sequence_starts_at_step_edges(W, R):
    """Steps with a sequence start among their taps take the masked path, the
    others the unmasked one; both must agree with the oracle everywhere."""
    T = 709
    wl, inp = inputs.small("lowrank", 1, T, 128, W, R=R, dtype="bf16", residual=True,
                           seed=11 * W + R)
    inp["cu_seqlens"] = _step_edge_cu(T)
    say(f"[lowrank] {wl.name} step-edge starts={inp['cu_seqlens'].tolist()}")
    y, dx, dz, dU = run_lowrank(inp, W, True)
    cu = inp["cu_seqlens"]
    x64, z64, U64, g64 = (to_f64(inp[k]) for k in ("x", "z", "U", "dy"))
    ry = oracle.lowrank_fwd(x64, z64, U64, W, cu_seqlens=cu, residual=True)
    rdx, rdz, rdU = oracle.lowrank_bwd(x64, z64, U64, g64, W, cu_seqlens=cu, residual=True)
    tol = TOL["bf16"]
    assert_close("y", y, ry, tol)
    assert_close("dx", dx, rdx, tol)
    assert_close("dz", dz, rdz, tol)
    assert_close("dU", dU, rdU, tol)


def test_headwise_repeat_is_bitwise_identical():
    wl, inp = inputs.small("headwise", 2, 300, 1024, 4, H=16, dtype="bf16", residual=True, seed=5)
    say(f"[headwise determinism] {wl.name}")
    a = run_headwise(inp, True)
    b = run_headwise(inp, True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ------------------------------------------------------------ full workloads


def _written(name: str, a: np.ndarray) -> None:
    """Every element of a full-size output was written (outputs start as NaN)."""
    bad = int(np.isnan(a).sum())
    say(f"    {name:4s} all {a.size} elements written" if not bad else f"    {name}: {bad} unwritten")
    assert bad == 0, f"{name}: {bad} elements not written"


def _row_chunks(N: int, parts: int) -> list[tuple[int, int]]:
    step = (N + parts - 1) // parts
    return [(lo, min(N, lo + step)) for lo in range(0, N, step)]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_full_size(cfg):
    """Every element of every output of the workload against the oracle."""
    wl = inputs.WORKLOADS[cfg]
    say(f"[workload {cfg}] {wl.name}: B={wl.B} T={wl.T} D={wl.D} W={wl.W} H={wl.H} R={wl.R} "
        f"{wl.dtype} residual={wl.residual} varlen={wl.varlen}")
    inp = inputs.make_inputs(wl)
    cu = inp["cu_seqlens"]
    tol = TOL[wl.dtype]
    N, D = wl.N, wl.D
    x64, g64 = to_f64(inp["x"]), to_f64(inp["dy"])
    if wl.kind == "headwise":
        y, dx, dw = run_headwise(inp, wl.residual)
        for name, a in (("y", y), ("dx", dx), ("dw", dw)):
            _written(name, a)
        w64 = to_f64(inp["w"])
        say("  oracle: all rows")
        ry = oracle.headwise_fwd(x64, w64, cu_seqlens=cu, residual=wl.residual)
        assert_close("y", y, ry, tol)
        del ry
        rdx, rdw = oracle.headwise_bwd(x64, w64, g64, cu_seqlens=cu, residual=wl.residual)
        assert_close("dx", dx, rdx, tol)
        assert_close("dw", dw, rdw, tol)
    else:
        W, R = wl.W, wl.R
        y, dx, dz, dU = run_lowrank(inp, W, wl.residual)
        for name, a in (("y", y), ("dx", dx), ("dz", dz), ("dU", dU)):
            _written(name, a)
        z64, U64 = to_f64(inp["z"]), to_f64(inp["U"])
        y, dx, dz = y.reshape(N, D), dx.reshape(N, D), dz.reshape(N, R)
        say("  oracle: all rows")
        ry = oracle.lowrank_fwd(x64, z64, U64, W, cu_seqlens=cu, residual=wl.residual).reshape(N, D)
        assert_close("y", y, ry, tol)
        del ry
        # the backward in row blocks (each compared against the whole
        # tensor's scale), dU in channel blocks: every element in the end
        rdx = np.empty((N, D))
        rdz = np.empty((N, R))
        for lo, hi in _row_chunks(N, 4):
            say(f"  oracle: dx, dz rows [{lo},{hi})")
            rdx[lo:hi], rdz[lo:hi], _ = oracle.lowrank_bwd(x64, z64, U64, g64, W, cu_seqlens=cu,
                                                           residual=wl.residual, rows=(lo, hi), channels=(0, 0))
        assert_close("dx", dx, rdx, tol)
        assert_close("dz", dz, rdz, tol)
        del rdx, rdz
        rdU = np.empty((R, D, W))
        for c0, c1 in _row_chunks(D, 4):
            say(f"  oracle: dU channels [{c0},{c1})")
            _, _, part = oracle.lowrank_bwd(x64, z64, U64, g64, W, cu_seqlens=cu, residual=wl.residual,
                                            rows=(0, 0), channels=(c0, c1))
            rdU[:, c0:c1] = part.reshape(R, c1 - c0, W)
        assert_close("dU", dU.reshape(R, D, W), rdU, tol)


def test_stream_argument_is_honoured():
    """Calls on a side stream complete in order on that stream."""
    wl, inp = inputs.small("headwise", 1, 256, 512, 4, H=8, dtype="bf16", residual=True, seed=9)
    say(f"[stream] {wl.name}")
    x, w = inp["x"].cuda(), inp["w"].cuda()
    y1 = torch.empty_like(x)
    y2 = torch.empty_like(x)
    binding.dsc_headwise_fwd(x, w, y1, residual=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.dsc_headwise_fwd(x, w, y2, residual=True, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.gpu
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_empty_batch(dt):
    """B*T = 0: every entry point succeeds; the low-rank dU (a sum over no tokens) is zero."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, D, W, H, R = 2, 64, 4, 8, 16
    say(f"[empty] {dt} B={B} T=0 D={D}")
    x = torch.empty((B, 0, D), dtype=dtype, device="cuda")
    dy, y, dx = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    w = torch.empty((B, 0, D // H, W), dtype=dtype, device="cuda")
    dw = torch.empty_like(w)
    z = torch.empty((B, 0, R), dtype=dtype, device="cuda")
    dz = torch.empty_like(z)
    U = torch.randn((R, D * W), device="cuda").to(dtype)
    dU = torch.full((R, D * W), float("nan"), device="cuda")
    binding.dsc_headwise_fwd(x, w, y)
    binding.dsc_headwise_bwd(x, w, dy, dx, dw)
    binding.dsc_lowrank_fwd(x, z, U, y, W=W)
    assert binding.dsc_lowrank_bwd_workspace_size(dtype, B, 0, D, W, R) == 0
    binding.dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, None, W=W)
    torch.cuda.synchronize()
    assert torch.equal(dU, torch.zeros_like(dU))
