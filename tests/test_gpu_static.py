"""GPU parity of the static short convolution (one fixed filter per channel)
through the C ABI against the fp64 oracle.

Small shapes are compared element by element on every output; the QKV ~150M
shape (B=8 T=2048 D=2304 W=4) is compared on sampled token windows for y and
dx and on every element of dc (a sum over all 16384 tokens).  Tolerance as for
the dynamic op: normwise max-relative 1e-5 (fp32) or 2e-2 (bf16 inputs, fp32
accumulation).
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, Guarded, assert_close, run_static, say
from input_dependent_short_amd import binding, inputs
from input_dependent_short_amd.inputs import to_f64

pytestmark = pytest.mark.gpu

# (dtype, B, T, D, W, residual, segment-length range or None)
ST_CASES = [
    ("fp32", 1, 64, 64, 4, False, None),        # the tiny per-channel shape
    ("fp32", 2, 37, 32, 3, True, None),
    ("fp32", 2, 50, 96, 8, True, (1, 9)),
    ("fp32", 1, 9, 4, 1, False, None),
    ("bf16", 2, 100, 128, 4, True, None),
    ("bf16", 1, 300, 1024, 4, False, (1, 40)),  # two groups of 64 chunks, a ragged group of tiles
    ("bf16", 3, 19, 48, 2, True, None),         # fewer chunks than lanes
    ("bf16", 1, 130, 64, 5, True, (1, 40)),     # 40 dc partials per thread: two reduction rounds
    ("bf16", 2, 66, 512, 7, False, None),
    ("bf16", 1, 40, 2304, 8, True, (1, 7)),     # a partial last chunk group, sequences of 1..7
    ("bf16", 4, 65, 2304, 4, True, None),
    ("bf16", 1, 1, 8, 3, False, None),          # one token
]


def _ids(cases):
    return [f"st-{c[0]}-B{c[1]}T{c[2]}D{c[3]}W{c[4]}-res{int(c[5])}-{'varlen' if c[6] else 'rows'}"
            for c in cases]


@pytest.mark.parametrize("case", ST_CASES, ids=_ids(ST_CASES))
def test_static_small(case):
    dt, B, T, D, W, res, seg = case
    wl, inp = inputs.small("static", B, T, D, W, dtype=dt, residual=res, varlen=seg is not None,
                           seglen_range=seg or (1, 8), seed=zlib.crc32(repr(case).encode()) % 1000)
    say(f"[static] {wl.name} residual={res} segments={inp['cu_seqlens']}")
    y, dx, dc = run_static(inp, res, repeat_bwd=2)
    cu = inp["cu_seqlens"]
    x64, c64, g64 = (to_f64(inp[k]) for k in ("x", "c", "dy"))
    ry = oracle.static_fwd(x64, c64, cu_seqlens=cu, residual=res)
    rdx, rdc = oracle.static_bwd(x64, c64, g64, cu_seqlens=cu, residual=res)
    tol = TOL[dt]
    assert_close("y", y, ry, tol)
    assert_close("dx", dx, rdx, tol)
    assert_close("dc", dc, rdc, tol)


def test_static_qkv_150m_full_size():
    wl = inputs.Workload("static-qkv-150m", "static", 8, 2048, 2304, 4, dtype="bf16", residual=True, cfg=6)
    inp = inputs.make_inputs(wl)
    say(f"[static] {wl.name}: B={wl.B} T={wl.T} D={wl.D} W={wl.W} bf16 residual")
    y, dx, dc = run_static(inp, True)
    x64, c64, g64 = (to_f64(inp[k]) for k in ("x", "c", "dy"))
    N, D = wl.N, wl.D
    tol = TOL["bf16"]
    yf, dxf = y.reshape(N, D), dx.reshape(N, D)
    for lo, hi in [(0, 40), (2040, 2060), (N // 2 - 7, N // 2 + 17), (N - 40, N)]:
        ry = oracle.static_fwd(x64, c64, residual=True, rows=(lo, hi))
        rdx, _ = oracle.static_bwd(x64, c64, g64, residual=True, rows=(lo, hi))
        assert_close("y", yf[lo:hi], ry, tol)
        assert_close("dx", dxf[lo:hi], rdx, tol)
    _, rdc = oracle.static_bwd(x64, c64, g64, residual=True, rows=(0, 0))
    assert_close("dc", dc, rdc, tol)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_static_empty_batch(dt):
    """B = 0: the forward writes nothing, the backward zero-fills dc."""
    tdt = inputs.DTYPES[dt]
    x = torch.empty(0, 16, 64, dtype=tdt, device="cuda")
    c = torch.randn(64, 4, device="cuda").to(tdt)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    dc = Guarded((64, 4), torch.float32)
    binding.dsc_static_fwd(x, c, y)
    binding.dsc_static_bwd(x, c, x, dx, dc.t)
    torch.cuda.synchronize()
    dc.check_guards("dc")
    assert np.all(dc.host() == 0.0)
