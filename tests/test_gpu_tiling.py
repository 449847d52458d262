"""Results that must not depend on the work split (GPU): the same rows run as
one batch and one row per call, so that the launches take different token
tiles and walk lengths.  At the MLP ~2B head-wise shape (B=4 T=4096 D=8192
H=16) the whole batch runs the backward with 64-token tiles and a single row
with 32-token tiles on MI355X (the tile follows the grid size); at the QKV
~150M low-rank shape (B=8 T=2048 D=2304 R=32) the backward's token chunks
and the forward's walks differ in length.  Every per-token result (y, dx,
dw) must agree bit for bit; dz and dU, summed with atomics in a different
order, within 1e-6 (fp32 dU) and one bf16 rounding (dz) normwise.  A race or
a tile-edge mistake would show up as a difference between the two runs."""
from __future__ import annotations

import pytest
import torch

from gpu_util import normwise_err, say
from input_dependent_short_amd import binding, inputs
from input_dependent_short_amd.inputs import to_f64

pytestmark = pytest.mark.gpu


def test_headwise_whole_batch_equals_row_by_row():
    wl = inputs.WORKLOADS[4]
    say(f"[tiling] {wl.name}: whole batch vs one row per call")
    inp = inputs.make_inputs(wl)
    x, w, dy = (inp[k].cuda() for k in ("x", "w", "dy"))
    outs = []
    for split in (False, True):
        y, dx, dw = torch.empty_like(x), torch.empty_like(x), torch.empty_like(w)
        parts = [slice(b, b + 1) for b in range(wl.B)] if split else [slice(0, wl.B)]
        for s in parts:
            binding.dsc_headwise_fwd(x[s], w[s], y[s], residual=wl.residual)
            binding.dsc_headwise_bwd(x[s], w[s], dy[s], dx[s], dw[s], residual=wl.residual)
        torch.cuda.synchronize()
        outs.append((y, dx, dw))
    for name, a, b in zip(("y", "dx", "dw"), *outs):
        assert torch.equal(a, b), f"{name} depends on the work split"


@pytest.mark.parametrize("cfg", [3, 5])
def test_lowrank_whole_batch_equals_row_by_row(cfg):
    wl = inputs.WORKLOADS[cfg]
    say(f"[tiling] {wl.name}: whole batch vs one row per call")
    inp = inputs.make_inputs(wl)
    if wl.varlen:  # rows as their own sequences in both runs: the packed offsets would cross rows
        inp["cu_seqlens"] = None
    x, z, U, dy = (inp[k].cuda() for k in ("x", "z", "U", "dy"))
    outs = []
    for split in (False, True):
        y, dx, dz = torch.empty_like(x), torch.empty_like(x), torch.empty_like(z)
        dU = torch.zeros(U.shape, dtype=torch.float32, device="cuda")
        rows = 1 if split else wl.B
        nws = binding.dsc_lowrank_bwd_workspace_size(x.dtype, rows, wl.T, wl.D, wl.W, wl.R)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
        part_dU = torch.empty_like(dU)
        for b0 in range(0, wl.B, rows):
            s = slice(b0, b0 + rows)
            binding.dsc_lowrank_fwd(x[s], z[s], U, y[s], W=wl.W, residual=wl.residual)
            binding.dsc_lowrank_bwd(x[s], z[s], U, dy[s], dx[s], dz[s], part_dU, ws, W=wl.W, residual=wl.residual)
            dU += part_dU
        torch.cuda.synchronize()
        outs.append((y, dx, dz, dU))
    (y0, dx0, dz0, dU0), (y1, dx1, dz1, dU1) = outs
    assert torch.equal(y0, y1), "y depends on the work split"
    assert torch.equal(dx0, dx1), "dx depends on the work split"
    e_dz = normwise_err(to_f64(dz1), to_f64(dz0))
    e_dU = normwise_err(to_f64(dU1), to_f64(dU0))
    say(f"  dz {e_dz:.2e}, dU {e_dU:.2e}")
    assert e_dz <= 1e-2 and e_dU <= 1e-6
