"""The training entry points under HIP graph capture (GPU).

Forward and backward of the head-wise, low-rank (with its zero-fill and cast
launches, and the fixed-order backward with its summing launches), static
(also its fixed-order backward) and head-wise + rotary layers are captured once as a single graph.  The graph is replayed three times; between replays the same calls run
eagerly on separate outputs, with synchronisation, and every replay is checked
against them: bit for bit where no atomic sum is involved, and within 1e-6
(fp32) or one bf16 rounding (bf16 dz) normwise for the sums accumulated with
atomics (dz, dU, dc), whose order of addition varies from run to run.  The
fixed-order backward passes' dz, dU and dc are compared bit for bit.
"""
from __future__ import annotations

import pytest
import torch

from gpu_util import normwise_err, say
from input_dependent_short_amd import binding, inputs
from input_dependent_short_amd.inputs import to_f64

pytestmark = pytest.mark.gpu


def _outputs(t: dict) -> dict:
    o = {}
    for k in ("hw", "rp"):
        o[k + "_y"], o[k + "_dx"], o[k + "_dw"] = (torch.empty_like(t["hx"]), torch.empty_like(t["hx"]),
                                                  torch.empty_like(t["hw"]))
    o["lr_y"], o["lr_dx"], o["lr_dz"] = torch.empty_like(t["lx"]), torch.empty_like(t["lx"]), torch.empty_like(t["z"])
    o["lr_dU"] = torch.empty(t["U"].shape, dtype=torch.float32, device="cuda")
    o["lr_ws"] = torch.empty(t["ws_bytes"], dtype=torch.uint8, device="cuda")
    o["ld_dx"], o["ld_dz"] = torch.empty_like(t["lx"]), torch.empty_like(t["z"])
    o["ld_dU"] = torch.empty(t["U"].shape, dtype=torch.float32, device="cuda")
    o["ld_ws"] = torch.empty(t["det_ws_bytes"], dtype=torch.uint8, device="cuda")
    o["st_y"], o["st_dx"] = torch.empty_like(t["sx"]), torch.empty_like(t["sx"])
    o["st_dc"] = torch.empty(t["c"].shape, dtype=torch.float32, device="cuda")
    o["sd_dx"] = torch.empty_like(t["sx"])
    o["sd_dc"] = torch.empty(t["c"].shape, dtype=torch.float32, device="cuda")
    o["sd_ws"] = torch.empty(t["st_ws_bytes"], dtype=torch.uint8, device="cuda")
    return o


def _calls(t: dict, o: dict) -> None:
    b = binding
    b.dsc_headwise_fwd(t["hx"], t["hw"], o["hw_y"], cu_seqlens=t["cu"], residual=True)
    b.dsc_headwise_bwd(t["hx"], t["hw"], t["hdy"], o["hw_dx"], o["hw_dw"], cu_seqlens=t["cu"], residual=True)
    b.dsc_lowrank_fwd(t["lx"], t["z"], t["U"], o["lr_y"], W=4)
    b.dsc_lowrank_bwd(t["lx"], t["z"], t["U"], t["ldy"], o["lr_dx"], o["lr_dz"], o["lr_dU"], o["lr_ws"], W=4)
    b.dsc_lowrank_bwd_deterministic(t["lx"], t["z"], t["U"], t["ldy"], o["ld_dx"], o["ld_dz"], o["ld_dU"],
                                    o["ld_ws"], W=4)
    b.dsc_static_fwd(t["sx"], t["c"], o["st_y"], residual=True)
    b.dsc_static_bwd(t["sx"], t["c"], t["sdy"], o["st_dx"], o["st_dc"], residual=True)
    b.dsc_static_bwd_deterministic(t["sx"], t["c"], t["sdy"], o["sd_dx"], o["sd_dc"], o["sd_ws"], residual=True)
    kw = dict(rot=512, head_dim=64, table=t["table"], cu_seqlens=t["cu"], residual=True)
    b.dsc_headwise_rope_fwd(t["hx"], t["hw"], o["rp_y"], **kw)
    b.dsc_headwise_rope_bwd(t["hx"], t["hw"], t["hdy"], o["rp_dx"], o["rp_dw"], **kw)


ATOMIC = {"lr_dz": 1e-2, "lr_dU": 1e-6, "st_dc": 1e-6}


def test_training_entry_points_replayed_as_a_graph():
    _, hi = inputs.small("headwise", 2, 300, 1024, 4, H=16, dtype="bf16", residual=True, varlen=True,
                         seglen_range=(1, 120), seed=31)
    _, li = inputs.small("lowrank", 2, 200, 256, 4, R=32, dtype="bf16", seed=32)
    _, si = inputs.small("static", 2, 300, 512, 4, dtype="bf16", residual=True, seed=33)
    t = {"hx": hi["x"].cuda(), "hw": hi["w"].cuda(), "hdy": hi["dy"].cuda(),
         "cu": torch.from_numpy(hi["cu_seqlens"]).cuda(),
         "lx": li["x"].cuda(), "z": li["z"].cuda(), "U": li["U"].cuda(), "ldy": li["dy"].cuda(),
         "sx": si["x"].cuda(), "c": si["c"].cuda(), "sdy": si["dy"].cuda()}
    t["ws_bytes"] = max(16, binding.dsc_lowrank_bwd_workspace_size(torch.bfloat16, 2, 200, 256, 4, 32))
    t["st_ws_bytes"] = max(16, binding.dsc_static_bwd_deterministic_workspace_size(torch.bfloat16, 2, 300, 512, 4))
    t["det_ws_bytes"] = max(16, binding.dsc_lowrank_bwd_deterministic_workspace_size(torch.bfloat16, 2, 200, 256, 4,
                                                                                     32))
    t["table"] = torch.empty(2 * 300, 32, 2, dtype=torch.float32, device="cuda")
    binding.dsc_rope_table(t["table"])
    say("[graph] head-wise, low-rank, static and head-wise + rotary, forward and backward")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture, on scratch outputs
        _calls(t, _outputs(t))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    og, oe = _outputs(t), _outputs(t)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _calls(t, og)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        _calls(t, oe)
        torch.cuda.synchronize()
        for k, a in og.items():
            if k in ("lr_ws", "ld_ws", "sd_ws"):
                continue
            b = oe[k]
            if k in ATOMIC:
                e = normwise_err(to_f64(a), to_f64(b))
                assert e <= ATOMIC[k], f"replay {rep}: {k} differs from the eager call by {e:.2e}"
            else:
                assert torch.equal(a, b), f"replay {rep}: {k} differs from the eager call"
