"""Seeded synthetic input recipe (CPU)."""
import numpy as np
import torch

from input_dependent_short_amd import inputs


def test_small_inputs_are_seeded_and_typed():
    wl, a = inputs.small("headwise", 2, 9, 16, 4, H=8, dtype="bf16", seed=3)
    _, b = inputs.small("headwise", 2, 9, 16, 4, H=8, dtype="bf16", seed=3)
    assert a["x"].dtype == torch.bfloat16 and a["x"].shape == (2, 9, 16)
    assert a["w"].shape == (2, 9, 2, 4)
    assert torch.equal(a["x"], b["x"]) and torch.equal(a["w"], b["w"])
    _, c = inputs.small("headwise", 2, 9, 16, 4, H=8, dtype="bf16", seed=4)
    assert not torch.equal(a["x"], c["x"])
    wl, d = inputs.small("lowrank", 1, 5, 8, 3, R=6, dtype="fp32", seed=0)
    assert d["z"].shape == (1, 5, 6) and d["U"].shape == (6, 24) and d["U"].dtype == torch.float32


def test_packed_segments_recipe():
    B, T = 4, 4096
    cu = inputs.packed_cu_seqlens(B, T, 256, 4096, inputs.seed_for(5, 4))
    assert cu[0] == 0 and cu[-1] == B * T and np.all(np.diff(cu) > 0)
    for b in range(B + 1):
        assert b * T in cu            # every row start is a segment start
    lens = np.diff(cu)
    ends = set((np.arange(1, B + 1) * T).tolist())
    for i, L in enumerate(lens):
        if int(cu[i + 1]) not in ends:  # only the last segment of a row may be cut short
            assert 256 <= L <= 4096


def test_scales_follow_recipe():
    wl = inputs.Workload("t", "lowrank", 2, 512, 64, 4, R=16, dtype="fp32", cfg=77)
    a = inputs.make_inputs(wl)
    assert abs(float(a["x"].std()) - 1.0) < 0.02
    assert abs(float(a["U"].std()) - 1.0 / np.sqrt(16 * 4)) < 0.01
    wl = inputs.Workload("t", "headwise", 2, 512, 64, 4, H=4, dtype="fp32", cfg=78)
    a = inputs.make_inputs(wl)
    assert abs(float(a["w"].std()) - 0.5) < 0.01


def test_workload_table():
    assert inputs.WORKLOADS[2].D == 2304 and inputs.WORKLOADS[2].H == 64
    assert inputs.WORKLOADS[4].D // inputs.WORKLOADS[4].H == 512
    assert inputs.WORKLOADS[5].varlen and inputs.WORKLOADS[5].R == 64
