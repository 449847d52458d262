"""Buffer offsets of the low-rank kernels' streams (CPU only).

x, dy, z, y and dx move through one raw buffer resource per token walk: a
lane's 32-bit offset is its place inside a 16-token step plus the step's
offset, and lanes with nothing to move (channels past D, ranks past R) start
at kFar, past the resource's clamped size, so the hardware range check drops
their accesses at every step.  The invariant that makes this safe is that no
offset of a 16-byte access, active or not, comes near 2^32: the launchers cap
the walk so that a walk, plus the steps fetched ahead of it, spans at most
kStreamSpan bytes, and kFar + kStreamSpan stays below 2^32.  An earlier
version gave idle lanes the offset 0xffffffff instead, where the 12 bytes
after the first of a 16-byte access lie past 2^32; the low-rank backward
faulted (memory aperture violation) on a shape with idle lanes (B=1 T=100
D=40 W=4 R=5, packed sequences), which stays a GPU parity case.

This test reads the constants from the kernel sources and checks the
invariant for the walk caps of the forward and backward kernels over a range
of channel counts, including D = 40 and the API's largest D.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "input_dependent_short_amd", "csrc")


def _const(path, name):
    text = open(os.path.join(CSRC, path)).read()
    m = re.search(rf"\b{name}\s*=\s*(0x[0-9a-fA-F]+|\d+)", text)
    assert m, f"{name} not found in {path}"
    return int(m.group(1).rstrip("uU"), 0)


K_FAR = _const("dsc_common.h", "kFar")
K_SPAN = _const("dsc_common.h", "kStreamSpan")
K_MAX_TOK = _const("lowrank_common.h", "kMaxTokPerWave")


def walk_cap(D, unit, overrun):
    """The launchers' walk cap (lowrank_common.h, walk_cap)."""
    span = K_SPAN // (2 * D) - overrun
    return (min(span, K_MAX_TOK) // unit) * unit


def test_far_offset_and_span_leave_room_below_2_32():
    assert K_FAR + K_SPAN <= 2**32 - 1
    assert K_FAR > K_SPAN  # idle lanes never alias an in-walk offset


@pytest.mark.parametrize("D", [8, 40, 64, 2304, 6144, 8192, 65536, 1 << 20, 1 << 24])
@pytest.mark.parametrize("ring", [2, 4, 6, 8])
def test_walk_offsets_never_reach_2_32(D, ring):
    unit, overrun = 16 * ring, 16 * (2 * ring + 2)
    cap = walk_cap(D, unit, overrun)
    if cap < unit:
        # no whole ring fits: the launchers take the vector-ALU kernels instead
        assert (unit + overrun) * 2 * D > K_SPAN
        return
    act_step = 16 * D * 2  # bytes of one 16-token step
    # the deepest step any lane fetches: the walk plus the steps loaded ahead
    # (at most ring + 1 of them) plus one step of margin
    last_step = cap // 16 + ring + 2
    assert (last_step * 16) * 2 * D <= (cap + overrun) * 2 * D <= K_SPAN
    # an active lane: its place in a step (token < 16, channel < D) plus the step
    active_max = (15 * D + (D - 8)) * 2 + last_step * act_step
    assert active_max + 16 <= K_SPAN + 1
    # an idle lane starts at kFar and walks the same steps
    idle_max = K_FAR + last_step * act_step
    assert idle_max + 16 <= 2**32, f"16-byte access at {idle_max:#x} crosses 2^32"
