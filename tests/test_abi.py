"""The C ABI of libdsc.so: exported symbols and host-side argument checks (CPU only).

Every call below fails validation, which the library performs before any HIP
call, so no GPU is touched.
"""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


@pytest.fixture(scope="module")
def lib():
    from input_dependent_short_amd import binding, build
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    return binding.lib()


def declared_symbols():
    """Every DSC_API function declared by a header under include/."""
    syms = []
    for h in HEADERS:
        syms += re.findall(r"DSC_API\s+[\w\s\*]+?\b(dsc_\w+)\s*\(", open(h).read())
    return syms


def test_header_declares_the_entry_points():
    syms = set(declared_symbols())
    for s in ("dsc_headwise_fwd", "dsc_headwise_bwd", "dsc_lowrank_fwd", "dsc_lowrank_bwd",
              "dsc_lowrank_bwd_workspace_size", "dsc_lowrank_bwd_deterministic",
              "dsc_lowrank_bwd_deterministic_workspace_size", "dsc_static_fwd", "dsc_static_bwd",
              "dsc_static_bwd_deterministic", "dsc_static_bwd_deterministic_workspace_size",
              "dsc_headwise_decode", "dsc_lowrank_decode", "dsc_state_from_prefill",
              "dsc_rope_table", "dsc_headwise_rope_fwd", "dsc_headwise_rope_bwd", "dsc_headwise_rope_decode",
              "dsc_lowrank_rope_fwd", "dsc_lowrank_rope_bwd", "dsc_headwise_gen_fwd", "dsc_headwise_gen_bwd",
              "dsc_headwise_gen_bwd_workspace_size", "dsc_generate_filters",
              "dsc_status_string", "dsc_last_error", "dsc_abi_version"):
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    for s in declared_symbols():
        assert hasattr(lib, s), f"{s} not exported"
    assert lib.dsc_abi_version() == 1
    assert lib.dsc_status_string(5) == b"DSC_ERR_ALIAS"


A = 1 << 20          # fake, 16-byte aligned device addresses (never dereferenced)
P = lambda k: ctypes.c_void_p(A * k)
S0 = ctypes.c_void_p(0)


def hw_fwd(lib, dtype=1, B=1, T=8, D=64, W=4, H=8, x=P(1), w=P(2), cu=None, ns=0, res=0, y=P(3)):
    return lib.dsc_headwise_fwd(S0, dtype, B, T, D, W, H, x, w, cu, ns, res, y)


def test_headwise_fwd_validation(lib):
    assert hw_fwd(lib, x=None) == 1
    assert hw_fwd(lib, W=0) == 2 and hw_fwd(lib, W=9) == 2
    assert hw_fwd(lib, D=60) == 2                 # bf16 needs D % 8 == 0
    assert hw_fwd(lib, H=7) == 2                  # H must divide D
    assert hw_fwd(lib, D=48, H=24, y=P(1)) == 5   # any H dividing D passes the shape checks
    assert hw_fwd(lib, D=48, H=3, y=P(1)) == 5 and hw_fwd(lib, D=48, H=48, y=P(1)) == 5
    assert hw_fwd(lib, dtype=7) == 3
    assert hw_fwd(lib, B=-1) == 2 and hw_fwd(lib, T=-3) == 2 and hw_fwd(lib, D=0) == 2
    assert hw_fwd(lib, H=7, B=0) == 2             # shapes are checked for an empty batch too
    assert hw_fwd(lib, x=ctypes.c_void_p(A + 2)) == 4
    assert hw_fwd(lib, y=P(1)) == 5               # in place
    assert hw_fwd(lib, y=ctypes.c_void_p(A + 64)) == 5   # partial overlap with x
    assert b"overlaps" in lib.dsc_last_error()
    assert hw_fwd(lib, res=2) == 2
    assert hw_fwd(lib, cu=P(9), ns=0) == 2        # pointer without count


def test_headwise_fwd_fp32_shape_reaches_launch_only_when_valid(lib):
    # fp32, D=60, H=4: valid shape; aliasing makes it fail before any HIP call
    assert hw_fwd(lib, dtype=0, D=60, H=4, y=P(1)) == 5


def test_headwise_bwd_validation(lib):
    f = lambda **k: lib.dsc_headwise_bwd(S0, 1, 1, 8, 64, 4, 8, k.get("x", P(1)), k.get("w", P(2)),
                                         k.get("dy", P(3)), None, 0, 0, k.get("dx", P(4)),
                                         k.get("dw", P(5)))
    assert f(dw=None) == 1
    assert f(dx=P(3)) == 5                        # dx aliases dy
    assert f(dw=P(4)) == 5                        # outputs overlap
    assert f(x=ctypes.c_void_p(A * 1 + 8)) == 4


def lr_bwd(lib, ws=P(8), wsb=1 << 20, **k):
    return lib.dsc_lowrank_bwd(S0, 1, 1, 8, 64, 4, k.get("R", 16), P(1), P(2), P(3), P(4), None, 0, 0,
                               k.get("dx", P(5)), k.get("dz", P(6)), k.get("dU", P(7)), ws, wsb)


def test_lowrank_validation(lib):
    assert lib.dsc_lowrank_fwd(S0, 1, 1, 8, 64, 4, 0, P(1), P(2), P(3), None, 0, 0, P(4)) == 2
    assert lib.dsc_lowrank_fwd(S0, 1, 1, 8, 64, 4, 129, P(1), P(2), P(3), None, 0, 0, P(4)) == 2
    assert lib.dsc_lowrank_fwd(S0, 1, 1, 8, 64, 4, 16, P(1), None, P(3), None, 0, 0, P(4)) == 1
    assert lib.dsc_lowrank_fwd(S0, 1, 1, 8, 64, 4, 16, P(1), P(2), P(3), None, 0, 0, P(3)) == 5
    need = lib.dsc_lowrank_bwd_workspace_size(1, 1, 8, 64, 4, 16)
    assert need >= 8 * 16 * 4
    assert lib.dsc_lowrank_bwd_workspace_size(0, 1, 8, 64, 4, 16) == 0   # fp32 accumulates in dz
    assert lib.dsc_lowrank_bwd_workspace_size(1, 1, 8, 63, 4, 16) == 0   # invalid sizes
    assert lr_bwd(lib, ws=None, wsb=0) == 6
    assert lr_bwd(lib, wsb=need - 1) == 6
    assert lr_bwd(lib, ws=P(1)) == 5              # workspace aliases x
    assert lr_bwd(lib, dU=P(5)) == 5
    assert lr_bwd(lib, dz=None) == 1


def test_lowrank_deterministic_validation(lib):
    G = lambda k: ctypes.c_void_p((1 << 30) * k)  # fake addresses 1 GiB apart: only the named overlaps
    f = lambda ws=G(8), wsb=1 << 30, **k: lib.dsc_lowrank_bwd_deterministic(
        S0, k.get("dtype", 1), 8, 2048, 2304, 4, 32, G(1), G(2), G(3), G(4), None, 0, 0, k.get("dx", G(5)),
        k.get("dz", G(6)), k.get("dU", G(7)), ws, wsb)
    size = lambda dtype, B, T, D, W, R: lib.dsc_lowrank_bwd_deterministic_workspace_size(dtype, B, T, D, W, R)
    # 16384 tokens, D = 2304 (18 blocks of 128 channels), R = 32: one fp32 dz region
    # per channel block, then one fp32 dU region (R x D*W) per token chunk; computed
    # on the host alone (no device here), so it cannot depend on the device
    need = size(1, 8, 2048, 2304, 4, 32)
    dz_bytes = 18 * 16384 * 32 * 4
    du_region = 32 * 2304 * 4 * 4
    chunks, rest = divmod(need - dz_bytes, du_region)
    assert need % 256 == 0 and rest < 256 and 1 <= chunks <= 16384 // 64
    assert size(1, 4, 4096, 6144, 4, 64) >= 48 * 16384 * 64 * 4 + 64 * 6144 * 4 * 4
    assert size(0, 1, 64, 64, 4, 16) == 0      # fp32: one thread per dz / dU element, no workspace
    assert size(1, 1, 64, 64, 4, 96) == 0      # bf16 shapes of the generic kernels: none either
    assert size(1, 1, 64, 64, 6, 40) == 0
    assert size(1, 1, 8, 63, 4, 16) == 0       # invalid sizes
    assert f(ws=None, wsb=0) == 6
    assert f(wsb=need - 1) == 6
    assert b"workspace of" in lib.dsc_last_error()
    assert f(ws=G(1)) == 5                     # workspace aliases x
    assert f(dz=G(5)) == 5                     # dz aliases dx
    assert f(dU=None) == 1
    assert f(dtype=0, ws=None, wsb=0, dU=G(4)) == 5   # fp32 needs no workspace; dU aliases dy


def st_fwd(lib, dtype=1, B=1, T=8, D=64, W=4, x=P(1), c=P(2), cu=None, ns=0, res=0, y=P(3)):
    return lib.dsc_static_fwd(S0, dtype, B, T, D, W, x, c, cu, ns, res, y)


def st_bwd(lib, dtype=1, B=1, T=8, D=64, W=4, x=P(1), c=P(2), dy=P(3), cu=None, ns=0, res=0,
           dx=P(4), dc=P(5)):
    return lib.dsc_static_bwd(S0, dtype, B, T, D, W, x, c, dy, cu, ns, res, dx, dc)


def test_static_validation(lib):
    assert st_fwd(lib, W=0) == 2
    assert st_fwd(lib, W=9) == 2
    assert st_fwd(lib, D=60) == 2                     # bf16 needs D % 8 == 0
    assert st_fwd(lib, dtype=0, D=62) == 2            # fp32 needs D % 4 == 0
    assert st_fwd(lib, dtype=2) == 3
    assert st_fwd(lib, res=2) == 2
    assert st_fwd(lib, c=None) == 1
    assert st_fwd(lib, c=ctypes.c_void_p(A * 2 + 8)) == 4
    assert st_fwd(lib, y=P(1)) == 5                  # y = x in place
    assert st_fwd(lib, y=ctypes.c_void_p(A * 2 + 16)) == 5   # y overlaps c (D*W*2 = 512 bytes)
    assert st_fwd(lib, cu=P(6), ns=0) == 2            # cu_seqlens and n_seqs disagree
    assert st_bwd(lib, dc=None) == 1
    assert st_bwd(lib, dx=P(3)) == 5                  # dx aliases dy
    assert st_bwd(lib, dc=P(2)) == 5                  # dc aliases c
    assert st_bwd(lib, dc=ctypes.c_void_p(A * 5 + 4)) == 4
    assert st_bwd(lib, W=9) == 2


def test_decode_validation(lib):
    hd = lambda dt=1, B=4, D=64, W=4, H=8, x=P(1), w=P(2), st=P(3), res=0, y=P(4): \
        lib.dsc_headwise_decode(S0, dt, B, D, W, H, x, w, st, res, y)
    ld = lambda dt=1, B=4, D=64, W=4, R=16, x=P(1), z=P(2), U=P(3), st=P(4), res=0, y=P(5): \
        lib.dsc_lowrank_decode(S0, dt, B, D, W, R, x, z, U, st, res, y)
    assert hd(W=0) == 2 and hd(W=9) == 2 and hd(D=60) == 2 and hd(H=3) == 2
    assert hd(H=12, D=96, y=P(1)) == 5              # groups across 16-byte chunks pass the shape checks
    assert hd(st=None) == 1
    assert hd(st=P(1)) == 5                         # state overlaps x
    assert hd(y=P(3)) == 5                          # y overlaps the state
    assert hd(x=ctypes.c_void_p(A + 8)) == 4
    assert hd(B=-1) == 2
    assert hd(B=0, x=None, w=None, st=None, y=None) == 0
    assert ld(R=0) == 2 and ld(R=129) == 2
    assert ld(U=None) == 1
    assert ld(st=P(3)) == 5                         # state overlaps U
    sp = lambda B=1, T=8, D=64, W=4, x=P(1), cu=None, ns=0, st=P(2): \
        lib.dsc_state_from_prefill(S0, 1, B, T, D, W, x, cu, ns, st)
    assert sp(W=9) == 2 and sp(st=None) == 1 and sp(st=P(1)) == 5
    assert sp(W=1, st=None) == 0                    # no slots: nothing to write
    assert sp(B=0, x=None, st=None) == 0


def test_rope_validation(lib):
    # head-wise + rotary: B=2 T=8 D=128 bf16, rot = 64 (one query and one key head of 32)
    def rf(dt=1, B=2, T=8, D=128, W=4, H=16, x=P(1), w=P(2), cu=None, ns=0, res=1, rot=64, hd=32,
           tab=P(3), maxp=8, y=P(4)):
        return lib.dsc_headwise_rope_fwd(S0, dt, B, T, D, W, H, x, w, cu, ns, res, rot, hd, tab, maxp, y)

    def rb(rot=64, hd=32, tab=P(3), maxp=8, dx=P(5), dw=P(6)):
        return lib.dsc_headwise_rope_bwd(S0, 1, 2, 8, 128, 4, 16, P(1), P(2), P(4), None, 0, 1, rot, hd, tab, maxp,
                                         dx, dw)
    assert rf(hd=31) == 2 and rf(hd=0) == 2          # odd / empty head
    assert rf(hd=4) == 3                             # a bf16 chunk of 8 channels would span two heads
    assert rf(dt=0, hd=4, rot=64, y=P(1)) == 5       # fp32 chunks are 4 channels: passes to the alias check
    assert rf(rot=48) == 2 and rf(rot=160) == 2 and rf(rot=-32) == 2
    assert rf(maxp=7) == 2                           # positions 0..T-1 need T rows
    assert rf(cu=P(9), ns=3, maxp=8) == 2            # packed: a sequence may be B*T long
    assert rf(tab=None) == 1
    assert rf(tab=ctypes.c_void_p(A * 3 + 8)) == 4
    assert rf(y=P(3)) == 5                           # y overlaps the table
    assert rf(rot=0, tab=None, maxp=0, y=P(1)) == 5  # rot = 0 needs no table; aliasing still checked
    assert rf(B=0, x=None, w=None, tab=None, y=None) == 0
    assert rb(dx=P(3)) == 5 and rb(dw=None) == 1 and rb(maxp=2) == 2
    assert lib.dsc_rope_table(S0, 8, 31, 10000.0, P(1)) == 2
    assert lib.dsc_rope_table(S0, 8, 32, 0.0, P(1)) == 2
    assert lib.dsc_rope_table(S0, 8, 32, float("nan"), P(1)) == 2
    assert lib.dsc_rope_table(S0, -1, 32, 10000.0, P(1)) == 2
    assert lib.dsc_rope_table(S0, 8, 32, 10000.0, None) == 1
    assert lib.dsc_rope_table(S0, 8, 32, 10000.0, ctypes.c_void_p(A + 4)) == 4
    assert lib.dsc_rope_table(S0, 0, 32, 10000.0, None) == 0
    # rotated decoding step: B=4 sequences, D=128, heads of 32, rot = 64
    def rd(B=4, hd=32, rot=64, tab=P(5), maxp=100, pos=P(6), y=P(4), st=P(3)):
        return lib.dsc_headwise_rope_decode(S0, 1, B, 128, 4, 16, P(1), P(2), st, 1, rot, hd, tab, maxp, pos, y)
    assert rd(hd=0, rot=0) == 2                      # head_dim is required
    assert rd(hd=4) == 3 and rd(rot=48) == 2 and rd(hd=31) == 2
    assert rd(pos=None) == 1 and rd(tab=None) == 1
    assert rd(pos=ctypes.c_void_p(A * 6 + 2)) == 4 and rd(tab=ctypes.c_void_p(A * 5 + 8)) == 4
    assert rd(maxp=0) == 2
    assert rd(y=P(6)) == 5                           # y overlaps the positions
    assert rd(st=P(5)) == 5                          # the state overlaps the table
    assert rd(B=0) == 0


def test_lowrank_rope_validation(lib):
    # low-rank + rotary: B=2 T=8 D=128 W=4 R=16 bf16, rot = 64 (heads of 32)
    def lf(dt=1, B=2, T=8, D=128, W=4, R=16, x=P(1), z=P(2), U=P(3), cu=None, ns=0, res=0, rot=64, hd=32,
           tab=P(4), maxp=8, y=P(5)):
        return lib.dsc_lowrank_rope_fwd(S0, dt, B, T, D, W, R, x, z, U, cu, ns, res, rot, hd, tab, maxp, y)

    def lb(dt=1, R=16, rot=64, hd=32, tab=P(4), maxp=8, dx=P(6), dz=P(7), dU=P(8), ws=P(9), wsb=1 << 20):
        return lib.dsc_lowrank_rope_bwd(S0, dt, 2, 8, 128, 4, R, P(1), P(2), P(3), P(5), None, 0, 0, rot, hd, tab,
                                         maxp, dx, dz, dU, ws, wsb)
    assert lf(R=0) == 2 and lf(R=129) == 2
    assert lf(hd=31) == 2 and lf(hd=4) == 3          # a bf16 chunk of 8 channels would span two heads
    assert lf(rot=48) == 2 and lf(rot=160) == 2
    assert lf(maxp=7) == 2                           # positions 0..T-1 need T rows
    assert lf(cu=P(10), ns=3, maxp=8) == 2           # packed: a sequence may be B*T long
    assert lf(tab=None) == 1
    assert lf(tab=ctypes.c_void_p(A * 4 + 8)) == 4
    assert lf(y=P(4)) == 5                           # y overlaps the table
    assert lf(rot=0, tab=None, maxp=0, y=P(1)) == 5  # rot = 0 needs no table; aliasing still checked
    assert lf(B=0, x=None, z=None, U=None, tab=None, y=None) == 0
    assert lb(dx=P(4)) == 5 and lb(dz=None) == 1 and lb(maxp=2) == 2
    assert lb(ws=None, wsb=0) == 6                   # bf16 needs the dz accumulator
    assert lb(wsb=16) == 6
    assert lb(ws=P(4)) == 5                          # the workspace overlaps the table
    assert lb(dt=0, ws=None, wsb=0, dx=P(1)) == 5    # fp32 needs no workspace: on to the alias check


def test_generator_validation(lib):
    # generated head-wise layer: B=2 T=8 D=128 W=4 H=16 (G=8, G*W=32), hidden width K=64, bf16
    def gf(dt=1, B=2, T=8, D=128, W=4, H=16, K=64, h=P(1), V=P(2), x=P(3), cu=None, ns=0, res=1, y=P(4)):
        return lib.dsc_headwise_gen_fwd(S0, dt, B, T, D, W, H, K, h, V, x, cu, ns, res, y)

    def gb(dt=1, K=64, dy=P(5), dx=P(6), dh=P(7), dV=P(8), ws=P(9), wsb=1 << 20, h=P(1)):
        return lib.dsc_headwise_gen_bwd(S0, dt, 2, 8, 128, 4, 16, K, h, P(2), P(3), dy, None, 0, 1, dx, dh, dV,
                                        ws, wsb)
    size = lambda dt=1, K=64, H=16, W=4: lib.dsc_headwise_gen_bwd_workspace_size(dt, 2, 8, 128, W, H, K)
    assert gf(dt=0) == 3                             # bf16 only
    assert gf(H=48) == 2 and gf(H=0) == 2            # H must divide D
    assert gf(K=0) == 2 and gf(K=12) == 3            # K a multiple of 8
    assert gf(W=3, H=64) == 3                        # G*W = 6 is not a multiple of 8
    assert gf(W=9) == 2
    assert gf(h=None) == 1 and gf(y=ctypes.c_void_p(A * 4 + 2)) == 4
    assert gf(y=P(3)) == 5 and gf(y=P(1)) == 5       # y overlaps x / h
    assert gf(B=0, h=None, V=None, x=None, y=None) == 0
    # dw (16 x 32), V^T (64 x 32), dw^T (32 x 32: tokens padded to 32), h^T (64 x 32), all bf16
    assert size() == 2 * (16 * 32 + 64 * 32 + 32 * 32 + 64 * 32)
    assert gf(h=P(3), y=P(3)) == 5                   # h may be x; y may not
    assert size(dt=0) == 0 and size(K=12) == 0
    assert gb(ws=None, wsb=0) == 6 and gb(wsb=100) == 6
    assert gb(dh=P(1)) == 5                          # dh overlaps h
    assert gb(dV=None) == 1 and gb(dx=ctypes.c_void_p(A * 6 + 8)) == 4
    assert gb(ws=P(5)) == 5                          # the workspace overlaps dy
    gen = lambda dt=1, N=16, K=64, C=32, h=P(1), V=P(2), w=P(3): lib.dsc_generate_filters(S0, dt, N, K, C, h, V, w)
    assert gen(dt=0) == 3 and gen(dt=7) == 2 and gen(K=12) == 3 and gen(C=20) == 3 and gen(K=0) == 2
    assert gen(w=None) == 1 and gen(w=P(1)) == 5 and gen(h=ctypes.c_void_p(A + 4)) == 4
    assert gen(N=0, h=None, V=None, w=None) == 0


def test_binding_raises_with_message(lib):
    import torch
    from input_dependent_short_amd import binding
    x = torch.zeros(1, 8, 60, dtype=torch.bfloat16)
    w = torch.zeros(1, 8, 60, 4, dtype=torch.bfloat16)
    with pytest.raises(binding.DscError, match="multiple of 8"):
        binding.dsc_headwise_fwd(x, w, x, stream=0)


def test_empty_batch_is_a_no_op(lib):
    # B or T = 0: nothing to compute and no HIP call, so NULL data pointers are
    # accepted (the low-rank backward, which zero-fills dU, is covered on the GPU)
    assert hw_fwd(lib, B=0, x=None, w=None, y=None) == 0
    assert hw_fwd(lib, T=0, x=None, w=None, y=None) == 0
    assert lib.dsc_headwise_bwd(S0, 1, 2, 0, 64, 4, 8, None, None, None, None, 0, 0, None, None) == 0
    assert lib.dsc_lowrank_fwd(S0, 1, 0, 8, 64, 4, 16, None, None, None, None, 0, 1, None) == 0
    assert lib.dsc_lowrank_fwd(S0, 1, 0, 8, 64, 4, 0, None, None, None, None, 0, 1, None) == 2  # R still checked
    assert lib.dsc_lowrank_bwd(S0, 1, 0, 8, 64, 4, 16, None, None, None, None, None, 0, 0,
                               None, None, None, None, 0) == 1   # dU is still required
    assert st_fwd(lib, B=0, x=None, c=None, y=None) == 0
    assert st_bwd(lib, T=0, x=None, c=None, dy=None, dx=None, dc=None) == 1   # dc is still required


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No fallback: without libdsc.so every binding call raises."""
    import torch
    from input_dependent_short_amd import binding
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "absent" / "libdsc.so"))
    monkeypatch.setattr(binding, "_lib", None)
    x = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    w = torch.zeros(1, 8, 8, 4, dtype=torch.bfloat16)
    with pytest.raises(ImportError, match="not built"):
        binding.dsc_headwise_fwd(x, w, x, stream=0)


def test_static_deterministic_validation(lib):
    G = lambda k: ctypes.c_void_p((1 << 30) * k)
    f = lambda ws=G(8), wsb=1 << 30, **k: lib.dsc_static_bwd_deterministic(
        S0, 1, 8, 2048, 2304, 4, G(1), G(2), G(3), None, 0, 0, k.get("dx", G(4)), k.get("dc", G(5)), ws, wsb)
    # D = 2304 bf16: 288 chunks of 8 channels, 32 per block (64 does not divide 288),
    # so 8 token tiles of 32 per block; 16384 tokens = 512 tiles = 64 tile groups,
    # each with one fp32 (D, W) region of dc
    need = lib.dsc_static_bwd_deterministic_workspace_size(1, 8, 2048, 2304, 4)
    assert need == 64 * 2304 * 4 * 4
    assert lib.dsc_static_bwd_deterministic_workspace_size(1, 0, 2048, 2304, 4) == 0
    assert lib.dsc_static_bwd_deterministic_workspace_size(1, 8, 2048, 2303, 4) == 0
    assert f(ws=None, wsb=0) == 6
    assert f(wsb=need - 1) == 6
    assert f(ws=G(1)) == 5                     # workspace aliases x
    assert f(dc=G(4)) == 5                     # dc aliases dx
    assert f(dx=None) == 1


def test_bench_stream_validation(lib):
    st = lambda src=P(1), rb=1 << 20, dst=P(9), wb=1 << 20, u=4, ln=0, sn=0, ch=0, bl=0: lib.dsc_bench_stream(
        S0, src, rb, dst, wb, u, ln, sn, ch, bl)
    assert st(rb=10) == 2 and st(wb=-16) == 2 and st(rb=1 << 40) == 2
    assert st(u=3) == 2 and st(ln=2) == 2 and st(ch=5) == 2 and st(bl=-1) == 2
    assert st(dst=None) == 1 and st(src=None) == 1
    assert st(src=ctypes.c_void_p(A + 8)) == 4
    assert st(dst=P(1)) == 5                      # dst overlaps src


def test_lowrank_bwd_noalloc_validation(lib):
    """The allocation-free backward checks everything, including its scratch
    limit (B*T*R <= 4,194,304), before any HIP call."""
    def call(B=1, T=8, D=64, R=16, x=P(1), dU=P(7)):
        return lib.dsc_lowrank_bwd_noalloc(S0, 1, B, T, D, 4, R, x, P(2), P(3), P(4), None, 0, 0,
                                           P(5), P(6), dU)
    assert call(x=None) == 1
    assert call(dU=ctypes.c_void_p(A * 7 + 4)) == 4
    assert call(R=0) == 2 and call(R=129) == 2
    assert call(T=(4 << 20) // 64 + 1, R=64) == 6     # one token past the scratch
    assert call(B=2, T=1 << 20, R=4) == 6
    assert b"built-in scratch" in lib.dsc_last_error()
