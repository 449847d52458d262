"""Dynamic short convolutions on AMD Instinct MI355X (gfx950).

The compute path is libdsc.so (hand-written HIP kernels behind the C ABI in
include/dsc.h); ``binding`` is its thin ctypes front end.  Importing the
package does not load the library; the first call does, and raises if it is
not built.
"""
from .binding import (DscError, dsc_abi_version, dsc_headwise_bwd, dsc_headwise_fwd,  # noqa: F401
                      dsc_lowrank_bwd, dsc_lowrank_bwd_workspace_size, dsc_lowrank_fwd)
