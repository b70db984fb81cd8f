"""Gated DeltaNet layer for AMD Instinct MI355X (gfx950).

The layer runs in the HIP kernels of libgdn.so (C ABI in include/gdn.h); this
package holds the build script and a thin ctypes binding with the same names.
"""
from .binding import (GDN_BF16, GDN_F32, GDN_FLAG_L2NORM_QK, GDN_OK, Desc, GdnError,  # noqa: F401
                      gdn_decode, gdn_prefill, gdn_prefill_profiled,
                      gdn_prefill_workspace_size, gdn_status_string, lib, make_desc)
