"""MI355X-native RWKV-7 WKV7 generalized-delta-rule forward and decode step.

The compute runs in hand-written HIP kernels for gfx950 behind the C-ABI
library ``libwkv7.so`` (declared in ``include/wkv7.h``); ``wkv7`` is the thin
ctypes binding.  Importing the package loads nothing; the library is loaded
on first use and a missing library raises.
"""
from .wkv7 import fwd, fwd_varlen, gdn_fwd, gdn_fwd_varlen, gdn_step, gdn_bwd, bwd, step, ALGO_AUTO, ALGO_RECURRENT, ALGO_CHUNKED  # noqa: F401
