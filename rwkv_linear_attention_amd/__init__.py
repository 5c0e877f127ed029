"""MI355X-native RWKV-7 WKV7 generalized delta rule (forward, backward,
decode step) and Gated DeltaNet on the same kernels.

The compute runs in hand-written HIP kernels for gfx950 behind the C-ABI
library ``libwkv7.so`` (declared in ``include/wkv7.h``); ``wkv7`` is the thin
ctypes binding, and ``api`` maps the rwkv-ops function names
(``generalized_delta_rule``, ``gated_delta_net_chunk``, ...) onto it with
torch.autograd.  Importing the package loads nothing; the library is loaded
on first use and a missing library raises.
"""
from .wkv7 import fwd, fwd_varlen, gdn_fwd, gdn_fwd_varlen, gdn_step, gdn_bwd, gdn_bwd_varlen, bwd, bwd_varlen, step, ALGO_AUTO, ALGO_RECURRENT, ALGO_CHUNKED  # noqa: F401
from .api import (generalized_delta_rule, generalized_delta_rule_inference, rwkv7_op, rwkv7_op_rnn,  # noqa: F401
                  gated_delta_net, gated_delta_net_recurrent, gated_delta_net_recurrent_inference,
                  gated_delta_net_recurrent_single_step, gated_delta_net_chunk)
