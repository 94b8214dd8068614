"""libtfla: chunkwise-parallel gated linear attention forward (mLSTMsig,
fixed per-head decay, per-key-channel gate) on AMD gfx950.

The compute path is the C-ABI library ``libtfla.so`` built from ``csrc/``;
:mod:`mlstm_sequence_amd.tfla` is its ctypes binding.
"""
from .tfla import (  # noqa: F401
    GLA_KEY, IO_BF16, MLSTM_SIG, SCALAR_DECAY, TflaError, forward, tfla_dbg_gates, tfla_dbg_states,
    tfla_fwd, tfla_fwd_ws, tfla_last_error, tfla_version, tfla_workspace_bytes, variant_of,
    workspace_for,
)
