"""Gated delta rule on AMD Instinct MI355X (gfx950): a C-ABI HIP library (libgdn.so) and its
Python binding.

    from gated_deltanet_delta_amd import gdn_chunk_fwd, gdn_recurrent_step

The binding only marshals torch tensors into the C ABI declared in include/gdn.h; the library must
be built (``python -m gated_deltanet_delta_amd.build``) and there is no CPU fallback.
"""
from .api import (chunk_gated_delta_rule, gdn_causal_conv1d, gdn_chunk_fwd,  # noqa: F401
                  gdn_chunk_bwd, gdn_chunk_bwd_ex, gdn_chunk_fwd_ex, gdn_chunk_fwd_gated_norm, gdn_chunk_fwd_gating, gdn_recurrent_step_ex,
                  gdn_chunk_fwd_indexed, gdn_chunk_fwd_noalloc, gdn_gated_rmsnorm, gdn_recurrent_step,
                  gdn_recurrent_step_gating,
                  gdn_recurrent_step_indexed, recurrent_gated_delta_rule, workspace_size)
from ._lib import GdnError  # noqa: F401
