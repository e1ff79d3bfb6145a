"""MI355X (gfx950) ragged extreme-GQA attention: forward and full VJP.

The compute path is the HIP library ``libragged_gqa_attn.so`` behind the C ABI
in include/attn_varlen.h; this package only marshals arguments to it.  The
entry points load the library on first use and raise if it is not built.
"""
from .api import (FullVJP, attention_varlen_feature_full_vjp, attn_varlen_bwd,
                  attn_varlen_full_vjp, attn_varlen_fwd, workspace_size)

__all__ = ["attention_varlen_feature_full_vjp", "attn_varlen_fwd", "attn_varlen_bwd",
           "attn_varlen_full_vjp", "FullVJP", "workspace_size"]
