"""MI355X (gfx950) fused attention forward: batch, varlen, GQA and paged-KV
decode, as hand-written HIP kernels behind the C ABI in include/attn.h.

The Python functions carry the C entry points' names and only marshal
arguments; the library must be built (``python -m paged_kv_attn_amd.build``).
"""

from ._lib import AttnError, AttnParams  # noqa: F401
from .api import (  # noqa: F401
    attn_fwd,
    attn_fwd_paged,
    attn_fwd_paged_noalloc,
    attn_fwd_varlen,
    attn_fwd_varlen_paged,
    attn_last_error,
    attn_num_splits,
    attn_params,
    attn_workspace_bytes,
)
