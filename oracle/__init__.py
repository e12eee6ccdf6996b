"""Plain, slow, fp64 CPU oracle for the fused attention forward pass.

This package is TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it. The product
path (``paged_kv_attn_amd``) never imports it, and it imports nothing from the
product path: the two share no kernels, helpers, tables or index logic. Only the
seeded input generators in ``synth`` feed both sides.

What it computes is the plain definition of attention written out (see
``attention.py``); every public function cites the passage of the source pages
it follows. The pages are three source listings:

* "flash-attention/hopper/epilogue_fwd.hpp" (FlashAttention-3 forward epilogue,
  ``CollectiveEpilogueFwd``),
* "Composable Kernel: fmha_fwd_pagedkv_kernel.hpp Source File"
  (``ck_tile::FmhaFwdPagedKVKernel``),
* "flash_attn_mma_share_kv_F32F16F16F32.cu" (CUDA-Learn-Notes FlashAttention-2
  forward with mma.sync).
"""

from .attention import (  # noqa: F401
    E4M3FN_TABLE,
    attention_batch,
    attention_paged,
    attention_varlen,
    attention_varlen_paged,
    bf16_bits_to_f64,
    e4m3fn_bits_to_f64,
    e4m3fn_value,
    head_attention,
    masked_allowed,
)
