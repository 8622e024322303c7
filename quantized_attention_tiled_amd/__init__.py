"""Fused, tiled attention for AMD MI355X (gfx950): forward and backward.

Python binding of the qattn C ABI (include/qattn.h). The kernels live in
``csrc/`` and are built into ``libqattn.so`` in this directory by
``python -m quantized_attention_tiled_amd.build``. Entry points:

* ``attn_fwd``                   dense bf16 / fp16: BNSD, BSND, BSH, SBH, TND varlen, GQA,
                                 causal, band, boolean masks, actual lengths, Dv <= D
* ``pack_atten_mask_bits``       byte atten_mask -> the bit-packed atten_mask attn_fwd takes
* ``build_kv_block_list``        128 x 128 block keep mask -> kept kv-block list
* ``build_qblock_order``         kept counts -> the order in which the sparse kernels take q-blocks
* ``attn_fwd_blocksparse``       bf16 / fp16 block-sparse attention over a kept list
* ``quantize_qk_perblock_int8``  Q/K INT8 per 128-token block
* ``quantize_v_perchannel_fp8``  V FP8 E4M3 per channel
* ``attn_fwd_qbsa``              INT8 Q.K / FP8 P.V quantised block-sparse attention
* ``attn_bwd``                   dQ, dK, dV of the dense forward (bf16 / fp16, every layout, GQA,
                                 causal, band, boolean masks, actual lengths; D, Dv multiples
                                 of 8 with Dv <= D <= 128; head ranges of whole GQA groups)
* ``attn_bwd_noalloc``           attn_bwd for callers that cannot allocate: its workspace is a
                                 static per-GPU buffer of the library

Each returns the attention output plus the per-row softmax max and sum where
the operation has them. Head and q-block subrange launches write only their
slice and reproduce the full call bit for bit.
"""

from .api import (  # noqa: F401
    attn_bwd,
    attn_bwd_noalloc,
    attn_fwd,
    attn_fwd_blocksparse,
    attn_fwd_qbsa,
    build_kv_block_list,
    build_qblock_order,
    make_desc,
    pack_atten_mask_bits,
    quantize_qk_perblock_int8,
    quantize_v_perchannel_fp8,
)
from ._lib import QattnError, load  # noqa: F401

__version__ = "0.1.0"
