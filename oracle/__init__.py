"""CPU oracle for the fused attention forward: TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, deliberately unoptimised reference. Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it; the HIP product path never does, and there is no CPU fallback through it.
It shares no code with the HIP path: it uses NumPy only.

What it computes, and which passage each part follows (the pages are the
``npu_fusion_attention`` guide, "Ascend NPU fused attention operator", and the
EagleQBSA article, "EagleQBSA quantised block-sparse attention"):

* ``attention``      softmax(mask(Q K^T scale)) V with the explicit score matrix,
                     in float64; softmax max and sum per row (fused attention
                     guide, section 2 formula and section 5 outputs; masks and
                     layouts from section 4; GQA from section 7).
* ``quant``          INT8 per-128-token-block Q/K and FP8 E4M3 per-channel V
                     quantisers in exact float32 steps; E4M3 encode/decode from
                     the format's definition; the kept-block list (EagleQBSA
                     article, scheme-design section and the API call at its end)
                     and the q-block order by kept count.
* ``backward``       the gradients dQ, dK, dV of the ``attention`` definition,
                     written out in float64 (the guide presents the operator
                     as a training operator but gives no backward algorithm).
* ``qbsa``           the quantised block-sparse forward, following the tiled
                     schedule with P cast to FP8 inside the loop (EagleQBSA
                     article, scheme-design and operator-optimisation sections).

Every function is pinned by tests in ``tests/test_oracle_*.py`` against
invariants, closed forms, brute force and independent library routines.
"""

from .backward import attention_backward, softmax_attention_backward  # noqa: F401
from .attention import (  # noqa: F401
    atten_mask_from_bits,
    attention,
    attention_block_sparse,
    attention_rows,
    softmax_attention,
)
from .quant import (  # noqa: F401
    qblock_order,
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    kept_block_list,
    quantize_qk_perblock_int8,
    quantize_v_perchannel_fp8,
)
from .qbsa import qbsa_attention, qbsa_plain_rows, qbsa_qblock  # noqa: F401
