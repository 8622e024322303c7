"""attn_bwd_noalloc against attn_bwd through the C ABI.

attn_bwd_noalloc runs the backward's kernels with the library's static per-GPU workspace in place
of the caller's buffer, so its gradients must equal attn_bwd's bit for bit. Two calls in a row, the
second with a smaller problem (a different layout and head dimension), check that the buffer's
contents from one call do not leak into the next.
"""

import numpy as np
import pytest
import torch

from gpu_util import banner, dev_bf16
from workloads import random_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _case(qa, shape_q, shape_k, seed, **kw):
    q = dev_bf16(random_bf16(seed, shape_q))
    k = dev_bf16(random_bf16(seed + 1, shape_k))
    v = dev_bf16(random_bf16(seed + 2, shape_k))
    do = dev_bf16(random_bf16(seed + 3, shape_q))
    o, m, l = qa.attn_fwd(q, k, v, **kw)
    ref = qa.attn_bwd(q, k, v, o, do, m, l, **kw)
    got = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    qa.attn_bwd_noalloc(q, k, v, o, do, m, l, *got, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert _same(a, b), f"{name} differs from attn_bwd"
        assert torch.isfinite(a.float()).all(), name


def test_noalloc_matches_attn_bwd_twice(qa):
    banner("noalloc backward: BNSD B=2 Nq=4 Nkv=2 S=300 D=128 causal")
    _case(qa, (2, 4, 300, 128), (2, 2, 300, 128), 1300, scale=128 ** -0.5, sparse_mode=2)
    banner("noalloc backward: TND 2 sequences (100, 57) Nq=2 Nkv=1 D=64 (smaller)")
    cu = [0, 100, 157]
    _case(qa, (157, 2, 64), (157, 1, 64), 1310, scale=0.125, layout="TND", cu_seqlens_q=cu, cu_seqlens_kv=cu,
          sparse_mode=3)


def test_noalloc_rejects_oversized_workspace(qa):
    from quantized_attention_tiled_amd._lib import NOALLOC_WORKSPACE_BYTES, QATTN_UNSUPPORTED, QattnError
    rows = NOALLOC_WORKSPACE_BYTES // 8 + 128          # one q-block of rows too many
    S = 128
    B = rows // S
    banner(f"noalloc backward: {rows} rows rejected")
    t = torch.zeros((B, 1, S, 64), dtype=torch.bfloat16, device="cuda")
    ml = torch.zeros((B, 1, S), dtype=torch.float32, device="cuda")
    with pytest.raises(QattnError) as e:
        qa.attn_bwd_noalloc(t, t, t, t, t, ml, ml, t, t, t, scale=0.125)
    assert e.value.status == QATTN_UNSUPPORTED
    assert np.isfinite(float(t[0, 0, 0, 0]))
