"""GPU parity of the attention backward at head dimensions other than D = Dv = 64 or 128.

The fused-attention guide lets the value head dimension be smaller than the query/key one
(D_v <= D_k, section 4.1) and allows other head sizes (section 7). The backward takes D and Dv
that are multiples of 8 with Dv <= D <= 128; it runs on the kernels built for width 64 or 128 with
every column past D (q, k) or Dv (v, o, dO) read as zero.

Checks, per case: the gradients against the float64 oracle (bound as in test_gpu_backward.py:
max-abs <= 2e-2 * max(1, max |reference|)); nothing written past the end of dq, dk, dv (each
output is a view at the start of a larger sentinel-filled buffer); and bit identity with the
same problem zero-padded to D = Dv = 64 or 128, the width of the kernels it runs on.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import banner, dev_bf16, f64, to_np
from workloads import random_bf16

pytestmark = pytest.mark.gpu

G_RTOL = 2e-2
SENTINEL = 0x7BAD


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _check(g, ref, what):
    g = to_np(g)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    bound = G_RTOL * max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)
    err = float(np.abs(g - ref).max()) if ref.size else 0.0
    banner(f"{what}: max-abs err {err:.3e} (bound {bound:.3e})")
    assert err <= bound, f"{what}: max abs error {err:.3e} > {bound:.3e}"


def _guarded(like: torch.Tensor):
    """A contiguous tensor shaped like `like` at the start of a buffer with 256 sentinel elements
    after it; returns (view, buffer)."""
    buf = torch.full((like.numel() + 256,), SENTINEL, dtype=torch.int16, device=like.device)
    return buf[:like.numel()].view(like.dtype).view(like.shape), buf


def _tail_intact(buf, n):
    assert torch.all(buf[n:] == SENTINEL), "a gradient was written past the end of its tensor"


def _pad(bits: np.ndarray, width: int) -> np.ndarray:
    out = np.zeros(bits.shape[:-1] + (width,), np.uint16)
    out[..., :bits.shape[-1]] = bits
    return out


@pytest.mark.parametrize("B,Nq,Nkv,Sq,Skv,D,Dv,mode", [
    (1, 2, 1, 300, 300, 128, 64, 0),    # Dv < D, GQA 2, ragged tail
    (2, 4, 2, 200, 333, 128, 64, 3),    # bottom-right causal, Sq != Skv
    (1, 2, 2, 256, 256, 96, 96, 2),     # D between the built widths
    (1, 4, 2, 300, 300, 120, 72, 0),
    (1, 2, 2, 130, 130, 64, 32, 2),     # the 64-wide kernels
    (1, 2, 1, 200, 200, 40, 40, 0),
    (1, 1, 1, 70, 90, 16, 8, 3),        # the smallest head dimensions
])
def test_backward_head_dims_against_oracle(qa, B, Nq, Nkv, Sq, Skv, D, Dv, mode):
    what = f"bwd B={B} Nq={Nq} Nkv={Nkv} Sq={Sq} Skv={Skv} D={D} Dv={Dv} mode={mode}"
    banner(what)
    seed = 1300 + D + Dv + mode
    qb = random_bf16(seed, (B, Nq, Sq, D))
    kb = random_bf16(seed + 1, (B, Nkv, Skv, D))
    vb = random_bf16(seed + 2, (B, Nkv, Skv, Dv))
    gb = random_bf16(seed + 3, (B, Nq, Sq, Dv))
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, sparse_mode=mode)
    assert o.shape == (B, Nq, Sq, Dv)
    (dq, bq), (dk, bk), (dv, bv) = _guarded(q), _guarded(k), _guarded(v)
    qa.attn_bwd(q, k, v, o, do, m, l, scale=scale, sparse_mode=mode, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t, buf in ((dq, bq), (dk, bk), (dv, bv)):
        _tail_intact(buf, t.numel())
    rq, rk, rv = oracle.attention_backward(f64(qb), f64(kb), f64(vb), f64(gb), scale, sparse_mode=mode)
    _check(dq, rq, what + " dQ")
    _check(dk, rk, what + " dK")
    _check(dv, rv, what + " dV")

    # the same problem with zero columns up to the width of the kernels it runs on (D = Dv = 64 or
    # 128): the same products in the same order, bit for bit
    W = 64 if D <= 64 else 128
    q2, k2 = dev_bf16(_pad(qb, W)), dev_bf16(_pad(kb, W))
    v2, do2 = dev_bf16(_pad(vb, W)), dev_bf16(_pad(gb, W))
    o2 = torch.zeros((B, Nq, Sq, W), dtype=torch.bfloat16, device=o.device)
    o2[..., :Dv] = o
    g2 = qa.attn_bwd(q2, k2, v2, o2, do2, m, l, scale=scale, sparse_mode=mode)
    torch.cuda.synchronize()
    for a, b, w in ((dq, g2[0], D), (dk, g2[1], D), (dv, g2[2], Dv)):
        assert torch.equal(a.view(torch.int16), b[..., :w].contiguous().view(torch.int16)), what + " vs padded"
        assert torch.all(b[..., w:] == 0)


@pytest.mark.parametrize("mode,Nq,Nkv,D,Dv", [(3, 4, 2, 128, 64), (0, 2, 2, 72, 48)])
def test_backward_head_dims_tnd(qa, mode, Nq, Nkv, D, Dv):
    """Varlen TND with Dv < D: unequal query and key lengths, an empty and a one-token sequence."""
    lq, lk = [300, 0, 1, 130, 64], [280, 5, 40, 130, 200]
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    what = f"bwd TND mode={mode} Nq={Nq} Nkv={Nkv} D={D} Dv={Dv}"
    banner(what)
    qb = random_bf16(141, (cq[-1], Nq, D))
    kb = random_bf16(142, (ck[-1], Nkv, D))
    vb = random_bf16(143, (ck[-1], Nkv, Dv))
    gb = random_bf16(144, (cq[-1], Nq, Dv))
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    kw = dict(scale=scale, sparse_mode=mode, layout="TND", cu_seqlens_q=cq.tolist(), cu_seqlens_kv=ck.tolist())
    o, m, l = qa.attn_fwd(q, k, v, **kw)
    (dq, bq), (dk, bk), (dv, bv) = _guarded(q), _guarded(k), _guarded(v)
    qa.attn_bwd(q, k, v, o, do, m, l, dq=dq, dk=dk, dv=dv, **kw)
    torch.cuda.synchronize()
    for t, buf in ((dq, bq), (dk, bk), (dv, bv)):
        _tail_intact(buf, t.numel())
    rq, rk, rv = oracle.attention_backward(f64(qb), f64(kb), f64(vb), f64(gb), scale, layout="TND", sparse_mode=mode,
                                           cu_seqlens_q=cq, cu_seqlens_kv=ck)
    _check(dq, rq, what + " dQ")
    _check(dk, rk, what + " dK")
    _check(dv, rv, what + " dV")


@pytest.mark.parametrize("layout", ["BSND", "BSH", "SBH"])
def test_backward_head_dims_layouts_match_bnsd(qa, layout):
    """Dv < D in the batched layouts (v, o and dO with their own head width): the same bits as BNSD."""
    B, Nq, Nkv, S, D, Dv = 2, 4, 2, 300, 128, 64
    banner(f"bwd layout {layout} D={D} Dv={Dv}")
    qb, kb = random_bf16(151, (B, Nq, S, D)), random_bf16(152, (B, Nkv, S, D))
    vb, gb = random_bf16(153, (B, Nkv, S, Dv)), random_bf16(154, (B, Nq, S, Dv))
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, sparse_mode=3)
    grads = qa.attn_bwd(q, k, v, o, do, m, l, scale=scale, sparse_mode=3)

    def to(x):  # BNSD -> layout
        if layout == "BSND":
            return x.transpose(1, 2).contiguous()
        y = x.permute(0, 2, 1, 3) if layout == "BSH" else x.permute(2, 0, 1, 3)
        return y.reshape(y.shape[0], y.shape[1], -1).contiguous()

    g2 = qa.attn_bwd(to(q), to(k), to(v), to(o), to(do), m, l, scale=scale, sparse_mode=3, layout=layout,
                     head_num=Nq)
    torch.cuda.synchronize()
    for a, b in zip(grads, g2):
        assert torch.equal(to(a).view(torch.int16), b.view(torch.int16))


def test_backward_head_dims_fp16(qa):
    """float16 with Dv < D, causal, GQA."""
    from workloads import random_f16
    B, Nq, Nkv, S, D, Dv = 1, 4, 2, 260, 128, 64
    banner(f"bwd fp16 D={D} Dv={Dv}")
    x = [random_f16(160 + i, s) for i, s in enumerate([(B, Nq, S, D), (B, Nkv, S, D), (B, Nkv, S, Dv),
                                                        (B, Nq, S, Dv)])]
    q, k, v, do = (torch.from_numpy(a).cuda() for a in x)
    scale = 1.0 / np.sqrt(D)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, sparse_mode=2)
    dq, dk, dv = qa.attn_bwd(q, k, v, o, do, m, l, scale=scale, sparse_mode=2)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(*(a.astype(np.float64) for a in x), scale, sparse_mode=2)
    _check(dq.float(), rq, "fp16 dQ")
    _check(dk.float(), rk, "fp16 dK")
    _check(dv.float(), rv, "fp16 dV")
