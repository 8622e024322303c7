"""GPU parity of the bf16 attention backward (dQ, dK, dV) against the float64 gradient oracle.

The forward runs on the GPU (its bf16 O and softmax max / sum are the backward's inputs, as in
training); the oracle differentiates the exact definition from the same bf16 Q, K, V and dO.

Tolerance, per gradient tensor: max-abs error <= 2e-2 * max(1, max |reference|). The kernels round
P and dS to bf16 before their products (relative 2^-9 each) and write bf16 (half an ulp, 2^-9
relative); the row term rowsum(dO * O) uses the forward's bf16 O. Each is a relative error of the
gradient's own magnitude, and together they stay below about 2^-7 of the largest entry; 2e-2 leaves
room for the sums over up to a few hundred keys or queries. Rows with no kept key must give dQ = 0
exactly, and repeated calls must give the same bits.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import banner, dev_bf16, f64, to_np
from workloads import random_bf16

pytestmark = pytest.mark.gpu

G_RTOL = 2e-2


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
    banner(f"{what}: max-abs err {err:.3e} (bound {bound:.3e}, max |ref| {np.abs(ref).max() if ref.size else 0:.3e})")
    assert err <= bound, f"{what}: max abs error {err:.3e} > {bound:.3e}"


def _run(qa, B, Nq, Nkv, Sq, Skv, D, mode, seed):
    qb = random_bf16(seed, (B, Nq, Sq, D))
    kb = random_bf16(seed + 1, (B, Nkv, Skv, D))
    vb = random_bf16(seed + 2, (B, Nkv, Skv, D))
    gb = random_bf16(seed + 3, (B, Nq, Sq, D))
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, sparse_mode=mode)
    dq, dk, dv = qa.attn_bwd(q, k, v, o, do, m, l, scale=scale, sparse_mode=mode)
    torch.cuda.synchronize()
    return (q, k, v, o, do, m, l, scale), (dq, dk, dv), (qb, kb, vb, gb)


@pytest.mark.parametrize("B,Nq,Nkv,Sq,Skv,D,mode", [
    (1, 2, 2, 256, 256, 64, 0),
    (2, 4, 2, 300, 300, 128, 0),     # ragged tails, GQA 2
    (1, 4, 1, 200, 333, 128, 0),     # Sq != Skv, GQA 4
    (1, 2, 2, 384, 384, 128, 2),
    (2, 4, 2, 300, 300, 64, 2),
    (1, 2, 1, 200, 450, 128, 3),     # bottom-right, Skv > Sq
    (1, 2, 2, 450, 200, 128, 3),     # bottom-right, Sq > Skv: leading rows see no key
    (1, 1, 1, 1, 1, 128, 0),
    (1, 1, 1, 5, 700, 64, 3),
])
def test_backward_against_oracle(qa, B, Nq, Nkv, Sq, Skv, D, mode):
    what = f"bwd B={B} Nq={Nq} Nkv={Nkv} Sq={Sq} Skv={Skv} D={D} mode={mode}"
    banner(what)
    fwd, (dq, dk, dv), (qb, kb, vb, gb) = _run(qa, B, Nq, Nkv, Sq, Skv, D, mode, 700 + Sq + Skv + D + mode)
    rq, rk, rv = oracle.attention_backward(f64(qb), f64(kb), f64(vb), f64(gb), fwd[7], sparse_mode=mode)
    _check(dq, rq, what + " dQ")
    _check(dk, rk, what + " dK")
    _check(dv, rv, what + " dV")
    if mode == 3 and Sq > Skv:  # rows i < Sq - Skv keep no key: their dQ is exactly 0
        assert torch.all(dq[:, :, :Sq - Skv] == 0)


def test_backward_deterministic(qa):
    fwd, g1, _ = _run(qa, 1, 4, 2, 640, 640, 128, 2, 901)
    q, k, v, o, do, m, l, scale = fwd
    for _ in range(2):
        g2 = qa.attn_bwd(q, k, v, o, do, m, l, scale=scale, sparse_mode=2)
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("mode,Nq,Nkv,D", [(3, 4, 2, 128), (0, 2, 2, 64), (2, 8, 2, 128)])
def test_backward_tnd(qa, mode, Nq, Nkv, D):
    """Varlen TND: sequences of unequal query and key lengths, including an empty and a one-token
    sequence; each sequence is its own problem."""
    lq, lk = [300, 0, 1, 130, 64], [280, 5, 40, 130, 200]
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    what = f"bwd TND mode={mode} Nq={Nq} Nkv={Nkv} D={D}"
    banner(what)
    qb = random_bf16(41, (cq[-1], Nq, D))
    kb = random_bf16(42, (ck[-1], Nkv, D))
    vb = random_bf16(43, (ck[-1], Nkv, D))
    gb = random_bf16(44, (cq[-1], Nq, D))
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    kw = dict(scale=scale, sparse_mode=mode, layout="TND", cu_seqlens_q=cq.tolist(), cu_seqlens_kv=ck.tolist())
    o, m, l = qa.attn_fwd(q, k, v, **kw)
    dq, dk, dv = qa.attn_bwd(q, k, v, o, do, m, l, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(f64(qb), f64(kb), f64(vb), f64(gb), scale, layout="TND", sparse_mode=mode,
                                           cu_seqlens_q=cq, cu_seqlens_kv=ck)
    _check(dq, rq, what + " dQ")
    _check(dk, rk, what + " dK")
    _check(dv, rv, what + " dV")


@pytest.mark.parametrize("layout", ["BSND", "BSH", "SBH"])
def test_backward_layouts_match_bnsd(qa, layout):
    """The batched layouts differ from BNSD only in the strides: the gradients must be the same bits."""
    B, Nq, Nkv, S, D = 2, 4, 2, 300, 128
    banner(f"bwd layout {layout}")
    fwd, grads, _ = _run(qa, B, Nq, Nkv, S, S, D, 3, 55)
    q, k, v, o, do, m, l, scale = fwd

    def to(x):  # BNSD -> layout
        if layout == "BSND":
            return x.transpose(1, 2).contiguous()
        y = x.permute(0, 2, 1, 3) if layout == "BSH" else x.permute(2, 0, 1, 3)
        return y.reshape(y.shape[0], y.shape[1], -1).contiguous()

    kw = dict(scale=scale, sparse_mode=3, layout=layout, head_num=Nq)
    g2 = qa.attn_bwd(to(q), to(k), to(v), to(o), to(do), m, l, **kw)
    torch.cuda.synchronize()
    for a, b in zip(grads, g2):
        assert torch.equal(to(a).view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("mode,D", [(0, 128), (3, 128), (2, 64)])
def test_backward_fp16(qa, mode, D):
    """float16 tensors: P and dS are rounded to fp16 (2^-11) and the gradients are written in fp16;
    the same relative bound holds with room to spare."""
    from workloads import random_f16
    B, Nq, Nkv, S = 1, 4, 2, 300
    what = f"bwd fp16 mode={mode} D={D}"
    banner(what)
    x = [random_f16(60 + i, shape) for i, shape in enumerate([(B, Nq, S, D), (B, Nkv, S, D), (B, Nkv, S, D),
                                                               (B, Nq, S, D)])]
    q, k, v, do = (torch.from_numpy(a).cuda() for a in x)
    scale = 1.0 / np.sqrt(D)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, sparse_mode=mode)
    dq, dk, dv = qa.attn_bwd(q, k, v, o, do, m, l, scale=scale, sparse_mode=mode)
    torch.cuda.synchronize()
    assert dq.dtype == torch.float16
    rq, rk, rv = oracle.attention_backward(*(a.astype(np.float64) for a in x), scale, sparse_mode=mode)
    _check(dq.float(), rq, what + " dQ")
    _check(dk.float(), rk, what + " dK")
    _check(dv.float(), rv, what + " dV")


@pytest.mark.parametrize("kw,D", [
    (dict(pre_tokens=100, next_tokens=20), 128),
    (dict(pre_tokens=0, next_tokens=0), 64),       # the diagonal only
    (dict(pre_tokens=-5, next_tokens=40), 128),    # a band off the diagonal
    (dict(pre_tokens=2147483647, next_tokens=-3), 128),  # one-sided
])
def test_backward_band(qa, kw, D):
    B, Nq, Nkv, Sq, Skv = 1, 4, 2, 330, 300
    what = f"bwd band {kw} D={D}"
    banner(what)
    qb, kb, vb, gb = (random_bf16(90 + i, s) for i, s in enumerate([(B, Nq, Sq, D), (B, Nkv, Skv, D), (B, Nkv, Skv, D),
                                                                    (B, Nq, Sq, D)]))
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, **kw)
    dq, dk, dv = qa.attn_bwd(q, k, v, o, do, m, l, scale=scale, **kw)
    torch.cuda.synchronize()
    band = {k2: (None if v2 == 2147483647 else v2) for k2, v2 in kw.items()}
    rq, rk, rv = oracle.attention_backward(f64(qb), f64(kb), f64(vb), f64(gb), scale, **band)
    _check(dq, rq, what + " dQ")
    _check(dk, rk, what + " dK")
    _check(dv, rv, what + " dV")


@pytest.mark.parametrize("kind,mode", [("SS", 0), ("B1SS", 2), ("BNSS", 3)])
def test_backward_boolean_mask(qa, kind, mode):
    B, Nq, Nkv, Sq, Skv, D = 2, 4, 2, 200, 260, 128
    what = f"bwd mask {kind} mode={mode}"
    banner(what)
    qb, kb, vb, gb = (random_bf16(95 + i, s) for i, s in enumerate([(B, Nq, Sq, D), (B, Nkv, Skv, D), (B, Nkv, Skv, D),
                                                                    (B, Nq, Sq, D)]))
    shape = {"SS": (Sq, Skv), "B1SS": (B, 1, Sq, Skv), "BNSS": (B, Nq, Sq, Skv)}[kind]
    mask = (np.random.default_rng(96).random(shape) < 0.3).astype(np.uint8)
    mask[..., 11, :] = 1  # a row with no kept key
    scale = 0.088
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    mt = torch.from_numpy(mask).cuda()
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, sparse_mode=mode, atten_mask=mt)
    dq, dk, dv = qa.attn_bwd(q, k, v, o, do, m, l, scale=scale, sparse_mode=mode, atten_mask=mt)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(f64(qb), f64(kb), f64(vb), f64(gb), scale, sparse_mode=mode,
                                           atten_mask=mask)
    _check(dq, rq, what + " dQ")
    _check(dk, rk, what + " dK")
    _check(dv, rv, what + " dV")
    assert torch.all(dq[:, :, 11] == 0)


@pytest.mark.parametrize("mode", [0, 3])
def test_backward_actual_lengths(qa, mode):
    """Padded BNSD with per-batch actual lengths: the padding of Q, K, V and dO is NaN and must never
    be read; padded rows of dQ and padded keys of dK / dV come out as zeros, whatever the output
    buffers held; the rest matches the oracle."""
    B, Nq, Nkv, Sq, Skv, D = 3, 4, 2, 330, 300, 128
    aq, akv = [330, 129, 0], [300, 77, 40]
    what = f"bwd actual lengths mode={mode}"
    banner(what)
    nan = np.uint16(0x7FC0)

    def padded(seed, shape, lens):
        x = random_bf16(seed, shape)
        for b, L in enumerate(lens):
            x[b, :, L:] = nan
        return x

    qb, kb, vb = padded(70, (B, Nq, Sq, D), aq), padded(71, (B, Nkv, Skv, D), akv), padded(72, (B, Nkv, Skv, D), akv)
    gb = padded(73, (B, Nq, Sq, D), aq)
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    kw = dict(scale=scale, sparse_mode=mode, actual_seq_lengths=aq, actual_seq_lengths_kv=akv)
    o, m, l = qa.attn_fwd(q, k, v, **kw)
    bufs = tuple(torch.full_like(x, 5.0) for x in (q, k, v))
    dq, dk, dv = qa.attn_bwd(q, k, v, o, do, m, l, dq=bufs[0], dk=bufs[1], dv=bufs[2], **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(np.nan_to_num(f64(qb)), np.nan_to_num(f64(kb)), np.nan_to_num(f64(vb)),
                                           np.nan_to_num(f64(gb)), scale, sparse_mode=mode, actual_seq_q=aq,
                                           actual_seq_kv=akv)
    _check(dq, rq, what + " dQ")
    _check(dk, rk, what + " dK")
    _check(dv, rv, what + " dV")
    for b in range(B):
        assert torch.all(dq[b, :, aq[b]:] == 0) and torch.all(dk[b, :, akv[b]:] == 0) and torch.all(dv[b, :, akv[b]:] == 0)
