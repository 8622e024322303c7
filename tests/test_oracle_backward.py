"""Pins for the backward oracle (CPU only).

* Central finite differences of L = sum(O * dO) on tiny inputs, for every causal mode, a boolean
  mask and GQA: independent of the gradient formulas.
* torch's float64 autograd on the plain definition (an independent library routine).
* Closed forms: with every value row equal, O does not depend on Q or K (dQ = dK = 0) and dV is
  the column sums of P weighted by dO; a row with no kept key contributes nothing.
"""

import numpy as np
import pytest
import torch

from oracle import attention, attention_backward

RNG = np.random.default_rng(31)


def _loss(q, k, v, do, scale, **kw):
    o, _, _ = attention(q, k, v, scale, **kw)
    return float((o * do).sum())


def _finite_diff(q, k, v, do, scale, eps=1e-6, **kw):
    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = _loss(q, k, v, do, scale, **kw)
            x[i] = old - eps
            lm = _loss(q, k, v, do, scale, **kw)
            x[i] = old
            g[i] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


@pytest.mark.parametrize("Sq,Skv,Nq,Nkv,kw", [
    (3, 4, 1, 1, dict(sparse_mode=0)),
    (4, 3, 2, 1, dict(sparse_mode=2)),
    (3, 5, 2, 2, dict(sparse_mode=3)),
    (5, 3, 1, 1, dict(sparse_mode=3)),      # leading rows see no key
    (4, 4, 2, 1, dict(pre_tokens=1, next_tokens=0)),
])
def test_finite_differences(Sq, Skv, Nq, Nkv, kw):
    D = 3
    q, k, v = RNG.normal(size=(1, Nq, Sq, D)), RNG.normal(size=(1, Nkv, Skv, D)), RNG.normal(size=(1, Nkv, Skv, D))
    do = RNG.normal(size=(1, Nq, Sq, D))
    dq, dk, dv = attention_backward(q, k, v, do, 0.8, **kw)
    fq, fk, fv = _finite_diff(q, k, v, do, 0.8, **kw)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-8)


def test_finite_differences_boolean_mask():
    Sq, Skv, D = 4, 5, 2
    q, k, v = RNG.normal(size=(1, 1, Sq, D)), RNG.normal(size=(1, 1, Skv, D)), RNG.normal(size=(1, 1, Skv, D))
    do = RNG.normal(size=(1, 1, Sq, D))
    mask = (RNG.random((Sq, Skv)) < 0.4).astype(np.uint8)
    mask[2, :] = 1  # a row with no kept key
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, atten_mask=mask)
    fq, fk, fv = _finite_diff(q, k, v, do, 0.5, atten_mask=mask)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-8)
    assert np.all(dq[0, 0, 2] == 0)


@pytest.mark.parametrize("mode", [0, 2, 3])
def test_matches_torch_autograd(mode):
    B, Nq, Nkv, Sq, Skv, D = 2, 4, 2, 37, 53, 8
    q, k, v = RNG.normal(size=(B, Nq, Sq, D)), RNG.normal(size=(B, Nkv, Skv, D)), RNG.normal(size=(B, Nkv, Skv, D))
    do = RNG.normal(size=(B, Nq, Sq, D))
    dq, dk, dv = attention_backward(q, k, v, do, 0.3, sparse_mode=mode)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(Nq // Nkv, dim=1)
    vv = tv.repeat_interleave(Nq // Nkv, dim=1)
    s = (tq @ kk.transpose(-1, -2)) * 0.3
    i = torch.arange(Sq)[:, None]
    j = torch.arange(Skv)[None, :]
    keep = torch.ones(Sq, Skv, dtype=torch.bool)
    if mode == 2:
        keep = j <= i
    elif mode == 3:
        keep = j <= i + (Skv - Sq)
    s = s.masked_fill(~keep, float("-inf"))
    o = torch.softmax(s, dim=-1) @ vv
    (o * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_constant_values_closed_form():
    Sq, Skv, D = 6, 9, 4
    q, k = RNG.normal(size=(1, 1, Sq, D)), RNG.normal(size=(1, 1, Skv, D))
    v = np.broadcast_to(RNG.normal(size=(1, 1, 1, D)), (1, 1, Skv, D)).copy()
    do = RNG.normal(size=(1, 1, Sq, D))
    dq, dk, dv = attention_backward(q, k, v, do, 0.7, sparse_mode=2)
    np.testing.assert_allclose(dq, 0, atol=1e-12)
    np.testing.assert_allclose(dk, 0, atol=1e-12)
    # dV_j = sum_i P_ij dO_i, with P rebuilt from the causal scores
    s = (q[0, 0] @ k[0, 0].T) * 0.7
    s = np.where(np.arange(Skv)[None, :] <= np.arange(Sq)[:, None], s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(dv[0, 0], p.T @ do[0, 0], rtol=1e-12, atol=1e-14)


def test_tnd_finite_differences():
    """TND: two sequences of different lengths, bottom-right causal, GQA; finite differences of the
    TND forward oracle (each sequence anchored inside itself)."""
    lq, lk, Nq, Nkv, D = [3, 2], [2, 4], 2, 1, 2
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    q, k, v = RNG.normal(size=(cq[-1], Nq, D)), RNG.normal(size=(ck[-1], Nkv, D)), RNG.normal(size=(ck[-1], Nkv, D))
    do = RNG.normal(size=(cq[-1], Nq, D))
    kw = dict(layout="TND", sparse_mode=3, cu_seqlens_q=cq, cu_seqlens_kv=ck)
    dq, dk, dv = attention_backward(q, k, v, do, 0.9, **kw)
    fq, fk, fv = _finite_diff(q, k, v, do, 0.9, **kw)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-8)


def test_actual_lengths_finite_differences():
    """Per-batch actual lengths on padded BNSD: the gradients are those of the actual-length forward
    (finite differences through it), and padded rows and keys get exactly zero."""
    B, Nq, Sq, Skv, D = 2, 1, 4, 5, 2
    q, k, v = RNG.normal(size=(B, Nq, Sq, D)), RNG.normal(size=(B, Nq, Skv, D)), RNG.normal(size=(B, Nq, Skv, D))
    do = RNG.normal(size=(B, Nq, Sq, D))
    kw = dict(sparse_mode=3, actual_seq_q=[3, 4], actual_seq_kv=[5, 2])
    dq, dk, dv = attention_backward(q, k, v, do, 0.6, **kw)
    fq, fk, fv = _finite_diff(q, k, v, do, 0.6, sparse_mode=3, actual_seq_q=[3, 4], actual_seq_kv=[5, 2])
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-8)
    assert np.all(dq[0, :, 3:] == 0) and np.all(dk[1, :, 2:] == 0) and np.all(dv[1, :, 2:] == 0)


@pytest.mark.parametrize("layout,kw", [("BNSD", dict(sparse_mode=2)), ("BNSD", dict(sparse_mode=0)),
                                       ("TND", dict(sparse_mode=3))])
def test_finite_differences_value_dim_below_d(layout, kw):
    """Dv < D (v, O and dO narrower than q and k; the fused-attention guide allows D_v <= D_k):
    finite differences through the forward oracle, GQA 2."""
    D, Dv, Nq, Nkv = 3, 2, 2, 1
    if layout == "TND":
        lq, lk = [3, 2], [2, 4]
        cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
        q, k = RNG.normal(size=(cq[-1], Nq, D)), RNG.normal(size=(ck[-1], Nkv, D))
        v, do = RNG.normal(size=(ck[-1], Nkv, Dv)), RNG.normal(size=(cq[-1], Nq, Dv))
        kw = dict(kw, layout="TND", cu_seqlens_q=cq, cu_seqlens_kv=ck)
    else:
        q, k = RNG.normal(size=(1, Nq, 4, D)), RNG.normal(size=(1, Nkv, 5, D))
        v, do = RNG.normal(size=(1, Nkv, 5, Dv)), RNG.normal(size=(1, Nq, 4, Dv))
    dq, dk, dv = attention_backward(q, k, v, do, 0.75, **kw)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    fq, fk, fv = _finite_diff(q, k, v, do, 0.75, **kw)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-8)
