"""Gradients of the plain attention definition (oracle; tests only).

The fused attention guide ("Ascend NPU fused attention operator", section 2)
presents the fused operator as a training operator: the softmax max and sum of
section 5 are kept for the backward pass, and the tiled form is said to bring
the backward memory from O(N^2) down to O(N). The pages give no backward
algorithm, so this module is the derivative of the section 2 definition
O = P V, P = softmax(mask(Q K^T scale)) row by row, written out in float64
with the explicit score matrix (masked pairs have P = 0):

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))      (the softmax Jacobian applied row-wise)
    dQ = scale * dS K
    dK = scale * dS^T Q

A row with no kept key has O = 0 and contributes nothing. Masks, causal modes,
GQA and layouts follow ``attention``'s readings (contiguous head groups: a
kv-head's gradient sums over the q-heads that read it).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import BLOCK, _allowed, _mask_for_head


def softmax_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                               allowed: np.ndarray):
    """Gradients for one head: q [R, D], k [Skv, D], v [Skv, Dv], do [R, Dv], allowed [R, Skv].

    Returns (dq [R, D], dk [Skv, D], dv [Skv, Dv])."""
    s = (q @ k.T) * scale
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    live = np.isfinite(m)
    p = np.exp(s - np.where(live, m, 0.0)[:, None])
    l = p.sum(axis=1)
    p = p / np.where(live, l, 1.0)[:, None]
    p[~live] = 0.0
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float, *,
                       layout: str = "BNSD", sparse_mode: int = 0, atten_mask: Optional[np.ndarray] = None,
                       pre_tokens: Optional[int] = None, next_tokens: Optional[int] = None,
                       cu_seqlens_q: Optional[np.ndarray] = None, cu_seqlens_kv: Optional[np.ndarray] = None,
                       actual_seq_q=None, actual_seq_kv=None):
    """Gradients (dq, dk, dv) shaped like q, k, v.

    BNSD: q [B, Nq, Sq, D], k/v [B, Nkv, Skv, D(v)], do [B, Nq, Sq, Dv].
    TND:  q [T, Nq, D], k/v [Tk, Nkv, D(v)], do [T, Nq, Dv], with cumulative lengths; each
          sequence is its own problem (causal anchors counted inside it).
    ``actual_seq_q`` / ``actual_seq_kv`` (BNSD): batch b is its first aq_b rows and akv_b keys,
    as in ``attention``; padded rows and keys get zero gradients."""
    if layout == "TND":
        if atten_mask is not None:
            raise ValueError("TND takes no boolean mask")
        dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
        for b in range(len(cu_seqlens_q) - 1):
            q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
            k0, k1 = int(cu_seqlens_kv[b]), int(cu_seqlens_kv[b + 1])
            gq, gk, gv = attention_backward(q[q0:q1].transpose(1, 0, 2)[None], k[k0:k1].transpose(1, 0, 2)[None],
                                            v[k0:k1].transpose(1, 0, 2)[None], do[q0:q1].transpose(1, 0, 2)[None],
                                            scale, sparse_mode=sparse_mode, pre_tokens=pre_tokens,
                                            next_tokens=next_tokens)
            dq[q0:q1] = gq[0].transpose(1, 0, 2)
            dk[k0:k1] = gk[0].transpose(1, 0, 2)
            dv[k0:k1] = gv[0].transpose(1, 0, 2)
        return dq, dk, dv
    if layout != "BNSD":
        raise ValueError("layout must be BNSD or TND")
    B, Nq, Sq, D = q.shape
    Nkv, Skv = k.shape[1], k.shape[2]
    if Nq % Nkv:
        raise ValueError("Nq must be a multiple of Nkv")
    g = Nq // Nkv
    aq = [Sq] * B if actual_seq_q is None else [int(x) for x in actual_seq_q]
    akv = [Skv] * B if actual_seq_kv is None else [int(x) for x in actual_seq_kv]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        lq, lk = aq[b], akv[b]
        rows = np.arange(lq)
        for h in range(Nq):
            mask = _mask_for_head(atten_mask, b, h)
            mask = None if mask is None else mask[:lq, :lk]
            a = _allowed(rows, lq, lk, sparse_mode, mask, None, pre_tokens, next_tokens)
            gq, gk, gv = softmax_attention_backward(q[b, h, :lq], k[b, h // g, :lk], v[b, h // g, :lk], do[b, h, :lq],
                                                    scale, a)
            dq[b, h, :lq] = gq
            dk[b, h // g, :lk] += gk
            dv[b, h // g, :lk] += gv
    return dq, dk, dv


__all__ = ["attention_backward", "softmax_attention_backward", "BLOCK"]
