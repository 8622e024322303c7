"""Plain float64 attention with the explicit score matrix (oracle; tests only).

Definition followed ("Ascend NPU fused attention operator" guide):
  * section 2: O = Softmax(Mask(Q K^T * scale)) V; no positional bias and no
    dropout are modelled.
  * section 6.1 spells out the unfused steps: scores = Q K^T * scale, add the
    mask, softmax over keys, multiply by V. This module is exactly those steps.
  * section 4.2: ``atten_mask`` uses 1 = masked, 0 = kept, shapes SS / B1SS / BNSS;
    section 8 recommends a compressed mask with the causal modes (``atten_mask_from_bits``
    states the bit layout read here).
  * section 4.3: ``sparse_mode`` 2 and 3 are causal lower triangles anchored at
    the top-left and bottom-right corners; ``sparse_mode`` 0 takes its range from
    ``pre_tokens`` and ``next_tokens`` (section 3's prototype defaults both to
    2147483647, i.e. no limit); varlen sequences are described by cumulative
    lengths (TND layout, section 4.1).
  * section 5: outputs are the attention result plus the softmax max and sum.
  * section 7: GQA requires Nq / Nkv to be an integer.
  * EagleQBSA article, API call: per-batch ``actual_seq_lengths`` /
    ``actual_seq_lengths_kv`` beside a padded BNSD tensor.

Readings where the guide is silent (each stated once here):
  * causal top-left keeps j <= i, bottom-right keeps j <= i + Skv - Sq, with i
    and j counted inside one sequence;
  * the sparse_mode 0 range keeps i - pre_tokens <= j <= i + next_tokens (a
    band around the top-left diagonal; pre/next None means no limit), also
    counted inside one sequence; the band is not combined with modes 2 and 3;
  * softmax_max m is the row maximum of the scaled, masked scores (natural-log
    domain) and softmax_sum l = sum_j exp(s_ij - m); a row with no unmasked key
    has O = 0, m = -inf, l = 0;
  * q-head h reads kv-head h // (Nq / Nkv) (contiguous groups);
  * block keep masks use 1 = keep on 128 x 128 blocks;
  * m and l are laid out [B, Nq, Sq] for BNSD and [Nq, T] for TND;
  * with actual lengths (aq_b, akv_b), batch b is the sequence of its first
    aq_b queries and akv_b keys (masks, causal anchors and the band counted
    inside it); its padded rows aq_b .. Sq - 1 are rows with no key (O = 0,
    m = -inf, l = 0).

Scores are formed 128 query rows at a time so long sequences fit in memory;
each slab is the plain definition on those rows.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

BLOCK = 128


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                      allowed: np.ndarray):
    """Plain attention on one head.

    q [R, D], k [Skv, D], v [Skv, Dv] (float64); ``allowed`` [R, Skv] bool.
    Returns (o [R, Dv], m [R], l [R]).
    """
    s = (q @ k.T) * scale
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    live = np.isfinite(m)
    p = np.exp(s - np.where(live, m, 0.0)[:, None])   # exp(-inf) = 0 for masked
    l = p.sum(axis=1)
    o = (p @ v) / np.where(live, l, 1.0)[:, None]
    o[~live] = 0.0
    return o, m, l


def _allowed(rows: np.ndarray, Sq: int, Skv: int, sparse_mode: int,
             mask_rows: Optional[np.ndarray], keep: Optional[np.ndarray],
             pre_tokens: Optional[int] = None, next_tokens: Optional[int] = None) -> np.ndarray:
    """Which (row, key) pairs survive the mask, for query rows ``rows`` of one sequence."""
    j = np.arange(Skv, dtype=np.int64)[None, :]
    i = rows.astype(np.int64)[:, None]
    a = np.ones((len(rows), Skv), dtype=bool)
    if sparse_mode == 2:
        a &= j <= i
    elif sparse_mode == 3:
        a &= j <= i + (Skv - Sq)
    elif sparse_mode != 0:
        raise ValueError("sparse_mode must be 0, 2 or 3")
    if pre_tokens is not None or next_tokens is not None:
        if sparse_mode != 0:
            raise ValueError("pre_tokens / next_tokens set the sparse_mode 0 range")
        if pre_tokens is not None:
            a &= j >= i - int(pre_tokens)
        if next_tokens is not None:
            a &= j <= i + int(next_tokens)
    if mask_rows is not None:
        a &= (mask_rows == 0)
    if keep is not None:
        a &= keep[rows // BLOCK][:, np.arange(Skv) // BLOCK].astype(bool)
    return a


def atten_mask_from_bits(words: np.ndarray, Skv: int) -> np.ndarray:
    """The uint8 atten_mask (1 = masked) that a bit-packed mask stands for.

    The guide advises a compressed atten_mask beside the causal sparse_modes (section 8, tuning
    advice) without giving its layout; section 4.2 fixes 1 = masked. Reading: one bit per key,
    each mask row held as ceil(Skv / 32) 32-bit words, key j in bit (j mod 32) of word
    (j div 32); bits past Skv carry nothing. ``words``: integer array [..., Sq, ceil(Skv / 32)]
    (SS, B1SS or BNSS). Returns uint8 [..., Sq, Skv].
    """
    w = np.asarray(words).astype(np.int64) & 0xFFFFFFFF
    if w.shape[-1] != (Skv + 31) // 32:
        raise ValueError(f"a bit-packed row of {Skv} keys has {(Skv + 31) // 32} words, got {w.shape[-1]}")
    j = np.arange(Skv)
    return ((w[..., j // 32] >> (j % 32)) & 1).astype(np.uint8)


def _mask_for_head(atten_mask: Optional[np.ndarray], b: int, h: int) -> Optional[np.ndarray]:
    """Select the [Sq, Skv] slice of an SS, B1SS or BNSS mask."""
    if atten_mask is None:
        return None
    if atten_mask.ndim == 2:
        return atten_mask
    if atten_mask.shape[1] == 1:
        return atten_mask[b, 0]
    return atten_mask[b, h]


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, rows: Sequence[int],
                   *, sparse_mode: int = 0, mask: Optional[np.ndarray] = None,
                   keep: Optional[np.ndarray] = None, pre_tokens: Optional[int] = None,
                   next_tokens: Optional[int] = None):
    """Attention for selected query rows of one head of one sequence.

    q [Sq, D], k [Skv, D], v [Skv, Dv]; ``mask`` [Sq, Skv] (1 = masked);
    ``keep`` [QB, KB] block keep bits. Returns (o, m, l) for those rows.
    """
    rows = np.asarray(rows, dtype=np.int64)
    Sq, Skv = q.shape[0], k.shape[0]
    a = _allowed(rows, Sq, Skv, sparse_mode, None if mask is None else mask[rows], keep, pre_tokens, next_tokens)
    return softmax_attention(q[rows], k, v, scale, a)


def _head(q, k, v, scale, sparse_mode, mask, keep, band=(None, None)):
    Sq = q.shape[0]
    o = np.zeros((Sq, v.shape[1]))
    m = np.zeros(Sq)
    l = np.zeros(Sq)
    for r0 in range(0, Sq, BLOCK):
        rows = np.arange(r0, min(Sq, r0 + BLOCK))
        o[rows], m[rows], l[rows] = attention_rows(q, k, v, scale, rows, sparse_mode=sparse_mode,
                                                   mask=mask, keep=keep, pre_tokens=band[0],
                                                   next_tokens=band[1])
    return o, m, l


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, *, layout: str = "BNSD",
              sparse_mode: int = 0, atten_mask: Optional[np.ndarray] = None,
              cu_seqlens_q: Optional[np.ndarray] = None, cu_seqlens_kv: Optional[np.ndarray] = None,
              block_keep: Optional[np.ndarray] = None, pre_tokens: Optional[int] = None,
              next_tokens: Optional[int] = None, actual_seq_q: Optional[Sequence[int]] = None,
              actual_seq_kv: Optional[Sequence[int]] = None):
    """Attention forward over a whole problem.

    BNSD: q [B, Nq, Sq, D], k/v [B, Nkv, Skv, D] -> o [B, Nq, Sq, D], m/l [B, Nq, Sq].
    TND:  q [T, Nq, D], k/v [Tk, Nkv, D] with cumulative lengths (B+1 entries,
          leading 0) -> o [T, Nq, D], m/l [Nq, T].
    ``atten_mask``: uint8, 1 = masked, [Sq, Skv] / [B, 1, Sq, Skv] / [B, Nq, Sq, Skv] (BNSD).
    ``block_keep``: uint8 [B, Nq, QB, KB], 1 = keep (BNSD).
    ``pre_tokens`` / ``next_tokens``: the sparse_mode 0 band (None = no limit).
    ``actual_seq_q`` / ``actual_seq_kv`` (BNSD): per-batch valid lengths (None = Sq / Skv).
    """
    band = (pre_tokens, next_tokens)
    if layout == "BNSD":
        B, Nq, Sq, D = q.shape
        Nkv = k.shape[1]
        if Nq % Nkv:
            raise ValueError("Nq must be a multiple of Nkv")
        g = Nq // Nkv
        Skv = k.shape[2]
        aq = [Sq] * B if actual_seq_q is None else [int(x) for x in actual_seq_q]
        akv = [Skv] * B if actual_seq_kv is None else [int(x) for x in actual_seq_kv]
        if len(aq) != B or len(akv) != B or not all(0 <= a <= Sq for a in aq) or \
                not all(0 <= a <= Skv for a in akv):
            raise ValueError("actual lengths must be B values within [0, Sq] and [0, Skv]")
        o = np.zeros(q.shape[:3] + (v.shape[3],))
        m = np.full((B, Nq, Sq), -np.inf)
        l = np.zeros((B, Nq, Sq))
        for b in range(B):
            lq, lk = aq[b], akv[b]
            for h in range(Nq):
                keep = None if block_keep is None else block_keep[b, h]
                mask = _mask_for_head(atten_mask, b, h)
                mask = None if mask is None else mask[:lq, :lk]
                o[b, h, :lq], m[b, h, :lq], l[b, h, :lq] = _head(q[b, h, :lq], k[b, h // g, :lk], v[b, h // g, :lk],
                                                                 scale, sparse_mode, mask, keep, band)
        return o, m, l
    if layout == "TND":
        if atten_mask is not None or block_keep is not None or actual_seq_q is not None or \
                actual_seq_kv is not None:
            raise ValueError("TND supports causal masks and the band only")
        T, Nq, D = q.shape
        Nkv = k.shape[1]
        if Nq % Nkv:
            raise ValueError("Nq must be a multiple of Nkv")
        g = Nq // Nkv
        o = np.zeros((T, Nq, v.shape[2]))
        m = np.zeros((Nq, T))
        l = np.zeros((Nq, T))
        for b in range(len(cu_seqlens_q) - 1):
            q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
            k0, k1 = int(cu_seqlens_kv[b]), int(cu_seqlens_kv[b + 1])
            for h in range(Nq):
                oh, mh, lh = _head(q[q0:q1, h], k[k0:k1, h // g], v[k0:k1, h // g], scale, sparse_mode,
                                   None, None, band)
                o[q0:q1, h], m[h, q0:q1], l[h, q0:q1] = oh, mh, lh
        return o, m, l
    raise ValueError("layout must be BNSD or TND")


def attention_block_sparse(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, keep: np.ndarray,
                           qblocks: Optional[Sequence[int]] = None):
    """Block-sparse attention for one head, gathering only the kept key blocks.

    q [Sq, D], k/v [Skv, D]; ``keep`` [QB, KB] (1 = keep). Keys outside kept
    blocks receive probability exactly 0 in the plain definition, so gathering
    the kept blocks' keys and running the plain softmax over them gives the
    same result with far less work. Returns (o, m, l) for the rows of the
    q-blocks in ``qblocks`` (all q-blocks by default), concatenated.
    """
    Sq, Skv = q.shape[0], k.shape[0]
    QB = (Sq + BLOCK - 1) // BLOCK
    qblocks = range(QB) if qblocks is None else qblocks
    outs, ms, ls = [], [], []
    for qb in qblocks:
        rows = np.arange(qb * BLOCK, min(Sq, (qb + 1) * BLOCK))
        kbs = np.nonzero(keep[qb])[0]
        cols = np.concatenate([np.arange(kb * BLOCK, min(Skv, (kb + 1) * BLOCK)) for kb in kbs]) \
            if len(kbs) else np.zeros(0, dtype=np.int64)
        a = np.ones((len(rows), len(cols)), dtype=bool)
        o, m, l = softmax_attention(q[rows], k[cols], v[cols], scale, a)
        outs.append(o)
        ms.append(m)
        ls.append(l)
    return np.concatenate(outs), np.concatenate(ms), np.concatenate(ls)
