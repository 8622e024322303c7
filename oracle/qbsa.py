"""Quantised block-sparse attention, EagleQBSA style (oracle; tests only).

Follows the EagleQBSA article ("EagleQBSA quantised block-sparse attention"):
  * scheme-design section (and figure 2.1, whose image is absent): Q.K^T runs
    on per-block INT8 Q/K; P and V enter the P.V product as FP8, V with one
    scale per channel; the S1 x S2 tile of P multiplies an S2 x D tile of V;
  * operator-optimisation section: P is cast to FP8 inside the tiled loop,
    after the softmax exponent, and is non-negative;
  * the API call: 128 x 128 blocks, a block-sparse mask, a softmax scale, a
    bf16 output.

Schedule-faithful form (``qbsa_qblock``): for one (batch, head, q-block) the
kept kv-blocks are visited in ascending order with the online softmax of the
fused attention guide (section 2, tiling with an online softmax):
    s      = (qc . kc^T) * sq[qb] * sk[kb] * scale
    m'     = max(m, rowmax s)
    alpha  = exp(m - m')            (1 when m == m', so no 0 * inf)
    p      = exp(s - m')
    l      = alpha * l + rowsum p   (unquantised p)
    acc    = alpha * acc + E4M3(p) . decode(vc)
    O      = acc * v_scale[d] / l
Readings: P is cast unscaled (p lies in [0, 1]); the cast rounds to nearest
even after rounding p to binary32, the precision the exponent is taken in on
the device; l sums the unquantised p. Integer dot products are formed with a
float64 matrix product, which is exact here (|sum| <= 127^2 * D < 2^53).
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .quant import BLOCK, e4m3_decode, e4m3_encode


def _fp8_round(p: np.ndarray) -> np.ndarray:
    """p in [0, 1] -> its E4M3FN value (via binary32, round to nearest even)."""
    return e4m3_decode(e4m3_encode(np.asarray(p, dtype=np.float32)))


def qbsa_qblock(qc: np.ndarray, kc: np.ndarray, vc: np.ndarray, sq: float, sk: np.ndarray,
                v_scale: np.ndarray, scale: float, kept: Sequence[int], qb: int, *, round_p: bool = True):
    """Schedule-faithful QBSA for one (batch, head, q-block).

    qc [Sq, D] int8 codes, kc [Skv, D] int8 codes, vc [Skv, D] E4M3 bytes,
    sq scalar (this q-block's scale), sk [KB] key-block scales, v_scale [D].
    ``kept``: ascending kv-block indices. ``round_p=False`` skips the FP8 cast
    of P (used to tie this oracle to the block-sparse one).
    Returns (o [R, D], m [R], l [R]) for the rows of q-block ``qb``.
    """
    Sq, D = qc.shape
    Skv = kc.shape[0]
    rows = slice(qb * BLOCK, min(Sq, (qb + 1) * BLOCK))
    q = qc[rows].astype(np.float64)
    R = q.shape[0]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, vc.shape[1]))
    vdec = None
    for kb in kept:
        cols = slice(kb * BLOCK, min(Skv, (kb + 1) * BLOCK))
        s = (q @ kc[cols].astype(np.float64).T) * (np.float64(sq) * np.float64(sk[kb]) * scale)
        m_new = np.maximum(m, s.max(axis=1))
        alpha = np.where(m == m_new, 1.0, np.exp(m - m_new))
        p = np.exp(s - m_new[:, None])
        l = alpha * l + p.sum(axis=1)
        pq = _fp8_round(p) if round_p else p
        vdec = e4m3_decode(vc[cols])
        acc = alpha[:, None] * acc + pq @ vdec
        m = m_new
    live = l > 0
    o = np.zeros_like(acc)
    o[live] = acc[live] * np.asarray(v_scale, dtype=np.float64)[None, :] / l[live, None]
    m = np.where(live, m, -np.inf)
    return o, m, l


def qbsa_attention(qc, kc, vc, q_scale, k_scale, v_scale, keep, scale,
                   qblocks: Optional[Sequence[tuple]] = None, *, round_p: bool = True,
                   actual_seq_q: Optional[Sequence[int]] = None, actual_seq_kv: Optional[Sequence[int]] = None):
    """QBSA over BNSD inputs.

    qc [B, Nq, S, D] int8, kc/vc [B, Nkv, S, D], q_scale [B, Nq, QB],
    k_scale [B, Nkv, KB], v_scale [B, Nkv, D], keep [B, Nq, QB, KB] (1 = keep).
    ``qblocks``: optional list of (b, h, qb) to compute; default all.
    ``actual_seq_q`` / ``actual_seq_kv`` (the API call's actual_seq_lengths and
    actual_seq_lengths_kv): batch b uses only its first aq_b query rows and akv_b
    keys; kept blocks past its keys hold no key. The scales stay those of the
    padded tensors (the quantisers see the whole buffers).
    Returns a dict {(b, h, qb): (o, m, l)} with the rows of q-block qb below aq_b
    (possibly none).
    """
    B, Nq, S, D = qc.shape
    Skv = kc.shape[2]
    g = Nq // kc.shape[1]
    QB = (S + BLOCK - 1) // BLOCK
    aq = [S] * B if actual_seq_q is None else [int(x) for x in actual_seq_q]
    akv = [Skv] * B if actual_seq_kv is None else [int(x) for x in actual_seq_kv]
    if qblocks is None:
        qblocks = [(b, h, qb) for b in range(B) for h in range(Nq) for qb in range(QB)]
    out = {}
    for (b, h, qb) in qblocks:
        kept = [kb for kb in np.nonzero(keep[b, h, qb])[0] if kb * BLOCK < akv[b]]
        out[(b, h, qb)] = qbsa_qblock(qc[b, h, :aq[b]], kc[b, h // g, :akv[b]], vc[b, h // g, :akv[b]],
                                      q_scale[b, h, qb], k_scale[b, h // g], v_scale[b, h // g], scale, kept, qb,
                                      round_p=round_p)
    return out


def qbsa_plain_rows(qc, kc, vc, sq, sk, v_scale, scale, kept, qb):
    """Non-tiled variant: one softmax over all kept keys with the final max,
    then P cast to FP8 once. Agrees with the tiled form within FP8 rounding."""
    Sq, D = qc.shape
    Skv = kc.shape[0]
    rows = slice(qb * BLOCK, min(Sq, (qb + 1) * BLOCK))
    cols = np.concatenate([np.arange(kb * BLOCK, min(Skv, (kb + 1) * BLOCK)) for kb in kept])
    col_scale = np.concatenate([np.full(min(Skv, (kb + 1) * BLOCK) - kb * BLOCK, np.float64(sk[kb]))
                                for kb in kept])
    s = (qc[rows].astype(np.float64) @ kc[cols].astype(np.float64).T) * np.float64(sq) * col_scale[None, :] * scale
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = (_fp8_round(p) @ e4m3_decode(vc[cols])) * np.asarray(v_scale, np.float64)[None, :] / l[:, None]
    return o, m, l
