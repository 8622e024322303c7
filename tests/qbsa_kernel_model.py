"""Float32 model of the quantised kernel's own arithmetic (test infrastructure).

The oracle (``oracle.qbsa``) computes each p = exp(s - m) in float64 and rounds
it to binary32 and then to E4M3. The kernel forms p in binary32 from the INT8
dot product d held as the float 1.5 * 2^23 + d:

    ct = fp32(fp32(q_scale * fp32(scale * log2 e)) * k_scale)   per kept block
    mh = fp32(d_max * ct)                                        per 64-key half
    m  = running max (base 2) through the end of the kept block
    cc = fp32(1.5 * 2^23 * ct + m)                               one rounding
    x  = fp32((1.5 * 2^23 + d) * ct - cc)                        one rounding (FMA)
    p  = exp2(x) in binary32, then E4M3 (round half even)

except for the first 64 keys of a block whose second half raised the max of some row of the
32-row wave: their p was formed against m1, the max through the first half, and is scaled, for
every row of that wave, by alpha = exp2(fp32(m1 - m)) in binary32 (1 where m1 = m):

    p  = fp32(exp2(x1) * alpha),  x1 with cc1 = fp32(1.5 * 2^23 * ct + m1)

The single rounding of cc shifts every x of a row and block by up to half an
ulp of 1.5 * 2^23 * ct, about 0.75 ct, i.e. a relative change of p of order
1e-4. Where the float64 p lies that close to an E4M3 midpoint, the kernel and
the oracle round it to neighbouring codes, one E4M3 step apart (up to 1/16 of p).
This model repeats the kernel's steps, so comparing the GPU output with it
separates those rounding decisions from any departure of the schedule.
Products and sums other than these are taken in float64; the model's
exp2 is correctly rounded, the hardware's is within one ulp.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from oracle.quant import BLOCK, e4m3_decode, e4m3_encode

_MAGIC = 12582912.0  # 1.5 * 2^23
_LOG2E = 1.4426950408889634


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def qbsa_qblock_model(qc: np.ndarray, kc: np.ndarray, vc: np.ndarray, sq: float, sk: np.ndarray,
                      v_scale: np.ndarray, scale: float, kept: Sequence[int], qb: int):
    """Rows of q-block ``qb`` as the kernel forms them (arguments as ``oracle.qbsa_qblock``).
    Returns o [R, D] (float64, before the bf16 store)."""
    Sq, D = qc.shape
    Skv = kc.shape[0]
    rows = slice(qb * BLOCK, min(Sq, (qb + 1) * BLOCK))
    q = qc[rows].astype(np.int64)
    R = q.shape[0]
    c = float(np.float32(scale * _LOG2E))
    qcs = _f32(np.float32(sq) * np.float64(c))
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, vc.shape[1]))
    for kb in kept:
        k0, k1 = kb * BLOCK, min(Skv, (kb + 1) * BLOCK)
        if k0 >= k1:
            continue
        ct = max(float(_f32(qcs * np.float64(np.float32(sk[kb])))), float(np.float32(1e-30)))
        d = q @ kc[k0:k1].astype(np.int64).T                      # exact integer dot products
        m_old = m.copy()
        m1 = m
        for h0 in (0, 64):                                       # the two 64-key halves
            dh = d[:, h0:h0 + 64]
            if dh.shape[1] == 0:
                continue
            mh = _f32(dh.max(axis=1).astype(np.float64) * ct)
            m = np.maximum(m, mh)
            if h0 == 0:
                m1 = m.copy()                                    # the max the first half's p is formed against
        alpha = np.where(m == m_old, 1.0, np.exp2(_f32(m_old - m)))
        cc = _f32(_MAGIC * ct + np.where(np.isneginf(m), 0.0, m))
        x = _f32((_MAGIC + d.astype(np.float64)) * ct - cc[:, None])
        p = _f32(np.exp2(x))
        # a 32-row wave whose second half raised some row's max forms its first half's p again
        # from the p against m1 times alpha1 (1 for the rows whose max did not move)
        cc1 = _f32(_MAGIC * ct + np.where(np.isneginf(m1), 0.0, m1))
        p1 = _f32(np.exp2(_f32((_MAGIC + d[:, :64].astype(np.float64)) * ct - cc1[:, None])))
        a1 = np.where(m == m1, 1.0, _f32(np.exp2(_f32(m1 - m))))
        p1 = _f32(p1 * a1[:, None])
        for w0 in range(0, R, 32):
            rows_w = slice(w0, min(R, w0 + 32))
            if np.any(m[rows_w] > m1[rows_w]):
                p[rows_w, :64] = p1[rows_w]
        pq = e4m3_decode(e4m3_encode(p.astype(np.float32)))
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + pq @ e4m3_decode(vc[k0:k1])
    o = np.zeros_like(acc)
    live = l > 0
    o[live] = acc[live] * np.asarray(v_scale, np.float64)[None, :] / l[live, None]
    return o
