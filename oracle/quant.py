"""Quantisers and the kept-block list (oracle; tests only).

Follows the EagleQBSA article ("EagleQBSA quantised block-sparse attention"):
  * scheme-design section: Q and K are quantised linearly to INT8 per block
    along the sequence (the article motivates it by the locality of video
    tokens); V is quantised to FP8 E4M3 per channel (one scale per head
    dimension), because a scale along the key axis would have to follow the
    P.V accumulation blocks;
  * the API call at the end: 128 x 128 block shape, INT8 query/key, E4M3FN
    value, separate query/key/value scale tensors, a block-sparse mask.

Readings where the article is silent (stated once here):
  * symmetric INT8 on [-127, 127]: scale = fp32(amax / 127),
    code = clip(round_half_even(fp32(x / scale)), -127, 127);
  * E4M3FN per channel: scale = fp32(amax / 448),
    code = E4M3_RNE(clip(fp32(x / scale), -448, 448)), sign kept (a negative
    value that rounds to zero encodes as 0x80);
  * both divisions are IEEE binary32 divisions, correctly rounded (NumPy
    float32 arithmetic);
  * a group whose amax is 0 gets scale 0 and all-zero codes;
  * Q/K groups are (batch, head, 128-token block); a ragged last block uses
    only the rows present. V groups are (batch, kv-head, channel) over all
    tokens;
  * the block-sparse mask is uint8 [B, Nq, QB, KB] with 1 = keep; its kept
    list holds, per (batch, q-head, q-block), the kept kv-block indices in
    ascending order followed by -1 padding, plus a count.

E4M3FN (the OCP 8-bit float torch calls ``float8_e4m3fn``): 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
m * 2^-9; there are no infinities; S.1111.111 is NaN; the largest finite
magnitude is 1.75 * 2^8 = 448.
"""

from __future__ import annotations

import numpy as np

BLOCK = 128
E4M3_MAX = 448.0
INT8_MAX = 127


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3FN bytes to float64 by the format's definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# All non-negative finite magnitudes, indexed by their code 0x00..0x7E; the
# table is increasing in the code.
_E4M3_TABLE = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round values to the nearest E4M3FN number, ties to the even code.

    The input must already lie in [-448, 448] (callers clamp first). Rounding
    works on the float64 value of ``x``: pick the nearer of the two
    representable neighbours; on a tie pick the one with an even mantissa,
    which is the one with an even code. The sign bit is kept for zeros.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3_encode expects finite values in [-448, 448]")
    a = np.abs(x)
    hi = np.searchsorted(_E4M3_TABLE, a, side="left")       # table[hi-1] < a <= table[hi]
    hi = np.clip(hi, 1, len(_E4M3_TABLE) - 1)
    lo = hi - 1
    d_lo = a - _E4M3_TABLE[lo]
    d_hi = _E4M3_TABLE[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(a == 0.0, 0, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_qk_perblock_int8(x: np.ndarray):
    """Symmetric INT8 per (batch, head, 128-token block).

    x [B, N, S, D] holding bf16 values (any float dtype). Returns
    (codes int8 [B, N, S, D], scales float32 [B, N, ceil(S/128)]).
    """
    B, N, S, D = x.shape
    nb = (S + BLOCK - 1) // BLOCK
    codes = np.zeros((B, N, S, D), dtype=np.int8)
    scales = np.zeros((B, N, nb), dtype=np.float32)
    x32 = np.asarray(x, dtype=np.float32)
    for blk in range(nb):
        xs = x32[:, :, blk * BLOCK:(blk + 1) * BLOCK, :]
        amax = np.abs(xs).max(axis=(2, 3))
        scale = amax / np.float32(INT8_MAX)                       # binary32 division
        safe = np.where(scale > 0, scale, np.float32(1.0))
        t = xs / safe[:, :, None, None]                           # binary32 division
        q = np.clip(np.rint(t), -INT8_MAX, INT8_MAX)
        q = np.where(scale[:, :, None, None] > 0, q, 0)
        codes[:, :, blk * BLOCK:(blk + 1) * BLOCK, :] = q.astype(np.int8)
        scales[:, :, blk] = scale
    return codes, scales


def quantize_v_perchannel_fp8(v: np.ndarray):
    """E4M3FN per (batch, head, channel) over all tokens.

    v [B, N, S, D] holding bf16 values. Returns (codes uint8 [B, N, S, D],
    scales float32 [B, N, D]).
    """
    v32 = np.asarray(v, dtype=np.float32)
    amax = np.abs(v32).max(axis=2)                                # [B, N, D]
    scale = amax / np.float32(E4M3_MAX)                           # binary32 division
    safe = np.where(scale > 0, scale, np.float32(1.0))
    t = v32 / safe[:, :, None, :]                                 # binary32 division
    t = np.clip(t, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = e4m3_encode(t)
    codes = np.where(scale[:, :, None, :] > 0, codes, np.uint8(0)).astype(np.uint8)
    return codes, scale.astype(np.float32)


def kept_block_list(keep: np.ndarray):
    """Compact a block keep mask [B, N, QB, KB] into (counts int32 [B, N, QB],
    idx int32 [B, N, QB, KB]) with ascending kept indices then -1 padding."""
    keep = np.asarray(keep)
    B, N, QB, KB = keep.shape
    counts = np.zeros((B, N, QB), dtype=np.int32)
    idx = np.full((B, N, QB, KB), -1, dtype=np.int32)
    for b in range(B):
        for n in range(N):
            for qb in range(QB):
                kept = [kb for kb in range(KB) if keep[b, n, qb, kb] != 0]
                counts[b, n, qb] = len(kept)
                idx[b, n, qb, :len(kept)] = kept
    return counts, idx


def qblock_order(counts: np.ndarray) -> np.ndarray:
    """Per (batch, head) row of kept counts [B, N, QB], the q-block indices sorted by kept count,
    largest first, ties in ascending q-block index: order[b, n, i] is the q-block of rank i.
    A scheduling order for the block-sparse launches (the kept lists of the EagleQBSA API call
    decide how much work each q-block has); written out as the plain sort by key
    (-count, index)."""
    counts = np.asarray(counts)
    B, N, QB = counts.shape
    order = np.zeros((B, N, QB), dtype=np.int32)
    for b in range(B):
        for n in range(N):
            order[b, n] = sorted(range(QB), key=lambda j: (-int(counts[b, n, j]), j))
    return order
