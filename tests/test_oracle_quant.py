"""Pins for the oracle's quantisers and kept-block list (CPU only).

The binary32 divisions and roundings are re-derived with exact rational
arithmetic (``fractions.Fraction``) on samples; the E4M3 codec is pinned to
the OCP definition points in tests/golden, exhaustively to its own
round-trip and tie rules, and to torch's float8_e4m3fn cast.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode, kept_block_list, quantize_qk_perblock_int8, quantize_v_perchannel_fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(11)


def _nearest_f32(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest binary32, ties to even mantissa."""
    approx = np.float32(float(fr))
    cands = {approx, np.nextafter(approx, np.float32(np.inf)), np.nextafter(approx, np.float32(-np.inf))}
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - fr)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def _e4m3_exact(fr: Fraction) -> int:
    """Nearest E4M3FN code to an exact rational in [-448, 448], ties to the even code."""
    neg = fr < 0 or (fr == 0 and False)
    a = abs(fr)
    best = None
    for c in range(0x7F):
        val = Fraction(float(e4m3_decode(np.uint8(c))))
        key = (abs(val - a), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1] | (0x80 if neg else 0)


def test_e4m3_decode_matches_spec_points():
    for line in open(os.path.join(GOLDEN, "e4m3fn_points.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = float(e4m3_decode(np.uint8(int(code, 16))))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), (code, got, val)


def test_e4m3_exhaustive_roundtrip_and_ties():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = e4m3_decode(codes)
    np.testing.assert_array_equal(e4m3_encode(vals), codes)
    pos = np.sort(e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2
    enc = e4m3_encode(mids)
    lo, hi = np.arange(0x7E), np.arange(1, 0x7F)
    np.testing.assert_array_equal(enc, np.where(lo % 2 == 0, lo, hi).astype(np.uint8))
    eps = np.abs(mids) * 1e-9
    np.testing.assert_array_equal(e4m3_encode(mids - eps), lo.astype(np.uint8))
    np.testing.assert_array_equal(e4m3_encode(mids + eps), hi.astype(np.uint8))
    # negative values that round to zero keep the sign
    assert e4m3_encode(np.array([-1e-6]))[0] == 0x80 and e4m3_encode(np.array([1e-6]))[0] == 0x00


def test_e4m3_encode_matches_torch_cast():
    x = np.concatenate([RNG.normal(size=20000) * 50, RNG.random(20000), RNG.random(5000) * 2 ** -7,
                        np.array([448.0, -448.0, 0.0])])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_encode(x), ref)


def test_int8_perblock_exact_rational():
    B, N, S, D = 1, 2, 300, 16            # ragged last block (44 rows)
    x = (RNG.normal(size=(B, N, S, D)) * np.exp(RNG.normal(size=(B, N, S, 1)))).astype(np.float32)
    codes, scales = quantize_qk_perblock_int8(x)
    assert codes.dtype == np.int8 and scales.shape == (B, N, 3)
    for n in range(N):
        for blk in range(3):
            xs = x[0, n, blk * 128:(blk + 1) * 128]
            amax = max(abs(Fraction(float(e))) for e in xs.ravel())
            sc = _nearest_f32(amax / 127)
            assert scales[0, n, blk] == sc
            for (r, d) in [(0, 0), (5, 3), (len(xs) - 1, D - 1)] + [tuple(RNG.integers(0, [len(xs), D])) for _ in range(20)]:
                t = _nearest_f32(Fraction(float(xs[r, d])) / Fraction(float(sc)))
                want = max(-127, min(127, round(Fraction(float(t)))))     # round() on Fraction: half to even
                assert codes[0, n, blk * 128 + r, d] == want
            amax_pos = np.unravel_index(np.argmax(np.abs(xs)), xs.shape)
            assert abs(int(codes[0, n, blk * 128 + amax_pos[0], amax_pos[1]])) == 127


def test_int8_properties_and_zero_block():
    x = RNG.normal(size=(2, 1, 256, 8)).astype(np.float32)
    x[1, 0, :128] = 0.0
    codes, scales = quantize_qk_perblock_int8(x)
    assert scales[1, 0, 0] == 0 and np.all(codes[1, 0, :128] == 0)
    deq = codes.astype(np.float64) * np.repeat(scales, 128, axis=2)[..., None]
    err = np.abs(deq - x)
    bound = np.repeat(scales, 128, axis=2)[..., None] * 0.5 * (1 + 1e-6)
    assert np.all(err <= bound)
    # half-way values go to the even integer
    y = np.zeros((1, 1, 128, 2), np.float32)
    y[0, 0, 0, 0] = 127.0
    y[0, 0, 1, 0] = 2.5
    y[0, 0, 2, 0] = -3.5
    y[0, 0, 3, 0] = 0.5
    c, s = quantize_qk_perblock_int8(y)
    assert s[0, 0, 0] == 1.0 and list(c[0, 0, :4, 0]) == [127, 2, -4, 0]


def test_v_perchannel_exact_rational():
    B, N, S, D = 1, 2, 200, 8
    v = (RNG.normal(size=(B, N, S, D)) * np.exp(RNG.normal(size=(1, N, 1, D)))).astype(np.float32)
    v[0, 1, :, 3] = 0.0                                   # all-zero channel
    codes, scales = quantize_v_perchannel_fp8(v)
    assert scales.shape == (B, N, D) and scales[0, 1, 3] == 0 and np.all(codes[0, 1, :, 3] == 0)
    for n in range(N):
        for d in range(D):
            col = v[0, n, :, d]
            amax = max(abs(Fraction(float(e))) for e in col)
            sc = _nearest_f32(amax / 448)
            assert scales[0, n, d] == sc
            if sc == 0:
                continue
            for s in list(RNG.integers(0, S, size=12)) + [int(np.argmax(np.abs(col)))]:
                t = _nearest_f32(Fraction(float(col[s])) / Fraction(float(sc)))
                t = min(Fraction(448), max(Fraction(-448), Fraction(float(t))))
                want = _e4m3_exact(t)
                if t == 0 and np.signbit(col[s]):
                    want = 0x80
                elif t < 0:
                    want |= 0x80
                assert codes[0, n, s, d] == want, (n, d, s)
            assert e4m3_decode(codes[0, n, int(np.argmax(np.abs(col))), d]) in (448.0, -448.0)


def test_kept_list_small_known_case():
    keep = np.array([[[[1, 0, 1, 1], [0, 0, 0, 0], [0, 1, 0, 0]]]], dtype=np.uint8)
    counts, idx = kept_block_list(keep)
    np.testing.assert_array_equal(counts, [[[3, 0, 1]]])
    np.testing.assert_array_equal(idx, [[[[0, 2, 3, -1], [-1, -1, -1, -1], [1, -1, -1, -1]]]])


def test_kept_list_properties():
    keep = (RNG.random((2, 3, 9, 17)) < 0.3).astype(np.uint8)
    counts, idx = kept_block_list(keep)
    np.testing.assert_array_equal(counts, keep.sum(axis=-1))
    for b, n, qb in np.ndindex(2, 3, 9):
        c = counts[b, n, qb]
        row = idx[b, n, qb]
        assert np.all(np.diff(row[:c]) > 0) and np.all(row[c:] == -1)
        assert np.all(keep[b, n, qb, row[:c]] == 1)


def test_qblock_order_hand_worked():
    """Counts 3, 7, 3, 0, 7 -> q-blocks 1, 4 (count 7, in index order), 0, 2 (count 3), 3."""
    from oracle import qblock_order
    o = qblock_order(np.array([[[3, 7, 3, 0, 7]]]))
    assert o.tolist() == [[[1, 4, 0, 2, 3]]]


def test_qblock_order_properties_and_stable_argsort():
    """A permutation per row, counts non-increasing along it, ties in ascending index; equal to
    numpy's stable argsort of the negated counts (an independent library routine)."""
    from oracle import qblock_order
    rng = np.random.default_rng(12)
    c = rng.integers(0, 6, size=(2, 3, 40))
    o = qblock_order(c)
    for b in range(2):
        for n in range(3):
            row = o[b, n]
            assert sorted(row.tolist()) == list(range(40))
            cs = c[b, n][row]
            assert np.all(cs[:-1] >= cs[1:])
            ties = cs[:-1] == cs[1:]
            assert np.all(row[:-1][ties] < row[1:][ties])
            np.testing.assert_array_equal(row, np.argsort(-c[b, n], kind="stable"))
