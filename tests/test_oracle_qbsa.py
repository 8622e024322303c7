"""Pins for the quantised block-sparse oracle (CPU only).

* With the FP8 cast of P switched off, the tiled QBSA oracle equals the plain
  block-sparse float64 oracle run on the dequantised Q, K, V: this checks the
  online-softmax recurrence, the per-block scale indexing and v_scale.
* The tiled form and the non-tiled form (one softmax, P cast once) agree
  within the quantised tolerance.
* The FP8 cast of P equals torch's float8_e4m3fn cast on [0, 1].
* Brute force on a tiny case with scalar loops.
"""

import math

import numpy as np
import torch

from oracle import (attention_block_sparse, e4m3_decode, kept_block_list, qbsa_attention, qbsa_plain_rows,
                    qbsa_qblock, quantize_qk_perblock_int8, quantize_v_perchannel_fp8)
from oracle.qbsa import _fp8_round

RNG = np.random.default_rng(23)


def _problem(S=384, D=16, N=2, p=0.5, chan=True):
    q = RNG.normal(size=(1, N, S, D)) + np.repeat(RNG.normal(size=(1, N, S // 128, D)) * 0.5, 128, axis=2)
    k = RNG.normal(size=(1, N, S, D)) + np.repeat(RNG.normal(size=(1, N, S // 128, D)) * 0.5, 128, axis=2)
    v = RNG.normal(size=(1, N, S, D))
    if chan:
        v = v * np.exp(RNG.normal(size=(1, N, 1, D)))
    q, k, v = (x.astype(np.float32) for x in (q, k, v))
    QB = S // 128
    keep = (RNG.random((1, N, QB, QB)) < p).astype(np.uint8)
    for i in range(QB):
        keep[0, :, i, i] = 1
    return q, k, v, keep


def test_unrounded_qbsa_equals_block_sparse_on_dequantised_inputs():
    q, k, v, keep = _problem()
    qc, qs = quantize_qk_perblock_int8(q)
    kc, ks = quantize_qk_perblock_int8(k)
    vc, vs = quantize_v_perchannel_fp8(v)
    scale = 0.25
    qh = qc.astype(np.float64) * np.repeat(qs, 128, axis=2)[..., None]
    kh = kc.astype(np.float64) * np.repeat(ks, 128, axis=2)[..., None]
    vh = e4m3_decode(vc) * vs[:, :, None, :]
    res = qbsa_attention(qc, kc, vc, qs, ks, vs, keep, scale, round_p=False)
    for h in range(q.shape[1]):
        o_ref, m_ref, l_ref = attention_block_sparse(qh[0, h], kh[0, h], vh[0, h], scale, keep[0, h])
        for qb in range(keep.shape[2]):
            o, m, l = res[(0, h, qb)]
            rows = slice(qb * 128, (qb + 1) * 128)
            np.testing.assert_allclose(o, o_ref[rows], atol=1e-11, rtol=1e-11)
            np.testing.assert_allclose(m, m_ref[rows], atol=1e-11)
            np.testing.assert_allclose(l, l_ref[rows], rtol=1e-11)


def test_tiled_and_plain_within_fp8_rounding_bound():
    """Rounding p to E4M3 moves it by at most max(2^-4 p, 2^-10) (half an ulp:
    3 mantissa bits in the normal range, 2^-9 steps below 2^-6). The tiled
    form rounds p relative to a running max m_t <= m_final, which scales that
    error by exp(m_t - m_final) <= 1, so both forms stay within
    sum_j max(2^-4 p_j, 2^-10) |v_j| / l of the unrounded result."""
    q, k, v, keep = _problem(S=512, D=32, N=1, p=0.6)
    qc, qs = quantize_qk_perblock_int8(q)
    kc, ks = quantize_qk_perblock_int8(k)
    vc, vs = quantize_v_perchannel_fp8(v)
    vhat = e4m3_decode(vc[0, 0]) * vs[0, 0][None, :]
    for qb in range(4):
        kept = np.nonzero(keep[0, 0, qb])[0]
        args = (qc[0, 0], kc[0, 0], vc[0, 0], qs[0, 0, qb], ks[0, 0], vs[0, 0], 0.2, kept, qb)
        o1, m1, l1 = qbsa_qblock(*args)
        o2, m2, l2 = qbsa_plain_rows(*args)
        o0, m0, l0 = qbsa_qblock(*args, round_p=False)
        np.testing.assert_allclose(m1, m2, atol=1e-12)
        np.testing.assert_allclose(l1, l2, rtol=1e-12)
        cols = np.concatenate([np.arange(kb * 128, kb * 128 + 128) for kb in kept])
        s = (qc[0, 0, qb * 128:(qb + 1) * 128].astype(np.float64) @ kc[0, 0, cols].astype(np.float64).T) \
            * qs[0, 0, qb] * np.repeat(ks[0, 0, kept], 128)[None, :] * 0.2
        p = np.exp(s - m0[:, None])
        bound = (np.maximum(2.0 ** -4 * p, 2.0 ** -10) @ np.abs(vhat[cols])) / l0[:, None] * (1 + 1e-9)
        assert np.all(np.abs(o1 - o0) <= bound) and np.all(np.abs(o2 - o0) <= bound)
        assert np.abs(o1 - o2).max() > 0          # the two schedules do round differently


def test_fp8_p_cast_matches_torch():
    p = np.concatenate([RNG.random(50000), RNG.random(20000) * 2 ** -8, [0.0, 1.0]])
    ref = torch.from_numpy(p.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(_fp8_round(p), ref)


def test_brute_force_tiny_qbsa():
    """Scalar loops over one q-block with two kept kv-blocks of a short, ragged problem."""
    D, Sq, Skv = 3, 5, 200
    qc = RNG.integers(-127, 128, size=(Sq, D)).astype(np.int8)
    kc = RNG.integers(-127, 128, size=(Skv, D)).astype(np.int8)
    vc = RNG.integers(0, 0x7E, size=(Skv, D)).astype(np.uint8) | (RNG.integers(0, 2, size=(Skv, D)) * 0x80).astype(np.uint8)
    sq, sk, vs = 0.013, np.array([0.02, 0.011]), np.array([0.5, 2.0, 0.1])
    kept = [0, 1]
    o, m, l = qbsa_qblock(qc, kc, vc, sq, sk, vs, 0.7, kept, 0)
    vdec = e4m3_decode(vc)
    for i in range(Sq):
        mm, ll, acc = -math.inf, 0.0, [0.0] * D
        for kb in kept:
            cols = range(kb * 128, min(Skv, kb * 128 + 128))
            s = {j: sum(int(qc[i, d]) * int(kc[j, d]) for d in range(D)) * sq * sk[kb] * 0.7 for j in cols}
            mn = max(mm, max(s.values()))
            a = 1.0 if mn == mm else math.exp(mm - mn)
            ps = {j: math.exp(x - mn) for j, x in s.items()}
            ll = a * ll + sum(ps.values())
            pr = {j: float(torch.tensor(float(np.float32(x))).to(torch.float8_e4m3fn).float()) for j, x in ps.items()}
            acc = [a * acc[d] + sum(pr[j] * vdec[j, d] for j in cols) for d in range(D)]
            mm = mn
        np.testing.assert_allclose(o[i], [acc[d] * vs[d] / ll for d in range(D)], rtol=1e-12, atol=1e-14)
        assert abs(m[i] - mm) <= 1e-12 * max(1, abs(mm)) and abs(l[i] - ll) <= 1e-12 * ll


def test_qbsa_uses_kept_list_order():
    q, k, v, keep = _problem(S=256, D=8, N=1, p=1.0)
    counts, idx = kept_block_list(keep)
    assert counts[0, 0, 0] == 2 and list(idx[0, 0, 0]) == [0, 1]


def test_actual_lengths_skip_padded_keys_and_rows():
    """QBSA with actual lengths: padded key codes that would dominate the softmax get no weight
    (the result equals the same codes cut to the valid keys), padded q-blocks are empty, and a
    kept block wholly past the valid keys contributes nothing."""
    q, k, v, keep = _problem(S=384, D=8, N=2, p=1.0)
    qc, qs = quantize_qk_perblock_int8(q)
    kc, ks = quantize_qk_perblock_int8(k)
    vc, vs = quantize_v_perchannel_fp8(v)
    akv, aq = 200, 250
    kc = kc.copy()
    kc[:, :, akv:] = 127 * np.sign(qc[:, :, :1]).astype(np.int8)  # aligned with query row 0
    out = qbsa_attention(qc, kc, vc, qs, ks, vs, keep, 0.3, actual_seq_q=[aq], actual_seq_kv=[akv])
    for h in range(2):
        for qb in range(3):
            o, m, l = out[(0, h, qb)]
            rows = max(0, min(aq, 128 * qb + 128) - 128 * qb)
            assert o.shape[0] == rows
            if rows == 0:
                continue
            ro, rm, rl = qbsa_qblock(qc[0, h, :aq], kc[0, h, :akv], vc[0, h, :akv], qs[0, h, qb], ks[0, h], vs[0, h],
                                     0.3, [0, 1], qb)
            np.testing.assert_array_equal(o, ro)
            np.testing.assert_array_equal(l, rl)
            # and against the plain (non-tiled) form on the valid keys only
            po, pm, pl = qbsa_plain_rows(qc[0, h, :aq], kc[0, h, :akv], vc[0, h, :akv], qs[0, h, qb], ks[0, h],
                                         vs[0, h], 0.3, [0, 1], qb)
            np.testing.assert_allclose(l, pl, rtol=1e-12)
            np.testing.assert_allclose(m, pm, rtol=1e-12)


def test_kernel_model_within_the_fp8_tolerance():
    """The float32 model of the quantised kernel's steps (a GPU-test helper) agrees with the
    oracle to the quantised tolerance; only E4M3 rounding decisions near midpoints differ."""
    import os
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    import oracle
    from qbsa_kernel_model import qbsa_qblock_model
    rng = np.random.default_rng(5)
    S, D = 384, 64
    q = rng.standard_normal((S, D)) + rng.normal(0, 0.5, (3, 1, D)).repeat(128, 0)[:S, 0]
    k = rng.standard_normal((S, D))
    v = rng.standard_normal((1, 1, S, D))
    qc, qs = oracle.quantize_qk_perblock_int8(q[None, None])
    kc, ks = oracle.quantize_qk_perblock_int8(k[None, None])
    vc, vs = oracle.quantize_v_perchannel_fp8(v)
    for qb, kept in [(0, [0, 2]), (1, [0, 1, 2]), (2, [2])]:
        o_ref, _, _ = oracle.qbsa_qblock(qc[0, 0], kc[0, 0], vc[0, 0], qs[0, 0, qb], ks[0, 0], vs[0, 0], 0.125,
                                         kept, qb)
        o_mod = qbsa_qblock_model(qc[0, 0], kc[0, 0], vc[0, 0], qs[0, 0, qb], ks[0, 0], vs[0, 0], 0.125, kept, qb)
        assert np.abs(o_mod - o_ref).max() <= 3e-2
