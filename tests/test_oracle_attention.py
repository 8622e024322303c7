"""Pins for the float64 attention oracle (CPU only).

Each test ties the oracle to something other than itself: scalar brute force,
closed forms, invariants of the softmax, special cases that must coincide, and
torch's CPU scaled_dot_product_attention as an independent library routine.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, attention_block_sparse, attention_rows, softmax_attention

RNG = np.random.default_rng(7)


def _brute(q, k, v, scale, keep_fn):
    """Scalar loops straight from the definition; keep_fn(i, j) -> bool."""
    Sq, D = q.shape
    Skv = k.shape[0]
    o = np.zeros((Sq, v.shape[1]))
    m = np.full(Sq, -math.inf)
    l = np.zeros(Sq)
    for i in range(Sq):
        sc = {}
        for j in range(Skv):
            if keep_fn(i, j):
                sc[j] = sum(float(q[i, d]) * float(k[j, d]) for d in range(D)) * scale
        if not sc:
            continue
        mx = max(sc.values())
        w = {j: math.exp(s - mx) for j, s in sc.items()}
        tot = sum(w.values())
        m[i], l[i] = mx, tot
        for c in range(v.shape[1]):
            o[i, c] = sum(w[j] * float(v[j, c]) for j in w) / tot
    return o, m, l


@pytest.mark.parametrize("Sq,Skv,D", [(1, 1, 1), (3, 5, 2), (5, 3, 4), (8, 8, 3), (7, 2, 4)])
@pytest.mark.parametrize("mode", [0, 2, 3])
def test_brute_force_causal_modes(Sq, Skv, D, mode):
    q, k, v = RNG.normal(size=(Sq, D)), RNG.normal(size=(Skv, D)), RNG.normal(size=(Skv, D))
    scale = 0.37
    if mode == 0:
        keep_fn = lambda i, j: True  # noqa: E731
    elif mode == 2:
        keep_fn = lambda i, j: j <= i  # noqa: E731  top-left anchored lower triangle
    else:
        keep_fn = lambda i, j: j - i <= Skv - Sq  # noqa: E731  bottom-right anchored lower triangle
    ob, mb, lb = _brute(q, k, v, scale, keep_fn)
    o, m, l = attention(q[None, None], k[None, None], v[None, None], scale, sparse_mode=mode)
    np.testing.assert_allclose(o[0, 0], ob, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(m[0, 0]), np.isinf(mb))
    fin = np.isfinite(mb)
    np.testing.assert_allclose(m[0, 0][fin], mb[fin], atol=1e-12)
    np.testing.assert_allclose(l[0, 0], lb, rtol=1e-12)


@pytest.mark.parametrize("kind", ["SS", "B1SS", "BNSS"])
def test_brute_force_boolean_mask(kind):
    B, N, Sq, Skv, D = 2, 3, 6, 7, 3
    q = RNG.normal(size=(B, N, Sq, D))
    k = RNG.normal(size=(B, N, Skv, D))
    v = RNG.normal(size=(B, N, Skv, D))
    shape = {"SS": (Sq, Skv), "B1SS": (B, 1, Sq, Skv), "BNSS": (B, N, Sq, Skv)}[kind]
    mask = (RNG.random(shape) < 0.4).astype(np.uint8)
    mask[..., 2, :] = 1                      # one row fully masked
    o, m, l = attention(q, k, v, 0.5, atten_mask=mask)
    for b in range(B):
        for h in range(N):
            mk = mask if kind == "SS" else (mask[b, 0] if kind == "B1SS" else mask[b, h])
            ob, mb, lb = _brute(q[b, h], k[b, h], v[b, h], 0.5, lambda i, j: mk[i, j] == 0)
            np.testing.assert_allclose(o[b, h], ob, atol=1e-12)
            np.testing.assert_allclose(l[b, h], lb, rtol=1e-12)
            assert np.isneginf(m[b, h, 2]) and l[b, h, 2] == 0 and np.all(o[b, h, 2] == 0)


def test_brute_force_block_keep():
    Sq, Skv, D = 300, 260, 2                 # ragged blocks on both axes
    q, k, v = RNG.normal(size=(Sq, D)), RNG.normal(size=(Skv, D)), RNG.normal(size=(Skv, 2))
    keep = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 0]], dtype=np.uint8)
    rows = [0, 127, 128, 255, 256, 299]
    ob, mb, lb = _brute(q[rows], k, v, 0.3, lambda i, j: keep[rows[i] // 128, j // 128] == 1)
    o, m, l = attention_rows(q, k, v, 0.3, rows, keep=keep)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(m, mb, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=1e-12)
    og, mg, lg = attention_block_sparse(q, k, v, 0.3, keep)
    of, mf, lf = attention(q[None, None], k[None, None], v[None, None], 0.3, block_keep=keep[None, None])
    np.testing.assert_allclose(og, of[0, 0], atol=1e-13)
    np.testing.assert_allclose(mg, mf[0, 0], atol=1e-13)
    np.testing.assert_allclose(lg, lf[0, 0], rtol=1e-13)


def test_probability_rows_sum_to_one_and_constant_v():
    Sq, Skv, D = 40, 300, 8
    q, k = RNG.normal(size=(Sq, D)) * 2, RNG.normal(size=(Skv, D)) * 2
    v = np.ones((Skv, 3))
    v[:, 1] = -2.5
    v[:, 2] = 7.0
    for mode in (0, 2, 3):
        o, m, l = attention(q[None, None], k[None, None], v[None, None], 0.4, sparse_mode=mode)
        live = np.isfinite(m[0, 0])
        np.testing.assert_allclose(o[0, 0][live], np.broadcast_to([1.0, -2.5, 7.0], (live.sum(), 3)),
                                   rtol=1e-13)


def test_single_key():
    q, k, v = RNG.normal(size=(9, 5)), RNG.normal(size=(1, 5)), RNG.normal(size=(1, 4))
    o, m, l = attention(q[None, None], k[None, None], v[None, None], 0.25)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0], (9, 4)), rtol=1e-14)
    np.testing.assert_allclose(m[0, 0], 0.25 * (q @ k[0]), rtol=1e-14)
    np.testing.assert_array_equal(l[0, 0], np.ones(9))


def test_shift_and_permutation_invariance():
    Sq, Skv, D = 16, 50, 6
    q, k, v = RNG.normal(size=(Sq, D)), RNG.normal(size=(Skv, D)), RNG.normal(size=(Skv, D))
    u = RNG.normal(size=D)
    o1, m1, l1 = attention(q[None, None], k[None, None], v[None, None], 0.3)
    o2, m2, l2 = attention(q[None, None], (k + u)[None, None], v[None, None], 0.3)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-12)
    np.testing.assert_allclose(m2[0, 0], m1[0, 0] + 0.3 * (q @ u), atol=1e-12)
    perm = RNG.permutation(Skv)
    o3, m3, l3 = attention(q[None, None], k[perm][None, None], v[perm][None, None], 0.3)
    np.testing.assert_allclose(o3, o1, atol=1e-12)
    np.testing.assert_allclose(m3, m1, atol=0)
    np.testing.assert_allclose(l3, l1, rtol=1e-12)


@pytest.mark.parametrize("Sq,Skv", [(200, 200), (130, 300), (300, 130)])
def test_zero_query_counts_unmasked_keys(Sq, Skv):
    """Q = 0 makes every allowed score 0: m = 0, l = number of allowed keys
    exactly, O = mean of the allowed V rows. This pins the mask geometry."""
    D = 4
    q = np.zeros((Sq, D))
    k, v = RNG.normal(size=(Skv, D)), RNG.normal(size=(Skv, 3))
    i = np.arange(Sq)
    for mode, count in ((2, np.minimum(i + 1, Skv)), (3, np.clip(i + 1 + Skv - Sq, 0, Skv))):
        o, m, l = attention(q[None, None], k[None, None], v[None, None], 1.0, sparse_mode=mode)
        np.testing.assert_array_equal(l[0, 0], count.astype(float))
        np.testing.assert_array_equal(m[0, 0], np.where(count > 0, 0.0, -np.inf))
        for r in (0, Sq // 2, Sq - 1):
            c = int(count[r])
            exp = v[:c].mean(axis=0) if c else np.zeros(3)
            np.testing.assert_allclose(o[0, 0, r], exp, atol=1e-13)
    # boolean mask: l = number of zeros per row
    mask = (RNG.random((Sq, Skv)) < 0.7).astype(np.uint8)
    o, m, l = attention(q[None, None], k[None, None], v[None, None], 1.0, atten_mask=mask)
    np.testing.assert_array_equal(l[0, 0], (mask == 0).sum(axis=1).astype(float))
    # block keep: l = kept key count
    QB, KB = (Sq + 127) // 128, (Skv + 127) // 128
    keep = (RNG.random((QB, KB)) < 0.5).astype(np.uint8)
    keep[0, 0] = 1
    o, m, l = attention(q[None, None], k[None, None], v[None, None], 1.0, block_keep=keep[None, None])
    blk_len = np.array([min(Skv, (kb + 1) * 128) - kb * 128 for kb in range(KB)])
    np.testing.assert_array_equal(l[0, 0], (keep[i // 128] * blk_len[None, :]).sum(axis=1).astype(float))


def test_special_cases_coincide():
    Sq = Skv = 140
    D = 8
    q, k, v = RNG.normal(size=(Sq, D)), RNG.normal(size=(Skv, D)), RNG.normal(size=(Skv, D))
    dense = attention(q[None, None], k[None, None], v[None, None], 0.5)
    allkept = attention(q[None, None], k[None, None], v[None, None], 0.5,
                        block_keep=np.ones((1, 1, 2, 2), np.uint8))
    for a, b in zip(dense, allkept):
        np.testing.assert_array_equal(a, b)
    causal = attention(q[None, None], k[None, None], v[None, None], 0.5, sparse_mode=2)
    np.testing.assert_allclose(causal[0][0, 0, 0], v[0], rtol=1e-14)   # row 0 sees key 0 only
    upper = np.triu(np.ones((Sq, Skv), np.uint8), k=1)                   # 1 = masked above diagonal
    viamask = attention(q[None, None], k[None, None], v[None, None], 0.5, atten_mask=upper)
    for a, b in zip(causal, viamask):
        np.testing.assert_array_equal(a, b)


def test_gqa_equals_mha_with_repeated_kv():
    B, Nq, Nkv, S, D = 2, 6, 2, 33, 4
    q = RNG.normal(size=(B, Nq, S, D))
    k, v = RNG.normal(size=(B, Nkv, S, D)), RNG.normal(size=(B, Nkv, S, D))
    og, mg, lg = attention(q, k, v, 0.5, sparse_mode=2)
    kr = torch.from_numpy(k).repeat_interleave(Nq // Nkv, dim=1).numpy()
    vr = torch.from_numpy(v).repeat_interleave(Nq // Nkv, dim=1).numpy()
    om, mm, lm = attention(q, kr, vr, 0.5, sparse_mode=2)
    np.testing.assert_array_equal(og, om)
    np.testing.assert_array_equal(mg, mm)
    np.testing.assert_array_equal(lg, lm)


def test_tnd_equals_per_sequence_bnsd():
    lens = [5, 130, 1, 64]
    Nq, Nkv, D = 4, 2, 4
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v = RNG.normal(size=(T, Nq, D)), RNG.normal(size=(T, Nkv, D)), RNG.normal(size=(T, Nkv, D))
    for mode in (0, 2, 3):
        o, m, l = attention(q, k, v, 0.7, layout="TND", sparse_mode=mode, cu_seqlens_q=cu, cu_seqlens_kv=cu)
        for b, L in enumerate(lens):
            s0 = cu[b]
            ob, mb, lb = attention(q[s0:s0 + L].transpose(1, 0, 2)[None], k[s0:s0 + L].transpose(1, 0, 2)[None],
                                   v[s0:s0 + L].transpose(1, 0, 2)[None], 0.7, sparse_mode=mode)
            np.testing.assert_array_equal(o[s0:s0 + L], ob[0].transpose(1, 0, 2))
            np.testing.assert_array_equal(m[:, s0:s0 + L], mb[0])
            np.testing.assert_array_equal(l[:, s0:s0 + L], lb[0])


def test_tnd_unequal_q_kv_lengths():
    lq, lk = [3, 200], [10, 150]
    cuq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cuk = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = np.zeros((sum(lq), 2, 4))
    k, v = RNG.normal(size=(sum(lk), 1, 4)), RNG.normal(size=(sum(lk), 1, 4))
    o, m, l = attention(q, k, v, 1.0, layout="TND", sparse_mode=3, cu_seqlens_q=cuq, cu_seqlens_kv=cuk)
    # bottom-right: row i of a sequence sees i + 1 + Lk - Lq keys
    for b in range(2):
        i = np.arange(lq[b])
        exp = np.clip(i + 1 + lk[b] - lq[b], 0, lk[b]).astype(float)
        np.testing.assert_array_equal(l[0, cuq[b]:cuq[b + 1]], exp)


@pytest.mark.parametrize("mode", [0, 2, "mask"])
def test_matches_torch_sdpa(mode):
    B, N, Sq, Skv, D = 1, 2, 70, 70, 16
    q = RNG.normal(size=(B, N, Sq, D))
    k, v = RNG.normal(size=(B, N, Skv, D)), RNG.normal(size=(B, N, Skv, D))
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    if mode == "mask":
        mask = (RNG.random((Sq, Skv)) < 0.3).astype(np.uint8)
        mask[:, 0] = 0
        o, _, _ = attention(q, k, v, 0.25, atten_mask=mask)
        # torch's boolean attn_mask marks positions to KEEP: the opposite polarity
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask == 0),
                                                               scale=0.25)
    else:
        o, _, _ = attention(q, k, v, 0.25, sparse_mode=mode)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=(mode == 2), scale=0.25)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)


def test_softmax_attention_empty_key_set():
    o, m, l = softmax_attention(np.ones((3, 2)), np.zeros((0, 2)), np.zeros((0, 2)), 1.0, np.zeros((3, 0), bool))
    assert np.all(o == 0) and np.all(np.isneginf(m)) and np.all(l == 0)


# ---- the sparse_mode 0 range: pre_tokens / next_tokens (fused attention guide, section 4.3) ----

@pytest.mark.parametrize("Sq,Skv", [(6, 6), (5, 9), (9, 4)])
@pytest.mark.parametrize("pre,nxt", [(0, 0), (2, 1), (1, 3), (-1, 2), (3, -2), (2147483647, 0), (0, 2147483647),
                                     (2147483647, 2147483647), (-3, 1)])
def test_brute_force_band(Sq, Skv, pre, nxt):
    D = 3
    q, k, v = RNG.normal(size=(Sq, D)), RNG.normal(size=(Skv, D)), RNG.normal(size=(Skv, D))
    ob, mb, lb = _brute(q, k, v, 0.6, lambda i, j: i - pre <= j <= i + nxt)
    o, m, l = attention(q[None, None], k[None, None], v[None, None], 0.6, pre_tokens=pre, next_tokens=nxt)
    np.testing.assert_allclose(o[0, 0], ob, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(m[0, 0]), np.isinf(mb))
    fin = np.isfinite(mb)
    np.testing.assert_allclose(m[0, 0][fin], mb[fin], atol=1e-12)
    np.testing.assert_allclose(l[0, 0], lb, rtol=1e-12)


@pytest.mark.parametrize("pre,nxt", [(100, 0), (0, 100), (37, 250), (300, -40), (-20, 90)])
def test_zero_query_counts_band_keys(pre, nxt):
    """Q = 0: every kept key has score 0, so l is the size of the row's range, which is
    max(0, min(Skv - 1, i + next) - max(0, i - pre) + 1)."""
    Sq, Skv, D = 260, 330, 4
    q = np.zeros((Sq, D))
    k, v = RNG.normal(size=(Skv, D)), RNG.normal(size=(Skv, 2))
    o, m, l = attention(q[None, None], k[None, None], v[None, None], 1.0, pre_tokens=pre, next_tokens=nxt)
    for i in range(Sq):
        n = max(0, min(Skv - 1, i + nxt) - max(0, i - pre) + 1)
        assert l[0, 0, i] == n
        assert (m[0, 0, i] == 0.0) if n else np.isneginf(m[0, 0, i])


def test_band_with_defaults_equals_unmasked_and_rejects_causal():
    q, k, v = RNG.normal(size=(1, 1, 20, 3)), RNG.normal(size=(1, 1, 30, 3)), RNG.normal(size=(1, 1, 30, 3))
    a = attention(q, k, v, 0.5)
    b = attention(q, k, v, 0.5, pre_tokens=2147483647, next_tokens=2147483647)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    with pytest.raises(ValueError):
        attention(q, k, v, 0.5, sparse_mode=2, pre_tokens=4)


def test_actual_lengths_brute_force_with_padding():
    """Per-batch actual lengths (EagleQBSA API call): padded keys get no weight even when they
    would score highest, and padded rows come out empty; scalar brute force on the valid part."""
    B, Nq, Sq, Skv, D = 3, 2, 9, 11, 3
    q, k, v = RNG.normal(size=(B, Nq, Sq, D)), RNG.normal(size=(B, Nq, Skv, D)), RNG.normal(size=(B, Nq, Skv, D))
    aq, akv = [9, 4, 0], [6, 11, 3]
    for b in range(B):  # padding that would dominate the softmax if it were read
        k[b, :, akv[b]:] = 50.0 * q[b, :, :1]
        v[b, :, akv[b]:] = 1e3
    for mode in (0, 2, 3):
        o, m, l = attention(q, k, v, 0.6, sparse_mode=mode, actual_seq_q=aq, actual_seq_kv=akv)
        for b in range(B):
            off = akv[b] - aq[b] if mode == 3 else 0
            for h in range(Nq):
                keep = (lambda i, j: True) if mode == 0 else (lambda i, j, off=off: j <= i + off)
                bo, bm, bl = _brute(q[b, h, :aq[b]], k[b, h, :akv[b]], v[b, h, :akv[b]], 0.6, keep)
                np.testing.assert_allclose(o[b, h, :aq[b]], bo, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(l[b, h, :aq[b]], bl, rtol=1e-12)
                np.testing.assert_array_equal(np.isneginf(m[b, h, :aq[b]]), np.isneginf(bm))
                assert np.all(o[b, h, aq[b]:] == 0) and np.all(np.isneginf(m[b, h, aq[b]:]))
                assert np.all(l[b, h, aq[b]:] == 0)


def test_actual_lengths_equal_tnd_and_full_lengths():
    """Padded BNSD with actual lengths equals TND over the same sequences (bottom-right causal
    and the band anchored inside each sequence); full actual lengths change nothing."""
    lq, lk = [5, 130, 64], [7, 100, 64]
    Nq, Nkv, D, S, Skv = 2, 1, 4, 140, 120
    q, k, v = RNG.normal(size=(3, Nq, S, D)), RNG.normal(size=(3, Nkv, Skv, D)), RNG.normal(size=(3, Nkv, Skv, D))
    cuq = np.concatenate([[0], np.cumsum(lq)])
    cuk = np.concatenate([[0], np.cumsum(lk)])
    qt = np.concatenate([q[b, :, :lq[b]].transpose(1, 0, 2) for b in range(3)])
    kt = np.concatenate([k[b, :, :lk[b]].transpose(1, 0, 2) for b in range(3)])
    vt = np.concatenate([v[b, :, :lk[b]].transpose(1, 0, 2) for b in range(3)])
    for kw in (dict(sparse_mode=3), dict(sparse_mode=2), dict(pre_tokens=9, next_tokens=-2)):
        o, m, l = attention(q, k, v, 0.5, actual_seq_q=lq, actual_seq_kv=lk, **kw)
        ot, mt, lt = attention(qt, kt, vt, 0.5, layout="TND", cu_seqlens_q=cuq, cu_seqlens_kv=cuk, **kw)
        for b in range(3):
            np.testing.assert_array_equal(o[b, :, :lq[b]], ot[cuq[b]:cuq[b + 1]].transpose(1, 0, 2))
            np.testing.assert_array_equal(m[b, :, :lq[b]], mt[:, cuq[b]:cuq[b + 1]])
            np.testing.assert_array_equal(l[b, :, :lq[b]], lt[:, cuq[b]:cuq[b + 1]])
    full = attention(q, k, v, 0.5, sparse_mode=3)
    same = attention(q, k, v, 0.5, sparse_mode=3, actual_seq_q=[S] * 3, actual_seq_kv=[Skv] * 3)
    for x, y in zip(full, same):
        np.testing.assert_array_equal(x, y)
    with pytest.raises(ValueError):
        attention(q, k, v, 0.5, actual_seq_q=[S + 1, 1, 1])


def test_bit_mask_layout_hand_worked():
    """Bit j % 32 of word j // 32 is key j, 1 = masked; bits past Skv are ignored."""
    from oracle import atten_mask_from_bits
    words = np.array([[0x80000005, 0x00000001], [0x00000000, 0xFFFFFFFE]], dtype=np.uint32)
    m = atten_mask_from_bits(words, 33)
    assert m.shape == (2, 33) and m.dtype == np.uint8
    assert np.nonzero(m[0])[0].tolist() == [0, 2, 31, 32]
    assert m[1].sum() == 0                       # bits 1..31 of the last word lie past key 32
    with pytest.raises(ValueError):
        atten_mask_from_bits(words, 65)


@pytest.mark.parametrize("Skv", [1, 31, 32, 33, 100, 257])
def test_bit_mask_inverts_numpy_packbits(Skv):
    """Against an independent routine: numpy's little-endian packbits of a byte mask, padded to
    whole 32-bit words and read as little-endian uint32, unpacks to the same byte mask (SS, B1SS
    and BNSS shapes)."""
    from oracle import atten_mask_from_bits
    for shape in ((5, Skv), (2, 1, 3, Skv), (2, 3, 4, Skv)):
        m = (RNG.random(shape) < 0.4).astype(np.uint8)
        W = (Skv + 31) // 32
        padded = np.zeros(shape[:-1] + (32 * W,), dtype=np.uint8)
        padded[..., :Skv] = m
        packed = np.packbits(padded, axis=-1, bitorder="little")          # bytes, 4 W per row
        words = np.ascontiguousarray(packed).view("<u4")
        assert words.shape == shape[:-1] + (W,)
        np.testing.assert_array_equal(atten_mask_from_bits(words, Skv), m)
        # and the attention it gives equals the byte mask's
        if len(shape) == 2:
            q, k, v = RNG.normal(size=(1, 1, 5, 4)), RNG.normal(size=(1, 1, Skv, 4)), RNG.normal(size=(1, 1, Skv, 4))
            a = attention(q, k, v, 0.5, atten_mask=m)
            b = attention(q, k, v, 0.5, atten_mask=atten_mask_from_bits(words, Skv))
            for x, y in zip(a, b):
                np.testing.assert_array_equal(x, y)
