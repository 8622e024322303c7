"""GPU parity of calls with more sequences (TND) or padded batches (per-batch actual lengths) than
one kernel launch carries (QATTN_MAX_SEQS = 256: the lengths travel in the kernel argument), which
the library runs as one launch per group of 256.

Each sequence or batch is its own problem, so a call over all of them must equal, bit for bit,
separate calls over parts of them; the groups must also hold against the float64 oracle (forward
O max-abs 1e-2, m/l relative 1e-3; the quantised path 3e-2 per channel scale; backward as in the
backward tests). The 1e-2 holds where |O| stays below about 2; thousands of short causal rows,
each with one to a few keys, reach |O| up to the largest |v|, where rounding P and O to bf16 alone
can pass it. There the bound is the arithmetic's own: P rounded to bf16 moves O by at most
2^-9 sum_j p_j |v_j| / l, and rounding O by half an ulp, at most 2^-9 |O|; the check allows twice
both, sum_j p_j |v_j| / l coming from the oracle run on |V|. Subrange launches whose q-block ranges straddle a group boundary must equal the
full call bit for bit, and rows past a batch's actual length come out as rows with no key.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import O_TOL_BF16, O_TOL_QUANT, banner, check_ml, check_o_channel_scaled, dev_bf16, f64, to_np
from workloads import make_block_keep, random_bf16

pytestmark = pytest.mark.gpu

G_RTOL = 1e-2  # backward: max-abs error relative to max(1, max |ref|), as in the backward tests


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _lengths(seed, n, hi, zeros=True):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0 if zeros else 1, hi + 1, size=n)
    return lens


def _check_o_rounding(o, ro, ro_abs, what):
    """O max-abs error within max(1e-2, 2^-8 (sum_j p_j |v_j| / l + |O|)) element by element."""
    if o.size == 0:  # a batch with no query row
        return
    err = np.abs(o - ro)
    bound = np.maximum(O_TOL_BF16, 2.0 ** -8 * (ro_abs + np.abs(ro)))
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    banner(f"{what}: O max-abs err {err.max():.3e}; tightest element err {err[worst]:.3e} bound {bound[worst]:.3e}")
    assert np.all(np.isfinite(o)), f"{what}: non-finite values"
    assert np.all(err <= bound), f"{what}: error {err[worst]:.3e} > {bound[worst]:.3e} at {worst}"


def _bits_equal(a, b):
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("mode", [0, 3])
def test_tnd_600_sequences(qa, mode):
    """600 sequences of 0..150 tokens (three launches): the oracle, then bit identity with three
    separate calls of 200 sequences each and with q-block subranges across the group edges."""
    n, Nq, Nkv, D = 600, 4, 2, 64
    lq = _lengths(1, n, 150)
    lk = lq.copy() if mode == 3 else _lengths(2, n, 150)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    what = f"TND {n} sequences mode={mode}"
    banner(what)
    qb, kb, vb = random_bf16(3, (cq[-1], Nq, D)), random_bf16(4, (ck[-1], Nkv, D)), random_bf16(5, (ck[-1], Nkv, D))
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    scale = 1.0 / np.sqrt(D)
    kw = dict(scale=scale, layout="TND", sparse_mode=mode)
    o, m, l = qa.attn_fwd(q, k, v, cu_seqlens_q=cq.tolist(), cu_seqlens_kv=ck.tolist(), **kw)
    torch.cuda.synchronize()
    ref = dict(layout="TND", sparse_mode=mode, cu_seqlens_q=cq, cu_seqlens_kv=ck)
    ro, rm, rl = oracle.attention(f64(qb), f64(kb), f64(vb), scale, **ref)
    ro_abs = oracle.attention(f64(qb), f64(kb), np.abs(f64(vb)), scale, **ref)[0]
    _check_o_rounding(to_np(o), ro, ro_abs, what)
    check_ml(to_np(m), to_np(l), rm, rl, what=what)
    # the same sequences as three calls of 200
    for s0 in range(0, n, 200):
        s1 = s0 + 200
        a, b = int(cq[s0]), int(cq[s1])
        c, d = int(ck[s0]), int(ck[s1])
        po, pm, pl = qa.attn_fwd(q[a:b].contiguous(), k[c:d].contiguous(), v[c:d].contiguous(),
                                 cu_seqlens_q=(cq[s0:s1 + 1] - a).tolist(), cu_seqlens_kv=(ck[s0:s1 + 1] - c).tolist(),
                                 **kw)
        torch.cuda.synchronize()
        assert _bits_equal(po, o[a:b]), f"sequences {s0}..{s1}: O"
        assert _bits_equal(pm, m[:, a:b]) and _bits_equal(pl, l[:, a:b]), f"sequences {s0}..{s1}: m, l"
    # q-block subranges whose edges fall inside the first and third groups
    nqb = int(sum((x + 127) // 128 for x in lq))
    cut = [0, nqb // 5, nqb // 2, (4 * nqb) // 5, nqb]
    out = tuple(torch.zeros_like(x) for x in (o, m, l))
    for i in range(4):
        qa.attn_fwd(q, k, v, cu_seqlens_q=cq.tolist(), cu_seqlens_kv=ck.tolist(), qblock_range=(cut[i], cut[i + 1]),
                    out=out[0], softmax_max=out[1], softmax_sum=out[2], **kw)
    torch.cuda.synchronize()
    for x, y in zip(out, (o, m, l)):
        assert _bits_equal(x, y)


def test_actual_lengths_300_batches(qa):
    """300 padded batches (two launches) with NaN padding: the oracle on every batch, bit identity
    with a separate call over batches 250..299, rows past each length written as rows with no key."""
    B, Nq, Nkv, Sq, Skv, D = 300, 2, 1, 160, 140, 64
    aq, akv = _lengths(6, B, Sq), _lengths(7, B, Skv)
    banner("actual lengths, 300 batches")
    nan = np.uint16(0x7FC0)
    qb, kb, vb = random_bf16(8, (B, Nq, Sq, D)), random_bf16(9, (B, Nkv, Skv, D)), random_bf16(10, (B, Nkv, Skv, D))
    for b in range(B):
        qb[b, :, aq[b]:] = nan
        kb[b, :, akv[b]:] = nan
        vb[b, :, akv[b]:] = nan
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    scale = 1.0 / np.sqrt(D)
    out = (torch.full((B, Nq, Sq, D), 7.0, dtype=torch.bfloat16, device="cuda"),
           torch.full((B, Nq, Sq), 5.0, device="cuda"), torch.full((B, Nq, Sq), 3.0, device="cuda"))
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, sparse_mode=3, actual_seq_lengths=aq.tolist(),
                          actual_seq_lengths_kv=akv.tolist(), out=out[0], softmax_max=out[1], softmax_sum=out[2])
    torch.cuda.synchronize()
    on, mn, ln = to_np(o), to_np(m), to_np(l)
    for b in range(B):
        assert np.all(on[b, :, aq[b]:] == 0) and np.all(np.isneginf(mn[b, :, aq[b]:])) and np.all(ln[b, :, aq[b]:] == 0)
    ref = dict(sparse_mode=3, actual_seq_q=aq, actual_seq_kv=akv)
    qr, kr, vr = (np.nan_to_num(f64(x)) for x in (qb, kb, vb))
    ro, rm, rl = oracle.attention(qr, kr, vr, scale, **ref)
    ro_abs = oracle.attention(qr, kr, np.abs(vr), scale, **ref)[0]
    for b in range(B):
        sl = slice(0, int(aq[b]))
        _check_o_rounding(on[b, :, sl], ro[b, :, sl], ro_abs[b, :, sl], f"batch {b}")
        check_ml(mn[b, :, sl], ln[b, :, sl], rm[b, :, sl], rl[b, :, sl], what=f"batch {b}")
    po, pm, pl = qa.attn_fwd(q[250:].contiguous(), k[250:].contiguous(), v[250:].contiguous(), scale=scale,
                             sparse_mode=3, actual_seq_lengths=aq[250:].tolist(),
                             actual_seq_lengths_kv=akv[250:].tolist())
    torch.cuda.synchronize()
    assert _bits_equal(po, o[250:]) and _bits_equal(pm, m[250:]) and _bits_equal(pl, l[250:])


def test_blocksparse_and_qbsa_270_batches(qa):
    """Block-sparse and quantised block-sparse with per-batch actual lengths over 270 batches (the
    kept-list walk of batch 256 on is that of its problem index). Block-sparse: every batch against
    the oracle. Quantised: bit for bit against separate calls over batches 0..255 and 256..269, then
    against the oracle with every key length full: its residual against the oracle is one E4M3 step
    of a p now and then (p formed in float32), which a row of a few keys (a diagonal block cut short
    by its batch's key length) weighs at up to |v|/16, beyond the 3e-2 stated for rows over many
    keys; with full key lengths every row sees at least its 128-key diagonal block."""
    B, Nq, Nkv, S, D = 270, 2, 2, 256, 128
    aq, akv = _lengths(11, B, S, zeros=False), _lengths(12, B, S, zeros=False)
    banner("block-sparse and QBSA, 270 batches")
    qb, kb, vb = random_bf16(13, (B, Nq, S, D)), random_bf16(14, (B, Nkv, S, D)), random_bf16(15, (B, Nkv, S, D))
    keep = make_block_keep(16, B, Nq, 2, 2, 0.5)
    counts, idx = qa.build_kv_block_list(torch.from_numpy(keep).cuda())
    scale = 1.0 / np.sqrt(D)
    lens = dict(actual_seq_lengths=aq.tolist(), actual_seq_lengths_kv=akv.tolist())
    o, m, l = qa.attn_fwd_blocksparse(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), counts, idx, scale=scale, **lens)
    torch.cuda.synchronize()
    ref = dict(block_keep=keep, actual_seq_q=aq, actual_seq_kv=akv)  # batches of 1..256 keys
    ro, rm, rl = oracle.attention(f64(qb), f64(kb), f64(vb), scale, **ref)
    ro_abs = oracle.attention(f64(qb), f64(kb), np.abs(f64(vb)), scale, **ref)[0]
    _check_o_rounding(to_np(o), ro, ro_abs, "block-sparse")
    check_ml(to_np(m), to_np(l), rm, rl, what="block-sparse")

    qq, qs = qa.quantize_qk_perblock_int8(dev_bf16(qb))
    kq, ks = qa.quantize_qk_perblock_int8(dev_bf16(kb))
    vq, vs = qa.quantize_v_perchannel_fp8(dev_bf16(vb))
    args = (qq, kq, vq, qs, ks, vs, counts, idx)
    o, m, l = qa.attn_fwd_qbsa(*args, scale=scale, **lens)
    torch.cuda.synchronize()
    for lo, hi in ((0, 256), (256, 270)):
        po, pm, pl = qa.attn_fwd_qbsa(*(x[lo:hi].contiguous() for x in args), scale=scale,
                                      actual_seq_lengths=aq[lo:hi].tolist(), actual_seq_lengths_kv=akv[lo:hi].tolist())
        torch.cuda.synchronize()
        assert _bits_equal(po, o[lo:hi]) and _bits_equal(pm, m[lo:hi]) and _bits_equal(pl, l[lo:hi]), f"{lo}..{hi}"

    o, m, l = qa.attn_fwd_qbsa(*args, scale=scale, actual_seq_lengths=aq.tolist())
    torch.cuda.synchronize()
    rqc, rqs = oracle.quantize_qk_perblock_int8(f64(qb))
    rkc, rks = oracle.quantize_qk_perblock_int8(f64(kb))
    rvc, rvs = oracle.quantize_v_perchannel_fp8(f64(vb))
    res = oracle.qbsa_attention(rqc, rkc, rvc, rqs, rks, rvs, keep, scale, actual_seq_q=aq)
    ro = np.zeros((B, Nq, S, D))
    rm = np.full((B, Nq, S), -np.inf)
    rl = np.zeros((B, Nq, S))
    for (b, h, qbk), (oo, mm, ll) in res.items():
        ro[b, h, qbk * 128:qbk * 128 + len(mm)] = oo
        rm[b, h, qbk * 128:qbk * 128 + len(mm)] = mm
        rl[b, h, qbk * 128:qbk * 128 + len(mm)] = ll
    check_o_channel_scaled(to_np(o), ro, f64(vb), O_TOL_QUANT)
    check_ml(to_np(m), to_np(l), rm, rl, what="qbsa")


def _check_grad(g, ref, what):
    g = to_np(g)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    bound = G_RTOL * max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)
    err = float(np.abs(g - ref).max()) if ref.size else 0.0
    banner(f"{what}: max-abs err {err:.3e} (bound {bound:.3e})")
    assert err <= bound, f"{what}: max abs error {err:.3e} > {bound:.3e}"


def test_backward_tnd_300_sequences(qa):
    """The backward over 300 sequences (two launches of its products): the oracle, then bit
    identity with separate calls over sequences 0..149 and 150..299."""
    n, Nq, Nkv, D = 300, 4, 2, 64
    lq, lk = _lengths(17, n, 100), _lengths(18, n, 100)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    banner(f"backward TND {n} sequences")
    qb, kb, vb = random_bf16(19, (cq[-1], Nq, D)), random_bf16(20, (ck[-1], Nkv, D)), random_bf16(21, (ck[-1], Nkv, D))
    gb = random_bf16(22, (cq[-1], Nq, D))
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    scale = 1.0 / np.sqrt(D)
    kw = dict(scale=scale, layout="TND", sparse_mode=0)
    o, m, l = qa.attn_fwd(q, k, v, cu_seqlens_q=cq.tolist(), cu_seqlens_kv=ck.tolist(), **kw)
    dq, dk, dv = qa.attn_bwd(q, k, v, o, do, m, l, cu_seqlens_q=cq.tolist(), cu_seqlens_kv=ck.tolist(), **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(f64(qb), f64(kb), f64(vb), f64(gb), scale, layout="TND", sparse_mode=0,
                                           cu_seqlens_q=cq, cu_seqlens_kv=ck)
    _check_grad(dq, rq, "dQ")
    _check_grad(dk, rk, "dK")
    _check_grad(dv, rv, "dV")
    for s0, s1 in ((0, 150), (150, 300)):
        a, b, c, d = int(cq[s0]), int(cq[s1]), int(ck[s0]), int(ck[s1])
        part = dict(cu_seqlens_q=(cq[s0:s1 + 1] - a).tolist(), cu_seqlens_kv=(ck[s0:s1 + 1] - c).tolist(), **kw)
        qs_, os_, dos_ = (x[a:b].contiguous() for x in (q, o, do))
        ks_, vs_ = k[c:d].contiguous(), v[c:d].contiguous()
        gq, gk, gv = qa.attn_bwd(qs_, ks_, vs_, os_, dos_, m[:, a:b].contiguous(), l[:, a:b].contiguous(), **part)
        torch.cuda.synchronize()
        assert _bits_equal(gq, dq[a:b]) and _bits_equal(gk, dk[c:d]) and _bits_equal(gv, dv[c:d]), f"{s0}..{s1}"


def test_backward_actual_lengths_270_batches(qa):
    """The backward over 270 padded batches with NaN padding: the oracle, and bit identity with a
    separate call over batches 200..269."""
    B, Nq, Nkv, Sq, Skv, D = 270, 2, 1, 150, 130, 64
    aq, akv = _lengths(23, B, Sq), _lengths(24, B, Skv)
    banner("backward actual lengths, 270 batches")
    nan = np.uint16(0x7FC0)

    def padded(seed, shape, lens):
        x = random_bf16(seed, shape)
        for b, L in enumerate(lens):
            x[b, :, L:] = nan
        return x

    qb, kb, vb = padded(25, (B, Nq, Sq, D), aq), padded(26, (B, Nkv, Skv, D), akv), padded(27, (B, Nkv, Skv, D), akv)
    gb = padded(28, (B, Nq, Sq, D), aq)
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    scale = 1.0 / np.sqrt(D)
    kw = dict(scale=scale, sparse_mode=2, actual_seq_lengths=aq.tolist(), actual_seq_lengths_kv=akv.tolist())
    o, m, l = qa.attn_fwd(q, k, v, **kw)
    dq, dk, dv = qa.attn_bwd(q, k, v, o, do, m, l, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(np.nan_to_num(f64(qb)), np.nan_to_num(f64(kb)), np.nan_to_num(f64(vb)),
                                           np.nan_to_num(f64(gb)), scale, sparse_mode=2, actual_seq_q=aq,
                                           actual_seq_kv=akv)
    _check_grad(dq, rq, "dQ")
    _check_grad(dk, rk, "dK")
    _check_grad(dv, rv, "dV")
    part = dict(scale=scale, sparse_mode=2, actual_seq_lengths=aq[200:].tolist(),
                actual_seq_lengths_kv=akv[200:].tolist())
    sl = lambda x: x[200:].contiguous()
    gq, gk, gv = qa.attn_bwd(sl(q), sl(k), sl(v), sl(o), sl(do), sl(m), sl(l), **part)
    torch.cuda.synchronize()
    assert _bits_equal(gq, dq[200:]) and _bits_equal(gk, dk[200:]) and _bits_equal(gv, dv[200:])
