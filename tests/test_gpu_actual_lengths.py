"""GPU parity with per-batch actual sequence lengths on padded BNSD tensors (EagleQBSA article,
API call: actual_seq_lengths / actual_seq_lengths_kv) against the float64 oracle.

Batch b is the sequence of its first aq_b queries and akv_b keys; its rows aq_b .. Sq - 1 must
come out exactly as rows with no key (O = 0, m = -inf, l = 0), whatever the output buffers held.
The padding of the 16-bit inputs is NaN, so any read of it would show. Tolerances as elsewhere:
O max-abs 1e-2 (16-bit path) or 3e-2 channel-scaled (quantised path), m/l relative 1e-3.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (O_TOL_BF16, O_TOL_QUANT, banner, check_ml, check_o, check_o_channel_scaled, dev_bf16, f64,
                      to_np)
from workloads import make_block_keep, random_bf16

pytestmark = pytest.mark.gpu

NAN_BF16 = np.uint16(0x7FC0)


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _padded(seed, B, N, S, D, lens, fill=NAN_BF16):
    """bf16 bits [B, N, S, D] whose rows from lens[b] on hold `fill`."""
    x = random_bf16(seed, (B, N, S, D))
    for b, L in enumerate(lens):
        x[b, :, L:] = fill
    return x


def _garbage_outputs(shape_o, shape_ml):
    return (torch.full(shape_o, 7.0, dtype=torch.bfloat16, device="cuda"),
            torch.full(shape_ml, 5.0, device="cuda"), torch.full(shape_ml, 3.0, device="cuda"))


def _check_padding(o, m, l, aq):
    o, m, l = to_np(o), to_np(m), to_np(l)
    for b, L in enumerate(aq):
        assert np.all(o[b, :, L:] == 0), f"batch {b}: padded rows of O not zero"
        assert np.all(np.isneginf(m[b, :, L:])), f"batch {b}: padded softmax_max not -inf"
        assert np.all(l[b, :, L:] == 0), f"batch {b}: padded softmax_sum not 0"


@pytest.mark.parametrize("mode,masked,band,D", [(0, False, None, 128), (2, False, None, 128), (3, False, None, 64),
                                                (0, True, None, 128), (0, False, (100, 10), 128),
                                                (3, True, None, 128)])
def test_dense(qa, mode, masked, band, D):
    B, Nq, Nkv, Sq, Skv = 4, 4, 2, 400, 460
    aq, akv = [400, 130, 0, 1], [460, 300, 5, 129]
    banner(f"actual lengths dense mode={mode} masked={masked} band={band} D={D}")
    q = _padded(1, B, Nq, Sq, D, aq)
    k = _padded(2, B, Nkv, Skv, D, akv)
    v = _padded(3, B, Nkv, Skv, D, akv)
    mask = None
    if masked:
        mask = (np.random.default_rng(4).random((B, 1, Sq, Skv)) < 0.25).astype(np.uint8)
    bk = {} if band is None else dict(pre_tokens=band[0], next_tokens=band[1])
    out = _garbage_outputs((B, Nq, Sq, D), (B, Nq, Sq))
    o, m, l = qa.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=0.09, sparse_mode=mode,
                          atten_mask=None if mask is None else torch.from_numpy(mask).cuda(), actual_seq_lengths=aq,
                          actual_seq_lengths_kv=akv, out=out[0], softmax_max=out[1], softmax_sum=out[2], **bk)
    torch.cuda.synchronize()
    _check_padding(o, m, l, aq)
    ro, rm, rl = oracle.attention(f64(q), f64(k), f64(v), 0.09, sparse_mode=mode, atten_mask=mask,
                                  actual_seq_q=aq, actual_seq_kv=akv, **bk)
    for b in range(B):
        sl = slice(0, aq[b])
        check_o(to_np(o)[b, :, sl], ro[b, :, sl], O_TOL_BF16, f"batch {b}")
        check_ml(to_np(m)[b, :, sl], to_np(l)[b, :, sl], rm[b, :, sl], rl[b, :, sl], what=f"batch {b}")


def test_kv_lengths_only_and_subranges(qa):
    """Only key lengths given; a head / q-block subrange covering the padding writes it too, and
    the pieces together equal the full call bit for bit."""
    B, Nq, S, D = 2, 2, 300, 128
    akv = [77, 300]
    qn, kn, vn = random_bf16(5, (B, Nq, S, D)), _padded(6, B, Nq, S, D, akv), _padded(7, B, Nq, S, D, akv)
    q, k, v = dev_bf16(qn), dev_bf16(kn), dev_bf16(vn)
    full = qa.attn_fwd(q, k, v, scale=0.1, sparse_mode=3, actual_seq_lengths_kv=akv)
    pieces = _garbage_outputs((B, Nq, S, D), (B, Nq, S))
    for hr, br in [((0, 1), (0, 3)), ((1, 2), (0, 1)), ((1, 2), (1, 3))]:
        qa.attn_fwd(q, k, v, scale=0.1, sparse_mode=3, actual_seq_lengths_kv=akv, head_range=hr, qblock_range=br,
                    out=pieces[0], softmax_max=pieces[1], softmax_sum=pieces[2])
    torch.cuda.synchronize()
    assert torch.equal(full[0].view(torch.int16), pieces[0].view(torch.int16))
    assert torch.equal(full[1], pieces[1]) and torch.equal(full[2], pieces[2])
    ro, rm, rl = oracle.attention(f64(qn), f64(kn), f64(vn), 0.1, sparse_mode=3, actual_seq_kv=akv)
    check_o(to_np(full[0]), ro, O_TOL_BF16)
    check_ml(to_np(full[1]), to_np(full[2]), rm, rl)


def test_blocksparse(qa):
    B, Nq, Nkv, S, D = 2, 4, 2, 640, 128
    aq, akv = [333, 640], [640, 200]
    banner("actual lengths block-sparse")
    q = _padded(11, B, Nq, S, D, aq)
    k = _padded(12, B, Nkv, S, D, akv)
    v = _padded(13, B, Nkv, S, D, akv)
    keep = make_block_keep(14, B, Nq, 5, 5, 0.5)
    counts, idx = qa.build_kv_block_list(torch.from_numpy(keep).cuda())
    out = _garbage_outputs((B, Nq, S, D), (B, Nq, S))
    o, m, l = qa.attn_fwd_blocksparse(dev_bf16(q), dev_bf16(k), dev_bf16(v), counts, idx, scale=0.088,
                                      actual_seq_lengths=aq, actual_seq_lengths_kv=akv, out=out[0],
                                      softmax_max=out[1], softmax_sum=out[2])
    torch.cuda.synchronize()
    _check_padding(o, m, l, aq)
    ro, rm, rl = oracle.attention(f64(q), f64(k), f64(v), 0.088, block_keep=keep, actual_seq_q=aq,
                                  actual_seq_kv=akv)
    for b in range(B):
        sl = slice(0, aq[b])
        check_o(to_np(o)[b, :, sl], ro[b, :, sl], O_TOL_BF16, f"batch {b}")
        check_ml(to_np(m)[b, :, sl], to_np(l)[b, :, sl], rm[b, :, sl], rl[b, :, sl], what=f"batch {b}")


def test_qbsa(qa):
    """The quantisers see the whole padded buffers (finite padding that would dominate the
    softmax if read); the attention uses only each batch's valid rows and keys."""
    B, Nq, Nkv, S, D = 2, 4, 2, 512, 128
    aq, akv = [512, 200], [300, 512]
    banner("actual lengths qbsa")
    q = random_bf16(21, (B, Nq, S, D), "block_offset")
    k = random_bf16(22, (B, Nkv, S, D), "block_offset")
    v = random_bf16(23, (B, Nkv, S, D), "block_offset")
    big = np.uint16(0x4200)  # 32.0
    for b in range(B):
        k[b, :, akv[b]:] = big
        v[b, :, akv[b]:] = big
    keep = make_block_keep(24, B, Nq, 4, 4, 0.6)
    qq, qs = qa.quantize_qk_perblock_int8(dev_bf16(q))
    kq, ks = qa.quantize_qk_perblock_int8(dev_bf16(k))
    vq, vs = qa.quantize_v_perchannel_fp8(dev_bf16(v))
    counts, idx = qa.build_kv_block_list(torch.from_numpy(keep).cuda())
    out = _garbage_outputs((B, Nq, S, D), (B, Nq, S))
    o, m, l = qa.attn_fwd_qbsa(qq, kq, vq, qs, ks, vs, counts, idx, scale=0.088, actual_seq_lengths=aq,
                               actual_seq_lengths_kv=akv, out=out[0], softmax_max=out[1], softmax_sum=out[2])
    torch.cuda.synchronize()
    _check_padding(o, m, l, aq)
    rqc, rqs = oracle.quantize_qk_perblock_int8(f64(q))
    rkc, rks = oracle.quantize_qk_perblock_int8(f64(k))
    rvc, rvs = oracle.quantize_v_perchannel_fp8(f64(v))
    res = oracle.qbsa_attention(rqc, rkc, rvc, rqs, rks, rvs, keep, 0.088, actual_seq_q=aq, actual_seq_kv=akv)
    ro = np.zeros((B, Nq, S, D))
    rm = np.full((B, Nq, S), -np.inf)
    rl = np.zeros((B, Nq, S))
    for (b, h, qb), (oo, mm, ll) in res.items():
        ro[b, h, qb * 128:qb * 128 + len(mm)] = oo
        rm[b, h, qb * 128:qb * 128 + len(mm)] = mm
        rl[b, h, qb * 128:qb * 128 + len(mm)] = ll
    vf = f64(v)
    for b in range(B):
        vf[b, :, akv[b]:] = 0.0  # the padding is not part of any channel's scale of reference
    check_o_channel_scaled(to_np(o), ro, vf, O_TOL_QUANT)
    check_ml(to_np(m), to_np(l), rm, rl)
