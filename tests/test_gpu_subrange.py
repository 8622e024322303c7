"""Subrange launches reproduce the full call bit for bit (power-cap page,
InsertComm and BlockAttn: attention split by head chunks and by query blocks,
results concatenated; the page checks that all modes give the same output).

Each test runs the full call once, then covers the same problem with several
head-chunk and q-block-range launches into fresh outputs, and compares bytes.
"""

import numpy as np
import pytest
import torch

from gpu_util import banner, dev_bf16
from workloads import make_block_keep, random_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _same(a, b):
    for x, y in zip(a, b):
        if x is None:
            continue
        xi = x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)
        yi = y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)
        assert torch.equal(xi, yi)


def _pieces(n_heads, n_qb):
    """Head chunks (1 head each, then 4-head chunks, then halves) crossed with
    q-block splits (halves, ragged thirds, single blocks at odd offsets)."""
    splits = []
    hc = [(h, h + 1) for h in range(n_heads)]
    h4 = [(h, min(n_heads, h + 4)) for h in range(0, n_heads, 4)]
    half = n_qb // 2
    qs = [[(0, half), (half, n_qb)], [(0, 1), (1, max(1, n_qb - 2)), (max(1, n_qb - 2), n_qb)],
          [(i, i + 1) for i in range(n_qb)]]
    splits.append([(h, (0, n_qb)) for h in hc])
    splits.append([(h, r) for h in h4 for r in qs[0]])
    splits.append([((0, n_heads), r) for r in qs[1] if r[0] < r[1]])
    splits.append([((0, n_heads), r) for r in qs[2]])
    return splits


# S = 1100: byte-mask rows read per element; S = 1104: 16-byte aligned byte-mask rows, staged in
# LDS; "bits": the same mask bit-packed (always staged in LDS)
@pytest.mark.parametrize("mode,masked,band,S", [(0, False, None, 1100), (2, False, None, 1100), (3, False, None, 1100),
                                               (0, True, None, 1100), (3, True, None, 1100), (0, False, (200, 30), 1100),
                                               (0, True, (64, 300), 1100), (0, True, None, 1104), (3, True, None, 1104),
                                               (0, True, (64, 300), 1104), (0, "bits", None, 1100),
                                               (3, "bits", None, 1104), (0, "bits", (64, 300), 1100)])
def test_dense_subranges(qa, mode, masked, band, S):
    B, Nq, Nkv, D = 1, 8, 4, 128
    banner(f"subrange dense mode={mode} masked={masked} S={S}")
    q = dev_bf16(random_bf16(1, (B, Nq, S, D)))
    k = dev_bf16(random_bf16(2, (B, Nkv, S, D)))
    v = dev_bf16(random_bf16(3, (B, Nkv, S, D)))
    mask = None
    if masked:  # B1SS boolean mask, about 20% of the keys masked
        g = torch.Generator(device="cuda").manual_seed(5)
        mask = (torch.rand((B, 1, S, S), generator=g, device="cuda") < 0.2).to(torch.uint8)
        if masked == "bits":
            from test_gpu_attention import pack_mask_bits
            mask = torch.from_numpy(pack_mask_bits(mask.cpu().numpy())).cuda()
    bk = {} if band is None else dict(pre_tokens=band[0], next_tokens=band[1])
    full = qa.attn_fwd(q, k, v, scale=0.1, sparse_mode=mode, atten_mask=mask, **bk)
    nqb = (S + 127) // 128
    for split in _pieces(Nq, nqb):
        out = (torch.zeros_like(full[0]), torch.zeros_like(full[1]), torch.zeros_like(full[2]))
        for hr, br in split:
            qa.attn_fwd(q, k, v, scale=0.1, sparse_mode=mode, atten_mask=mask, head_range=hr, qblock_range=br,
                        out=out[0], softmax_max=out[1], softmax_sum=out[2], **bk)
        torch.cuda.synchronize()
        _same(full, out)


@pytest.mark.parametrize("mode", [0, 3])
def test_tnd_subranges(qa, mode):
    lens = [300, 5, 700, 128]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    T, Nq, Nkv, D = cu[-1], 4, 2, 128
    q = dev_bf16(random_bf16(11, (T, Nq, D)))
    k = dev_bf16(random_bf16(12, (T, Nkv, D)))
    v = dev_bf16(random_bf16(13, (T, Nkv, D)))
    full = qa.attn_fwd(q, k, v, scale=0.1, layout="TND", sparse_mode=mode, cu_seqlens_q=cu)
    nqb = sum((x + 127) // 128 for x in lens)
    for split in _pieces(Nq, nqb):
        out = (torch.zeros_like(full[0]), torch.zeros_like(full[1]), torch.zeros_like(full[2]))
        for hr, br in split:
            qa.attn_fwd(q, k, v, scale=0.1, layout="TND", sparse_mode=mode, cu_seqlens_q=cu, head_range=hr,
                        qblock_range=br, out=out[0], softmax_max=out[1], softmax_sum=out[2])
        torch.cuda.synchronize()
        _same(full, out)


def test_blocksparse_and_qbsa_subranges(qa):
    S, Nq, D = 1024, 4, 128
    nb = S // 128
    qb_ = random_bf16(21, (1, Nq, S, D), "block_offset")
    kb_ = random_bf16(22, (1, Nq, S, D), "block_offset")
    vb_ = random_bf16(23, (1, Nq, S, D), "block_offset")
    keep = torch.from_numpy(make_block_keep(24, 1, Nq, nb, nb, 0.4)).cuda()
    q, k, v = dev_bf16(qb_), dev_bf16(kb_), dev_bf16(vb_)
    counts, idx = qa.build_kv_block_list(keep)
    full = qa.attn_fwd_blocksparse(q, k, v, counts, idx, scale=0.1)
    qq, qs = qa.quantize_qk_perblock_int8(q)
    kq, ks = qa.quantize_qk_perblock_int8(k)
    vq, vs = qa.quantize_v_perchannel_fp8(v)
    fullq = qa.attn_fwd_qbsa(qq, kq, vq, qs, ks, vs, counts, idx, scale=0.1)
    for split in _pieces(Nq, nb):
        out = (torch.zeros_like(full[0]), torch.zeros_like(full[1]), torch.zeros_like(full[2]))
        outq = (torch.zeros_like(full[0]), torch.zeros_like(full[1]), torch.zeros_like(full[2]))
        for hr, br in split:
            qa.attn_fwd_blocksparse(q, k, v, counts, idx, scale=0.1, head_range=hr, qblock_range=br, out=out[0],
                                    softmax_max=out[1], softmax_sum=out[2])
            qa.attn_fwd_qbsa(qq, kq, vq, qs, ks, vs, counts, idx, scale=0.1, head_range=hr, qblock_range=br,
                             out=outq[0], softmax_max=outq[1], softmax_sum=outq[2])
        torch.cuda.synchronize()
        _same(full, out)
        _same(fullq, outq)


@pytest.mark.parametrize("mode,qbr", [(0, (1, 3)), (0, (1, 2)), (0, (3, 4)), (3, (1, 2))])
def test_subrange_leaves_rest_untouched(qa, mode, qbr):
    """Only the slice's rows are written, also when a workgroup's second q-block lies outside it."""
    B, Nq, S, D = 1, 2, 512, 64
    q = dev_bf16(random_bf16(31, (B, Nq, S, D)))
    sentinel = torch.full((B, Nq, S, D), 7.0, dtype=torch.bfloat16, device="cuda")
    m = torch.full((B, Nq, S), 7.0, device="cuda")
    l = torch.full((B, Nq, S), 7.0, device="cuda")
    qa.attn_fwd(q, q, q, scale=0.1, sparse_mode=mode, head_range=(1, 2), qblock_range=qbr, out=sentinel,
                softmax_max=m, softmax_sum=l)
    torch.cuda.synchronize()
    touched = torch.zeros((B, Nq, S), dtype=torch.bool, device="cuda")
    touched[:, 1, 128 * qbr[0]:128 * qbr[1]] = True
    assert torch.all(sentinel[~touched] == 7.0) and torch.all(m[~touched] == 7.0) and torch.all(l[~touched] == 7.0)
    assert not torch.any(sentinel[touched] == 7.0)
    assert not torch.any(sentinel[touched] == 7.0)
