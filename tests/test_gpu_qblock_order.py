"""GPU tests of the q-block order: build_qblock_order and the block-sparse launches that take it.

* build_qblock_order equals the oracle's plain sort by (-kept count, index), bit for bit.
* The quantised kernel computes every row the same way in any order: with the order its outputs
  are the same bits as without, over whole problems, head and q-block subranges, and a padded
  batch of more than 256 batches (one launch per group of 256, the order offset per group).
* The bf16 block-sparse kernel walks each row's kept blocks from the first when given the order:
  its outputs match the oracle, and subrange launches with the order reproduce the full ordered
  call bit for bit and write nothing outside their slice.
* A bf16 block-sparse launch of 350 items (more than one chunk of 256 over the 8 XCDs, not a
  multiple of it) writes every row and matches the oracle, with and without the order.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import O_TOL_BF16, banner, check_ml, check_o, dev_bf16, f64, to_np
from workloads import make_block_keep, random_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same(a, b):
    for x, y in zip(a, b):
        assert torch.equal(_bits(x), _bits(y))


def test_order_matches_oracle(qa):
    B, N, QB = 2, 3, 100
    banner("build_qblock_order against the oracle")
    keep = torch.from_numpy(make_block_keep(301, B, N, QB, QB, 0.3)).cuda()
    counts, _ = qa.build_kv_block_list(keep)
    order = qa.build_qblock_order(counts)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    assert len(np.unique(c)) < c.size                      # ties present
    np.testing.assert_array_equal(order.cpu().numpy(), oracle.qblock_order(c))
    # a row of equal counts keeps the index order
    eq = torch.full((1, 1, 37), 5, dtype=torch.int32, device="cuda")
    o2 = qa.build_qblock_order(eq)
    torch.cuda.synchronize()
    assert o2.cpu().numpy().ravel().tolist() == list(range(37))


def _qbsa_inputs(qa, B, N, S, seed):
    q = dev_bf16(random_bf16(seed, (B, N, S, 128), "block_offset"))
    k = dev_bf16(random_bf16(seed + 1, (B, N, S, 128), "block_offset"))
    v = dev_bf16(random_bf16(seed + 2, (B, N, S, 128), "block_offset"))
    QB = (S + 127) // 128
    keep = torch.from_numpy(make_block_keep(seed + 3, B, N, QB, QB, 0.37)).cuda()
    qq, qs = qa.quantize_qk_perblock_int8(q)
    kq, ks = qa.quantize_qk_perblock_int8(k)
    vq, vs = qa.quantize_v_perchannel_fp8(v)
    counts, idx = qa.build_kv_block_list(keep)
    return (qq, kq, vq, qs, ks, vs, counts, idx), QB


def test_qbsa_same_bits_with_order(qa):
    B, N, S = 1, 4, 2048
    banner("QBSA with and without the q-block order, full and subranges")
    args, QB = _qbsa_inputs(qa, B, N, S, 310)
    order = qa.build_qblock_order(args[6])
    ref = qa.attn_fwd_qbsa(*args, scale=128 ** -0.5)
    got = qa.attn_fwd_qbsa(*args, scale=128 ** -0.5, qblock_order=order)
    torch.cuda.synchronize()
    _same(ref, got)
    # head x q-block subranges with the order, into outputs that start as a sentinel
    out = torch.full_like(ref[0], 7.0)
    m = torch.full_like(ref[1], 7.0)
    l = torch.full_like(ref[2], 7.0)
    for hr in ((0, 1), (1, 4)):
        for qr in ((0, 5), (5, QB - 1), (QB - 1, QB)):
            qa.attn_fwd_qbsa(*args, scale=128 ** -0.5, qblock_order=order, head_range=hr, qblock_range=qr, out=out,
                             softmax_max=m, softmax_sum=l)
    torch.cuda.synchronize()
    _same(ref, (out, m, l))
    # one subrange alone writes only its slice
    out2 = torch.full_like(ref[0], 7.0)
    qa.attn_fwd_qbsa(*args, scale=128 ** -0.5, qblock_order=order, head_range=(1, 3), qblock_range=(2, 9), out=out2,
                     return_softmax=False)
    torch.cuda.synchronize()
    sl = (slice(None), slice(1, 3), slice(2 * 128, 9 * 128))
    assert torch.equal(_bits(out2[sl]), _bits(ref[0][sl]))
    mask = torch.ones_like(out2, dtype=torch.bool)
    mask[sl] = False
    assert torch.all(out2[mask] == 7.0)


def test_qbsa_order_over_batch_groups(qa):
    """More than 256 padded batches: one launch per group of 256, the order offset per group."""
    B, N, S = 270, 1, 256
    banner("QBSA with the q-block order over 270 padded batches")
    args, QB = _qbsa_inputs(qa, B, N, S, 320)
    rng = np.random.default_rng(321)
    aq = rng.integers(1, S + 1, size=B).tolist()
    akv = rng.integers(1, S + 1, size=B).tolist()
    order = qa.build_qblock_order(args[6])
    kw = dict(scale=128 ** -0.5, actual_seq_lengths=aq, actual_seq_lengths_kv=akv)
    ref = qa.attn_fwd_qbsa(*args, **kw)
    got = qa.attn_fwd_qbsa(*args, qblock_order=order, **kw)
    torch.cuda.synchronize()
    _same(ref, got)


def test_bsa_with_order_against_oracle_and_subranges(qa):
    B, Nq, Nkv, S, D = 1, 4, 2, 1100, 128
    banner("BSA with the q-block order: oracle and subranges")
    QB = (S + 127) // 128
    qb_, kb_, vb_ = (random_bf16(330 + i, s) for i, s in enumerate([(B, Nq, S, D), (B, Nkv, S, D), (B, Nkv, S, D)]))
    keep_np = make_block_keep(333, B, Nq, QB, QB, 0.3)
    keep = torch.from_numpy(keep_np).cuda()
    q, k, v = dev_bf16(qb_), dev_bf16(kb_), dev_bf16(vb_)
    counts, idx = qa.build_kv_block_list(keep)
    order = qa.build_qblock_order(counts)
    full = qa.attn_fwd_blocksparse(q, k, v, counts, idx, scale=0.09, qblock_order=order)
    torch.cuda.synchronize()
    o_np = full[0].float().cpu().numpy().astype(np.float64)
    m_np, l_np = to_np(full[1]), to_np(full[2])
    for h in range(Nq):   # GQA: q-head h reads kv-head h // 2
        ro, rm, rl = oracle.attention_block_sparse(f64(qb_[0, h]), f64(kb_[0, h // 2]), f64(vb_[0, h // 2]), 0.09,
                                                   keep_np[0, h])
        check_o(o_np[0, h], ro, O_TOL_BF16)
        check_ml(m_np[0, h], l_np[0, h], rm, rl)
    out = torch.full_like(full[0], 7.0)
    m = torch.full_like(full[1], 7.0)
    l = torch.full_like(full[2], 7.0)
    for hr in ((0, 2), (2, 4)):
        for qr in ((0, 3), (3, QB)):
            qa.attn_fwd_blocksparse(q, k, v, counts, idx, scale=0.09, qblock_order=order, head_range=hr,
                                    qblock_range=qr, out=out, softmax_max=m, softmax_sum=l)
            torch.cuda.synchronize()
    _same(full, (out, m, l))


@pytest.mark.parametrize("ordered", [False, True])
def test_bsa_ragged_item_count(qa, ordered):
    """350 items (5 heads of 70 q-blocks, the last one ragged): more than one chunk of 256 items
    over the 8 XCDs and not a multiple of it. Every row is written, and sampled q-blocks of every
    head match the oracle."""
    B, N, D = 1, 5, 128
    S = 70 * 128 - 37
    QB = (S + 127) // 128
    banner(f"BSA over {N * QB} items, S={S}, q-block order {ordered}")
    qb_, kb_, vb_ = (random_bf16(340 + i, (B, N, S, D)) for i in range(3))
    keep_np = make_block_keep(343, B, N, QB, QB, 0.1)
    q, k, v = dev_bf16(qb_), dev_bf16(kb_), dev_bf16(vb_)
    counts, idx = qa.build_kv_block_list(torch.from_numpy(keep_np).cuda())
    order = qa.build_qblock_order(counts) if ordered else None
    out = torch.full((B, N, S, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    m = torch.full((B, N, S), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((B, N, S), float("nan"), dtype=torch.float32, device="cuda")
    qa.attn_fwd_blocksparse(q, k, v, counts, idx, scale=0.09, qblock_order=order, out=out, softmax_max=m,
                            softmax_sum=l)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any() and not torch.isnan(m).any() and not torch.isnan(l).any()
    o_np = out.float().cpu().numpy().astype(np.float64)
    m_np, l_np = to_np(m), to_np(l)
    sample = [0, 1, 33, QB - 2, QB - 1]
    rows = np.concatenate([np.arange(j * 128, min(S, (j + 1) * 128)) for j in sample])
    for h in range(N):
        ro, rm, rl = oracle.attention_block_sparse(f64(qb_[0, h]), f64(kb_[0, h]), f64(vb_[0, h]), 0.09,
                                                   keep_np[0, h], qblocks=sample)
        check_o(o_np[0, h][rows], ro, O_TOL_BF16)
        check_ml(m_np[0, h][rows], l_np[0, h][rows], rm, rl)
