"""GPU tests of the backward over head subranges (whole groups of q-heads that share kv-heads).

A launch over q-heads [h0, h1), h0 and h1 multiples of Nq / Nkv, writes dQ of those q-heads and
dK, dV of kv-heads [h0 / g, h1 / g), and nothing else. Run chunk by chunk over the heads, it must
reproduce the full call bit for bit: each work item's arithmetic does not depend on which heads
the launch holds. Outputs start filled with a sentinel to show which heads a launch writes.
"""

import numpy as np
import pytest
import torch

from gpu_util import banner, dev_bf16
from workloads import random_bf16

pytestmark = pytest.mark.gpu

SENTINEL = 0x7BAD


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _sentinel(like):
    return torch.full(like.shape, SENTINEL, dtype=torch.int16, device=like.device).view(like.dtype)


def _bits(t):
    return t.view(torch.int16)


def _chunked(qa, chunks, head_axis, kv_axis, group, args, kw):
    """Backward over each head chunk in turn into sentinel-filled outputs; checks after each chunk
    that exactly the chunk's heads (and their kv-heads) have been written so far."""
    q, k, v = args[0], args[1], args[2]
    dq, dk, dv = _sentinel(q), _sentinel(k), _sentinel(v)
    done_q = []
    for h0, h1 in chunks:
        qa.attn_bwd(*args, dq=dq, dk=dk, dv=dv, head_range=(h0, h1), workspace=None, **kw)
        torch.cuda.synchronize()
        done_q += list(range(h0, h1))
        for h in range(q.shape[head_axis]):
            untouched = bool(torch.all(_bits(dq.select(head_axis, h)) == SENTINEL))
            assert untouched == (h not in done_q), f"dq head {h} after chunk [{h0}, {h1})"
        for g in range(k.shape[kv_axis]):
            for t in (dk, dv):
                untouched = bool(torch.all(_bits(t.select(kv_axis, g)) == SENTINEL))
                assert untouched == (g * group not in done_q), f"dk/dv kv-head {g} after chunk [{h0}, {h1})"
    return dq, dk, dv


@pytest.mark.parametrize("B,Nq,Nkv,S,D,Dv,mode,chunks", [
    (2, 8, 4, 300, 128, 128, 3, [(0, 2), (2, 6), (6, 8)]),
    (1, 8, 2, 330, 128, 64, 0, [(4, 8), (0, 4)]),       # Dv < D, chunks out of order
    (1, 4, 4, 200, 64, 64, 2, [(0, 1), (1, 2), (2, 3), (3, 4)]),  # one head per chunk (no GQA)
])
def test_backward_head_chunks_match_full(qa, B, Nq, Nkv, S, D, Dv, mode, chunks):
    what = f"bwd head chunks B={B} Nq={Nq} Nkv={Nkv} S={S} D={D} Dv={Dv} mode={mode} {chunks}"
    banner(what)
    seed = 2100 + D + Dv + mode
    q, k = dev_bf16(random_bf16(seed, (B, Nq, S, D))), dev_bf16(random_bf16(seed + 1, (B, Nkv, S, D)))
    v, do = dev_bf16(random_bf16(seed + 2, (B, Nkv, S, Dv))), dev_bf16(random_bf16(seed + 3, (B, Nq, S, Dv)))
    scale = 1.0 / np.sqrt(D)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, sparse_mode=mode)
    full = qa.attn_bwd(q, k, v, o, do, m, l, scale=scale, sparse_mode=mode)
    torch.cuda.synchronize()
    parts = _chunked(qa, chunks, 1, 1, Nq // Nkv, (q, k, v, o, do, m, l), dict(scale=scale, sparse_mode=mode))
    for a, b in zip(full, parts):
        assert torch.equal(_bits(a), _bits(b)), what


def test_backward_head_chunks_tnd(qa):
    """Varlen TND (heads are the middle axis), GQA 2, bottom-right causal."""
    lq, lk = [300, 1, 130, 64], [280, 40, 130, 200]
    cq, ck = np.concatenate([[0], np.cumsum(lq)]).tolist(), np.concatenate([[0], np.cumsum(lk)]).tolist()
    Nq, Nkv, D = 4, 2, 128
    banner("bwd head chunks TND")
    q, k = dev_bf16(random_bf16(2201, (cq[-1], Nq, D))), dev_bf16(random_bf16(2202, (ck[-1], Nkv, D)))
    v, do = dev_bf16(random_bf16(2203, (ck[-1], Nkv, D))), dev_bf16(random_bf16(2204, (cq[-1], Nq, D)))
    kw = dict(scale=1.0 / np.sqrt(D), sparse_mode=3, layout="TND", cu_seqlens_q=cq, cu_seqlens_kv=ck)
    o, m, l = qa.attn_fwd(q, k, v, **kw)
    full = qa.attn_bwd(q, k, v, o, do, m, l, **kw)
    torch.cuda.synchronize()
    parts = _chunked(qa, [(2, 4), (0, 2)], 1, 1, Nq // Nkv, (q, k, v, o, do, m, l), kw)
    for a, b in zip(full, parts):
        assert torch.equal(_bits(a), _bits(b))


def test_backward_head_chunks_mask_and_actual_lengths(qa):
    """A per-head (BNSS) boolean mask, whose head offset moves with the chunk, and per-batch actual
    lengths, whose batches run in groups: chunked equals full."""
    B, Nq, Nkv, Sq, Skv, D = 3, 4, 2, 260, 230, 128
    aq, akv = [260, 129, 7], [230, 77, 40]
    banner("bwd head chunks BNSS mask + actual lengths")
    q, k = dev_bf16(random_bf16(2301, (B, Nq, Sq, D))), dev_bf16(random_bf16(2302, (B, Nkv, Skv, D)))
    v, do = dev_bf16(random_bf16(2303, (B, Nkv, Skv, D))), dev_bf16(random_bf16(2304, (B, Nq, Sq, D)))
    mask = torch.from_numpy((np.random.default_rng(2305).random((B, Nq, Sq, Skv)) < 0.3).astype(np.uint8)).cuda()
    kw = dict(scale=0.09, sparse_mode=2, atten_mask=mask, actual_seq_lengths=aq, actual_seq_lengths_kv=akv)
    o, m, l = qa.attn_fwd(q, k, v, **kw)
    full = qa.attn_bwd(q, k, v, o, do, m, l, **kw)
    torch.cuda.synchronize()
    parts = _chunked(qa, [(0, 2), (2, 4)], 1, 1, Nq // Nkv, (q, k, v, o, do, m, l), kw)
    for a, b in zip(full, parts):
        assert torch.equal(_bits(a), _bits(b))


def test_backward_head_range_rejected(qa):
    """Head ranges that split a group of q-heads sharing a kv-head, and q-block ranges, are refused."""
    from quantized_attention_tiled_amd import QattnError
    q = dev_bf16(random_bf16(2401, (1, 4, 128, 64)))
    k = dev_bf16(random_bf16(2402, (1, 2, 128, 64)))
    o, m, l = qa.attn_fwd(q, k, k)
    for hr in ((1, 3), (0, 1)):
        with pytest.raises(QattnError, match="UNSUPPORTED"):
            qa.attn_bwd(q, k, k, o, o, m, l, head_range=hr)
