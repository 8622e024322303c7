"""Launches with more work items than the GPU has CUs (each CU then runs several workgroups in
turn), checked two ways: sampled rows against the oracle, and bit identity with launches of one
head each (the fused-attention guide's operator computed over head chunks, as the power-cap page's
split launches do). Cases: ragged query and key lengths with GQA, head dimensions 64/96/128,
Dv < D and float16; rows that take the second key pass (a peaked Q); padded batches with rows and
whole work items of padding. Tolerances: O max-abs 1e-2, softmax max/sum relative 1e-3.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import O_TOL_BF16, banner, check_ml, check_o, dev_bf16, f64, to_np
from workloads import f32_to_bf16_bits, random_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _per_head(qa, q, k, v, scale, **kw):
    """The same problem as one launch per head (into one set of outputs)."""
    B, Nq, Sq = q.shape[:3]
    o = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=q.dtype, device=q.device)
    m = torch.empty((B, Nq, Sq), dtype=torch.float32, device=q.device)
    l = torch.empty_like(m)
    for h in range(Nq):
        qa.attn_fwd(q, k, v, scale=scale, head_range=(h, h + 1), out=o, softmax_max=m, softmax_sum=l, **kw)
    return o, m, l


def _same(a, b, what):
    for x, y, name in zip(a, b, ("O", "m", "l")):
        assert torch.equal(_bits(x), _bits(y)), f"{what}: {name} differs from the one-head launches"


def _rows(qbs, S):
    return np.concatenate([np.arange(qb * 128, min(S, qb * 128 + 128)) for qb in qbs])


@pytest.mark.parametrize("D,Dv,dtype", [(128, 128, "bf16"), (64, 64, "bf16"), (96, 96, "bf16"), (128, 64, "bf16"),
                                        (128, 128, "fp16")])
def test_many_items_against_oracle_and_one_head_launches(qa, D, Dv, dtype):
    B, Nq, Nkv, Sq, Skv = 2, 24, 4, 3000, 1500  # 2 x 24 x 12 q-block pairs = 576 items
    banner(f"many items D={D} Dv={Dv} {dtype}")
    qb_, kb_, vb_ = (random_bf16(seed, shape) for seed, shape in
                     ((71, (B, Nq, Sq, D)), (72, (B, Nkv, Skv, D)), (73, (B, Nkv, Skv, Dv))))
    q, k, v = dev_bf16(qb_), dev_bf16(kb_), dev_bf16(vb_)
    if dtype == "fp16":
        q, k, v = q.half(), k.half(), v.half()  # bf16 values are exact in float16 at this scale
    scale = 1.0 / np.sqrt(D)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale)
    ref = _per_head(qa, q, k, v, scale)
    torch.cuda.synchronize()
    _same((o, m, l), ref, "many items")
    g = Nq // Nkv
    for b, h, qbs in ((0, 0, [0, 11, 23]), (1, 13, [1, 22]), (1, 23, [12, 23])):
        rows = _rows(qbs, Sq)
        ro, rm, rl = oracle.attention_rows(f64(qb_[b, h]), f64(kb_[b, h // g]), f64(vb_[b, h // g]), scale, rows)
        check_o(to_np(o[b, h, rows]), ro, O_TOL_BF16, f"b{b} h{h}")
        check_ml(to_np(m[b, h, rows]), to_np(l[b, h, rows]), rm, rl, what=f"b{b} h{h}")


def test_many_items_second_pass(qa):
    """Rows whose scores grow, after their first keys, far beyond the reference maximum the kernel
    fixes there (spiked rows of the even heads see a few spiked keys: about 2^190 in p) take the
    second key pass."""
    B, Nq, S, D = 1, 40, 2048, 128  # 40 x 8 = 320 items
    banner("many items second pass")
    rng = np.random.default_rng(321)
    q = rng.standard_normal((B, Nq, S, D)) * 0.2
    k = rng.standard_normal((B, Nq, S, D)) * 0.2
    v = rng.standard_normal((B, Nq, S, D))
    k[..., :2] = 0.0                 # channel 0 carries only the spikes
    q[:, ::2, 1000:1040, 0] = 12.0   # these rows score about 132 on keys 900..909
    k[:, ::2, 900:910, 0] = 11.0
    qb_, kb_, vb_ = (f32_to_bf16_bits(a.astype(np.float32)) for a in (q, k, v))
    q, k, v = dev_bf16(qb_), dev_bf16(kb_), dev_bf16(vb_)
    o, m, l = qa.attn_fwd(q, k, v, scale=1.0)
    ref = _per_head(qa, q, k, v, 1.0)
    torch.cuda.synchronize()
    _same((o, m, l), ref, "second pass")
    for h, qbs in ((0, [7, 8, 15]), (1, [7]), (38, [0, 7])):
        rows = _rows(qbs, S)
        ro, rm, rl = oracle.attention_rows(f64(qb_[0, h]), f64(kb_[0, h]), f64(vb_[0, h]), 1.0, rows)
        check_o(to_np(o[0, h, rows]), ro, O_TOL_BF16, f"h{h}")
        check_ml(to_np(m[0, h, rows]), to_np(l[0, h, rows]), rm, rl, what=f"h{h}")


def test_many_items_padded_batches(qa):
    """Per-batch actual lengths: items whose rows are all padding (no tiles), items of one key,
    ragged ends; padded rows come out as rows with no key."""
    B, Nq, S, D = 6, 16, 2048, 128  # 6 x 16 x 8 = 768 items
    aq = [2048, 1, 0, 1000, 2047, 300]
    akv = [2048, 70, 0, 1999, 1, 512]
    banner(f"many items padded batches aq={aq} akv={akv}")
    qb_, kb_, vb_ = (random_bf16(90 + i, (B, Nq, S, D)) for i in range(3))
    q, k, v = dev_bf16(qb_), dev_bf16(kb_), dev_bf16(vb_)
    scale = 1.0 / np.sqrt(D)
    kw = dict(actual_seq_lengths=aq, actual_seq_lengths_kv=akv)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, **kw)
    ref = _per_head(qa, q, k, v, scale, **kw)
    torch.cuda.synchronize()
    _same((o, m, l), ref, "padded batches")
    on, mn, ln = to_np(o), to_np(m), to_np(l)
    for b in range(B):
        pad = slice(aq[b], S)
        assert np.all(on[b, :, pad] == 0) and np.all(np.isneginf(mn[b, :, pad])) and np.all(ln[b, :, pad] == 0)
        if aq[b] == 0:
            continue
        h = (5 * b + 3) % Nq
        rows = _rows(sorted({0, (aq[b] - 1) // 128}), aq[b])
        ro, rm, rl = oracle.attention_rows(f64(qb_[b, h, :aq[b]]), f64(kb_[b, h, :akv[b]]), f64(vb_[b, h, :akv[b]]),
                                           scale, rows)
        check_o(on[b, h, rows], ro, O_TOL_BF16, f"b{b} h{h}")
        check_ml(mn[b, h, rows], ln[b, h, rows], rm, rl, what=f"b{b} h{h}")
