"""GPU parity of the quantisers (bit-exact codes and scales) and of the
quantised block-sparse attention against the oracle. The oracle quantises the
same bf16 inputs itself; nothing it uses comes from the GPU.

Quantised-attention tolerance: O max-abs <= 3e-2 in units of each V channel's
RMS (floored at 1), softmax max/sum relative <= 1e-3. The 3e-2 bound is stated
for N(0,1)-scale inputs, while these V tensors carry log-normal per-channel
scales; measuring each channel's error in its own scale is the same test on
N(0,1)-scale V. gfx950's FP8 MFMA sums each group of 16 products with
truncation to about 12 significant bits before the exact fp32 accumulation,
so its error grows with the channel's magnitude; the oracle is exact.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import O_TOL_QUANT, banner, check_ml, check_o_channel_scaled, dev_bf16, f64, to_np
from workloads import make_block_keep, make_workload, random_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


@pytest.mark.parametrize("B,N,S,D,recipe", [(1, 2, 256, 128, "block_offset"), (2, 3, 300, 64, "normal"),
                                            (1, 1, 1, 128, "normal"), (1, 2, 1000, 128, "block_offset")])
def test_quant_qk_bitexact(qa, B, N, S, D, recipe):
    banner(f"quant_qk B={B} N={N} S={S} D={D}")
    x = random_bf16(200 + S, (B, N, S, D), recipe)
    if S >= 256:
        x[0, 0, 128:256] = 0                                   # an all-zero block
    codes, scale = qa.quantize_qk_perblock_int8(dev_bf16(x))
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_qk_perblock_int8(f64(x))
    assert np.array_equal(to_np(scale).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(to_np(codes), rc)


@pytest.mark.parametrize("B,N,S,D", [(1, 2, 256, 128), (2, 3, 300, 64), (1, 1, 1, 128), (1, 2, 5000, 128)])
def test_quant_v_bitexact(qa, B, N, S, D):
    banner(f"quant_v B={B} N={N} S={S} D={D}")
    x = random_bf16(300 + S, (B, N, S, D))
    chan = np.exp(np.random.default_rng(S).normal(size=(B, N, 1, D))).astype(np.float32)
    from workloads import bf16_bits_to_f32, f32_to_bf16_bits
    x = f32_to_bf16_bits(bf16_bits_to_f32(x) * chan)
    x[0, 0, :, 3] = 0                                           # all-zero channel
    x[0, 0, 0, 5] = 0x8000                                      # -0.0
    codes, scale = qa.quantize_v_perchannel_fp8(dev_bf16(x))
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_v_perchannel_fp8(f64(x))
    assert np.array_equal(to_np(scale).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(to_np(codes), rc)


def _qbsa_case(qa, S, Nq, Nkv, D, p, seed):
    q = random_bf16(seed, (1, Nq, S, D), "block_offset")
    k = random_bf16(seed + 1, (1, Nkv, S, D), "block_offset")
    from workloads import bf16_bits_to_f32, f32_to_bf16_bits
    chan = np.exp(np.random.default_rng(seed).normal(size=(1, Nkv, 1, D))).astype(np.float32)
    v = f32_to_bf16_bits(bf16_bits_to_f32(random_bf16(seed + 2, (1, Nkv, S, D), "block_offset")) * chan)
    nb = (S + 127) // 128
    keep = make_block_keep(seed + 3, 1, Nq, nb, nb, p)
    return q, k, v, keep


@pytest.mark.parametrize("S,Nq,Nkv,D,p", [(512, 2, 2, 128, 0.37), (640, 4, 2, 128, 0.6), (300, 2, 1, 64, 0.5),
                                          (1024, 1, 1, 128, 1.0)])
def test_qbsa(qa, S, Nq, Nkv, D, p):
    banner(f"qbsa S={S} Nq={Nq} Nkv={Nkv} D={D} p={p}")
    q, k, v, keep = _qbsa_case(qa, S, Nq, Nkv, D, p, 400 + S)
    keep[0, 0, 1, :] = 0
    scale = 1.0 / np.sqrt(D)
    qq, qs = qa.quantize_qk_perblock_int8(dev_bf16(q))
    kq, ks = qa.quantize_qk_perblock_int8(dev_bf16(k))
    vq, vs = qa.quantize_v_perchannel_fp8(dev_bf16(v))
    counts, idx = qa.build_kv_block_list(torch.from_numpy(keep).cuda())
    o, m, l = qa.attn_fwd_qbsa(qq, kq, vq, qs, ks, vs, counts, idx, scale=scale)
    torch.cuda.synchronize()
    rqc, rqs = oracle.quantize_qk_perblock_int8(f64(q))
    rkc, rks = oracle.quantize_qk_perblock_int8(f64(k))
    rvc, rvs = oracle.quantize_v_perchannel_fp8(f64(v))
    res = oracle.qbsa_attention(rqc, rkc, rvc, rqs, rks, rvs, keep, scale)
    nb = keep.shape[2]
    ro = np.zeros((1, Nq, S, D))
    rm = np.zeros((1, Nq, S))
    rl = np.zeros((1, Nq, S))
    for h in range(Nq):
        for qb in range(nb):
            oo, mm, ll = res[(0, h, qb)]
            ro[0, h, qb * 128:qb * 128 + len(mm)] = oo
            rm[0, h, qb * 128:qb * 128 + len(mm)] = mm
            rl[0, h, qb * 128:qb * 128 + len(mm)] = ll
    check_o_channel_scaled(to_np(o), ro, f64(v), O_TOL_QUANT)
    check_ml(to_np(m), to_np(l), rm, rl)


def test_qbsa_without_softmax_outputs(qa):
    q, k, v, keep = _qbsa_case(qa, 256, 1, 1, 128, 1.0, 77)
    qq, qs = qa.quantize_qk_perblock_int8(dev_bf16(q))
    kq, ks = qa.quantize_qk_perblock_int8(dev_bf16(k))
    vq, vs = qa.quantize_v_perchannel_fp8(dev_bf16(v))
    counts, idx = qa.build_kv_block_list(torch.from_numpy(keep).cuda())
    o1, _, _ = qa.attn_fwd_qbsa(qq, kq, vq, qs, ks, vs, counts, idx, scale=0.1, return_softmax=False)
    o2, _, _ = qa.attn_fwd_qbsa(qq, kq, vq, qs, ks, vs, counts, idx, scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_c5_recipe_scaled(qa):
    """The quantised config's recipe at S = 2048, 2 heads."""
    w = make_workload("c5_qbsa_60k", S=2048, N=2)
    banner("c5-shaped S=2048")
    qq, qs = qa.quantize_qk_perblock_int8(dev_bf16(w.q))
    kq, ks = qa.quantize_qk_perblock_int8(dev_bf16(w.k))
    vq, vs = qa.quantize_v_perchannel_fp8(dev_bf16(w.v))
    counts, idx = qa.build_kv_block_list(torch.from_numpy(w.keep).cuda())
    o, m, l = qa.attn_fwd_qbsa(qq, kq, vq, qs, ks, vs, counts, idx, scale=w.scale)
    torch.cuda.synchronize()
    rqc, rqs = oracle.quantize_qk_perblock_int8(f64(w.q))
    rkc, rks = oracle.quantize_qk_perblock_int8(f64(w.k))
    rvc, rvs = oracle.quantize_v_perchannel_fp8(f64(w.v))
    assert np.array_equal(to_np(qq), rqc) and np.array_equal(to_np(kq), rkc) and np.array_equal(to_np(vq), rvc)
    for (h, qb) in [(0, 0), (0, 7), (1, 15), (1, 3)]:
        oo, mm, ll = oracle.qbsa_qblock(rqc[0, h], rkc[0, h], rvc[0, h], rqs[0, h, qb], rks[0, h], rvs[0, h], w.scale,
                                        np.nonzero(w.keep[0, h, qb])[0], qb)
        rows = slice(qb * 128, qb * 128 + 128)
        check_o_channel_scaled(to_np(o[0, h, rows])[None, None], oo[None, None], f64(w.v)[:, h:h + 1], O_TOL_QUANT)
        check_ml(to_np(m[0, h, rows]), to_np(l[0, h, rows]), mm, ll)
