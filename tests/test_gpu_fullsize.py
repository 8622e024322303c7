"""Parity at the five workloads' full sizes, in the launch configuration the
benchmark times (one call over all heads and q-blocks). The oracle computes
sampled rows one by one: whole q-blocks of a few heads, chosen to include the
first, last and interior blocks. The backward at C2 and C3 size is checked on
whole heads (C2) or a whole GQA group (C3), whose gradients do not depend on
the other heads.

Tolerances as in the other GPU tests: bf16 O max-abs 1e-2; quantised O max-abs
3e-2 in units of each V channel's RMS; softmax max/sum relative 1e-3;
quantisation codes, scales and the kept list bit-exact on sampled heads.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (O_TOL_BF16, O_TOL_QUANT, banner, check_ml, check_o, check_o_channel_scaled, dev_bf16, f64,
                      to_np)
from workloads import f32_to_bf16_bits, make_workload

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _rows_of(qbs, S):
    return np.concatenate([np.arange(qb * 128, min(S, qb * 128 + 128)) for qb in qbs])


def test_c2_dense_8k_full(qa):
    w = make_workload("c2_dense_8k")
    banner(f"c2 full {w.q.shape}")
    o, m, l = qa.attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), scale=w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    for h in (0, 17, 39):
        qbs = [0, 31, 63] if h != 17 else [5, 40]
        rows = _rows_of(qbs, w.Sq)
        ro, rm, rl = oracle.attention_rows(f64(w.q[0, h]), f64(w.k[0, h]), f64(w.v[0, h]), w.scale, rows)
        check_o(to_np(o[0, h, rows]), ro, O_TOL_BF16, f"c2 h{h}")
        check_ml(to_np(m[0, h, rows]), to_np(l[0, h, rows]), rm, rl, what=f"c2 h{h}")


def test_dense_64k_sampled(qa):
    """Dense attention at the long end of the 8K-64K range the throughput target spans (S = 65536,
    the C2 recipe with 8 heads: every work item is the one of the 40-head launch), sampled
    q-blocks against the oracle."""
    w = make_workload("c2_dense_8k", S=65536, N=8)
    banner(f"dense 64k {w.q.shape}")
    o, m, l = qa.attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), scale=w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    for h, qbs in ((0, [0, 511]), (5, [257])):
        rows = _rows_of(qbs, w.Sq)
        ro, rm, rl = oracle.attention_rows(f64(w.q[0, h]), f64(w.k[0, h]), f64(w.v[0, h]), w.scale, rows)
        check_o(to_np(o[0, h, rows]), ro, O_TOL_BF16, f"dense64k h{h}")
        check_ml(to_np(m[0, h, rows]), to_np(l[0, h, rows]), rm, rl, what=f"dense64k h{h}")


def test_c3_varlen_full(qa):
    w = make_workload("c3_varlen_gqa_causal")
    banner(f"c3 full T={w.Sq} lens={np.diff(w.cu_seqlens_q).tolist()}")
    o, m, l = qa.attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), scale=w.scale, layout="TND",
                          sparse_mode=w.sparse_mode, cu_seqlens_q=w.cu_seqlens_q.tolist(),
                          cu_seqlens_kv=w.cu_seqlens_kv.tolist())
    torch.cuda.synchronize()
    cu = w.cu_seqlens_q
    g = w.Nq // w.Nkv
    for b in range(w.B):
        L = int(cu[b + 1] - cu[b])
        nqb = (L + 127) // 128
        for h in ((b * 5) % w.Nq, (b * 11 + 7) % w.Nq):
            qbs = sorted({0, nqb // 2, nqb - 1})
            rows = _rows_of(qbs, L)
            s0, s1 = int(cu[b]), int(cu[b + 1])
            ro, rm, rl = oracle.attention_rows(f64(w.q[s0:s1, h]), f64(w.k[s0:s1, h // g]), f64(w.v[s0:s1, h // g]),
                                               w.scale, rows, sparse_mode=w.sparse_mode)
            check_o(to_np(o[s0 + rows, h]), ro, O_TOL_BF16, f"c3 seq{b} h{h}")
            check_ml(to_np(m[h, s0 + rows]), to_np(l[h, s0 + rows]), rm, rl, what=f"c3 seq{b} h{h}")


def test_c4_blocksparse_64k_full(qa):
    w = make_workload("c4_blocksparse_64k")
    banner(f"c4 full {w.q.shape} kept fraction {w.keep.mean():.4f}")
    keep = torch.from_numpy(w.keep).cuda()
    counts, idx = qa.build_kv_block_list(keep)
    o, m, l = qa.attn_fwd_blocksparse(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), counts, idx, scale=w.scale)
    torch.cuda.synchronize()
    for h in (0, 23, 39):
        rc, ri = oracle.kept_block_list(w.keep[:, h:h + 1])
        assert np.array_equal(to_np(counts[:, h:h + 1]), rc) and np.array_equal(to_np(idx[:, h:h + 1]), ri)
        qbs = [0, 255, 511] if h != 23 else [100, 400]
        ro, rm, rl = oracle.attention_block_sparse(f64(w.q[0, h]), f64(w.k[0, h]), f64(w.v[0, h]), w.scale,
                                                   w.keep[0, h], qblocks=qbs)
        rows = _rows_of(qbs, w.Sq)
        check_o(to_np(o[0, h, rows]), ro, O_TOL_BF16, f"c4 h{h}")
        check_ml(to_np(m[0, h, rows]), to_np(l[0, h, rows]), rm, rl, what=f"c4 h{h}")


def test_c5_qbsa_60k_full(qa):
    w = make_workload("c5_qbsa_60k")
    banner(f"c5 full {w.q.shape} kept fraction {w.keep.mean():.4f}")
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    qq, qs = qa.quantize_qk_perblock_int8(q)
    kq, ks = qa.quantize_qk_perblock_int8(k)
    vq, vs = qa.quantize_v_perchannel_fp8(v)
    counts, idx = qa.build_kv_block_list(torch.from_numpy(w.keep).cuda())
    o, m, l = qa.attn_fwd_qbsa(qq, kq, vq, qs, ks, vs, counts, idx, scale=w.scale)
    torch.cuda.synchronize()
    for h in (0, 31):
        rqc, rqs = oracle.quantize_qk_perblock_int8(f64(w.q[:, h:h + 1]))
        rkc, rks = oracle.quantize_qk_perblock_int8(f64(w.k[:, h:h + 1]))
        rvc, rvs = oracle.quantize_v_perchannel_fp8(f64(w.v[:, h:h + 1]))
        assert np.array_equal(to_np(qq[:, h:h + 1]), rqc) and np.array_equal(to_np(qs[:, h:h + 1]).view(np.uint32),
                                                                            rqs.view(np.uint32))
        assert np.array_equal(to_np(kq[:, h:h + 1]), rkc) and np.array_equal(to_np(ks[:, h:h + 1]).view(np.uint32),
                                                                            rks.view(np.uint32))
        assert np.array_equal(to_np(vq[:, h:h + 1]), rvc) and np.array_equal(to_np(vs[:, h:h + 1]).view(np.uint32),
                                                                            rvs.view(np.uint32))
        for qb in (0, 239, 479):
            oo, mm, ll = oracle.qbsa_qblock(rqc[0, 0], rkc[0, 0], rvc[0, 0], rqs[0, 0, qb], rks[0, 0], rvs[0, 0],
                                            w.scale, np.nonzero(w.keep[0, h, qb])[0], qb)
            rows = slice(qb * 128, qb * 128 + 128)
            check_o_channel_scaled(to_np(o[0, h, rows])[None, None], oo[None, None], f64(w.v[:, h:h + 1]),
                                   O_TOL_QUANT, f"c5 h{h} qb{qb}")
            check_ml(to_np(m[0, h, rows]), to_np(l[0, h, rows]), mm, ll, what=f"c5 h{h} qb{qb}")


def test_sweep_128k_sampled(qa):
    """The long end of the EagleQBSA article's operator sweep (Fig. 4.1: S up to 128K at N = 40,
    D = 128): dense, block-sparse (sparsity 0.9) and quantised block-sparse (sparsity 0.63) at
    S = 131072 on 2 heads. A row's arithmetic does not depend on how many heads a launch holds
    (the subrange tests check it bit for bit), so 2 heads at the full length are the work items of
    the 40-head sweep. Sampled q-blocks (first, interior, last) against the oracle."""
    S = 131072
    wd = make_workload("c2_dense_8k", S=S, N=2)
    banner(f"128k dense {wd.q.shape}")
    o, m, l = qa.attn_fwd(dev_bf16(wd.q), dev_bf16(wd.k), dev_bf16(wd.v), scale=wd.scale)
    torch.cuda.synchronize()
    for h, qbs in ((0, [0, 1023]), (1, [512])):
        rows = _rows_of(qbs, S)
        ro, rm, rl = oracle.attention_rows(f64(wd.q[0, h]), f64(wd.k[0, h]), f64(wd.v[0, h]), wd.scale, rows)
        check_o(to_np(o[0, h, rows]), ro, O_TOL_BF16, f"dense128k h{h}")
        check_ml(to_np(m[0, h, rows]), to_np(l[0, h, rows]), rm, rl, what=f"dense128k h{h}")
    del wd, o, m, l

    wb = make_workload("c4_blocksparse_64k", S=S, N=2)
    banner(f"128k block-sparse {wb.q.shape} kept fraction {wb.keep.mean():.4f}")
    counts, idx = qa.build_kv_block_list(torch.from_numpy(wb.keep).cuda())
    o, m, l = qa.attn_fwd_blocksparse(dev_bf16(wb.q), dev_bf16(wb.k), dev_bf16(wb.v), counts, idx, scale=wb.scale)
    torch.cuda.synchronize()
    for h, qbs in ((0, [0, 1023]), (1, [300, 777])):
        ro, rm, rl = oracle.attention_block_sparse(f64(wb.q[0, h]), f64(wb.k[0, h]), f64(wb.v[0, h]), wb.scale,
                                                   wb.keep[0, h], qblocks=qbs)
        rows = _rows_of(qbs, S)
        check_o(to_np(o[0, h, rows]), ro, O_TOL_BF16, f"bsa128k h{h}")
        check_ml(to_np(m[0, h, rows]), to_np(l[0, h, rows]), rm, rl, what=f"bsa128k h{h}")
    del wb, o, m, l, counts, idx

    wq = make_workload("c5_qbsa_60k", S=S, N=2)
    banner(f"128k quantised block-sparse {wq.q.shape} kept fraction {wq.keep.mean():.4f}")
    qq, qs = qa.quantize_qk_perblock_int8(dev_bf16(wq.q))
    kq, ks = qa.quantize_qk_perblock_int8(dev_bf16(wq.k))
    vq, vs = qa.quantize_v_perchannel_fp8(dev_bf16(wq.v))
    counts, idx = qa.build_kv_block_list(torch.from_numpy(wq.keep).cuda())
    o, m, l = qa.attn_fwd_qbsa(qq, kq, vq, qs, ks, vs, counts, idx, scale=wq.scale)
    torch.cuda.synchronize()
    for h in (0, 1):
        rqc, rqs = oracle.quantize_qk_perblock_int8(f64(wq.q[:, h:h + 1]))
        rkc, rks = oracle.quantize_qk_perblock_int8(f64(wq.k[:, h:h + 1]))
        rvc, rvs = oracle.quantize_v_perchannel_fp8(f64(wq.v[:, h:h + 1]))
        assert np.array_equal(to_np(qq[:, h:h + 1]), rqc) and np.array_equal(to_np(kq[:, h:h + 1]), rkc)
        assert np.array_equal(to_np(vq[:, h:h + 1]), rvc)
        assert np.array_equal(to_np(vs[:, h:h + 1]).view(np.uint32), rvs.view(np.uint32))
        for qb in ((0, 1023) if h == 0 else (640,)):
            oo, mm, ll = oracle.qbsa_qblock(rqc[0, 0], rkc[0, 0], rvc[0, 0], rqs[0, 0, qb], rks[0, 0], rvs[0, 0],
                                            wq.scale, np.nonzero(wq.keep[0, h, qb])[0], qb)
            rows = slice(qb * 128, qb * 128 + 128)
            check_o_channel_scaled(to_np(o[0, h, rows])[None, None], oo[None, None], f64(wq.v[:, h:h + 1]),
                                   O_TOL_QUANT, f"qbsa128k h{h} qb{qb}")
            check_ml(to_np(m[0, h, rows]), to_np(l[0, h, rows]), mm, ll, what=f"qbsa128k h{h} qb{qb}")


def _grad_check(g, ref, what, rtol=2e-2):
    """The backward tests' bound: max-abs error <= rtol * max(1, max |reference|)."""
    g = to_np(g).astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    bound = rtol * max(1.0, float(np.abs(ref).max()))
    err = float(np.abs(g - ref).max())
    banner(f"{what}: max-abs err {err:.3e} (bound {bound:.3e})")
    assert err <= bound, f"{what}: {err:.3e} > {bound:.3e}"


def test_c2_backward_full(qa):
    """The backward at C2's full size in the launch the backward benchmark times (all 40 heads in
    one call), against the oracle's full gradients of two heads (each head is its own problem)."""
    w = make_workload("c2_dense_8k")
    banner(f"c2 backward full {w.q.shape}")
    gb = f32_to_bf16_bits(np.random.default_rng(2024).standard_normal(w.q.shape, dtype=np.float32))
    q, k, v, do = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), dev_bf16(gb)
    o, m, l = qa.attn_fwd(q, k, v, scale=w.scale)
    dq, dk, dv = qa.attn_bwd(q, k, v, o, do, m, l, scale=w.scale)
    torch.cuda.synchronize()
    for h in (0, 39):
        sl = slice(h, h + 1)
        rq, rk, rv = oracle.attention_backward(f64(w.q[:, sl]), f64(w.k[:, sl]), f64(w.v[:, sl]), f64(gb[:, sl]),
                                               w.scale)
        _grad_check(dq[:, sl], rq, f"c2 bwd h{h} dQ")
        _grad_check(dk[:, sl], rk, f"c2 bwd h{h} dK")
        _grad_check(dv[:, sl], rv, f"c2 bwd h{h} dV")


def test_c3_backward_full(qa):
    """The backward at C3's full size (TND varlen, GQA 32/8, bottom-right causal) in one call;
    the oracle computes the gradients of kv-head 0's group (q-heads 0..3) over every sequence."""
    w = make_workload("c3_varlen_gqa_causal")
    banner(f"c3 backward full {w.q.shape}")
    gb = f32_to_bf16_bits(np.random.default_rng(2025).standard_normal(w.q.shape, dtype=np.float32))
    cu = w.cu_seqlens_q.tolist()
    kw = dict(scale=w.scale, layout="TND", sparse_mode=w.sparse_mode, cu_seqlens_q=cu, cu_seqlens_kv=cu)
    q, k, v, do = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), dev_bf16(gb)
    o, m, l = qa.attn_fwd(q, k, v, **kw)
    dq, dk, dv = qa.attn_bwd(q, k, v, o, do, m, l, **kw)
    torch.cuda.synchronize()
    g = w.Nq // w.Nkv
    rq, rk, rv = oracle.attention_backward(f64(w.q[:, :g]), f64(w.k[:, :1]), f64(w.v[:, :1]), f64(gb[:, :g]), w.scale,
                                           layout="TND", sparse_mode=w.sparse_mode, cu_seqlens_q=w.cu_seqlens_q,
                                           cu_seqlens_kv=w.cu_seqlens_kv)
    _grad_check(dq[:, :g], rq, "c3 bwd dQ (q-heads 0..3)")
    _grad_check(dk[:, :1], rk, "c3 bwd dK (kv-head 0)")
    _grad_check(dv[:, :1], rv, "c3 bwd dV (kv-head 0)")
