"""GPU parity of the bf16 attention forward (dense, causal, masks, TND, GQA,
block-sparse) against the float64 oracle, element by element.

Tolerances: O max-abs <= 1e-2; softmax max/sum relative <= 1e-3 (with
|m| floored at 1); rows with no kept key must be exactly O = 0, m = -inf, l = 0.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import O_TOL_BF16, banner, check_ml, check_o, dev_bf16, f64, to_np
from workloads import bf16_bits_to_f32, make_block_keep, make_workload, random_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _bnsd(seed, B, Nq, Nkv, Sq, Skv, D, recipe="normal"):
    q = random_bf16(seed, (B, Nq, Sq, D), recipe)
    k = random_bf16(seed + 1, (B, Nkv, Skv, D), recipe)
    v = random_bf16(seed + 2, (B, Nkv, Skv, D), recipe)
    return q, k, v


def test_c1_dense_small(qa):
    w = make_workload("c1_dense_small")
    banner(f"c1 {w.q.shape}")
    o, m, l = qa.attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), scale=w.scale)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(w.q), f64(w.k), f64(w.v), w.scale)
    check_o(to_np(o), ro, O_TOL_BF16)
    check_ml(to_np(m), to_np(l), rm, rl)


@pytest.mark.parametrize("B,Nq,Nkv,Sq,Skv,D,mode", [
    (1, 2, 2, 256, 256, 64, 0),
    (2, 4, 2, 300, 300, 128, 0),      # ragged q and kv tails, GQA 2
    (1, 4, 1, 200, 333, 64, 0),       # Sq != Skv, GQA 4
    (1, 8, 1, 130, 130, 128, 0),      # GQA 8
    (1, 2, 2, 384, 384, 128, 2),
    (2, 4, 2, 300, 300, 64, 2),
    (1, 2, 1, 200, 450, 128, 3),      # bottom-right with Skv > Sq
    (1, 2, 2, 450, 200, 128, 3),      # bottom-right with Sq > Skv: leading rows see no key
    (1, 2, 2, 450, 200, 64, 2),
    (1, 1, 1, 1, 1, 128, 0),
    (1, 1, 1, 5, 700, 64, 3),
])
def test_dense_and_causal(qa, B, Nq, Nkv, Sq, Skv, D, mode):
    banner(f"dense B={B} Nq={Nq} Nkv={Nkv} Sq={Sq} Skv={Skv} D={D} mode={mode}")
    q, k, v = _bnsd(100 + Sq + D + mode, B, Nq, Nkv, Sq, Skv, D)
    scale = 1.0 / np.sqrt(D)
    o, m, l = qa.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=scale, sparse_mode=mode)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(q), f64(k), f64(v), scale, sparse_mode=mode)
    check_o(to_np(o), ro, O_TOL_BF16)
    check_ml(to_np(m), to_np(l), rm, rl)


# Skv = 260: mask rows not 16-byte aligned, read per element from global memory; Skv = 272 (and
# 1024): aligned rows, staged in LDS beside the K tiles
@pytest.mark.parametrize("kind,mode,Skv", [("SS", 0, 260), ("B1SS", 0, 260), ("BNSS", 0, 260), ("SS", 2, 260),
                                           ("BNSS", 3, 260), ("SS", 0, 272), ("B1SS", 0, 272), ("BNSS", 0, 272),
                                           ("SS", 2, 272), ("BNSS", 3, 272), ("B1SS", 3, 1024)])
def test_boolean_masks(qa, kind, mode, Skv):
    B, Nq, Nkv, Sq, D = 2, 4, 2, 200, 128
    banner(f"mask {kind} mode={mode} Skv={Skv}")
    q, k, v = _bnsd(7 + mode, B, Nq, Nkv, Sq, Skv, D)
    rng = np.random.default_rng(5)
    shape = {"SS": (Sq, Skv), "B1SS": (B, 1, Sq, Skv), "BNSS": (B, Nq, Sq, Skv)}[kind]
    mask = (rng.random(shape) < 0.3).astype(np.uint8)
    mask[..., 17, :] = 1                                   # a fully masked row
    scale = 0.09
    o, m, l = qa.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=scale, sparse_mode=mode,
                          atten_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(q), f64(k), f64(v), scale, sparse_mode=mode, atten_mask=mask)
    check_o(to_np(o), ro, O_TOL_BF16)
    check_ml(to_np(m), to_np(l), rm, rl)
    assert np.all(to_np(o)[:, :, 17] == 0)


def pack_mask_bits(mask: np.ndarray) -> np.ndarray:
    """Bit-packed form of a uint8 mask: rows of ceil(Skv / 32) little-endian 32-bit words, key j
    in bit j % 32 of word j // 32 (numpy's little-endian packbits, padded to whole words)."""
    Skv = mask.shape[-1]
    W = (Skv + 31) // 32
    padded = np.zeros(mask.shape[:-1] + (32 * W,), dtype=np.uint8)
    padded[..., :Skv] = mask != 0
    return np.ascontiguousarray(np.packbits(padded, axis=-1, bitorder="little")).view("<i4")


# bit-packed masks: every shape and causal mode, ragged rows (Skv = 260: 9 words per row; 33: two
# words, the second one bit), checked against the oracle and bit for bit against the byte mask
@pytest.mark.parametrize("kind,mode,Skv,dt,Dv", [("SS", 0, 260, "bf16", 128), ("B1SS", 0, 260, "bf16", 128),
                                                ("BNSS", 0, 260, "bf16", 128), ("SS", 2, 260, "bf16", 128),
                                                ("BNSS", 3, 260, "bf16", 128), ("SS", 0, 1024, "bf16", 128),
                                                ("B1SS", 3, 1024, "bf16", 128), ("BNSS", 2, 272, "bf16", 128),
                                                ("SS", 0, 33, "bf16", 128), ("B1SS", 2, 300, "fp16", 64),
                                                ("SS", 3, 500, "bf16", 64)])
def test_bit_packed_masks(qa, kind, mode, Skv, dt, Dv):
    B, Nq, Nkv, Sq, D = 2, 4, 2, 200, 128
    banner(f"bit mask {kind} mode={mode} Skv={Skv} {dt} Dv={Dv}")
    q, k, v = _bnsd(70 + mode, B, Nq, Nkv, Sq, Skv, D)
    v = np.ascontiguousarray(v[..., :Dv])
    rng = np.random.default_rng(50 + Skv)
    shape = {"SS": (Sq, Skv), "B1SS": (B, 1, Sq, Skv), "BNSS": (B, Nq, Sq, Skv)}[kind]
    mask = (rng.random(shape) < 0.3).astype(np.uint8)
    mask[..., 17, :] = 1                                   # a fully masked row
    mask[..., 40, :] = 0                                   # and an unmasked one
    words = pack_mask_bits(mask)
    up = (lambda x: dev_bf16(x)) if dt == "bf16" else \
        (lambda x: torch.from_numpy(bf16_bits_to_f32(x).astype(np.float16)).cuda())
    qd, kd, vd = up(q), up(k), up(v)
    scale = 0.09
    o, m, l = qa.attn_fwd(qd, kd, vd, scale=scale, sparse_mode=mode, atten_mask=torch.from_numpy(words).cuda())
    ob, mb, lb = qa.attn_fwd(qd, kd, vd, scale=scale, sparse_mode=mode, atten_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ob.view(torch.int16)), "bits and bytes masks differ"
    assert torch.equal(m, mb) and torch.equal(l, lb)
    unpacked = oracle.atten_mask_from_bits(words, Skv)
    assert np.array_equal(unpacked, mask)
    ro, rm, rl = oracle.attention(f64(q), f64(k), f64(v), scale, sparse_mode=mode, atten_mask=unpacked)
    check_o(o.float().cpu().numpy().astype(np.float64), ro, O_TOL_BF16)
    check_ml(to_np(m), to_np(l), rm, rl)
    assert np.all(o.float().cpu().numpy()[:, :, 17] == 0)


@pytest.mark.parametrize("lens_q,lens_kv,mode,Nq,Nkv,D", [
    ([1, 5, 130, 257], None, 3, 4, 2, 128),
    ([300, 0, 64, 129], None, 2, 2, 2, 64),
    ([100, 260], [300, 120], 3, 4, 1, 128),                 # kv longer / shorter than q per sequence
    ([128, 256, 384], None, 0, 2, 2, 128),
    ([3, 0, 7], [5, 9, 0], 3, 2, 2, 64),                     # empty q and empty kv sequences
])
def test_tnd_varlen(qa, lens_q, lens_kv, mode, Nq, Nkv, D):
    lens_kv = lens_q if lens_kv is None else lens_kv
    banner(f"tnd lens_q={lens_q} lens_kv={lens_kv} mode={mode}")
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lens_kv)]).astype(np.int32)
    q = random_bf16(31, (int(cq[-1]), Nq, D))
    k = random_bf16(32, (int(ck[-1]), Nkv, D))
    v = random_bf16(33, (int(ck[-1]), Nkv, D))
    scale = 1.0 / np.sqrt(D)
    o, m, l = qa.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=scale, layout="TND", sparse_mode=mode,
                          cu_seqlens_q=cq.tolist(), cu_seqlens_kv=ck.tolist())
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(q), f64(k), f64(v), scale, layout="TND", sparse_mode=mode,
                                  cu_seqlens_q=cq, cu_seqlens_kv=ck)
    check_o(to_np(o), ro, O_TOL_BF16)
    check_ml(to_np(m), to_np(l), rm, rl)


def test_varlen_config_scaled(qa):
    """The causal GQA varlen recipe at reduced lengths (full size is in the full-size tests)."""
    w = make_workload("c3_varlen_gqa_causal", lengths=[512, 700, 1029, 640])
    banner(f"c3-shaped T={w.Sq}")
    o, m, l = qa.attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), scale=w.scale, layout="TND",
                          sparse_mode=w.sparse_mode, cu_seqlens_q=w.cu_seqlens_q.tolist(),
                          cu_seqlens_kv=w.cu_seqlens_kv.tolist())
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(w.q), f64(w.k), f64(w.v), w.scale, layout="TND", sparse_mode=w.sparse_mode,
                                  cu_seqlens_q=w.cu_seqlens_q, cu_seqlens_kv=w.cu_seqlens_kv)
    check_o(to_np(o), ro, O_TOL_BF16)
    check_ml(to_np(m), to_np(l), rm, rl)


def test_block_list_bitexact(qa):
    keep = make_block_keep(77, 2, 3, 37, 70, 0.3)
    keep[0, 1, 5, :] = 0                                      # an empty row
    keep[1, 2, 6, :] = 1                                      # a full row
    counts, idx = qa.build_kv_block_list(torch.from_numpy(keep).cuda())
    torch.cuda.synchronize()
    rc, ri = oracle.kept_block_list(keep)
    assert np.array_equal(to_np(counts), rc) and np.array_equal(to_np(idx), ri)


@pytest.mark.parametrize("S,Nq,Nkv,D,p", [(640, 2, 2, 128, 0.3), (333, 4, 2, 64, 0.5), (1024, 2, 1, 128, 0.1)])
def test_blocksparse(qa, S, Nq, Nkv, D, p):
    banner(f"blocksparse S={S} Nq={Nq} Nkv={Nkv} D={D} p={p}")
    q, k, v = _bnsd(900 + S, 1, Nq, Nkv, S, S, D, recipe="block_offset")
    nb = (S + 127) // 128
    keep = make_block_keep(901, 1, Nq, nb, nb, p)
    keep[0, 0, 1, :] = 0                                      # q-block with no kept block
    scale = 1.0 / np.sqrt(D)
    counts, idx = qa.build_kv_block_list(torch.from_numpy(keep).cuda())
    o, m, l = qa.attn_fwd_blocksparse(dev_bf16(q), dev_bf16(k), dev_bf16(v), counts, idx, scale=scale)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(q), f64(k), f64(v), scale, block_keep=keep)
    check_o(to_np(o), ro, O_TOL_BF16)
    check_ml(to_np(m), to_np(l), rm, rl)


def test_blocksparse_all_kept_equals_dense(qa):
    S, D = 512, 128
    q, k, v = _bnsd(55, 1, 2, 2, S, S, D)
    keep = np.ones((1, 2, 4, 4), np.uint8)
    counts, idx = qa.build_kv_block_list(torch.from_numpy(keep).cuda())
    a = qa.attn_fwd_blocksparse(dev_bf16(q), dev_bf16(k), dev_bf16(v), counts, idx, scale=0.1)
    b = qa.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=0.1)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(q), f64(k), f64(v), 0.1)
    for out in (a, b):
        check_o(to_np(out[0]), ro, O_TOL_BF16)
        check_ml(to_np(out[1]), to_np(out[2]), rm, rl)


def test_deterministic(qa):
    q, k, v = _bnsd(66, 1, 4, 4, 1000, 1000, 128)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    a = qa.attn_fwd(dq, dk, dv, scale=0.1, sparse_mode=2)
    b = qa.attn_fwd(dq, dk, dv, scale=0.1, sparse_mode=2)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y.view(torch.int32))


# ---- the other batched layouts of the fused attention guide (section 4.1): BSND, BSH, SBH ----

def _to_layout(x, layout):
    """BNSD [B, N, S, D] device tensor -> the same values in `layout`."""
    B, N, S, D = x.shape
    if layout == "BSND":
        return x.permute(0, 2, 1, 3).contiguous()
    if layout == "BSH":
        return x.permute(0, 2, 1, 3).reshape(B, S, N * D).contiguous()
    return x.permute(2, 0, 1, 3).reshape(S, B, N * D).contiguous()  # SBH


def _from_layout(x, layout, B, N, S, D):
    if layout == "BSND":
        return x.permute(0, 2, 1, 3)
    if layout == "BSH":
        return x.reshape(B, S, N, D).permute(0, 2, 1, 3)
    return x.reshape(S, B, N, D).permute(1, 2, 0, 3)


def _bits(x):
    return x.contiguous().view(torch.int16) if x.dtype == torch.bfloat16 else x.contiguous().view(torch.int32)


@pytest.mark.parametrize("layout", ["BSND", "BSH", "SBH"])
@pytest.mark.parametrize("mode,masked,D", [(0, False, 128), (3, False, 128), (0, True, 64), (2, False, 64)])
def test_layouts_match_bnsd(qa, layout, mode, masked, D):
    """A row's arithmetic does not depend on the strides, so every layout reproduces the BNSD call
    bit for bit (O, softmax_max, softmax_sum)."""
    B, Nq, Nkv, S = 2, 4, 2, 300
    banner(f"layout {layout} mode={mode} masked={masked} D={D}")
    q, k, v = (dev_bf16(x) for x in _bnsd(500 + D + mode, B, Nq, Nkv, S, S, D))
    mask = None
    if masked:
        g = torch.Generator(device="cuda").manual_seed(9)
        mask = (torch.rand((B, 1, S, S), generator=g, device="cuda") < 0.25).to(torch.uint8)
    ref = qa.attn_fwd(q, k, v, scale=0.125, sparse_mode=mode, atten_mask=mask)
    hn = Nq if layout in ("BSH", "SBH") else None
    out = qa.attn_fwd(_to_layout(q, layout), _to_layout(k, layout), _to_layout(v, layout), scale=0.125,
                      sparse_mode=mode, atten_mask=mask, layout=layout, head_num=hn)
    torch.cuda.synchronize()
    assert torch.equal(_bits(_from_layout(out[0], layout, B, Nq, S, D)), _bits(ref[0]))
    assert torch.equal(_bits(out[1]), _bits(ref[1])) and torch.equal(_bits(out[2]), _bits(ref[2]))


def test_bsnd_against_oracle(qa):
    B, Nq, Nkv, S, D = 1, 4, 2, 400, 128
    q, k, v = _bnsd(601, B, Nq, Nkv, S, S, D)
    o, m, l = qa.attn_fwd(_to_layout(dev_bf16(q), "BSND"), _to_layout(dev_bf16(k), "BSND"),
                          _to_layout(dev_bf16(v), "BSND"), scale=0.09, sparse_mode=3, layout="BSND")
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(q), f64(k), f64(v), 0.09, sparse_mode=3)
    check_o(to_np(_from_layout(o, "BSND", B, Nq, S, D).contiguous()), ro, O_TOL_BF16)
    check_ml(to_np(m), to_np(l), rm, rl)


@pytest.mark.parametrize("layout", ["BSND", "SBH"])
def test_blocksparse_layouts_match_bnsd(qa, layout):
    B, Nq, Nkv, S, D = 1, 4, 2, 640, 128
    q, k, v = (dev_bf16(x) for x in _bnsd(700, B, Nq, Nkv, S, S, D))
    nb = (S + 127) // 128
    keep = torch.from_numpy(make_block_keep(701, B, Nq, nb, nb, 0.4)).cuda()
    counts, idx = qa.build_kv_block_list(keep)
    ref = qa.attn_fwd_blocksparse(q, k, v, counts, idx, scale=0.1)
    hn = Nq if layout == "SBH" else None
    out = qa.attn_fwd_blocksparse(_to_layout(q, layout), _to_layout(k, layout), _to_layout(v, layout), counts, idx,
                                  scale=0.1, layout=layout, head_num=hn)
    torch.cuda.synchronize()
    assert torch.equal(_bits(_from_layout(out[0], layout, B, Nq, S, D)), _bits(ref[0]))
    assert torch.equal(_bits(out[1]), _bits(ref[1])) and torch.equal(_bits(out[2]), _bits(ref[2]))


# ---- the sparse_mode 0 range: pre_tokens / next_tokens (fused attention guide, section 4.3) ----

@pytest.mark.parametrize("B,Nq,Nkv,Sq,Skv,D,pre,nxt", [
    (1, 2, 2, 512, 512, 128, 100, 0),       # sliding window ending at the diagonal
    (2, 4, 2, 300, 300, 64, 64, 64),        # symmetric band, ragged tails, GQA 2
    (1, 2, 1, 700, 450, 128, 130, 200),     # Sq > Skv
    (1, 2, 2, 260, 900, 128, 0, 300),       # only keys at or after the diagonal
    (1, 2, 2, 640, 640, 64, 2147483647, 31),
    (1, 2, 2, 640, 640, 128, 300, -40),     # band strictly below the diagonal
    (1, 1, 1, 400, 400, 128, -10, 5),       # narrow band strictly above it
    (1, 1, 1, 300, 300, 128, -20, 10),      # empty band: every row fully masked
])
def test_band(qa, B, Nq, Nkv, Sq, Skv, D, pre, nxt):
    banner(f"band B={B} Nq={Nq} Nkv={Nkv} Sq={Sq} Skv={Skv} D={D} pre={pre} next={nxt}")
    q, k, v = _bnsd(800 + Sq + D, B, Nq, Nkv, Sq, Skv, D)
    scale = 1.0 / np.sqrt(D)
    o, m, l = qa.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=scale, pre_tokens=pre, next_tokens=nxt)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(q), f64(k), f64(v), scale, pre_tokens=pre, next_tokens=nxt)
    check_o(to_np(o), ro, O_TOL_BF16)
    check_ml(to_np(m), to_np(l), rm, rl)


def test_band_with_boolean_mask_and_tnd(qa):
    B, Nq, Nkv, S, D = 2, 2, 2, 333, 128
    q, k, v = _bnsd(901, B, Nq, Nkv, S, S, D)
    mask = (np.random.default_rng(902).random((B, 1, S, S)) < 0.3).astype(np.uint8)
    o, m, l = qa.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=0.1, atten_mask=torch.from_numpy(mask).cuda(),
                          pre_tokens=90, next_tokens=20)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(q), f64(k), f64(v), 0.1, atten_mask=mask, pre_tokens=90, next_tokens=20)
    check_o(to_np(o), ro, O_TOL_BF16)
    check_ml(to_np(m), to_np(l), rm, rl)
    lens = [300, 5, 700, 130]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    qt = random_bf16(903, (T, 4, D))
    kt = random_bf16(904, (T, 2, D))
    vt = random_bf16(905, (T, 2, D))
    o, m, l = qa.attn_fwd(dev_bf16(qt), dev_bf16(kt), dev_bf16(vt), scale=0.1, layout="TND", cu_seqlens_q=cu.tolist(),
                          pre_tokens=150, next_tokens=0)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(qt), f64(kt), f64(vt), 0.1, layout="TND", cu_seqlens_q=cu, cu_seqlens_kv=cu,
                                  pre_tokens=150, next_tokens=0)
    check_o(to_np(o), ro, O_TOL_BF16)
    check_ml(to_np(m), to_np(l), rm, rl)
