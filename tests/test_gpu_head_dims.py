"""GPU parity of the 16-bit forward at head dimensions other than 64 and 128 (fused attention guide,
section 4.1: D_q = D_k >= D_v; section 7: head dimensions from 1 up to 768), against the float64
oracle, element by element.

The kernels are built for D = 64, 128 and 256 (value dimension 64 or 128). A problem's D and Dv,
multiples of 8, run on the next size up: the Q registers and the K/V tiles hold zeros past them,
and O is stored up to Dv. A value dimension above 128 runs as two launches, one per column range
of V and O. The oracle scores with the problem's own D, so a padded column that read anything but
zero would show; the BSND cases put NaN right after each computed head's row, where a padded chunk
would read. Tolerances as elsewhere: O max-abs 1e-2 (bf16) or 4e-3 (fp16), softmax max/sum
relative 1e-3, for N(0, 1) inputs with scale 1/sqrt(D) (the pages' setting; a larger scale makes
rows that one key dominates, where bf16 rounding of P and of |O| > 2 alone can pass 1e-2);
subrange launches bit for bit against the full call.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import O_TOL_BF16, banner, check_ml, check_o, dev_bf16, f64, to_np
from workloads import make_block_keep, random_bf16, random_f16

pytestmark = pytest.mark.gpu

O_TOL_F16 = 4e-3
NAN_BF16 = np.uint16(0x7FC0)


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _inputs(dtype, seed, shapes):
    """Device tensors of the given type and their float64 values for the oracle."""
    out = []
    for i, shape in enumerate(shapes):
        if dtype == "fp16":
            x = random_f16(seed + i, shape)
            out.append((torch.from_numpy(x).cuda(), x.astype(np.float64)))
        else:
            bits = random_bf16(seed + i, shape)
            out.append((dev_bf16(bits), f64(bits)))
    return out


def _check(dtype, o, m, l, ro, rm, rl, what):
    og = o.float().cpu().numpy().astype(np.float64)
    err = check_o(og, ro, O_TOL_F16 if dtype == "fp16" else O_TOL_BF16, what)
    banner(f"{what}: O max-abs err {err:.3e}")
    check_ml(to_np(m), to_np(l), rm, rl, what=what)


def _pack_bits(mask: np.ndarray) -> np.ndarray:
    """Rows of ceil(Skv / 32) little-endian 32-bit words, key j in bit j % 32 of word j // 32."""
    Skv = mask.shape[-1]
    padded = np.zeros(mask.shape[:-1] + (32 * ((Skv + 31) // 32),), dtype=np.uint8)
    padded[..., :Skv] = mask != 0
    return np.ascontiguousarray(np.packbits(padded, axis=-1, bitorder="little")).view("<i4")


# (dtype, D, Dv, sparse_mode): every kernel size (64, 128, 256), padded and exact, Dv < D within
# and across sizes, and Dv above 128 (two column launches)
_DIMS = [("bf16", 8, 8, 0), ("bf16", 40, 40, 2), ("bf16", 72, 72, 0), ("bf16", 80, 48, 3), ("bf16", 96, 96, 0),
         ("fp16", 96, 96, 2), ("bf16", 112, 64, 0), ("bf16", 120, 120, 3), ("bf16", 136, 136, 0),
         ("bf16", 160, 8, 2), ("bf16", 192, 128, 0), ("fp16", 192, 192, 3), ("bf16", 256, 256, 0),
         ("bf16", 256, 256, 2), ("bf16", 256, 200, 3), ("fp16", 256, 256, 0), ("bf16", 256, 64, 0),
         ("bf16", 256, 136, 2)]


@pytest.mark.parametrize("dtype,D,Dv,mode", _DIMS)
def test_dense_and_causal(qa, dtype, D, Dv, mode):
    B, Nq, Nkv, Sq, Skv = 2, 4, 2, 300, 333
    what = f"{dtype} D={D} Dv={Dv} mode={mode}"
    banner(what)
    (q, qr), (k, kr), (v, vr) = _inputs(dtype, 500 + D + Dv + mode,
                                        [(B, Nq, Sq, D), (B, Nkv, Skv, D), (B, Nkv, Skv, Dv)])
    scale = 1.0 / np.sqrt(D)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, sparse_mode=mode)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (B, Nq, Sq, Dv)
    ro, rm, rl = oracle.attention(qr, kr, vr, scale, sparse_mode=mode)
    _check(dtype, o, m, l, ro, rm, rl, what)


# byte masks staged in LDS (Skv = 320: rows of 320 bytes) and read per element (Skv = 333), bit
# masks, with a band or a causal mode
@pytest.mark.parametrize("D,Dv,kind,Skv,mode", [(96, 96, "bytes", 320, 0), (96, 56, "bytes", 333, 3),
                                                (96, 96, "bits", 333, 2), (256, 256, "bytes", 320, 2),
                                                (256, 256, "bytes", 333, 0), (200, 160, "bits", 333, 3)])
def test_masks(qa, D, Dv, kind, Skv, mode):
    B, Nq, Nkv, Sq = 2, 4, 2, 260
    what = f"mask {kind} D={D} Dv={Dv} Skv={Skv} mode={mode}"
    banner(what)
    (q, qr), (k, kr), (v, vr) = _inputs("bf16", 600 + D + Skv, [(B, Nq, Sq, D), (B, Nkv, Skv, D), (B, Nkv, Skv, Dv)])
    mask = (np.random.default_rng(D + Skv).random((B, 1, Sq, Skv)) < 0.3).astype(np.uint8)
    mask[..., 7, :] = 1  # a row with every key masked
    band = dict(pre_tokens=90, next_tokens=30) if mode == 0 else {}
    dmask = torch.from_numpy(_pack_bits(mask) if kind == "bits" else mask).cuda()
    scale = 1.0 / np.sqrt(D)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, sparse_mode=mode, atten_mask=dmask, **band)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(qr, kr, vr, scale, sparse_mode=mode, atten_mask=mask, **band)
    _check("bf16", o, m, l, ro, rm, rl, what)


@pytest.mark.parametrize("dtype,D,Dv,mode", [("bf16", 72, 40, 3), ("fp16", 104, 104, 0), ("bf16", 256, 256, 3),
                                             ("bf16", 176, 96, 2)])
def test_tnd(qa, dtype, D, Dv, mode):
    lens_q, lens_kv = [300, 1, 129, 64], [280, 40, 129, 500]
    cq = np.concatenate([[0], np.cumsum(lens_q)])
    ck = np.concatenate([[0], np.cumsum(lens_kv)])
    Nq, Nkv = 4, 2
    what = f"{dtype} TND D={D} Dv={Dv} mode={mode}"
    banner(what)
    (q, qr), (k, kr), (v, vr) = _inputs(dtype, 700 + D, [(cq[-1], Nq, D), (ck[-1], Nkv, D), (ck[-1], Nkv, Dv)])
    scale = 1.0 / np.sqrt(D)
    o, m, l = qa.attn_fwd(q, k, v, scale=scale, layout="TND", sparse_mode=mode, cu_seqlens_q=cq.tolist(),
                          cu_seqlens_kv=ck.tolist())
    torch.cuda.synchronize()
    assert tuple(o.shape) == (cq[-1], Nq, Dv)
    ro, rm, rl = oracle.attention(qr, kr, vr, scale, layout="TND", sparse_mode=mode, cu_seqlens_q=cq,
                                  cu_seqlens_kv=ck)
    _check(dtype, o, m, l, ro, rm, rl, what)


@pytest.mark.parametrize("dtype,D,Dv", [("bf16", 96, 96), ("bf16", 40, 24), ("fp16", 256, 256), ("bf16", 256, 128)])
def test_blocksparse(qa, dtype, D, Dv):
    B, Nq, Nkv, S = 1, 4, 2, 640
    QB = KB = (S + 127) // 128
    what = f"{dtype} block-sparse D={D} Dv={Dv}"
    banner(what)
    (q, qr), (k, kr), (v, vr) = _inputs(dtype, 800 + D, [(B, Nq, S, D), (B, Nkv, S, D), (B, Nkv, S, Dv)])
    keep = make_block_keep(61 + D, B, Nq, QB, KB, 0.4)
    counts, idx = qa.build_kv_block_list(torch.from_numpy(keep).cuda())
    scale = 1.0 / np.sqrt(D)
    o, m, l = qa.attn_fwd_blocksparse(q, k, v, counts, idx, scale=scale)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(qr, kr, vr, scale, block_keep=keep)
    _check(dtype, o, m, l, ro, rm, rl, what)


@pytest.mark.parametrize("D,Dv,mode", [(40, 40, 0), (96, 64, 2), (256, 256, 0), (232, 232, 3)])
def test_bsnd_neighbours_not_read(qa, D, Dv, mode):
    """BSND rows hold all heads of a token side by side, so the chunk after a head's last one is
    the next head's first. Heads outside the computed range (q-heads 2, 3 and kv-head 1) are NaN:
    a padded chunk read from there would turn the scores or the output NaN."""
    B, Nq, Nkv, S = 2, 4, 2, 300
    what = f"BSND neighbours D={D} Dv={Dv} mode={mode}"
    banner(what)
    qb, kb, vb = (random_bf16(900 + D + i, s) for i, s in
                  enumerate([(B, Nq, S, D), (B, Nkv, S, D), (B, Nkv, S, Dv)]))
    qb[:, 2:] = NAN_BF16
    kb[:, 1:] = NAN_BF16
    vb[:, 1:] = NAN_BF16
    q, k, v = (dev_bf16(x).transpose(1, 2).contiguous() for x in (qb, kb, vb))
    o = torch.zeros((B, S, Nq, Dv), dtype=torch.bfloat16, device="cuda")
    m = torch.zeros((B, Nq, S), device="cuda")
    l = torch.zeros((B, Nq, S), device="cuda")
    scale = 1.0 / np.sqrt(D)
    qa.attn_fwd(q, k, v, scale=scale, sparse_mode=mode, layout="BSND", head_range=(0, 2), out=o, softmax_max=m,
                softmax_sum=l)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attention(f64(qb[:, :2]), f64(kb[:, :1]), f64(vb[:, :1]), scale, sparse_mode=mode)
    og = o.transpose(1, 2)[:, :2].float().cpu().numpy().astype(np.float64)
    err = check_o(og, ro, O_TOL_BF16, what)
    banner(f"{what}: O max-abs err {err:.3e}")
    check_ml(to_np(m)[:, :2], to_np(l)[:, :2], rm, rl, what=what)
    assert torch.all(o[:, :, 2:] == 0)  # heads outside the range untouched


@pytest.mark.parametrize("D,Dv,mode", [(96, 96, 0), (96, 48, 3), (256, 256, 0), (256, 200, 2)])
def test_subranges_bitexact(qa, D, Dv, mode):
    B, Nq, Nkv, S = 1, 4, 2, 700
    banner(f"subranges D={D} Dv={Dv} mode={mode}")
    (q, _), (k, _), (v, _) = _inputs("bf16", 1000 + D, [(B, Nq, S, D), (B, Nkv, S, D), (B, Nkv, S, Dv)])
    full = qa.attn_fwd(q, k, v, scale=0.1, sparse_mode=mode)
    nqb = (S + 127) // 128
    for split in ([((h, h + 1), (0, nqb)) for h in range(Nq)], [((0, Nq), (i, i + 1)) for i in range(nqb)],
                  [((0, 2), (0, 3)), ((0, 2), (3, nqb)), ((2, Nq), (0, 1)), ((2, Nq), (1, nqb))]):
        out = tuple(torch.zeros_like(x) for x in full)
        for hr, br in split:
            qa.attn_fwd(q, k, v, scale=0.1, sparse_mode=mode, head_range=hr, qblock_range=br, out=out[0],
                        softmax_max=out[1], softmax_sum=out[2])
        torch.cuda.synchronize()
        assert torch.equal(full[0].view(torch.int16), out[0].view(torch.int16))
        assert torch.equal(full[1].view(torch.int32), out[1].view(torch.int32))
        assert torch.equal(full[2].view(torch.int32), out[2].view(torch.int32))


def test_exact_sizes_match_padded_path(qa):
    """D = 120 and D = 128 with the last 8 columns of Q and K zero (Dv = 120 both times) give the
    same scores, so the same outputs bit for bit: the padded path differs from the exact one only
    in what it loads."""
    B, Nq, Nkv, S = 1, 2, 1, 400
    banner("D=120 against D=128 with zero columns")
    qb, kb, vb = (random_bf16(1100 + i, s) for i, s in enumerate([(B, Nq, S, 120), (B, Nkv, S, 120),
                                                                  (B, Nkv, S, 120)]))
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:-1] + (8,), np.uint16)], axis=-1)
    a = qa.attn_fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), scale=0.1)
    b = qa.attn_fwd(dev_bf16(pad(qb)), dev_bf16(pad(kb)), dev_bf16(vb), scale=0.1)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))
