"""GPU tests of pack_atten_mask_bits: a byte atten_mask packed on the device into the bit form the
forward takes with QATTN_MASK_BITS.

The packed words must unpack, through the oracle's reading of the bit layout
(``oracle.atten_mask_from_bits``, pinned against numpy's packbits), to exactly the byte mask, with
every bit past Skv zero; and the forward must give the same bits with the packed mask as with the
byte mask it came from.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import banner, dev_bf16
from workloads import random_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_tiled_amd as qa
    qa.load()
    return qa


def _check_words(words: np.ndarray, mask: np.ndarray):
    Skv = mask.shape[-1]
    assert words.shape == mask.shape[:-1] + ((Skv + 31) // 32,)
    np.testing.assert_array_equal(oracle.atten_mask_from_bits(words, Skv), (mask != 0).astype(np.uint8))
    if Skv % 32:
        assert np.all((words[..., -1].astype(np.int64) & 0xFFFFFFFF) >> (Skv % 32) == 0), "bits past Skv"


@pytest.mark.parametrize("shape", [(200, 300), (2, 4, 130, 1000), (3, 1, 17, 33), (5, 1), (4, 31), (4, 32),
                                   (4, 64), (2, 65), (1, 2, 8, 1024)])
def test_pack_matches_oracle_reading(qa, shape):
    banner(f"pack_atten_mask_bits {shape}")
    rng = np.random.default_rng(sum(shape))
    mask = (rng.random(shape) < 0.3).astype(np.uint8)
    mask[..., 0, :] = 1                                     # a fully masked row
    if shape[-2] > 1:
        mask[..., 1, :] = 0                                 # an unmasked one
    mask[rng.random(shape) < 0.05] = 7                      # any nonzero byte masks
    words = qa.pack_atten_mask_bits(torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    _check_words(words.cpu().numpy(), mask)
    wb = qa.pack_atten_mask_bits(torch.from_numpy(mask != 0).cuda())   # bool input
    torch.cuda.synchronize()
    assert torch.equal(words, wb)


def test_pack_strided_rows_through_the_abi(qa):
    """Rows further apart than Skv bytes (a mask cut out of a wider one), through the C ABI."""
    from quantized_attention_tiled_amd import _lib
    lib = _lib.load()
    rows, Skv, stride = 50, 77, 77 + 51
    rng = np.random.default_rng(3)
    wide = (rng.random((rows, stride)) < 0.4).astype(np.uint8)
    wd = torch.from_numpy(wide).cuda()
    out = torch.full((rows, (Skv + 31) // 32), -1, dtype=torch.int32, device="cuda")
    rc = lib.pack_atten_mask_bits(ctypes.c_void_p(wd.data_ptr()), rows, Skv, stride, ctypes.c_void_p(out.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == 0
    _check_words(out.cpu().numpy(), wide[:, :Skv])


@pytest.mark.parametrize("kind,mode", [("SS", 0), ("BNSS", 2)])
def test_forward_with_packed_mask_equals_byte_mask(qa, kind, mode):
    B, Nq, Nkv, Sq, Skv, D = 2, 4, 2, 200, 333, 128
    banner(f"forward with a device-packed {kind} mask, mode {mode}")
    q = dev_bf16(random_bf16(80, (B, Nq, Sq, D)))
    k = dev_bf16(random_bf16(81, (B, Nkv, Skv, D)))
    v = dev_bf16(random_bf16(82, (B, Nkv, Skv, D)))
    shape = (Sq, Skv) if kind == "SS" else (B, Nq, Sq, Skv)
    mask = torch.from_numpy((np.random.default_rng(83).random(shape) < 0.3).astype(np.uint8)).cuda()
    bits = qa.pack_atten_mask_bits(mask)
    o1, m1, l1 = qa.attn_fwd(q, k, v, scale=0.09, sparse_mode=mode, atten_mask=mask)
    o2, m2, l2 = qa.attn_fwd(q, k, v, scale=0.09, sparse_mode=mode, atten_mask=bits)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(m1, m2) and torch.equal(l1, l2)
