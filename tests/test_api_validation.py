"""Host-side checks of the Python binding (no GPU needed).

The C ABI sees only pointers, so the binding must reject every caller buffer
whose dtype, shape or length does not match the problem: otherwise the kernels
would read or write past its end. The binding checks dtype and shape before
the device, so CPU tensors are enough to reach each shape error here.
"""

import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_attention_tiled_amd", "libqattn.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libqattn.so not built")

from quantized_attention_tiled_amd import api  # noqa: E402

bf16, i8, u8, f32, i32 = torch.bfloat16, torch.int8, torch.uint8, torch.float32, torch.int32


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def raises_shape(name, fn, *a, **kw):
    with pytest.raises(ValueError, match=name):
        fn(*a, **kw)


def raises_device(fn, *a, **kw):
    """Shapes all right: the first complaint is the CPU device."""
    with pytest.raises(ValueError, match="GPU device"):
        fn(*a, **kw)


def test_require_order():
    t = z((2, 3), f32)
    with pytest.raises(TypeError):
        api._require(t, "t", bf16)
    with pytest.raises(ValueError, match=r"shape \(3, 2\)"):
        api._require(t, "t", f32, shape=(3, 2))
    with pytest.raises(ValueError, match="contiguous"):
        api._require(t.t(), "t", f32, shape=(3, 2))
    api._require(t, "t", f32, shape=(2, 3))
    with pytest.raises(ValueError, match="u must be on a GPU device"):
        api._placed(torch.device("cuda:0"), t=None, u=t)


def test_attn_fwd_buffers():
    q, k, v = z((1, 2, 256, 64), bf16), z((1, 2, 256, 64), bf16), z((1, 2, 256, 64), bf16)
    raises_device(api.attn_fwd, q, k, v)
    raises_shape("out", api.attn_fwd, q, k, v, out=z((1, 2, 255, 64), bf16))
    raises_shape("softmax_max", api.attn_fwd, q, k, v, softmax_max=z((1, 2, 128), f32))
    raises_shape("softmax_sum", api.attn_fwd, q, k, v, softmax_sum=z((2, 256), f32))
    with pytest.raises(TypeError):
        api.attn_fwd(q, k, v, out=z((1, 2, 256, 64), torch.float16))
    raises_shape("atten_mask", api.attn_fwd, q, k, v, atten_mask=z((256, 255), u8))
    raises_shape("actual_seq_lengths", api.attn_fwd, q, k, v, actual_seq_lengths=[128, 128])
    raises_shape("actual_seq_lengths_kv", api.attn_fwd, q, k, v, actual_seq_lengths_kv=[])
    with pytest.raises(ValueError, match="3-D"):
        api.attn_fwd(q, k, v, layout="TND", cu_seqlens_q=[0, 256])


def test_block_list_buffers():
    keep = z((1, 2, 3, 4), u8)
    raises_device(api.build_kv_block_list, keep)
    raises_shape("keep", api.build_kv_block_list, z((2, 3, 4), u8))
    raises_shape("counts", api.build_kv_block_list, keep, counts=z((1, 2, 4), i32))
    raises_shape("idx", api.build_kv_block_list, keep, idx=z((1, 2, 3, 3), i32))


def test_blocksparse_buffers():
    q = k = v = z((1, 2, 256, 128), bf16)
    c, ix = z((1, 2, 2), i32), z((1, 2, 2, 2), i32)
    raises_device(api.attn_fwd_blocksparse, q, k, v, c, ix)
    raises_shape("counts", api.attn_fwd_blocksparse, q, k, v, z((1, 2, 3), i32), ix)
    raises_shape("idx", api.attn_fwd_blocksparse, q, k, v, c, z((1, 2, 2, 3), i32))
    raises_shape("softmax_max", api.attn_fwd_blocksparse, q, k, v, c, ix, softmax_max=z((1, 2, 255), f32))
    raises_shape("softmax_sum", api.attn_fwd_blocksparse, q, k, v, c, ix, softmax_sum=z((1, 1, 256), f32))
    raises_shape("out", api.attn_fwd_blocksparse, q, k, v, c, ix, out=z((1, 2, 256, 64), bf16))
    raises_shape("actual_seq_lengths", api.attn_fwd_blocksparse, q, k, v, c, ix, actual_seq_lengths=[1, 2, 3])


def test_quantizer_buffers():
    x = z((1, 2, 300, 128), bf16)
    raises_device(api.quantize_qk_perblock_int8, x)
    raises_shape("x_q", api.quantize_qk_perblock_int8, x, x_q=z((1, 2, 256, 128), i8))
    raises_shape("scale", api.quantize_qk_perblock_int8, x, scale=z((1, 2, 2), f32))
    raises_shape("x must be 4-D", api.quantize_qk_perblock_int8, z((2, 300, 128), bf16))
    raises_device(api.quantize_v_perchannel_fp8, x)
    raises_shape("v_q", api.quantize_v_perchannel_fp8, x, v_q=z((1, 2, 300, 64), u8))
    raises_shape("scale", api.quantize_v_perchannel_fp8, x, scale=z((1, 2, 300), f32))
    raises_shape("v must be 4-D", api.quantize_v_perchannel_fp8, z((300, 128), bf16))


def test_qbsa_buffers():
    B, Nq, Nkv, S, D = 1, 4, 2, 300, 128
    QB = KB = 3
    qq, kq, vq = z((B, Nq, S, D), i8), z((B, Nkv, S, D), i8), z((B, Nkv, S, D), u8)
    sc = (z((B, Nq, QB), f32), z((B, Nkv, KB), f32), z((B, Nkv, D), f32))
    c, ix = z((B, Nq, QB), i32), z((B, Nq, QB, KB), i32)

    def call(**kw):
        a = dict(q_q=qq, k_q=kq, v_q=vq, q_scale=sc[0], k_scale=sc[1], v_scale=sc[2], counts=c, idx=ix)
        a.update(kw)
        return api.attn_fwd_qbsa(a.pop("q_q"), a.pop("k_q"), a.pop("v_q"), a.pop("q_scale"), a.pop("k_scale"),
                                 a.pop("v_scale"), a.pop("counts"), a.pop("idx"), scale=0.1, **a)

    raises_device(call)
    raises_shape("k_q", call, k_q=z((B, Nkv, S, 64), i8))
    raises_shape("k_q", call, k_q=z((2, Nkv, S, D), i8))
    raises_shape("v_q", call, v_q=z((B, Nkv, S - 1, D), u8))
    raises_shape("q_scale", call, q_scale=z((B, Nq, 2), f32))
    raises_shape("k_scale", call, k_scale=z((B, Nq, KB), f32))
    raises_shape("v_scale", call, v_scale=z((B, Nkv, 64), f32))
    raises_shape("counts", call, counts=z((B, Nkv, QB), i32))
    raises_shape("idx", call, idx=z((B, Nq, QB, 2), i32))
    raises_shape("out", call, out=z((B, Nq, S, 64), bf16))
    with pytest.raises(TypeError):
        call(out=z((B, Nq, S, D), f32))
    raises_shape("softmax_max", call, softmax_max=z((B, Nq, S + 1), f32))
    raises_shape("softmax_sum", call, softmax_sum=z((B, Nq), f32))
    raises_shape("softmax_max", call, return_softmax=False, softmax_max=z((Nq, S), f32))
    raises_shape("actual_seq_lengths_kv", call, actual_seq_lengths_kv=[S, S])
    raises_shape("4-D", call, q_q=z((Nq, S, D), i8))


def test_backward_buffers():
    q = k = v = o = do = z((1, 2, 256, 64), bf16)
    m = l = z((1, 2, 256), f32)
    raises_device(api.attn_bwd, q, k, v, o, do, m, l)
    raises_shape("dq", api.attn_bwd, q, k, v, o, do, m, l, dq=z((1, 2, 255, 64), bf16))
    raises_shape("dk", api.attn_bwd, q, k, v, o, do, m, l, dk=z((1, 1, 256, 64), bf16))
    raises_shape("dv", api.attn_bwd, q, k, v, o, do, m, l, dv=z((1, 2, 256, 32), bf16))
    raises_shape("softmax_max", api.attn_bwd, q, k, v, o, do, z((1, 2, 255), f32), l)
    raises_shape("atten_mask", api.attn_bwd, q, k, v, o, do, m, l, atten_mask=z((1, 3, 256, 256), u8))
    raises_shape("actual_seq_lengths", api.attn_bwd, q, k, v, o, do, m, l, actual_seq_lengths=[1, 2])
    # Dv < D: out, dout and dv take v's head dimension
    v32 = o32 = z((1, 2, 256, 32), bf16)
    raises_device(api.attn_bwd, q, k, v32, o32, o32, m, l)
    raises_shape("out and dout", api.attn_bwd, q, k, v32, o, o32, m, l)
    raises_shape("out and dout", api.attn_bwd, q, k, v32, o32, do, m, l)
    raises_shape("dv", api.attn_bwd, q, k, v32, o32, o32, m, l, dv=z((1, 2, 256, 64), bf16))
    raises_shape("does not match k", api.attn_bwd, q, k, z((1, 2, 255, 32), bf16), o32, o32, m, l)


def test_pack_mask_buffers():
    m = z((4, 70), u8)
    raises_device(api.pack_atten_mask_bits, m)
    raises_shape("out", api.pack_atten_mask_bits, m, out=z((4, 2), i32))
    with pytest.raises(TypeError):
        api.pack_atten_mask_bits(z((4, 70), f32))
    raises_shape("Sq, Skv", api.pack_atten_mask_bits, z((70,), u8))


def test_qblock_order_buffers():
    c = z((1, 2, 4), i32)
    raises_device(api.build_qblock_order, c)
    raises_shape("order", api.build_qblock_order, c, order=z((1, 2, 5), i32))
    raises_shape("3-D", api.build_qblock_order, z((2, 4), i32))
    q = k = v = z((1, 2, 512, 64), bf16)
    counts, idx = z((1, 2, 4), i32), z((1, 2, 4, 4), i32)
    raises_shape("qblock_order", api.attn_fwd_blocksparse, q, k, v, counts, idx, qblock_order=z((1, 2, 3), i32))
