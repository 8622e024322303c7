"""ctypes loader for libqattn.so and the C structures of include/qattn.h.

The library is built in-tree (``python -m quantized_attention_tiled_amd.build``).
There is no fallback: if the shared library is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqattn.so")

QATTN_OK = 0
QATTN_INVALID_ARGUMENT = 1
QATTN_UNSUPPORTED = 2
QATTN_MISALIGNED = 3
QATTN_HIP_ERROR = 4

LAYOUT_BNSD = 0
LAYOUT_TND = 1
LAYOUT_BSND = 2  # also BSH
LAYOUT_SBH = 3
MASK_SS, MASK_B1SS, MASK_BNSS = 0, 1, 2
MASK_BITS = 0x100  # OR'ed into mask_kind: one bit per key
DTYPE_BF16, DTYPE_FP16 = 0, 1
MAX_SEQS = 256  # QATTN_MAX_SEQS: sequences or padded batches per kernel launch (calls may hold more)

STATUS_NAMES = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "MISALIGNED", 4: "HIP_ERROR"}

# Every symbol include/qattn.h declares.
EXPORTS = ("attn_fwd", "pack_atten_mask_bits", "build_qblock_order", "build_kv_block_list", "attn_fwd_blocksparse",
           "quantize_qk_perblock_int8", "quantize_v_perchannel_fp8", "attn_fwd_qbsa", "attn_bwd",
           "attn_bwd_workspace_bytes", "attn_bwd_noalloc", "qattn_last_error", "qattn_version")
NOALLOC_WORKSPACE_BYTES = 32 << 20  # QATTN_NOALLOC_WORKSPACE_BYTES


class QattnError(RuntimeError):
    """A qattn call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class QattnDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("layout", ctypes.c_int32),
        ("B", ctypes.c_int32),
        ("Nq", ctypes.c_int32),
        ("Nkv", ctypes.c_int32),
        ("Sq", ctypes.c_int32),
        ("Skv", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("sparse_mode", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.POINTER(ctypes.c_int32)),
        ("cu_seqlens_kv", ctypes.POINTER(ctypes.c_int32)),
        ("atten_mask", ctypes.c_void_p),
        ("mask_kind", ctypes.c_int32),
        ("head_begin", ctypes.c_int32),
        ("head_end", ctypes.c_int32),
        ("qblock_begin", ctypes.c_int32),
        ("qblock_end", ctypes.c_int32),
        ("pre_tokens", ctypes.c_int32),
        ("next_tokens", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("Dv", ctypes.c_int32),
        ("actual_seq_lengths", ctypes.POINTER(ctypes.c_int32)),
        ("actual_seq_lengths_kv", ctypes.POINTER(ctypes.c_int32)),
        ("qblock_order", ctypes.c_void_p),
    ]


NO_LIMIT = 2147483647  # pre_tokens / next_tokens default: no band limit


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqattn.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m quantized_attention_tiled_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, i32, f32p, i32p = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    desc_p = ctypes.POINTER(QattnDesc)
    lib.attn_fwd.argtypes = [desc_p, vp, vp, vp, vp, f32p, f32p, vp]
    lib.build_kv_block_list.argtypes = [vp, i32, i32, i32, i32, i32p, i32p, vp]
    lib.pack_atten_mask_bits.argtypes = [vp, ctypes.c_int64, i32, ctypes.c_int64, i32p, vp]
    lib.build_qblock_order.argtypes = [i32p, i32, i32, i32, i32p, vp]
    lib.attn_fwd_blocksparse.argtypes = [desc_p, vp, vp, vp, vp, f32p, f32p, i32p, i32p, vp]
    lib.attn_bwd.argtypes = [desc_p, vp, vp, vp, vp, vp, f32p, f32p, vp, vp, vp, f32p, vp]
    lib.attn_bwd_noalloc.argtypes = [desc_p, vp, vp, vp, vp, vp, f32p, f32p, vp, vp, vp, vp]
    lib.attn_bwd_workspace_bytes.argtypes = [desc_p]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.quantize_qk_perblock_int8.argtypes = [vp, i32, i32, i32, i32, vp, f32p, vp]
    lib.quantize_v_perchannel_fp8.argtypes = [vp, i32, i32, i32, i32, vp, f32p, vp]
    lib.attn_fwd_qbsa.argtypes = [desc_p, vp, vp, vp, f32p, f32p, f32p, i32p, i32p, vp, f32p, f32p, vp]
    for name in ("attn_fwd", "pack_atten_mask_bits", "build_qblock_order", "build_kv_block_list", "attn_fwd_blocksparse",
                 "quantize_qk_perblock_int8", "quantize_v_perchannel_fp8", "attn_fwd_qbsa", "attn_bwd",
                 "attn_bwd_noalloc", "qattn_version"):
        getattr(lib, name).restype = ctypes.c_int
    lib.qattn_last_error.argtypes = []
    lib.qattn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != QATTN_OK:
        msg = load().qattn_last_error().decode(errors="replace")
        raise QattnError(status, msg)
