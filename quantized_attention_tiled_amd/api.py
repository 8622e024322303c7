"""PyTorch-facing wrappers over the qattn C ABI.

These functions only marshal arguments: they check dtypes, shapes and
devices, allocate outputs with torch when the caller passes none, and call the
library on the current HIP stream. Every step of the computation runs in the
library's kernels.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import (DTYPE_BF16, DTYPE_FP16, LAYOUT_BNSD, LAYOUT_BSND, LAYOUT_SBH, LAYOUT_TND, MASK_B1SS, MASK_BITS,
                   MASK_BNSS, MASK_SS, NO_LIMIT, QattnDesc, check, load)

BLOCK = 128
_DTYPES = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_FP16}


def _vp(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t: torch.Tensor, name: str, dtype, shape=None) -> None:
    """Type, dtype, shape and contiguity of a buffer the library reads or writes. The C ABI sees
    only pointers, so a wrong shape would mean out-of-bounds device accesses. Each entry point
    checks every buffer here first and all their devices (``_placed``) just before the call."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _placed(device: torch.device, **bufs) -> None:
    """Every named buffer (None = absent) lives on the GPU `device`."""
    for name, t in bufs.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU device")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _cu(x) -> Optional[ctypes.Array]:
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().tolist()
    vals = [int(v) for v in x]
    return (ctypes.c_int32 * len(vals))(*vals)


def _lengths(x, B: int, name: str) -> Optional[ctypes.Array]:
    """Per-batch actual lengths as a host int32 array of exactly B entries (the library reads B)."""
    arr = _cu(x)
    if arr is not None and len(arr) != B:
        raise ValueError(f"{name} must hold one length per batch ({B}), got {len(arr)}")
    return arr


def _ranges(head_range, qblock_range):
    h = (-1, -1) if head_range is None else (int(head_range[0]), int(head_range[1]))
    b = (-1, -1) if qblock_range is None else (int(qblock_range[0]), int(qblock_range[1]))
    return h, b


def make_desc(*, layout: int, B: int, Nq: int, Nkv: int, Sq: int, Skv: int, D: int, scale: float,
              sparse_mode: int = 0, cu_q=None, cu_kv=None, atten_mask: Optional[torch.Tensor] = None,
              mask_kind: int = MASK_SS, head_range=None, qblock_range=None, pre_tokens: int = NO_LIMIT,
              next_tokens: int = NO_LIMIT, dtype: int = DTYPE_BF16, Dv: int = 0, actual_q=None,
              actual_kv=None, qblock_order: Optional[torch.Tensor] = None) -> QattnDesc:
    d = QattnDesc()
    d.struct_size = ctypes.sizeof(QattnDesc)
    d.layout, d.B, d.Nq, d.Nkv, d.Sq, d.Skv, d.D = layout, B, Nq, Nkv, Sq, Skv, D
    d.scale = float(scale)
    d.sparse_mode = int(sparse_mode)
    d.cu_seqlens_q = ctypes.cast(cu_q, ctypes.POINTER(ctypes.c_int32)) if cu_q is not None else None
    d.cu_seqlens_kv = ctypes.cast(cu_kv, ctypes.POINTER(ctypes.c_int32)) if cu_kv is not None else None
    d.atten_mask = atten_mask.data_ptr() if atten_mask is not None else None
    d.mask_kind = int(mask_kind)
    (d.head_begin, d.head_end), (d.qblock_begin, d.qblock_end) = _ranges(head_range, qblock_range)
    d.pre_tokens, d.next_tokens = int(pre_tokens), int(next_tokens)
    d.dtype, d.Dv = int(dtype), int(Dv)
    d.actual_seq_lengths = ctypes.cast(actual_q, ctypes.POINTER(ctypes.c_int32)) if actual_q is not None else None
    d.actual_seq_lengths_kv = ctypes.cast(actual_kv, ctypes.POINTER(ctypes.c_int32)) if actual_kv is not None else None
    d.qblock_order = qblock_order.data_ptr() if qblock_order is not None else None
    return d


def _dims(layout: str, q: torch.Tensor, k: torch.Tensor, head_num: Optional[int]):
    """(layout code, B, Nq, Sq, Nkv, Skv, D) of the batched layouts: BNSD and BSND are 4-D, BSH and
    SBH 3-D with H = head_num * D (head_num counts the query heads; the kv heads follow from k).
    D is the query/key head dimension; v's follows from v (``_value_dim``)."""
    if layout in ("BNSD", "BSND"):
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError(f"{layout} tensors must be 4-D")
        if layout == "BNSD":
            (B, Nq, Sq, D), (Bk, Nkv, Skv, Dk), code = q.shape, k.shape, LAYOUT_BNSD
        else:
            (B, Sq, Nq, D), (Bk, Skv, Nkv, Dk), code = q.shape, k.shape, LAYOUT_BSND
    elif layout in ("BSH", "SBH"):
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError(f"{layout} tensors must be 3-D")
        if head_num is None or head_num < 1 or q.shape[2] % head_num:
            raise ValueError(f"{layout} needs head_num dividing H = {q.shape[2]}")
        Nq, D = int(head_num), q.shape[2] // int(head_num)
        if k.shape[2] % D:
            raise ValueError(f"k's H = {k.shape[2]} is not a multiple of D = {D}")
        Nkv, Dk = k.shape[2] // D, D
        if layout == "BSH":
            (B, Sq), (Bk, Skv), code = q.shape[:2], k.shape[:2], LAYOUT_BSND
        else:
            (Sq, B), (Skv, Bk), code = q.shape[:2], k.shape[:2], LAYOUT_SBH
    else:
        raise ValueError("layout must be 'BNSD', 'BSND', 'BSH', 'SBH' or 'TND'")
    if Bk != B or Dk != D:
        raise ValueError(f"k/v do not match q in {layout}")
    return code, B, Nq, Sq, Nkv, Skv, D


def _value_dim(layout: str, k: torch.Tensor, v: torch.Tensor, Nkv: int) -> int:
    """Head dimension of v, whose other dimensions must match k's."""
    if v.dim() != k.dim() or v.shape[:-1] != k.shape[:-1]:
        raise ValueError(f"v {tuple(v.shape)} does not match k {tuple(k.shape)} outside the head dimension")
    if layout in ("BSH", "SBH"):
        if v.shape[-1] % Nkv:
            raise ValueError(f"v's H = {v.shape[-1]} is not a multiple of Nkv = {Nkv}")
        return v.shape[-1] // Nkv
    return v.shape[-1]


def _check_dtypes(q, k, v) -> int:
    if not isinstance(q, torch.Tensor) or q.dtype not in _DTYPES:
        raise TypeError(f"q must be a bfloat16 or float16 tensor, got {getattr(q, 'dtype', type(q))}")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, q.dtype)
    return _DTYPES[q.dtype]


def _mask_kind(mask: torch.Tensor, B: int, Nq: int, Sq: int, Skv: int) -> int:
    """mask_kind of an atten_mask: uint8 (one byte per key) or int32 (bit-packed, ceil(Skv / 32)
    words per row, key j in bit j % 32 of word j // 32), shaped SS, B1SS or BNSS."""
    bits = mask.dtype == torch.int32
    W = (Skv + 31) // 32 if bits else Skv
    flag = MASK_BITS if bits else 0
    if mask.dim() == 2 and tuple(mask.shape) == (Sq, W):
        return MASK_SS | flag
    if mask.dim() == 4 and tuple(mask.shape) == (B, 1, Sq, W):
        return MASK_B1SS | flag
    if mask.dim() == 4 and tuple(mask.shape) == (B, Nq, Sq, W):
        return MASK_BNSS | flag
    raise ValueError(f"atten_mask shape {tuple(mask.shape)} is not SS, B1SS or BNSS for B={B} Nq={Nq} Sq={Sq} "
                     f"Skv={Skv}" + (f" (bit-packed: {W} int32 words per row)" if bits else ""))


def _atten_mask(atten_mask: torch.Tensor) -> torch.Tensor:
    """bool / uint8 byte masks as uint8; int32 bit-packed masks as they are."""
    if atten_mask.dtype == torch.bool:
        atten_mask = atten_mask.view(torch.uint8)
    if atten_mask.dtype not in (torch.uint8, torch.int32):
        raise TypeError(f"atten_mask must be bool / uint8 (one byte per key) or int32 (bit-packed), "
                        f"got {atten_mask.dtype}")
    _require(atten_mask, "atten_mask", atten_mask.dtype)
    return atten_mask


def _outputs(q, out, softmax_max, softmax_sum, ml_shape, o_shape=None):
    if out is None:
        out = torch.empty(q.shape if o_shape is None else o_shape, dtype=q.dtype, device=q.device)
    if softmax_max is None:
        softmax_max = torch.empty(ml_shape, dtype=torch.float32, device=q.device)
    if softmax_sum is None:
        softmax_sum = torch.empty(ml_shape, dtype=torch.float32, device=q.device)
    return out, softmax_max, softmax_sum


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: float = 1.0, layout: str = "BNSD",
             sparse_mode: int = 0, atten_mask: Optional[torch.Tensor] = None,
             cu_seqlens_q: Optional[Sequence[int]] = None, cu_seqlens_kv: Optional[Sequence[int]] = None,
             head_range: Optional[Tuple[int, int]] = None, qblock_range: Optional[Tuple[int, int]] = None,
             out: Optional[torch.Tensor] = None, softmax_max: Optional[torch.Tensor] = None,
             softmax_sum: Optional[torch.Tensor] = None, head_num: Optional[int] = None,
             pre_tokens: int = NO_LIMIT, next_tokens: int = NO_LIMIT,
             actual_seq_lengths: Optional[Sequence[int]] = None,
             actual_seq_lengths_kv: Optional[Sequence[int]] = None):
    """Dense attention forward on bfloat16 or float16 q, k, v (one type); returns (out,
    softmax_max, softmax_sum), out in that type.

    BNSD: q [B, Nq, Sq, D], k/v [B, Nkv, Skv, D]; BSND: q [B, Sq, Nq, D], k/v [B, Skv, Nkv, D];
    BSH: q [B, Sq, Nq * D], SBH: q [Sq, B, Nq * D] (k/v alike, with head_num = Nq); m/l [B, Nq, Sq].
    TND:  q [T, Nq, D], k/v [Tk, Nkv, D] plus cumulative lengths; m/l [Nq, T].
    v may have a smaller head dimension Dv; out then has Dv where q has D. D and Dv: multiples of 8 with
    Dv <= D <= 256.
    ``atten_mask`` (uint8 or bool, 1/True = masked) is SS, B1SS or BNSS (not with TND); an int32
    mask is bit-packed: ceil(Skv / 32) words per row, key j in bit j % 32 of word j // 32.
    With sparse_mode 0, ``pre_tokens`` / ``next_tokens`` keep key j for query i when
    i - pre_tokens <= j <= i + next_tokens (2147483647 = no limit).
    ``actual_seq_lengths`` / ``actual_seq_lengths_kv`` (not TND): per-batch valid query / key
    lengths of padded tensors; padded rows come out as rows with no key.
    With a head or q-block range only that slice of the outputs is written.
    """
    lib = load()
    dev = q.device
    dtype = _check_dtypes(q, k, v)
    if layout != "TND":
        lay, B, Nq, Sq, Nkv, Skv, D = _dims(layout, q, k, head_num)
        cu_q, cu_kv, ml_shape = None, None, (B, Nq, Sq)
    else:
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("TND tensors must be 3-D [T, N, D]")
        Sq, Nq, D = q.shape
        Skv, Nkv = k.shape[0], k.shape[1]
        if k.shape[2] != D:
            raise ValueError("k/v must be [Tk, Nkv, D] matching q")
        cu_q, cu_kv = _cu(cu_seqlens_q), _cu(cu_seqlens_kv if cu_seqlens_kv is not None else cu_seqlens_q)
        if cu_q is None:
            raise ValueError("TND needs cu_seqlens_q")
        if len(cu_q) != len(cu_kv):
            raise ValueError("cu_seqlens_q and cu_seqlens_kv differ in length")
        B = len(cu_q) - 1
        lay, ml_shape = LAYOUT_TND, (Nq, Sq)
    Dv = _value_dim(layout, k, v, Nkv)
    o_shape = q.shape[:-1] + (q.shape[-1] // D * Dv,)
    kind = MASK_SS
    if atten_mask is not None:
        atten_mask = _atten_mask(atten_mask)
        if layout == "TND":
            raise ValueError("atten_mask is not available with TND")
        kind = _mask_kind(atten_mask, B, Nq, Sq, Skv)
    out, softmax_max, softmax_sum = _outputs(q, out, softmax_max, softmax_sum, ml_shape, o_shape)
    _require(out, "out", q.dtype, o_shape)
    _require(softmax_max, "softmax_max", torch.float32, ml_shape)
    _require(softmax_sum, "softmax_sum", torch.float32, ml_shape)
    # host arrays, alive until the call returns
    aq_arr = _lengths(actual_seq_lengths, B, "actual_seq_lengths")
    akv_arr = _lengths(actual_seq_lengths_kv, B, "actual_seq_lengths_kv")
    _placed(dev, q=q, k=k, v=v, atten_mask=atten_mask, out=out, softmax_max=softmax_max, softmax_sum=softmax_sum)
    desc = make_desc(layout=lay, B=B, Nq=Nq, Nkv=Nkv, Sq=Sq, Skv=Skv, D=D, scale=scale, sparse_mode=sparse_mode,
                     cu_q=cu_q, cu_kv=cu_kv, atten_mask=atten_mask, mask_kind=kind, head_range=head_range,
                     qblock_range=qblock_range, pre_tokens=pre_tokens, next_tokens=next_tokens, dtype=dtype, Dv=Dv,
                     actual_q=aq_arr, actual_kv=akv_arr)
    with torch.cuda.device(dev):
        check(lib.attn_fwd(ctypes.byref(desc), _vp(q), _vp(k), _vp(v), _vp(out), _vp(softmax_max), _vp(softmax_sum),
                           _stream(dev)))
    return out, softmax_max, softmax_sum


def pack_atten_mask_bits(atten_mask: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The bit-packed form of a byte atten_mask (uint8 or bool, nonzero / True = masked, shape
    [..., Sq, Skv] with contiguous rows): int32 [..., Sq, ceil(Skv / 32)], key j in bit j % 32 of
    word j // 32. attn_fwd takes the result as an atten_mask of the same kind (SS, B1SS, BNSS)."""
    lib = load()
    if atten_mask.dtype == torch.bool:
        atten_mask = atten_mask.view(torch.uint8)
    _require(atten_mask, "atten_mask", torch.uint8)
    if atten_mask.dim() < 2:
        raise ValueError(f"atten_mask must be [..., Sq, Skv], got shape {tuple(atten_mask.shape)}")
    Skv = atten_mask.shape[-1]
    if Skv < 1:
        raise ValueError("atten_mask needs at least one key")
    shape = tuple(atten_mask.shape[:-1]) + ((Skv + 31) // 32,)
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=atten_mask.device)
    _require(out, "out", torch.int32, shape)
    _placed(atten_mask.device, atten_mask=atten_mask, out=out)
    rows = atten_mask.numel() // Skv
    with torch.cuda.device(atten_mask.device):
        check(lib.pack_atten_mask_bits(_vp(atten_mask), rows, Skv, Skv, _vp(out), _stream(atten_mask.device)))
    return out


def build_qblock_order(counts: torch.Tensor, order: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per (batch, head) of the kept counts int32 [B, N, QB] (from build_kv_block_list) the
    q-blocks by kept count, largest first, ties in ascending order: int32 [B, N, QB], the
    ``qblock_order`` of attn_fwd_blocksparse and attn_fwd_qbsa. QB <= 16384."""
    lib = load()
    _require(counts, "counts", torch.int32)
    if counts.dim() != 3:
        raise ValueError(f"counts must be 3-D [B, N, QB], got shape {tuple(counts.shape)}")
    B, N, QB = counts.shape
    if order is None:
        order = torch.empty((B, N, QB), dtype=torch.int32, device=counts.device)
    _require(order, "order", torch.int32, (B, N, QB))
    _placed(counts.device, counts=counts, order=order)
    with torch.cuda.device(counts.device):
        check(lib.build_qblock_order(_vp(counts), B, N, QB, _vp(order), _stream(counts.device)))
    return order


def build_kv_block_list(keep: torch.Tensor, counts: Optional[torch.Tensor] = None,
                        idx: Optional[torch.Tensor] = None):
    """Kept-block list of a block keep mask uint8 [B, N, QB, KB] (nonzero = keep).

    Returns (counts int32 [B, N, QB], idx int32 [B, N, QB, KB])."""
    lib = load()
    if keep.dtype == torch.bool:
        keep = keep.view(torch.uint8)
    _require(keep, "keep", torch.uint8)
    if keep.dim() != 4:
        raise ValueError(f"keep must be 4-D [B, N, QB, KB], got shape {tuple(keep.shape)}")
    B, N, QB, KB = keep.shape
    if counts is None:
        counts = torch.empty((B, N, QB), dtype=torch.int32, device=keep.device)
    if idx is None:
        idx = torch.empty((B, N, QB, KB), dtype=torch.int32, device=keep.device)
    _require(counts, "counts", torch.int32, (B, N, QB))
    _require(idx, "idx", torch.int32, (B, N, QB, KB))
    _placed(keep.device, keep=keep, counts=counts, idx=idx)
    with torch.cuda.device(keep.device):
        check(lib.build_kv_block_list(_vp(keep), B, N, QB, KB, _vp(counts), _vp(idx), _stream(keep.device)))
    return counts, idx


def attn_fwd_blocksparse(q, k, v, counts, idx, *, scale: float = 1.0, head_range=None, qblock_range=None,
                         out=None, softmax_max=None, softmax_sum=None, layout: str = "BNSD",
                         head_num: Optional[int] = None, actual_seq_lengths=None, actual_seq_lengths_kv=None,
                         qblock_order: Optional[torch.Tensor] = None):
    """Block-sparse attention over a kept-block list on bfloat16 or float16 q, k, v (BNSD, BSND,
    BSH or SBH, shapes and Dv as for attn_fwd); returns (out, m [B, Nq, Sq], l).
    ``qblock_order``: optional int32 [B, Nq, QB] from build_qblock_order (the order in which each
    head's q-blocks are taken; each row then walks its kept blocks from the first)."""
    lib = load()
    dev = q.device
    dtype = _check_dtypes(q, k, v)
    lay, B, Nq, Sq, Nkv, Skv, D = _dims(layout, q, k, head_num)
    Dv = _value_dim(layout, k, v, Nkv)
    o_shape = q.shape[:-1] + (q.shape[-1] // D * Dv,)
    QB, KB = (Sq + BLOCK - 1) // BLOCK, (Skv + BLOCK - 1) // BLOCK
    _require(counts, "counts", torch.int32, (B, Nq, QB))
    _require(idx, "idx", torch.int32, (B, Nq, QB, KB))
    if qblock_order is not None:
        _require(qblock_order, "qblock_order", torch.int32, (B, Nq, QB))
    out, softmax_max, softmax_sum = _outputs(q, out, softmax_max, softmax_sum, (B, Nq, Sq), o_shape)
    _require(out, "out", q.dtype, o_shape)
    _require(softmax_max, "softmax_max", torch.float32, (B, Nq, Sq))
    _require(softmax_sum, "softmax_sum", torch.float32, (B, Nq, Sq))
    # host arrays, alive until the call returns
    aq_arr = _lengths(actual_seq_lengths, B, "actual_seq_lengths")
    akv_arr = _lengths(actual_seq_lengths_kv, B, "actual_seq_lengths_kv")
    _placed(dev, q=q, k=k, v=v, counts=counts, idx=idx, out=out, softmax_max=softmax_max, softmax_sum=softmax_sum,
            qblock_order=qblock_order)
    desc = make_desc(layout=lay, B=B, Nq=Nq, Nkv=Nkv, Sq=Sq, Skv=Skv, D=D, scale=scale,
                     head_range=head_range, qblock_range=qblock_range, dtype=dtype, Dv=Dv,
                     actual_q=aq_arr, actual_kv=akv_arr, qblock_order=qblock_order)
    with torch.cuda.device(dev):
        check(lib.attn_fwd_blocksparse(ctypes.byref(desc), _vp(q), _vp(k), _vp(v), _vp(out), _vp(softmax_max),
                                       _vp(softmax_sum), _vp(counts), _vp(idx), _stream(dev)))
    return out, softmax_max, softmax_sum


def quantize_qk_perblock_int8(x: torch.Tensor, x_q: Optional[torch.Tensor] = None,
                              scale: Optional[torch.Tensor] = None):
    """INT8 per (batch, head, 128-token block); returns (codes int8, scale fp32 [B, N, ceil(S/128)])."""
    lib = load()
    _require(x, "x", torch.bfloat16)
    if x.dim() != 4:
        raise ValueError(f"x must be 4-D BNSD [B, N, S, D], got shape {tuple(x.shape)}")
    B, N, S, D = x.shape
    if x_q is None:
        x_q = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty((B, N, (S + BLOCK - 1) // BLOCK), dtype=torch.float32, device=x.device)
    _require(x_q, "x_q", torch.int8, x.shape)
    _require(scale, "scale", torch.float32, (B, N, (S + BLOCK - 1) // BLOCK))
    _placed(x.device, x=x, x_q=x_q, scale=scale)
    with torch.cuda.device(x.device):
        check(lib.quantize_qk_perblock_int8(_vp(x), B, N, S, D, _vp(x_q), _vp(scale), _stream(x.device)))
    return x_q, scale


def quantize_v_perchannel_fp8(v: torch.Tensor, v_q: Optional[torch.Tensor] = None,
                              scale: Optional[torch.Tensor] = None):
    """E4M3FN per (batch, head, channel); returns (codes uint8, scale fp32 [B, N, D])."""
    lib = load()
    _require(v, "v", torch.bfloat16)
    if v.dim() != 4:
        raise ValueError(f"v must be 4-D BNSD [B, N, S, D], got shape {tuple(v.shape)}")
    B, N, S, D = v.shape
    if v_q is None:
        v_q = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    if v_q.dtype == torch.float8_e4m3fn:
        v_q = v_q.view(torch.uint8)
    if scale is None:
        scale = torch.empty((B, N, D), dtype=torch.float32, device=v.device)
    _require(v_q, "v_q", torch.uint8, v.shape)
    _require(scale, "scale", torch.float32, (B, N, D))
    _placed(v.device, v=v, v_q=v_q, scale=scale)
    with torch.cuda.device(v.device):
        check(lib.quantize_v_perchannel_fp8(_vp(v), B, N, S, D, _vp(v_q), _vp(scale), _stream(v.device)))
    return v_q, scale


def attn_fwd_qbsa(q_q, k_q, v_q, q_scale, k_scale, v_scale, counts, idx, *, scale: float,
                  head_range=None, qblock_range=None, out=None, softmax_max=None, softmax_sum=None,
                  return_softmax: bool = True, actual_seq_lengths=None, actual_seq_lengths_kv=None,
                  qblock_order: Optional[torch.Tensor] = None):
    """Quantised block-sparse attention (BNSD); returns (out, m, l) or (out, None, None).
    ``actual_seq_lengths`` / ``actual_seq_lengths_kv``: per-batch valid lengths, as for attn_fwd.
    ``qblock_order``: optional int32 [B, Nq, QB] from build_qblock_order (the order in which each
    head's q-blocks are taken; the results are the same bits either way)."""
    lib = load()
    dev = q_q.device
    _require(q_q, "q_q", torch.int8)
    if q_q.dim() != 4 or k_q.dim() != 4:
        raise ValueError("q_q and k_q must be 4-D BNSD")
    B, Nq, Sq, D = q_q.shape
    Nkv, Skv = k_q.shape[1], k_q.shape[2]
    _require(k_q, "k_q", torch.int8, (B, Nkv, Skv, D))
    if v_q.dtype == torch.float8_e4m3fn:
        v_q = v_q.view(torch.uint8)
    _require(v_q, "v_q", torch.uint8, (B, Nkv, Skv, D))
    QB, KB = (Sq + BLOCK - 1) // BLOCK, (Skv + BLOCK - 1) // BLOCK
    _require(q_scale, "q_scale", torch.float32, (B, Nq, QB))
    _require(k_scale, "k_scale", torch.float32, (B, Nkv, KB))
    _require(v_scale, "v_scale", torch.float32, (B, Nkv, D))
    _require(counts, "counts", torch.int32, (B, Nq, QB))
    _require(idx, "idx", torch.int32, (B, Nq, QB, KB))
    if qblock_order is not None:
        _require(qblock_order, "qblock_order", torch.int32, (B, Nq, QB))
    if out is None:
        out = torch.empty(q_q.shape, dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, (B, Nq, Sq, D))
    if return_softmax:
        if softmax_max is None:
            softmax_max = torch.empty((B, Nq, Sq), dtype=torch.float32, device=dev)
        if softmax_sum is None:
            softmax_sum = torch.empty((B, Nq, Sq), dtype=torch.float32, device=dev)
    for t, n in ((softmax_max, "softmax_max"), (softmax_sum, "softmax_sum")):
        if t is not None:
            _require(t, n, torch.float32, (B, Nq, Sq))
    # host arrays, alive until the call returns
    aq_arr = _lengths(actual_seq_lengths, B, "actual_seq_lengths")
    akv_arr = _lengths(actual_seq_lengths_kv, B, "actual_seq_lengths_kv")
    _placed(dev, q_q=q_q, k_q=k_q, v_q=v_q, q_scale=q_scale, k_scale=k_scale, v_scale=v_scale, counts=counts,
            idx=idx, out=out, softmax_max=softmax_max, softmax_sum=softmax_sum, qblock_order=qblock_order)
    desc = make_desc(layout=LAYOUT_BNSD, B=B, Nq=Nq, Nkv=Nkv, Sq=Sq, Skv=Skv, D=D, scale=scale,
                     head_range=head_range, qblock_range=qblock_range, actual_q=aq_arr, actual_kv=akv_arr,
                     qblock_order=qblock_order)
    with torch.cuda.device(dev):
        check(lib.attn_fwd_qbsa(ctypes.byref(desc), _vp(q_q), _vp(k_q), _vp(v_q), _vp(q_scale), _vp(k_scale),
                                _vp(v_scale), _vp(counts), _vp(idx), _vp(out), _vp(softmax_max), _vp(softmax_sum),
                                _stream(dev)))
    return out, softmax_max, softmax_sum


def _bwd_args(q, k, v, out, dout, softmax_max, softmax_sum, scale, sparse_mode, layout, cu_seqlens_q,
              cu_seqlens_kv, head_num, atten_mask, pre_tokens, next_tokens, actual_seq_lengths,
              actual_seq_lengths_kv, dq, dk, dv, allocate_grads: bool, head_range=None):
    """Checked arguments of the backward entry points: (desc, host arrays kept alive, mask, dq, dk, dv)."""
    dtype = _check_dtypes(q, k, v)
    for t, n in ((out, "out"), (dout, "dout")):
        _require(t, n, q.dtype)
    for t, n in ((softmax_max, "softmax_max"), (softmax_sum, "softmax_sum")):
        _require(t, n, torch.float32)
    cu_q = cu_kv = None
    if layout == "TND":
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("TND tensors must be 3-D [T, N, D]")
        Sq, Nq, D = q.shape
        Skv, Nkv = k.shape[0], k.shape[1]
        if k.shape[2] != D:
            raise ValueError("k/v must be [Tk, Nkv, D] matching q")
        cu_q, cu_kv = _cu(cu_seqlens_q), _cu(cu_seqlens_kv if cu_seqlens_kv is not None else cu_seqlens_q)
        if cu_q is None or len(cu_q) != len(cu_kv):
            raise ValueError("TND needs cu_seqlens_q (and cu_seqlens_kv of the same length)")
        B, lay, ml_shape = len(cu_q) - 1, LAYOUT_TND, (Nq, Sq)
    else:
        lay, B, Nq, Sq, Nkv, Skv, D = _dims(layout, q, k, head_num)
        ml_shape = (B, Nq, Sq)
    Dv = _value_dim(layout, k, v, Nkv)
    o_shape = q.shape[:-1] + (q.shape[-1] // D * Dv,)
    if out.shape != o_shape or dout.shape != o_shape:
        raise ValueError(f"out and dout must be {tuple(o_shape)} (q's shape with v's head dimension)")
    if tuple(softmax_max.shape) != ml_shape or tuple(softmax_sum.shape) != ml_shape:
        raise ValueError(f"softmax_max / softmax_sum must be {ml_shape}")
    kind = MASK_SS
    if atten_mask is not None:
        atten_mask = _atten_mask(atten_mask)
        if layout == "TND":
            raise ValueError("atten_mask is not available with TND")
        kind = _mask_kind(atten_mask, B, Nq, Sq, Skv)
    if allocate_grads:
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        if t is None:
            raise ValueError(f"{n} must be given (this entry point allocates nothing)")
        _require(t, n, q.dtype, ref.shape)
    # host arrays, alive until the call returns
    keep = (cu_q, cu_kv, _lengths(actual_seq_lengths, B, "actual_seq_lengths"),
            _lengths(actual_seq_lengths_kv, B, "actual_seq_lengths_kv"))
    desc = make_desc(layout=lay, B=B, Nq=Nq, Nkv=Nkv, Sq=Sq, Skv=Skv, D=D, scale=scale, sparse_mode=sparse_mode,
                     cu_q=cu_q, cu_kv=cu_kv, dtype=dtype, atten_mask=atten_mask, mask_kind=kind,
                     pre_tokens=pre_tokens, next_tokens=next_tokens, actual_q=keep[2], actual_kv=keep[3], Dv=Dv,
                     head_range=head_range)
    return desc, keep, atten_mask, dq, dk, dv


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
             softmax_max: torch.Tensor, softmax_sum: torch.Tensor, *, scale: float = 1.0, sparse_mode: int = 0,
             layout: str = "BNSD", cu_seqlens_q: Optional[Sequence[int]] = None,
             cu_seqlens_kv: Optional[Sequence[int]] = None, head_num: Optional[int] = None,
             atten_mask: Optional[torch.Tensor] = None, pre_tokens: int = NO_LIMIT, next_tokens: int = NO_LIMIT,
             actual_seq_lengths: Optional[Sequence[int]] = None,
             actual_seq_lengths_kv: Optional[Sequence[int]] = None, dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, head_range: Optional[Tuple[int, int]] = None):
    """Gradients (dq, dk, dv) of attn_fwd on bfloat16 or float16 q, k, v (one type) in any layout
    attn_fwd takes (shapes as there; D and Dv multiples of 8 with Dv <= D <= 128), given the
    forward's out and softmax_max / softmax_sum and the output gradient dout (shaped like out). The masks are the forward's: sparse_mode,
    ``atten_mask`` (not with TND), the ``pre_tokens`` / ``next_tokens`` band and per-batch
    ``actual_seq_lengths`` / ``actual_seq_lengths_kv`` (padded rows and keys get zero gradients).
    ``workspace``: optional fp32 device tensor of at least attn_bwd_workspace_bytes / 4 elements
    (2 B Nq Sq; TND: 2 Nq T). ``head_range`` (h0, h1): whole groups of Nq / Nkv q-heads; only dq of
    those q-heads and dk, dv of their kv-heads are written, bit for bit as by the full call."""
    lib = load()
    dev = q.device
    desc, _keep, atten_mask, dq, dk, dv = _bwd_args(
        q, k, v, out, dout, softmax_max, softmax_sum, scale, sparse_mode, layout, cu_seqlens_q, cu_seqlens_kv,
        head_num, atten_mask, pre_tokens, next_tokens, actual_seq_lengths, actual_seq_lengths_kv, dq, dk, dv, True,
        head_range)
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(desc)) // 4
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.float32, device=dev)
    _require(workspace, "workspace", torch.float32)
    if workspace.numel() < need:
        raise ValueError(f"workspace needs {need} float32 elements")
    _placed(dev, q=q, k=k, v=v, out=out, dout=dout, softmax_max=softmax_max, softmax_sum=softmax_sum,
            atten_mask=atten_mask, dq=dq, dk=dk, dv=dv, workspace=workspace)
    with torch.cuda.device(dev):
        check(lib.attn_bwd(ctypes.byref(desc), _vp(q), _vp(k), _vp(v), _vp(out), _vp(dout), _vp(softmax_max),
                           _vp(softmax_sum), _vp(dq), _vp(dk), _vp(dv), _vp(workspace), _stream(dev)))
    return dq, dk, dv


def attn_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                     softmax_max: torch.Tensor, softmax_sum: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor,
                     dv: torch.Tensor, *, scale: float = 1.0, sparse_mode: int = 0, layout: str = "BNSD",
                     cu_seqlens_q: Optional[Sequence[int]] = None, cu_seqlens_kv: Optional[Sequence[int]] = None,
                     head_num: Optional[int] = None, atten_mask: Optional[torch.Tensor] = None,
                     pre_tokens: int = NO_LIMIT, next_tokens: int = NO_LIMIT,
                     actual_seq_lengths: Optional[Sequence[int]] = None,
                     actual_seq_lengths_kv: Optional[Sequence[int]] = None,
                     head_range: Optional[Tuple[int, int]] = None):
    """attn_bwd for callers that cannot allocate: the caller passes every input and the outputs
    dq, dk, dv; the workspace is the library's static per-GPU buffer (at most
    NOALLOC_WORKSPACE_BYTES, i.e. 4194304 query rows). Allocates no device memory. Calls that
    overlap on one GPU share that buffer and must be serialised by the caller. ``head_range`` as
    for attn_bwd."""
    lib = load()
    dev = q.device
    desc, _keep, atten_mask, dq, dk, dv = _bwd_args(
        q, k, v, out, dout, softmax_max, softmax_sum, scale, sparse_mode, layout, cu_seqlens_q, cu_seqlens_kv,
        head_num, atten_mask, pre_tokens, next_tokens, actual_seq_lengths, actual_seq_lengths_kv, dq, dk, dv, False,
        head_range)
    _placed(dev, q=q, k=k, v=v, out=out, dout=dout, softmax_max=softmax_max, softmax_sum=softmax_sum,
            atten_mask=atten_mask, dq=dq, dk=dk, dv=dv)
    with torch.cuda.device(dev):
        check(lib.attn_bwd_noalloc(ctypes.byref(desc), _vp(q), _vp(k), _vp(v), _vp(out), _vp(dout),
                                   _vp(softmax_max), _vp(softmax_sum), _vp(dq), _vp(dk), _vp(dv), _stream(dev)))
    return dq, dk, dv


__all__ = ["attn_bwd", "attn_bwd_noalloc", "attn_fwd", "attn_fwd_blocksparse", "attn_fwd_qbsa", "build_kv_block_list",
           "build_qblock_order", "pack_atten_mask_bits", "quantize_qk_perblock_int8",
           "quantize_v_perchannel_fp8", "make_desc", "_lib"]
