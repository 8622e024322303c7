"""C-ABI host checks that need no GPU.

* the built library exports every function include/qattn.h declares;
* the ctypes mirror of qattn_desc has the C layout (checked against gcc);
* argument validation returns the documented status codes before any
  launch (fake, never-dereferenced device pointers are enough for that).
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qattn.h")
LIB = os.path.join(ROOT, "quantized_attention_tiled_amd", "libqattn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libqattn.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def q():
    from quantized_attention_tiled_amd import _lib
    return _lib


def test_exports_every_declared_symbol(q):
    lib = q.load()
    declared = _declared_functions()
    assert set(declared) == set(q.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    for name in declared:
        assert re.search(rf"\bT {name}$", nm, flags=re.M), name
    assert lib.qattn_version() == 100


def test_desc_layout_matches_c(q, tmp_path):
    fields = [f for f, _ in q.QattnDesc._fields_]
    src = tmp_path / "probe.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "qattn.h"', "int main(void) {",
             '  printf("%zu\\n", sizeof(qattn_desc));']
    lines += [f'  printf("%zu\\n", offsetof(qattn_desc, {f}));' for f in fields]
    lines += ["  return 0;", "}"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(q.QattnDesc)
    for f, off in zip(fields, out[1:]):
        assert getattr(q.QattnDesc, f).offset == off, f


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def _desc(q, **kw):
    d = q.QattnDesc()
    d.struct_size = ctypes.sizeof(q.QattnDesc)
    base = dict(layout=0, B=1, Nq=4, Nkv=2, Sq=256, Skv=256, D=128, scale=0.1, sparse_mode=0, mask_kind=0,
                head_begin=-1, head_end=-1, qblock_begin=-1, qblock_end=-1, pre_tokens=2147483647,
                next_tokens=2147483647, dtype=0, Dv=0)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def _fwd(q, d, qp=FAKE, kp=FAKE, vp=FAKE, op=FAKE, m=0, l=0):
    lib = q.load()
    return lib.attn_fwd(ctypes.byref(d) if d is not None else None, qp, kp, vp, op, m or None, l or None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=100), 2), (dict(D=264), 2), (dict(D=0), 1), (dict(D=769), 1), (dict(Nq=3, Nkv=2), 1), (dict(scale=0.0), 1), (dict(scale=-1.0), 1),
    (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(sparse_mode=1), 1), (dict(layout=4), 1),
    (dict(layout=-1), 1), (dict(sparse_mode=2, pre_tokens=5), 1), (dict(sparse_mode=3, next_tokens=0), 1), (dict(layout=3, B=64, Nq=64, Nkv=64, Skv=1 << 17, Sq=128), 2),
    (dict(layout=2, Nq=64, Nkv=64, Skv=1 << 20, Sq=128), 2),
    (dict(B=0), 1), (dict(Sq=-1), 1), (dict(Nkv=0), 1), (dict(head_begin=0, head_end=5), 1),
    (dict(head_begin=3, head_end=2), 1), (dict(qblock_begin=0, qblock_end=3), 1), (dict(qblock_begin=-2, qblock_end=1), 1),
    (dict(dtype=2), 1), (dict(dtype=-1), 1), (dict(Dv=-64), 1), (dict(Dv=256), 1), (dict(D=64, Dv=128), 1),
    (dict(Dv=36), 2), (dict(Dv=100), 2), (dict(D=64, Dv=20), 2), (dict(D=96, Dv=4), 2),
])
def test_invalid_descriptions(q, kw, status):
    assert _fwd(q, _desc(q, **kw)) == status
    assert q.load().qattn_last_error()


def test_struct_size_and_null_desc(q):
    d = _desc(q)
    d.struct_size = 12
    assert _fwd(q, d) == 1
    assert _fwd(q, None) == 1


def test_pointer_checks(q):
    assert _fwd(q, _desc(q), qp=0) == 1
    assert _fwd(q, _desc(q), vp=FAKE + 8) == 3
    assert _fwd(q, _desc(q), m=FAKE + 2) == 3
    assert b"not 16-byte aligned" in q.load().qattn_last_error() or b"4-byte" in q.load().qattn_last_error()


def test_tnd_validation(q):
    lib = q.load()

    def tnd(cu_q, cu_kv, **kw):
        aq = (ctypes.c_int32 * len(cu_q))(*cu_q)
        ak = (ctypes.c_int32 * len(cu_kv))(*cu_kv)
        d = _desc(q, layout=1, B=len(cu_q) - 1, Sq=cu_q[-1], Skv=cu_kv[-1], **kw)
        d.cu_seqlens_q = ctypes.cast(aq, ctypes.POINTER(ctypes.c_int32))
        d.cu_seqlens_kv = ctypes.cast(ak, ctypes.POINTER(ctypes.c_int32))
        return lib.attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None)

    assert tnd([1, 5], [0, 5]) == 1                      # does not start at 0
    assert tnd([0, 5, 3], [0, 5, 6]) == 1                # decreasing
    d = _desc(q, layout=1, B=2, Sq=10, Skv=10)           # missing arrays
    assert lib.attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None) == 1
    # more sequences than one launch carries: still validated entry by entry (the call would run in
    # groups of QATTN_MAX_SEQS; these fail validation before any launch)
    big = list(range(0, 301))
    bad = big[:280] + [big[279] - 1] + big[281:]
    assert tnd(bad, big) == 1                            # decreasing at sequence 279
    assert tnd(big, big[:290] + [big[289] - 2] + big[291:]) == 1   # kv lengths decreasing at sequence 289
    aq = (ctypes.c_int32 * 3)(0, 4, 9)
    d = _desc(q, layout=1, B=2, Sq=10, Skv=9)            # last entry != Sq
    d.cu_seqlens_q = ctypes.cast(aq, ctypes.POINTER(ctypes.c_int32))
    d.cu_seqlens_kv = ctypes.cast(aq, ctypes.POINTER(ctypes.c_int32))
    assert lib.attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None) == 1
    # a boolean mask needs BNSD
    d2 = _desc(q, layout=1, B=1, Sq=5, Skv=5)
    a5 = (ctypes.c_int32 * 2)(0, 5)
    d2.cu_seqlens_q = ctypes.cast(a5, ctypes.POINTER(ctypes.c_int32))
    d2.cu_seqlens_kv = ctypes.cast(a5, ctypes.POINTER(ctypes.c_int32))
    d2.atten_mask = FAKE
    assert lib.attn_fwd(ctypes.byref(d2), FAKE, FAKE, FAKE, FAKE, None, None, None) == 2


def test_actual_lengths_validation(q):
    lib = q.load()

    def call(aq, akv, **kw):
        d = _desc(q, B=2, **kw)
        keep = []
        if aq is not None:
            keep.append((ctypes.c_int32 * len(aq))(*aq))
            d.actual_seq_lengths = ctypes.cast(keep[-1], ctypes.POINTER(ctypes.c_int32))
        if akv is not None:
            keep.append((ctypes.c_int32 * len(akv))(*akv))
            d.actual_seq_lengths_kv = ctypes.cast(keep[-1], ctypes.POINTER(ctypes.c_int32))
        return lib.attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None)

    assert call([257, 3], None) == 1       # longer than Sq = 256
    assert call([3, -1], None) == 1
    assert call(None, [0, 257]) == 1
    d = _desc(q, B=300, Nq=2, Nkv=2, Sq=4, Skv=4)   # more batches than one launch carries: every entry checked
    arr = (ctypes.c_int32 * 300)(*([1] * 299 + [5]))
    d.actual_seq_lengths = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    assert lib.attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None) == 1   # batch 299: 5 > Sq
    d = _desc(q, layout=1, B=1, Sq=5, Skv=5)  # TND takes cu_seqlens instead
    a5 = (ctypes.c_int32 * 2)(0, 5)
    d.cu_seqlens_q = ctypes.cast(a5, ctypes.POINTER(ctypes.c_int32))
    d.cu_seqlens_kv = ctypes.cast(a5, ctypes.POINTER(ctypes.c_int32))
    d.actual_seq_lengths = ctypes.cast(a5, ctypes.POINTER(ctypes.c_int32))
    assert lib.attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None) == 1


def test_pack_mask_validation(q):
    lib = q.load()

    def pack(mask=FAKE, rows=4, Skv=33, stride=33, bits=FAKE):
        return lib.pack_atten_mask_bits(mask, rows, Skv, stride, bits, None)

    assert pack(rows=0) == 0                 # nothing to do, nothing launched
    assert pack(mask=None) == 1
    assert pack(bits=None) == 1
    assert pack(Skv=0) == 1
    assert pack(rows=-1) == 1
    assert pack(stride=32) == 1              # rows overlap
    assert pack(Skv=1 << 28, stride=1 << 28) == 1
    assert pack(bits=FAKE + 2) == 3          # words need 4-byte alignment
    assert b"aligned" in lib.qattn_last_error()


def test_qblock_order_validation(q):
    lib = q.load()
    assert lib.build_qblock_order(FAKE, 0, 4, 8, FAKE, None) == 0      # nothing to do
    assert lib.build_qblock_order(None, 1, 4, 8, FAKE, None) == 1
    assert lib.build_qblock_order(FAKE, 1, 4, 8, None, None) == 1
    assert lib.build_qblock_order(FAKE, -1, 4, 8, FAKE, None) == 1
    assert lib.build_qblock_order(FAKE, 1, 4, 16385, FAKE, None) == 2   # QB above 16384
    assert lib.build_qblock_order(FAKE + 2, 1, 4, 8, FAKE, None) == 3
    # the descriptor's qblock_order: block-sparse entry points only, 4-byte aligned
    d = _desc(q)
    d.qblock_order = FAKE
    assert _fwd(q, d) == 1 and b"block-sparse" in lib.qattn_last_error()
    assert lib.attn_bwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    d = _desc(q, Nkv=4)
    d.qblock_order = FAKE + 2
    assert lib.attn_fwd_blocksparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None) == 3


def test_backward_validation(q):
    lib = q.load()

    def bwd(d, ws=FAKE, m=FAKE):
        return lib.attn_bwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, m, FAKE, FAKE, FAKE, FAKE, ws, None)

    assert lib.attn_bwd_workspace_bytes(ctypes.byref(_desc(q, B=2, Nq=4, Sq=100))) == 8 * 2 * 4 * 100
    assert lib.attn_bwd_workspace_bytes(None) == 0
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(_desc(q, layout=1, B=3, Nq=4, Sq=100))) == 8 * 4 * 100  # TND
    # head dimensions: multiples of 8 with Dv <= D <= 128 (D = 96, Dv = 64 and the like are taken)
    for kw in (dict(Dv=60), dict(D=100), dict(D=256), dict(D=136, Dv=64), dict(D=4),
               dict(head_begin=0, head_end=1), dict(head_begin=1, head_end=3), dict(qblock_begin=0, qblock_end=1),
               dict(head_begin=0, head_end=2, qblock_begin=0, qblock_end=1)):
        # head ranges must hold whole groups (Nq / Nkv = 2 q-heads) and every q-block
        assert bwd(_desc(q, **kw)) == 2, kw
    assert bwd(_desc(q, head_begin=2, head_end=5)) == 1  # past Nq
    assert bwd(_desc(q, Dv=136)) == 1  # Dv > D
    assert bwd(_desc(q), ws=None) == 1
    assert bwd(_desc(q), m=FAKE + 2) == 3
    assert bwd(_desc(q, sparse_mode=1)) == 1
    assert lib.attn_bwd(ctypes.byref(_desc(q)), FAKE, FAKE, FAKE, FAKE, FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        None) == 3  # dout misaligned
    # the no-allocation variant: the same checks, and problems beyond its static workspace are refused
    # on the host (4194304 query rows of 8 bytes fit its 32 MiB)
    def noalloc(d):
        return lib.attn_bwd_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)

    assert noalloc(_desc(q, Nq=64, Nkv=64, Sq=65538, Skv=128)) == 2
    assert b"static buffer" in lib.qattn_last_error()
    assert noalloc(_desc(q, Dv=60)) == 2
    assert noalloc(_desc(q, sparse_mode=1)) == 1
    assert lib.attn_bwd_noalloc(ctypes.byref(_desc(q)), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                None) == 1


def test_blocksparse_and_qbsa_validation(q):
    lib = q.load()
    d = _desc(q, sparse_mode=2)
    assert lib.attn_fwd_blocksparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None) == 2
    d = _desc(q)
    d.atten_mask = FAKE
    assert lib.attn_fwd_blocksparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None) == 2
    d = _desc(q)
    assert lib.attn_fwd_blocksparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None) == 1
    for kw in (dict(D=100), dict(D=264), dict(Dv=36)):  # head dimensions as for attn_fwd
        assert lib.attn_fwd_blocksparse(ctypes.byref(_desc(q, **kw)), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE,
                                        None) == 2, kw
    d = _desc(q, pre_tokens=10)  # the band is a dense-entry-point option
    assert lib.attn_fwd_blocksparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None) == 2
    assert lib.attn_fwd_qbsa(ctypes.byref(_desc(q, next_tokens=0)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, None, None, None) == 2
    assert lib.attn_fwd_qbsa(ctypes.byref(_desc(q, layout=1)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             None, None, None) == 2
    for lay in (2, 3):  # BSND and SBH are bf16-only layouts
        assert lib.attn_fwd_qbsa(ctypes.byref(_desc(q, layout=lay)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, None, None, None) == 2
    for kw in (dict(dtype=1), dict(Dv=64), dict(D=96), dict(D=256)):  # bf16 out, D = Dv = 64 or 128
        assert lib.attn_fwd_qbsa(ctypes.byref(_desc(q, **kw)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, None, None, None) == 2
    assert lib.attn_fwd_qbsa(ctypes.byref(_desc(q)), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                             None, None, None) == 1
    assert lib.attn_fwd_qbsa(ctypes.byref(_desc(q)), FAKE, FAKE, FAKE, FAKE + 1, FAKE, FAKE, FAKE, FAKE, FAKE,
                             None, None, None) == 3


def test_quantizer_and_list_validation(q):
    lib = q.load()
    assert lib.quantize_qk_perblock_int8(FAKE, 1, 1, 128, 96, FAKE, FAKE, None) == 2
    assert lib.quantize_qk_perblock_int8(FAKE, 1, -1, 128, 128, FAKE, FAKE, None) == 1
    assert lib.quantize_qk_perblock_int8(FAKE + 4, 1, 1, 128, 128, FAKE, FAKE, None) == 3
    assert lib.quantize_qk_perblock_int8(FAKE, 1, 1, 128, 128, FAKE, None, None) == 1
    assert lib.quantize_v_perchannel_fp8(FAKE, 1, 1, 128, 32, FAKE, FAKE, None) == 2
    assert lib.quantize_v_perchannel_fp8(FAKE, 1, 1, 128, 128, FAKE, None, None) == 1
    assert lib.build_kv_block_list(None, 1, 1, 4, 4, FAKE, FAKE, None) == 1
    assert lib.build_kv_block_list(FAKE, 1, 1, 4, 4, FAKE + 2, FAKE, None) == 3
    # empty problems are a successful no-op that launches nothing
    assert lib.quantize_qk_perblock_int8(FAKE, 0, 1, 128, 128, FAKE, FAKE, None) == 0
    assert lib.build_kv_block_list(FAKE, 1, 0, 4, 4, FAKE, FAKE, None) == 0
    assert _fwd(q, _desc(q, Sq=0)) == 0
    assert _fwd(q, _desc(q, head_begin=1, head_end=1)) == 0
