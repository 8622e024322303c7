"""Synthetic workloads shaped like the pages' attention benchmarks.

Recipes (all values drawn in float32 and rounded once, to nearest-even, to
bfloat16, or to float16 for the float16 inputs):

* ``normal``        x ~ N(0, 1)
* ``block_offset``  x ~ N(0, 1) + o[blk, d], o ~ N(0, 0.5^2), one offset vector
                    per (batch, head, 128-token block); it mimics the
                    spatio-temporal locality the EagleQBSA article gives as the
                    reason for per-block Q/K quantisation.
* ``block_offset_channel``  as ``block_offset``, then every channel d of a
                    (batch, head) is multiplied by exp(g_d), g_d ~ N(0, 1)
                    (log-normal per-channel magnitudes for V).

Block keep masks are ``uint8 [B, Nq, QB, KB]`` with 1 = keep: the diagonal
block is always kept and every other block is kept independently with
probability ``p_keep``.

Seeds: config k uses base seed ``1000 + k``; every tensor, head and mask row
set has its own ``SeedSequence([base, tensor_id, b, n])``.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BLOCK = 128

# tensor ids inside a config's seed space
_T_Q, _T_K, _T_V = 1, 2, 3
_T_OFF = 10          # + tensor id: block offsets
_T_CHAN = 20         # channel log-scales (V)
_T_KEEP = 30         # block keep mask
_T_LENS = 99         # varlen lengths


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def _draw_head(base: int, tid: int, b: int, n: int, S: int, D: int, recipe: str) -> np.ndarray:
    """One (batch, head) slice [S, D] in float32 before bf16 rounding."""
    x = _rng(base, tid, b, n).standard_normal((S, D), dtype=np.float32)
    if recipe in ("block_offset", "block_offset_channel"):
        nblk = (S + BLOCK - 1) // BLOCK
        off = _rng(base, _T_OFF + tid, b, n).standard_normal((nblk, D), dtype=np.float32) * np.float32(0.5)
        x += np.repeat(off, BLOCK, axis=0)[:S]
    if recipe == "block_offset_channel":
        g = _rng(base, _T_CHAN, b, n).standard_normal(D, dtype=np.float32)
        x *= np.exp(g).astype(np.float32)[None, :]
    elif recipe not in ("normal", "block_offset"):
        raise ValueError(f"unknown recipe {recipe}")
    return x


def random_bf16(seed: int, shape, recipe: str = "normal") -> np.ndarray:
    """bf16 bits of an arbitrary-shape tensor: N(0, 1) values (``normal``) or
    N(0, 1) plus a per-(leading index, 128-row block) offset N(0, 0.5^2) along
    the second-to-last axis (``block_offset``)."""
    shape = tuple(int(s) for s in shape)
    x = _rng(seed, 0).standard_normal(shape, dtype=np.float32)
    if recipe == "block_offset":
        S = shape[-2]
        nblk = (S + BLOCK - 1) // BLOCK
        off = _rng(seed, _T_OFF).standard_normal(shape[:-2] + (nblk, shape[-1]), dtype=np.float32) * np.float32(0.5)
        x += np.repeat(off, BLOCK, axis=-2)[..., :S, :]
    elif recipe != "normal":
        raise ValueError(f"unknown recipe {recipe}")
    return f32_to_bf16_bits(x)


def random_f16(seed: int, shape, recipe: str = "normal") -> np.ndarray:
    """float16 values of an arbitrary-shape tensor (the recipes of ``random_bf16``, drawn in
    float32 from the same seed and rounded once, to nearest-even, to IEEE binary16)."""
    shape = tuple(int(s) for s in shape)
    x = _rng(seed, 0).standard_normal(shape, dtype=np.float32)
    if recipe == "block_offset":
        S = shape[-2]
        nblk = (S + BLOCK - 1) // BLOCK
        off = _rng(seed, _T_OFF).standard_normal(shape[:-2] + (nblk, shape[-1]), dtype=np.float32) * np.float32(0.5)
        x += np.repeat(off, BLOCK, axis=-2)[..., :S, :]
    elif recipe != "normal":
        raise ValueError(f"unknown recipe {recipe}")
    return x.astype(np.float16)


def make_block_keep(base: int, B: int, N: int, QB: int, KB: int, p_keep: float,
                    heads: Optional[list] = None) -> np.ndarray:
    """Block keep mask uint8 [B, N, QB, KB] (1 = keep); diagonal always kept."""
    heads = list(range(N)) if heads is None else list(heads)
    keep = np.zeros((B, len(heads), QB, KB), dtype=np.uint8)
    diag = np.arange(min(QB, KB))
    for b in range(B):
        for j, n in enumerate(heads):
            m = _rng(base, _T_KEEP, b, n).random((QB, KB)) < p_keep
            m[diag, diag] = True
            keep[b, j] = m
    return keep


def varlen_lengths(base: int, nseq: int, lo: int, hi: int) -> np.ndarray:
    """Sequence lengths uniform on the integers [lo, hi]."""
    return _rng(base, _T_LENS).integers(lo, hi + 1, size=nseq).astype(np.int64)


@dataclasses.dataclass
class Workload:
    name: str
    kind: str                 # "dense" | "blocksparse" | "qbsa"
    layout: str               # "BNSD" | "TND"
    B: int
    Nq: int
    Nkv: int
    Sq: int                   # BNSD length, or total tokens T for TND
    Skv: int
    D: int
    scale: float
    sparse_mode: int          # 0 none, 2 causal top-left, 3 causal bottom-right
    q: np.ndarray             # bf16 bits, layout-shaped
    k: np.ndarray
    v: np.ndarray
    heads: list               # q-heads generated (all, unless a subset was asked for)
    cu_seqlens_q: Optional[np.ndarray] = None   # int32 [B+1] (TND)
    cu_seqlens_kv: Optional[np.ndarray] = None
    keep: Optional[np.ndarray] = None           # uint8 [B, len(heads), QB, KB]
    p_keep: Optional[float] = None
    description: str = ""


# The five workloads: a small dense case, the 8K dense operator shape, a causal
# GQA varlen batch, 64K block-sparse at sparsity 0.9 and the 60K-token
# quantised block-sparse case at sparsity 0.63.
CONFIGS = {
    "c1_dense_small": dict(kind="dense", layout="BNSD", B=1, Nq=2, Nkv=2, S=256, D=64,
                           recipe_qk="normal", recipe_v="normal", seed=1001,
                           description="dense B=1 N=2 S=256 D=64 BNSD, N(0,1), no mask"),
    "c2_dense_8k": dict(kind="dense", layout="BNSD", B=1, Nq=40, Nkv=40, S=8192, D=128,
                        recipe_qk="normal", recipe_v="normal", seed=1002,
                        description="dense B=1 N=40 S=8192 D=128 BNSD, N(0,1), no mask"),
    "c3_varlen_gqa_causal": dict(kind="dense", layout="TND", B=8, Nq=32, Nkv=8, D=128,
                                 len_lo=512, len_hi=4096, sparse_mode=3,
                                 recipe_qk="normal", recipe_v="normal", seed=1003,
                                 description="TND varlen, 8 sequences U[512,4096], Nq=32 Nkv=8 D=128, "
                                             "bottom-right causal"),
    "c4_blocksparse_64k": dict(kind="blocksparse", layout="BNSD", B=1, Nq=40, Nkv=40, S=65536, D=128,
                               recipe_qk="block_offset", recipe_v="block_offset", p_keep=0.1, seed=1004,
                               description="block-sparse B=1 N=40 S=65536 D=128, 128x128 blocks, "
                                           "diagonal + p=0.1 (sparsity 0.9)"),
    "c5_qbsa_60k": dict(kind="qbsa", layout="BNSD", B=1, Nq=40, Nkv=40, S=61440, D=128,
                        recipe_qk="block_offset", recipe_v="block_offset_channel", p_keep=0.37, seed=1005,
                        description="quantised block-sparse B=1 N=40 S=61440 D=128, INT8 Q/K per block, "
                                    "FP8 V per channel, diagonal + p=0.37 (sparsity 0.63)"),
}


def make_workload(name: str, *, S: Optional[int] = None, N: Optional[int] = None,
                  Nkv: Optional[int] = None, D: Optional[int] = None, B: Optional[int] = None,
                  heads: Optional[list] = None, lengths: Optional[list] = None,
                  sparse_mode: Optional[int] = None, p_keep: Optional[float] = None,
                  seed: Optional[int] = None) -> Workload:
    """Build a workload by name, optionally at a reduced size.

    ``heads`` restricts generation to a subset of q-heads (BNSD only; the
    kv-heads they map to are generated alongside, at the same indices when
    Nq == Nkv). Overrides keep the recipe; the seed stays the config's unless
    ``seed`` is given.
    """
    c = dict(CONFIGS[name])
    base = int(seed if seed is not None else c["seed"])
    D_ = int(D if D is not None else c["D"])
    Nq = int(N if N is not None else c["Nq"])
    Nk = int(Nkv if Nkv is not None else (c["Nkv"] if N is None else (Nq if c["Nq"] == c["Nkv"] else c["Nkv"])))
    if Nq % Nk:
        raise ValueError("Nq must be a multiple of Nkv")
    smode = int(sparse_mode if sparse_mode is not None else c.get("sparse_mode", 0))
    scale = float(1.0 / np.sqrt(D_))
    if c["layout"] == "TND":
        if lengths is None:
            nseq = int(B if B is not None else c["B"])
            lengths = varlen_lengths(base, nseq, c["len_lo"], c["len_hi"])
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        T = int(cu[-1])

        def tnd(tid, nh, recipe):
            out = np.empty((T, nh, D_), dtype=np.uint16)
            for n in range(nh):
                out[:, n, :] = f32_to_bf16_bits(_draw_head(base, tid, 0, n, T, D_, recipe))
            return out

        return Workload(name=name, kind=c["kind"], layout="TND", B=len(lengths), Nq=Nq, Nkv=Nk,
                        Sq=T, Skv=T, D=D_, scale=scale, sparse_mode=smode,
                        q=tnd(_T_Q, Nq, c["recipe_qk"]), k=tnd(_T_K, Nk, c["recipe_qk"]),
                        v=tnd(_T_V, Nk, c["recipe_v"]), heads=list(range(Nq)),
                        cu_seqlens_q=cu, cu_seqlens_kv=cu.copy(), description=c["description"])

    S_ = int(S if S is not None else c["S"])
    B_ = int(B if B is not None else c["B"])
    hq = list(range(Nq)) if heads is None else [int(h) for h in heads]
    group = Nq // Nk
    hk = sorted({h // group for h in hq}) if heads is not None else list(range(Nk))

    def bnsd(tid, hl, recipe):
        out = np.empty((B_, len(hl), S_, D_), dtype=np.uint16)
        for b in range(B_):
            for j, n in enumerate(hl):
                out[b, j] = f32_to_bf16_bits(_draw_head(base, tid, b, n, S_, D_, recipe))
        return out

    keep = None
    pk = None
    if c["kind"] in ("blocksparse", "qbsa"):
        pk = float(p_keep if p_keep is not None else c["p_keep"])
        nb = (S_ + BLOCK - 1) // BLOCK
        keep = make_block_keep(base, B_, Nq, nb, nb, pk, heads=hq)
    return Workload(name=name, kind=c["kind"], layout="BNSD", B=B_, Nq=Nq, Nkv=Nk, Sq=S_, Skv=S_, D=D_,
                    scale=scale, sparse_mode=smode, q=bnsd(_T_Q, hq, c["recipe_qk"]),
                    k=bnsd(_T_K, hk, c["recipe_qk"]), v=bnsd(_T_V, hk, c["recipe_v"]), heads=hq,
                    keep=keep, p_keep=pk, description=c["description"])
