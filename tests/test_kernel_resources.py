"""Build invariants of the gfx950 kernels, checked from the compiler's resource report (hipcc
cross-compiles here; no GPU needed).

* No kernel keeps data in private (scratch) memory, except the boolean-mask instantiations of the
  16-bit kernel, whose per-element mask loads spill a few dozen registers. Scratch use elsewhere has
  meant an outlined lambda that demoted the kernel arguments and register arrays to memory.
* Both attention kernels run two waves per SIMD (at most 256 VGPRs). A forward workgroup of one
  q-block (four waves) uses at most 80 KiB of LDS, so that two share a CU; one of two q-blocks
  (eight waves, the CU's only workgroup) at most 160 KiB. The exception is the 16-bit forward
  built for head dimension 256: one q-block, one wave per SIMD (its Q^T and O^T registers alone
  take 192 VGPRs), the CU's only workgroup, its extra registers in AGPRs rather than scratch.
"""

import functools
import os
import re
import shutil
import subprocess

import pytest

from quantized_attention_tiled_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")

MASK_MODES = {2, 3}  # kMask, kCausal | kMask


@functools.lru_cache(maxsize=None)
def _compile(src):
    """Device assembly and per-kernel resource report of one source (one hipcc run)."""
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           f"-I{B.INCLUDE}", f"-I{B.CSRC}", *B.DEVICE_FLAGS, *B.SOURCE_FLAGS.get(src, []),
           os.path.join(B.CSRC, src), "-o", "-", "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = {}
    cur = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return kernels, r.stdout


def _resources(src):
    return _compile(src)[0]


FWD_SOURCES = ["attn_fwd_bf16.hip", "attn_fwd_f16.hip"]
# element type, D, Dv, mode, q-blocks per workgroup
FWD_NAME = re.compile(r"attn_fwd_kernelI(DF16b|DF16_)Li(\d+)ELi(\d+)ELi(\d+)ELi(\d+)EEE")


@pytest.fixture(scope="module", params=FWD_SOURCES)
def fwd(request):
    return _resources(request.param)


def test_fwd_instantiations(fwd):
    """Each element type gets every (D, Dv) pair in all eleven modes."""
    shapes = set()
    for name in fwd:
        m = FWD_NAME.search(name)
        assert m, name
        shapes.add((int(m.group(2)), int(m.group(3)), int(m.group(4))))
    # 18, 19: kMask (| kCausal) | kMaskTile; 50, 51: the same with kMaskBits (bit-packed masks)
    modes = [0, 1, 2, 3, 4, 8, 9, 18, 19, 50, 51]
    assert shapes == {(d, dv, mode) for d, dv in [(64, 64), (128, 128), (128, 64), (256, 128)] for mode in modes}
    assert len({FWD_NAME.search(n).group(1) for n in fwd}) == 1


def test_fwd_kernels_use_no_scratch(fwd):
    assert fwd, "no kernels reported"
    for name, res in fwd.items():
        mode = int(FWD_NAME.search(name).group(4))
        if mode in MASK_MODES:
            continue
        assert res.get("ScratchSize", 0) == 0, (name, res)
        if int(FWD_NAME.search(name).group(2)) <= 128:
            assert res.get("VGPRs Spill", 0) == 0, (name, res)


def test_fwd_two_waves_per_simd_and_lds(fwd):
    for name, res in fwd.items():
        m = FWD_NAME.search(name)
        d, nqb = int(m.group(2)), int(m.group(5))
        if d > 128:
            assert nqb == 1 and res.get("Occupancy", 0) == 1, (name, res)
            assert res.get("LDS Size", 0) <= 160 * 1024, (name, res)
            continue
        assert res.get("Occupancy", 0) >= 2, (name, res)
        assert res.get("LDS Size", 0) <= (80 if nqb == 1 else 160) * 1024, (name, res)


@pytest.fixture(scope="module")
def qbsa():
    return _resources("attn_qbsa.hip")


def test_qbsa_kernels_use_no_scratch(qbsa):
    assert qbsa, "no kernels reported"
    for name, res in qbsa.items():
        assert res.get("ScratchSize", 0) == 0, (name, res)
        assert res.get("VGPRs Spill", 0) == 0, (name, res)


def test_qbsa_two_waves_per_simd_and_lds(qbsa):
    for name, res in qbsa.items():
        assert res.get("Occupancy", 0) >= 2, (name, res)
        assert res.get("LDS Size", 0) <= 80 * 1024, (name, res)


def test_quant_kernels_use_no_scratch():
    ks = _resources("quant.hip")
    assert ks
    for name, res in ks.items():
        assert res.get("ScratchSize", 0) == 0, (name, res)


def _asm(src):
    return _compile(src)[1]


BWD_NAME = re.compile(r"bwd_(dq|dkdv)_kernelI(DF16b|DF16_)Li(\d+)ELi(\d+)EEE")


def test_bwd_kernels_use_no_scratch_and_fit():
    """The backward kernels keep everything in registers, except the boolean-mask instantiations
    of the dQ kernel, whose per-element mask bytes spill a few dozen registers; the dQ kernel runs
    two workgroups per CU (two waves per SIMD, 64 KiB of LDS each), the dK/dV kernel one (its
    accumulators take up to 512 registers per lane)."""
    ks = _resources("attn_bwd.hip")
    # preparation (2 D x 2 types), dQ and dK/dV (4 modes x 2 D x 2 types each)
    assert len(ks) == 4 + 2 * 16, list(ks)
    for name, res in ks.items():
        m = BWD_NAME.search(name)
        if m and int(m.group(4)) in MASK_MODES:
            continue
        assert res.get("ScratchSize", 0) == 0, (name, res)
        assert res.get("VGPRs Spill", 0) == 0, (name, res)
        if "bwd_dq_kernel" in name:
            assert res.get("Occupancy", 0) >= 2 and res.get("LDS Size", 0) <= 80 * 1024, (name, res)
        if "bwd_dkdv_kernel" in name:
            assert res.get("Occupancy", 0) >= 1 and res.get("LDS Size", 0) <= 160 * 1024, (name, res)


@pytest.mark.parametrize("src", FWD_SOURCES + ["attn_qbsa.hip", "attn_bwd.hip"])
def test_m0_only_feeds_direct_lds_loads(src):
    """The direct HBM -> LDS loads set M0 in inline asm, where the compiler does not preserve it:
    no other instruction of these kernels may read or write M0."""
    lines = [ln.split(";")[0].strip() for ln in _asm(src).splitlines()]
    lines = [ln for ln in lines if ln and not ln.startswith((".", "//"))]
    uses = 0
    for i, ln in enumerate(lines):
        if not re.search(r"\bm0\b", ln):
            continue
        uses += 1
        assert re.match(r"s_mov_b32 m0, s\d+$", ln), ln
        nxt = [x for x in lines[i + 1:i + 4] if not x.startswith("s_nop")]
        assert nxt and re.match(r"buffer_load_dword(x4)? .* offen lds$", nxt[0]), (ln, lines[i + 1:i + 4])
    assert uses > 0
