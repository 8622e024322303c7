"""The C ABI's host code under AddressSanitizer (no GPU needed).

qattn_abi.hip is compiled with its host code instrumented (-Xarch_host -fsanitize=address; device
code untouched) and linked with launch stubs (tests/abi_launch_stubs.hip) into a library of its
own. The ABI and binding validation tests (test_abi_cpu.py, test_api_validation.py) then run
against that library in a child process with the sanitizer runtime preloaded: every host-side read
of the descriptor, the cumulative-length and actual-length arrays, and the caller's buffers'
metadata is checked. A second child makes a call that breaks the documented contract (a
300-entry actual_seq_lengths array for B = 301) to show that the sanitizer is live: it must
report the library's read past that array.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_attention_tiled_amd", "csrc")
HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and RUNTIME),
                                reason="hipcc or the clang AddressSanitizer runtime is missing")


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("asan")
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    common = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-c", *inc]
    abi, stubs, lib = d / "abi.o", d / "stubs.o", d / "libqattn_host_asan.so"
    subprocess.run([*common, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                    os.path.join(CSRC, "qattn_abi.hip"), "-o", str(abi)], check=True, capture_output=True)
    subprocess.run([*common, "--cuda-host-only", os.path.join(ROOT, "tests", "abi_launch_stubs.hip"), "-o",
                    str(stubs)], check=True, capture_output=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", str(abi), str(stubs), "-o", str(lib)],
                   check=True, capture_output=True)
    return str(lib)


def _child(code: str):
    env = dict(os.environ, LD_PRELOAD=RUNTIME[-1], ASAN_OPTIONS="detect_leaks=0")
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


def test_validation_suites_clean_under_asan(asan_lib):
    code = (f"import sys; sys.path.insert(0, {ROOT!r})\n"
            "import quantized_attention_tiled_amd._lib as L\n"
            f"L.load({asan_lib!r})\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi_cpu.py', "
            "'tests/test_api_validation.py']))\n")
    r = _child(code)
    assert "AddressSanitizer" not in r.stderr + r.stdout, (r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout


def test_sanitizer_is_live(asan_lib):
    code = (f"import ctypes, sys; sys.path.insert(0, {ROOT!r})\n"
            "import quantized_attention_tiled_amd._lib as L\n"
            f"lib = L.load({asan_lib!r})\n"
            "libc = ctypes.CDLL(None); libc.malloc.restype = ctypes.c_void_p\n"
            "buf = libc.malloc(300 * 4); ctypes.memset(buf, 0, 300 * 4)\n"
            "d = L.QattnDesc(); d.struct_size = ctypes.sizeof(L.QattnDesc)\n"
            "for k, v in dict(layout=0, B=301, Nq=2, Nkv=2, Sq=4, Skv=4, D=128, scale=0.1, head_begin=-1,\n"
            "                 head_end=-1, qblock_begin=-1, qblock_end=-1, pre_tokens=2147483647,\n"
            "                 next_tokens=2147483647).items(): setattr(d, k, v)\n"
            "d.actual_seq_lengths = ctypes.cast(buf, ctypes.POINTER(ctypes.c_int32))\n"
            "lib.attn_fwd(ctypes.byref(d), 0x10000, 0x10000, 0x10000, 0x10000, None, None, None)\n")
    r = _child(code)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr and "setup_common" in r.stderr, r.stderr[-3000:]
