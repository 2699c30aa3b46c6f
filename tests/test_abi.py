"""Host-side checks of the C ABI: the library loads, exports every function include/fp4.h
declares, and rejects invalid arguments before any HIP call (no compute happens here, so
these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from microscaled_fp4_quantization_block_amd import binding as B
from oracle import dualscale

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4.h")

needs_lib = pytest.mark.skipif(not os.path.exists(B.library_path()),
                               reason="libfp4.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(B.EXPORTED)


@needs_lib
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", B.library_path()], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared():
        assert name in syms, name
    L = B.lib()
    for name in _declared():
        assert hasattr(L, name)


@needs_lib
def test_status_strings():
    L = B.lib()
    for code, name in B._STATUS.items():
        assert L.fp4_status_str(code).decode() == name
    assert L.fp4_status_str(99).decode() == "FP4_E_UNKNOWN"


@needs_lib
def test_pack_bytes_matches_layout():
    L = B.lib()
    for M, K in [(1, 128), (3, 384), (8192, 8192), (7, 1024)]:
        assert L.fp4_pack_bytes(M, K) == dualscale.layout(M, K)["total"]
    assert L.fp4_pack_bytes(4, 100) == 0 and L.fp4_pack_bytes(-1, 128) == 0


FAKE = 0x10000   # never dereferenced: every call below fails validation first
MIS = 0x10008    # 8-byte aligned only


def _status(fn, *args):
    L = B.lib()
    s = getattr(L, fn)(*args)
    return s, L.fp4_last_error().decode()


@needs_lib
@pytest.mark.parametrize("args,want", [
    ((FAKE, 1, 4, 33, 1, 0, FAKE, FAKE, None, 0, None, None), 2),       # K not a multiple of 32
    ((FAKE, 1, -1, 32, 1, 0, FAKE, FAKE, None, 0, None, None), 2),      # negative M
    ((FAKE, 1, 4, 32, 1, 8, FAKE, FAKE, None, 0, None, None), 4),       # unsupported rotation
    ((FAKE, 1, 4, 256, 1, 64, FAKE, FAKE, None, 0, None, None), 4),     # unsupported rotation
    ((FAKE, 1, 4, 96, 1, 128, FAKE, FAKE, None, 0, None, None), 2),     # two-level 128 with K % 128 != 0
    ((FAKE, 1, 4, 32, 2, 0, FAKE, FAKE, None, 0, None, None), 4),       # unknown format
    ((FAKE, 7, 4, 32, 1, 0, FAKE, FAKE, None, 0, None, None), 4),       # unknown dtype
    ((FAKE, 1, 4, 32, 0, 0, FAKE, FAKE, None, 0, None, None), 1),       # NVFP4 without tensor scale
    ((FAKE, 1, 4, 32, 1, 0, FAKE, FAKE, FAKE, 0, None, None), 4),       # MXFP4 with a tensor scale
    ((None, 1, 4, 32, 1, 0, FAKE, FAKE, None, 0, None, None), 1),       # null input
    ((MIS, 1, 4, 32, 1, 0, FAKE, FAKE, None, 0, None, None), 3),        # misaligned input
    ((FAKE, 1, 4, 32, 1, 0, FAKE, FAKE + 2, None, 0, None, None), 3),   # misaligned scales
])
def test_quantize_validation(args, want):
    s, msg = _status("fp4_quantize", *args)
    assert s == want and msg.startswith("fp4_quantize")


@needs_lib
def test_other_entry_points_validation():
    assert _status("fp4_dequantize", FAKE, FAKE, None, 4, 48, 1, 0, FAKE, 0, None)[0] == 2
    assert _status("fp4_dequantize", FAKE, FAKE, None, 4, 64, 0, 0, FAKE, 0, None)[0] == 1
    assert _status("fp4_dequantize", FAKE, FAKE, None, 4, 64, 1, 64, FAKE, 0, None)[0] == 4
    assert _status("fp4_dequantize", FAKE, FAKE, None, 4, 96, 1, 128, FAKE, 0, None)[0] == 2
    args = [FAKE, 4, 64, None, ctypes.c_float(1e-6), FAKE, 16, FAKE, FAKE, FAKE, 0, None, None]
    bad = list(args); bad[6] = 24                                      # S not a multiple of 16
    assert _status("fp4_residual_quantize", *bad)[0] == 2
    bad = list(args); bad[6] = 80                                      # S > K
    assert _status("fp4_residual_quantize", *bad)[0] == 2
    bad = list(args); bad[5] = None                                    # no permutation
    assert _status("fp4_residual_quantize", *bad)[0] == 1
    bad = list(args); bad[2] = 32768                                   # K beyond the LDS row
    assert _status("fp4_residual_quantize", *bad)[0] == 2
    mx = [FAKE, 4, 64, None, ctypes.c_float(1e-6), FAKE, 32, FAKE, FAKE, None, None]
    bad = list(mx); bad[6] = 16                                        # S not a multiple of 32
    assert _status("fp4_residual_quantize_mx", *bad)[0] == 2
    bad = list(mx); bad[2] = 48                                        # K not a multiple of 32
    assert _status("fp4_residual_quantize_mx", *bad)[0] == 2
    bad = list(mx); bad[5] = None
    assert _status("fp4_residual_quantize_mx", *bad)[0] == 1
    bad = list(mx); bad[7] = FAKE + 8                                  # codes not 16-byte aligned
    assert _status("fp4_residual_quantize_mx", *bad)[0] == 3
    assert _status("fp4_pack", FAKE, 4, 100, FAKE, None, None)[0] == 2
    assert _status("fp4_pack", FAKE, 4, 128, FAKE + 16, None, None)[0] == 3
    assert _status("fp4_unpack", None, 4, 128, FAKE, None)[0] == 1
    assert _status("fp4_gemm", FAKE, FAKE, FAKE, FAKE, 4, 4, 100, FAKE, 1, None)[0] == 2
    assert _status("fp4_gemm", FAKE, FAKE, FAKE, FAKE, 4, 4, 0, FAKE, 1, None)[0] == 2
    assert _status("fp4_gemm", FAKE, None, FAKE, FAKE, 4, 4, 128, FAKE, 1, None)[0] == 1
    assert _status("fp4_gemm", FAKE, FAKE, FAKE, FAKE, 4, 4, 128, FAKE, 3, None)[0] == 4


@needs_lib
def test_empty_shapes_are_no_ops():
    # M = 0 returns OK without touching the (null) buffers or the GPU
    assert _status("fp4_quantize", None, 1, 0, 64, 1, 32, None, None, None, 0, None, None)[0] == 0
    assert _status("fp4_dequantize", None, None, None, 0, 64, 1, 0, None, 0, None)[0] == 0
    assert _status("fp4_pack", None, 0, 128, None, None, None)[0] == 0
    assert _status("fp4_residual_quantize_mx", None, 0, 64, None, ctypes.c_float(1e-6), FAKE, 32, None, None,
                   None, None)[0] == 0
    assert _status("fp4_gemm", None, None, None, None, 0, 5, 128, None, 1, None)[0] == 0


def test_missing_library_fails_loudly(monkeypatch):
    """No fallback: without libfp4.so the first call raises instead of computing anywhere else."""
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "_LIB_PATH", os.path.join(ROOT, "no_such_dir", "libfp4.so"))
    with pytest.raises(RuntimeError, match="HIP library missing"):
        B.lib()
    with pytest.raises(RuntimeError, match="HIP library missing"):
        B.fp4_pack_bytes(4, 128)


@needs_lib
def test_injected_launch_failure_reports_hip_status(monkeypatch):
    """FP4_FAULT_INJECT=launch: each entry point that passes validation reports FP4_E_HIP
    through the library's HIP-status mapping, with a readable detail, and enqueues nothing
    (the fake pointers below are never touched, so this runs without a GPU).  Validation
    still decides first, and a clean environment makes the same call validate again."""
    monkeypatch.setenv("FP4_FAULT_INJECT", "launch")
    cases = [
        ("fp4_quantize", (FAKE, 1, 4, 32, 1, 32, FAKE, FAKE, None, 0, None, None)),
        ("fp4_dequantize", (FAKE, FAKE, None, 4, 64, 1, 0, FAKE, 0, None)),
        ("fp4_residual_quantize", (FAKE, 4, 64, None, ctypes.c_float(1e-6), FAKE, 16, FAKE, FAKE, FAKE, 0,
                                   None, None)),
        ("fp4_residual_quantize_mx", (FAKE, 4, 64, None, ctypes.c_float(1e-6), FAKE, 32, FAKE, FAKE, None, None)),
        ("fp4_pack", (FAKE, 4, 128, FAKE, None, None)),
        ("fp4_unpack", (FAKE, 4, 128, FAKE, None)),
        ("fp4_gemm", (FAKE, FAKE, FAKE, FAKE, 4, 4, 128, FAKE, 1, None)),
    ]
    for name, args in cases:
        s, msg = _status(name, *args)
        assert s == 5, (name, s, msg)
        assert msg.startswith(name) and "injected" in msg and len(msg) > len(name) + 12, msg
        assert B.lib().fp4_status_str(s).decode() == "FP4_E_HIP"
    assert _status("fp4_quantize", FAKE, 1, 4, 33, 1, 0, FAKE, FAKE, None, 0, None, None)[0] == 2
    monkeypatch.setenv("FP4_FAULT_INJECT", "none")
    assert _status("fp4_gemm", FAKE, FAKE, FAKE, FAKE, 4, 4, 100, FAKE, 1, None)[0] == 2


PROBE_HEADER = os.path.join(ROOT, "include", "fp4_probe.h")
PROBE_LIB = os.path.join(os.path.dirname(B.library_path()), "libfp4probe.so")


@pytest.mark.skipif(not os.path.exists(PROBE_LIB), reason="libfp4probe.so not built")
def test_probe_library_exports_its_header_and_rejects_bad_arguments():
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(fp4probe_[a-z_]+)\s*\(", text)))
    assert names == ["fp4probe_gemm_fused_a", "fp4probe_hbm_read", "fp4probe_mfma_loop"]
    L = ctypes.CDLL(PROBE_LIB)
    for n in names:
        assert hasattr(L, n)
    L.fp4probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.fp4probe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert L.fp4probe_hbm_read(None, 1024, FAKE, 4, None) == 1
    assert L.fp4probe_hbm_read(FAKE, 1000, FAKE, 4, None) == 1      # not a multiple of 16
    assert L.fp4probe_mfma_loop(10, 3, 4, FAKE, None) == 1            # unknown operand mode
    assert L.fp4probe_mfma_loop(10, 0, 0, FAKE, None) == 1
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.fp4probe_gemm_fused_a.argtypes = [vp, vp, vp, i64, i64, i64, vp, ctypes.c_int, vp]
    assert L.fp4probe_gemm_fused_a(FAKE, FAKE, FAKE, 4, 4, 384, FAKE, 1, None) == 1   # K % 256 != 0
    assert L.fp4probe_gemm_fused_a(None, FAKE, FAKE, 4, 4, 256, FAKE, 1, None) == 1
    assert L.fp4probe_gemm_fused_a(FAKE + 8, FAKE, FAKE, 4, 4, 256, FAKE, 1, None) == 1
    assert L.fp4probe_gemm_fused_a(None, None, None, 0, 4, 256, None, 1, None) == 0  # empty: no-op
