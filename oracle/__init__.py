"""CPU oracle for micro-scaled FP4 quantization (plain float64 numpy).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import anything here.  It shares no code, table or
constant with the HIP library and imports nothing from it.  Every function evaluates
the definition it cites in the plainest way (float64, whole-array steps, a matmul or a
sort as library primitives), without blocking, fusion or reordering.

Modules
-------
formats    E2M1 / E4M3 / E8M0 encode and decode, nibble packing, bf16 rounding
hadamard   Sylvester block Hadamard (16/32) and the two-level 16 x 8 FWHT of 128-groups
nvfp4      NVFP4 (E4M3 per 16 + binary32 tensor scale) quantize / dequantize
mxfp4      MXFP4 (E8M0 per 32) quantize / dequantize with optional rotation
dualscale  FP4Quant micro-grouped dual-scale pack / unpack (binary32 per 128 + E4M3 per 16)
arcquant   ARCQuant RMSNorm + reorder + primary and residual NVFP4, [K | S] layout
gemm       W4A4 MXFP4 GEMM of dequantized operands, float64 accumulation

Parity status: every function is pinned by tests/test_oracle_*.py against closed forms,
library routines (torch's float8_e4m3fn cast, numpy's half-to-even rounding), brute
force in exact rational arithmetic, and invariants.  The ARCQuant "alignment overhead"
constant quoted on its page is not modelled (parity unpinned: the page does not define
the quantity).
"""
from . import formats, hadamard, nvfp4, mxfp4, dualscale, arcquant, gemm  # noqa: F401
