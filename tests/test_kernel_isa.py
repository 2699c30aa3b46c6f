"""Checks on the gfx950 assembly of every kernel source, compiled here with the library's
own flags (no GPU needed):

* every buffer instruction takes its resource descriptor from SGPRs.  The GEMM issues its
  global -> LDS loads from inline assembly whose descriptor operand is constrained to
  scalar registers; a descriptor the compiler computes in vector registers still fills
  that operand, and the load then runs on whatever the encoding points at;
* no kernel spills to scratch (the fused-quantization experiment excepted);
* no packed fp32 arithmetic (v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32) in device code.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from microscaled_fp4_quantization_block_amd import build as B

SOURCES = [s for s in B.SOURCES + B.PROBE_SOURCES if s.endswith(".hip")]


def _have_hipcc():
    try:
        return os.path.exists(B.hipcc())
    except RuntimeError:
        return False


pytestmark = pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")


def _asm(src):
    out = os.path.join(B.BUILD, os.path.splitext(src)[0] + ".isa.s")
    os.makedirs(B.BUILD, exist_ok=True)
    cmd = [B.hipcc(), *B.flags(), "--cuda-device-only", "-S", "-x", "hip", os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def isa():
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        return dict(zip(SOURCES, ex.map(_asm, SOURCES)))


def _instructions(text):
    for line in text.splitlines():
        line = line.split(";", 1)[0].strip()
        if line and not line.startswith(".") and not line.endswith(":"):
            yield line


def test_buffer_descriptors_are_scalar(isa):
    """Operands: vdata, vaddr, srsrc, soffset -- or, loading straight into LDS, vaddr,
    srsrc, soffset.  The descriptor must be a range of four SGPRs."""
    n = 0
    for src, text in isa.items():
        for ins in _instructions(text):
            if not ins.startswith("buffer_"):
                continue
            n += 1
            ops = [o.strip() for o in ins.split(None, 1)[1].split(",")]
            rsrc = ops[1] if re.search(r"\blds\b", ops[-1]) else ops[2]
            m = re.fullmatch(r"s\[(\d+):(\d+)\]", rsrc)
            assert m and int(m.group(2)) - int(m.group(1)) == 3, f"{src}: descriptor operand of '{ins}'"
    assert n > 0


#: the fused-quantization experiment keeps the activation quantization's registers beside
#: the GEMM's 128 accumulators per lane and spills; its measurement includes that traffic
SPILL_ALLOWED = {"gemm_fused.hip"}


def test_no_scratch(isa):
    for src, text in isa.items():
        if src in SPILL_ALLOWED:
            continue
        sizes = [int(v) for v in re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", text)]
        assert sizes and max(sizes) == 0, f"{src}: a kernel uses {max(sizes)} bytes of scratch"


def test_no_packed_fp32(isa):
    for src, text in isa.items():
        bad = [i for i in _instructions(text) if re.match(r"v_pk_(add|mul|fma)_f32\b", i)]
        assert not bad, f"{src}: {bad[:3]}"


def test_m0_only_around_the_lds_dma(isa):
    """The GEMM's global -> LDS loads set M0 inside their own asm statement and list it as
    clobbered.  M0 is a register the compiler reserves, so it does not promise to keep a
    value of its own in M0 across such a statement: check that no compiler-generated
    instruction uses M0 at all, i.e. every M0 reference is an asm `s_mov_b32 m0, ...`
    directly followed by its `s_nop 0` and the `buffer_load ... lds`."""
    for src, text in isa.items():
        ins = list(_instructions(text))
        for i, line in enumerate(ins):
            if not re.search(r"\bm0\b", line):
                continue
            assert line.startswith("s_mov_b32 m0,"), f"{src}: compiler use of M0: '{line}'"
            assert ins[i + 1] == "s_nop 0" and re.match(r"buffer_load_dwordx4 .* lds$", ins[i + 2]), \
                f"{src}: M0 write not followed by its LDS DMA: {ins[i:i + 3]}"
