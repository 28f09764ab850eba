"""The pipelined W4A4 GEMMs issue their LDS DMAs through inline assembly that
writes M0 (the DMA's LDS base).  M0 is a register the compiler reserves and
does not preserve around inline assembly, so this is only sound while
nothing else in that kernel uses M0.  Compile the GEMM source for gfx950 and
check, in the kernel's AMD assembly, that every M0 access is one of those
DMA sequences: an M0 write, one wait state, the DMA."""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "mxfp4_activation_quantizer_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _kernel_body(asm: str, name: str) -> list:
    start = re.search(rf"^{re.escape(name)}:", asm, re.M)
    assert start, f"{name} not in the assembly"
    end = asm.find(".Lfunc_end", start.end())
    return [l.split(";")[0].strip() for l in asm[start.end():end].splitlines()]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_pipelined_gemm_m0_only_in_dma_sequences(tmp_path):
    out = tmp_path / "kq_gemm.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, "kq_gemm.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    asm = out.read_text()
    names = re.findall(r"^(_ZN2kq21w4a4_gemm_pipe_kernel\w*):", asm, re.M)
    assert len(names) == 2, names  # fixed and moving stage mapping
    for name in names:
        body = [l for l in _kernel_body(asm, name) if l and not l.startswith((".", "//"))]
        dmas = 0
        for i, line in enumerate(body):
            if not re.search(r"\bm0\b", line):
                continue
            assert line.startswith("s_mov_b32 m0,"), f"{name}: M0 used outside a DMA sequence: {line!r}"
            assert body[i + 1] == "s_nop 0", f"{name}: no wait state after the M0 write: {body[i + 1]!r}"
            assert body[i + 2].startswith("global_load_lds_dwordx4"), \
                f"{name}: M0 write not followed by a DMA: {body[i + 2]!r}"
            dmas += 1
        # and every DMA of the kernel comes from such a sequence
        assert dmas > 0
        assert dmas == sum(1 for l in body if l.startswith("global_load_lds"))


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_wide_gemm_m0_only_in_dma_sequences_and_no_scratch(tmp_path):
    """The 256 x 256-tile GEMM issues its LDS DMAs (buffer loads of 16-byte
    code chunks and 4-byte scale words with an LDS destination) the same way;
    it must also keep every value in registers, since its explicit vmcnt
    waits count only its own DMAs."""
    out = tmp_path / "kq_gemm_wide.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, "kq_gemm_wide.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    asm = out.read_text()
    names = re.findall(r"^(_ZN2kq4wide16gemm_wide_kernel\w*):", asm, re.M)
    assert len(names) == 1, names
    body = [l for l in _kernel_body(asm, names[0]) if l and not l.startswith((".", "//"))]
    is_dma = lambda l: re.match(r"buffer_load_dword(x4)?\b.*\blds$", l) is not None
    dmas = 0
    for i, line in enumerate(body):
        if not re.search(r"\bm0\b", line):
            continue
        assert line.startswith("s_mov_b32 m0,"), f"M0 used outside a DMA sequence: {line!r}"
        assert body[i + 1] == "s_nop 0", f"no wait state after the M0 write: {body[i + 1]!r}"
        assert is_dma(body[i + 2]), f"M0 write not followed by a DMA: {body[i + 2]!r}"
        dmas += 1
    assert dmas > 0
    assert dmas == sum(1 for l in body if is_dma(l))
    # no memory traffic besides the DMAs and the output stores
    assert not any(l.startswith(("scratch_", "buffer_store")) for l in body), \
        "the wide GEMM kernel spills to scratch"
    assert all(is_dma(l) for l in body if l.startswith("buffer_load"))
    m = re.search(r"\.private_segment_fixed_size:\s+(\d+)", asm)
    assert m and int(m.group(1)) == 0
