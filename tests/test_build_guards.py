"""Compile-time guards for properties the kernels rely on (CPU only).

The direct-to-LDS pipelines wait for their tiles with explicit
`s_waitcnt vmcnt(N)`, where N counts the vector-memory instructions a
wavefront issues after the tile's loads.  Register spills (scratch loads and
stores are vector-memory instructions too) would change that count, and the
inline-asm loads clobber M0, which must therefore not carry anything else.
"""
import os
import re
import subprocess
import tempfile

import pytest

from attention_sink_fwd_amd.build import FLAGS, HIPCC

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_sink_fwd_amd", "csrc")


def _asm(source):
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
        cmd = [HIPCC, *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-S",
               "--cuda-device-only", os.path.join(CSRC, source), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def _kernels(asm):
    """{kernel symbol: body text} for every kernel in the assembly."""
    out = {}
    for m in re.finditer(r"^(_Z\S+):\s*(?:;.*)?$", asm, flags=re.M):
        name = m.group(1)
        end = asm.find(".Lfunc_end", m.end())
        out[name] = asm[m.end():end]
    return out


@pytest.mark.parametrize("source", ["fwd_kernel.hip", "bwd_kernels.hip"])
def test_no_scratch_and_m0_only_in_dma_blocks(source):
    asm = _asm(source)
    kernels = _kernels(asm)
    assert kernels, "no kernels found"
    for name, body in kernels.items():
        assert "scratch_" not in body, f"{name} spills registers"
        lines = [l.strip() for l in body.splitlines()]
        for i, line in enumerate(lines):
            if re.search(r"\bm0\b", line) and not line.startswith(";"):
                ok = (line.startswith("s_mov_b32 m0,") and lines[i + 1] == "s_nop 0"
                      and "global_load_lds" in lines[i + 2])
                ok = ok or line.startswith("global_load_lds")
                assert ok, f"{name}: unexpected use of M0: {line}"
    for m in re.finditer(r"\.private_segment_fixed_size:\s+(\d+)", asm):
        assert int(m.group(1)) == 0
