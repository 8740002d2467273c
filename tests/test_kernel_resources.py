"""Every HIP kernel of the library compiles for gfx950 without private
(scratch) memory and without VGPR spills.

The block kernels are tuned to a register budget (two waves per SIMD for
the forward and dQ kernels, one for dK/dV); a change that pushes one over
it does not fail any parity test, it only makes the kernel slow, because
the compiler then spills to scratch or demotes arrays to private memory.
This test compiles each source with the library's own flags (device code
only, to assembly) and reads the code object metadata of every kernel.
No GPU is needed.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from long_context_transformers_amd import build as hip_build

SOURCES = [s for s in hip_build.SOURCES if s != "ra_host.hip"]


def _compile(src, outdir):
    out = os.path.join(outdir, src.replace(".hip", ".s"))
    cmd = [hip_build.HIPCC] + hip_build.flags() + ["--cuda-device-only", "-S",
                                                   os.path.join(hip_build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"hipcc failed on {src}:\n{r.stderr[-2000:]}"
    return out


def _kernel_metadata(asm_text):
    """(name, private_segment_fixed_size, vgpr_spill_count, sgpr_spill_count)
    for every kernel entry of the AMDGPU metadata block."""
    out = []
    for entry in re.split(r"\n  - \.agpr_count:", asm_text.split("amdhsa.kernels:", 1)[-1])[1:]:
        name = re.search(r"\.name:\s+(\S+)", entry)
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", entry)
        vsp = re.search(r"\.vgpr_spill_count:\s+(\d+)", entry)
        ssp = re.search(r"\.sgpr_spill_count:\s+(\d+)", entry)
        if name and priv and vsp:
            out.append((name.group(1), int(priv.group(1)), int(vsp.group(1)), int(ssp.group(1)) if ssp else 0))
    return out


@pytest.mark.skipif(not os.path.exists(hip_build.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not available")
def test_kernels_use_no_scratch_and_do_not_spill():
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(max_workers=4) as ex:
            outs = list(ex.map(lambda s: _compile(s, d), SOURCES))
        kernels = []
        for o in outs:
            with open(o) as f:
                kernels += _kernel_metadata(f.read())
    names = [k[0] for k in kernels]
    for expected in ("fwd_bf16_kernel", "dkdv_kernel", "dq_kernel", "decode_split_kernel", "gemm_nt_kernel",
                     "finalize_kernel", "merge_o_kernel"):
        assert any(expected in n for n in names), f"no kernel matching {expected} found"
    bad = [(n, p, v) for n, p, v, _ in kernels if p != 0 or v != 0]
    assert not bad, "kernels with private memory or VGPR spills (name, private bytes, spilled VGPRs): " + repr(bad)
