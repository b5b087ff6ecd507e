"""Resource checks of the hot kernels, from their gfx950 code objects (CPU only).

The bf16 sampling step kernels run five wavefronts per SIMD, which their
register count allows only up to 96 VGPRs; the wide LM-head kernel needs its
128 KiB of LDS and at most 256 VGPRs (two wavefronts per SIMD).  No kernel may
keep anything in scratch memory: a private array (for instance an accumulator
indexed at run time) or a VGPR spill would move to scratch and slow every step
without changing a result, so only these checks would notice.  SGPR spills go
to VGPR lanes, not memory, and are allowed.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_verification_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _kernels(source, tmp_path):
    """{kernel name: metadata fields} of one source's device code."""
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc is not available")
    out = tmp_path / (source + ".s")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "--offload-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, source), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    meta = text[text.index("amdhsa.kernels"):]
    kernels = {}
    for blk in meta.split("  - .agpr_count")[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk).group(1)
        fields = {}
        for key in ("vgpr_count", "vgpr_spill_count", "private_segment_fixed_size",
                    "group_segment_fixed_size"):
            m = re.search(r"\." + key + r":\s+(\d+)", blk)
            fields[key] = int(m.group(1)) if m else 0
        kernels[name] = fields
    assert kernels, "no kernels found"
    return kernels


def _no_scratch(kernels):
    for name, f in kernels.items():
        assert f["private_segment_fixed_size"] == 0, f"{name} uses scratch memory"
        assert f["vgpr_spill_count"] == 0, f"{name} spills VGPRs"


def test_step_kernels(tmp_path):
    kernels = _kernels("isd_step.hip", tmp_path)
    _no_scratch(kernels)
    # bf16, aligned rows, sample mode: the default, Gumbel-max, one-hot and both variants
    sampling = [n for n in kernels if "step_kernel" in n and "ItLb1ELi0EL" in n]
    assert len(sampling) == 4, sorted(kernels)
    for n in sampling:
        assert kernels[n]["vgpr_count"] <= 96, (n, kernels[n])


def test_lm_head_kernels(tmp_path):
    kernels = _kernels("isd_lm_head.hip", tmp_path)
    _no_scratch(kernels)
    wide = [n for n in kernels if "lm_head_pp_kernel" in n]
    # plain, two-segment and statistics, each also with the K-split tail
    assert len(wide) == 6, sorted(kernels)
    for n in wide:
        assert kernels[n]["group_segment_fixed_size"] == 128 * 1024, kernels[n]
        assert kernels[n]["vgpr_count"] <= 256, kernels[n]
