"""Code-generation guards for the HIP kernels (CPU only: hipcc cross-compiles
gfx950 assembly here).  They catch the performance regressions that tests of
results cannot see:
  * a buffer descriptor the compiler cannot prove uniform makes it wrap every
    buffer load in a readfirstlane loop ("waterfall"), which once slowed the
    ragged batch by a fifth;
  * register spills to scratch memory;
  * a kernel with one row tile that no longer fits twice on a CU (at most
    80 KiB of LDS and 256 VGPRs), which the INT8 batch, the masked scan and
    the short D=256 layers need for their speed."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRCS = [os.path.join(ROOT, "decode_attention_flash_amd", "csrc", name) for name in ("ck_decode_attn.hip", "ck_topk.hip")]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    text = ""
    for n, src in enumerate(SRCS):
        out = tmp_path_factory.mktemp("asm") / f"k{n}.s"
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
               src, "-o", str(out)]
        subprocess.run(cmd, check=True, capture_output=True)
        text += out.read_text()
    return text


def kernels(text):
    names = re.findall(r"^(_ZN4ck(?:da|tk)\w+):", text, flags=re.M)
    for n in names:
        i = text.index(n + ":")
        j = text.index(".Lfunc_end", i)
        yield n, text[i:j]


def test_decode_kernels_have_no_waterfall_loops(asm):
    found = 0
    for name, body in kernels(asm):
        if "decode_kernel" not in name:
            continue
        found += 1
        n_rfl = body.count("v_readfirstlane")
        assert n_rfl <= 40, f"{name}: {n_rfl} v_readfirstlane (a per-lane buffer descriptor?)"
    # D 128 and 256, modes 0-3: one row tile alone or in shared groups, two
    # row tiles; plus the VALU contractions (dot2 and fp32, 4 or 8 rows) for
    # modes 0 and 2, and the phase-stamping instance of plain decode
    assert found == 42


def test_no_scratch_spills(asm):
    n = 0
    for name, body in kernels(asm):
        n += 1
        assert "scratch_store" not in body and "scratch_load" not in body, f"{name}: spills to scratch"
    assert n >= 19


def kernel_resources(text):
    """(LDS bytes, VGPRs incl. AGPRs) per kernel, from the code object metadata."""
    meta = text[text.index("amdhsa.kernels:"):]
    res = {}
    for block in meta.split("\n  - ")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        lds = re.search(r"\.group_segment_fixed_size:\s+(\d+)", block)
        vgpr = re.search(r"\.vgpr_count:\s+(\d+)", block)
        if name and lds and vgpr:
            res[name.group(1)] = (int(lds.group(1)), int(vgpr.group(1)))
    return res


def test_one_row_tile_kernels_fit_twice_per_cu(asm):
    res = kernel_resources(asm)
    found = 0
    for name, (lds, vgpr) in res.items():
        if not re.search(r"decode_kernelILi(128|256)ELi1E", name):
            continue
        found += 1
        assert lds <= 80 * 1024, f"{name}: {lds} bytes of LDS, two workgroups no longer fit on a CU"
        assert vgpr <= 256, f"{name}: {vgpr} VGPRs, two waves no longer fit on a SIMD"
    # D 128 and 256, modes 0-3, alone or in shared groups; VALU (dot2 and
    # fp32) 4 and 8 rows, modes 0 and 2; phase stamps
    assert found == 34
