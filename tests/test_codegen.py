"""Code-generation guards for the HIP kernels (CPU only: hipcc cross-compiles
gfx950 assembly here).  They catch the performance regressions that tests of
results cannot see:
  * a buffer descriptor the compiler cannot prove uniform makes it wrap every
    buffer load in a readfirstlane loop ("waterfall"), which once slowed the
    ragged batch by a fifth;
  * register spills to scratch memory."""
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
    assert found == 16


def test_no_scratch_spills(asm):
    n = 0
    for name, body in kernels(asm):
        n += 1
        assert "scratch_store" not in body and "scratch_load" not in body, f"{name}: spills to scratch"
    assert n >= 19
