"""Code generation checks for the gfx950 kernels (CPU only, needs hipcc).

The device assembly must contain no scalar-memory writes or atomics (all
stores go through vector memory), no packed fp32 arithmetic (the build
disables it), and the hot kernels must not use scratch memory.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "draft_tree_retrieval_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

SCALAR_WRITE = re.compile(r"^\s+s_(store|atomic|dcache_wb|buffer_store|scratch_store)", re.M)
PACKED_F32 = re.compile(r"^\s+v_pk_(add|mul|fma)_f32", re.M)


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not HIPCC:
        pytest.skip("hipcc not available")
    from draft_tree_retrieval_amd.build import FLAGS
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in ("k_topk.hip", "k_small.hip", "k_attn.hip"):
        dst = d / (src + ".s")
        flags = [f for f in FLAGS if f not in ("-fPIC", "-Wall")]
        subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src),
                        "-o", str(dst)], check=True, capture_output=True)
        out[src] = dst.read_text()
    return out


def kernels(text):
    """name -> metadata block of every kernel in an assembly file."""
    res = {}
    for blk in re.split(r"\n\s+- \.agpr_count", text)[1:]:
        m = re.search(r"\.name:\s+(\S+)", blk)
        if m:
            res[m.group(1)] = blk
    return res


def field(blk, key):
    m = re.search(r"\.%s:\s+(\d+)" % key, blk)
    return int(m.group(1)) if m else None


def test_no_scalar_memory_writes(asm):
    for src, text in asm.items():
        assert not SCALAR_WRITE.search(text), src


def test_no_packed_fp32(asm):
    for src, text in asm.items():
        assert not PACKED_F32.search(text), src


def test_hot_kernels_use_no_scratch(asm):
    hot = {**kernels(asm["k_topk.hip"]), **kernels(asm["k_attn.hip"])}
    assert len(hot) >= 6
    for name, blk in hot.items():
        assert field(blk, "private_segment_fixed_size") == 0, name
        assert field(blk, "vgpr_spill_count") == 0, name
