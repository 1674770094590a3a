"""Register and scratch use of the forward kernels as built (CPU only).

The forward kernels' speed rests on their register budget: the forms that
run two waves per SIMD (bf16 d = 64 and 128 with 2 to 8 waves per
workgroup, fp8 d <= 128) must fit 256 registers per lane, and no hot-path
form may spill vector registers or use scratch memory (a spilling build of
the fused iteration measured 2-6x slower).  These tests read the AMDGPU
kernel metadata of the gfx950 code objects that build.py compiled, so a
compiler or source change that breaks the budget fails here, before any
GPU run.
"""
import os
import re
import subprocess

import pytest

from exact_attention_07_amd import build

LLVM = "/opt/rocm/llvm/bin"
TOOLS = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

pytestmark = pytest.mark.skipif(not all(os.path.exists(t) for t in TOOLS), reason="ROCm LLVM tools not found")


def _objects():
    objs = {s: os.path.join(build.HERE, "_build", s + ".o") for s in ("fa_fwd.hip", "fa_fwd_fp8.hip")}
    if not all(os.path.exists(o) for o in objs.values()):
        build.build()
    return objs


def kernel_metadata(obj, tmp):
    """{kernel symbol: {metadata key: value}} of the gfx950 code object inside obj."""
    fatbin = os.path.join(tmp, os.path.basename(obj) + ".fatbin")
    dev = os.path.join(tmp, os.path.basename(obj) + ".gfx950.o")
    subprocess.run([TOOLS[0], f"--dump-section=.hip_fatbin={fatbin}", obj], check=True)
    subprocess.run([TOOLS[1], "--type=o", f"--targets={TARGET}", f"--input={fatbin}", f"--output={dev}",
                    "--unbundle"], check=True)
    notes = subprocess.run([TOOLS[2], "--notes", dev], check=True, capture_output=True, text=True).stdout
    # kernel entries of amdhsa.kernels open with "  - .key:", their own keys
    # sit at four spaces; argument lists are nested deeper
    kernels, cur = {}, None
    for line in notes.splitlines():
        m = re.match(r"^  (- |  )\.([a-z_]+):\s+(\S+)", line)
        if not m:
            continue
        opener, key, val = m.groups()
        if opener == "- ":
            cur = {}
        if cur is None:
            continue
        cur[key] = val
        if key == "name":
            kernels[val] = cur
    return kernels


@pytest.fixture(scope="module")
def meta(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("codeobj"))
    return {src: kernel_metadata(obj, tmp) for src, obj in _objects().items()}


BF16 = re.compile(r"fa_fwd_bf16_kernelILi(\d+)ELb(\d)ELi(\d+)ELi(\d+)E")
FP8 = re.compile(r"fa_fwd_fp8_kernelILi(\d+)ELb(\d)ELi(\d+)E")


def _forms(kernels, pattern):
    out = {}
    for name, k in kernels.items():
        m = pattern.search(name)
        if m and not name.endswith(".kd"):
            out[tuple(int(g) for g in m.groups())] = k
    return out


def _regs(k):
    """Registers per lane: .vgpr_count counts the unified VGPR and AGPR file."""
    assert int(k["vgpr_count"]) >= int(k["agpr_count"]), k
    return int(k["vgpr_count"])


def test_metadata_lists_every_instantiation(meta):
    bf16, fp8 = _forms(meta["fa_fwd.hip"], BF16), _forms(meta["fa_fwd_fp8.hip"], FP8)
    for d in (64, 128, 256):
        for causal in (0, 1):
            assert (d, causal, 4, 0) in bf16 and (d, causal, 4) in fp8
    assert (128, 1, 8, 0) in bf16 and (128, 0, 8, 0) in bf16


@pytest.mark.parametrize("d,nw", [(64, 2), (64, 4), (128, 4), (128, 8)])
@pytest.mark.parametrize("causal", [0, 1])
def test_two_wave_bf16_forms_fit_without_spills(meta, d, nw, causal):
    k = _forms(meta["fa_fwd.hip"], BF16)[(d, causal, nw, 0)]
    assert k["private_segment_fixed_size"] == "0", k
    assert k["vgpr_spill_count"] == "0", k
    assert _regs(k) <= 256, k


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_two_wave_fp8_forms_fit_without_spills(meta, d, causal):
    k = _forms(meta["fa_fwd_fp8.hip"], FP8)[(d, causal, 4)]
    assert k["private_segment_fixed_size"] == "0", k
    assert k["vgpr_spill_count"] == "0", k
    assert _regs(k) <= 256, k


@pytest.mark.parametrize("causal", [0, 1])
def test_head_dim_256_forms_use_no_scratch(meta, causal):
    """One wave per SIMD at d = 256: more than 256 registers, the overflow
    kept in AGPRs, never in scratch memory."""
    for k in (_forms(meta["fa_fwd.hip"], BF16)[(256, causal, 4, 0)], _forms(meta["fa_fwd_fp8.hip"], FP8)[(256, causal, 4)]):
        assert k["private_segment_fixed_size"] == "0", k
        assert _regs(k) <= 512, k
