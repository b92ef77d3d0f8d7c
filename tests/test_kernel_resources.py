"""Resource checks on the built gfx950 code objects (CPU only): no kernel of
the library may use private (scratch) memory or spill vector registers.  A
kernel that does would stream far below HBM bandwidth, and an array indexed
at run time that the compiler moved to scratch is easy to miss while every
parity test still passes.  Scalar-register spills are allowed: the rank
pointer arrays (up to 32 + 32 addresses) exceed the scalar register file, and
the compiler keeps the overflow in lanes of a vector register, not in memory
(the private segment stays 0).  The metadata is read from the objects
build.py leaves in allreduce_reduction_nranks_amd/_build."""
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "allreduce_reduction_nranks_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
OBJECTS = sorted(glob.glob(os.path.join(BUILD, "*.hip.o")))


def kernel_metadata(obj, tmp_path):
    """[(kernel name, {key: int})] from the object's gfx950 code object."""
    fatbin = tmp_path / "fatbin"
    co = tmp_path / "code_object"
    dump = subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                           ".hip_fatbin=%s" % fatbin, obj], capture_output=True, text=True)
    if dump.returncode != 0 and "not found" in dump.stderr:
        return []  # host-only object
    dump.check_returncode()
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                    "--targets=" + TARGET, "--input=%s" % fatbin, "--output=%s" % co],
                   check=True, capture_output=True)
    notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", str(co)], check=True,
                           capture_output=True, text=True).stdout
    section = notes[notes.index("amdhsa.kernels:"):]
    kernels = []
    for entry in re.split(r"\n  - ", section)[1:]:
        name = re.search(r"^    \.name:\s+(\S+)", entry, re.M)
        vals = {k: int(v) for k, v in re.findall(
            r"^    \.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count):\s+(\d+)",
            entry, re.M)}
        if name:
            kernels.append((name.group(1), vals))
    return kernels


@pytest.mark.skipif(not OBJECTS or not os.path.exists(os.path.join(LLVM, "clang-offload-bundler")),
                    reason="library objects or ROCm LLVM tools not present")
@pytest.mark.parametrize("obj", OBJECTS, ids=[os.path.basename(o) for o in OBJECTS])
def test_no_kernel_uses_scratch_memory(obj, tmp_path):
    kernels = kernel_metadata(obj, tmp_path)
    if os.path.basename(obj) != "api.hip.o":
        assert kernels, "no kernels found in %s" % obj
    bad = [(n, v) for n, v in kernels
           if v.get("private_segment_fixed_size", 0) or v.get("vgpr_spill_count", 0)]
    assert not bad, "kernels using scratch memory or spilling vector registers: %s" % bad[:5]
