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


def code_object(obj, tmp_path):
    """Path of the object's gfx950 code object, or None for a host-only object."""
    fatbin = tmp_path / "fatbin"
    co = tmp_path / "code_object"
    dump = subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                           ".hip_fatbin=%s" % fatbin, obj], capture_output=True, text=True)
    if dump.returncode != 0 and "not found" in dump.stderr:
        return None
    dump.check_returncode()
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                    "--targets=" + TARGET, "--input=%s" % fatbin, "--output=%s" % co],
                   check=True, capture_output=True)
    return co


def kernel_metadata(obj, tmp_path):
    """[(kernel name, {key: int})] from the object's gfx950 code object."""
    co = code_object(obj, tmp_path)
    if co is None:
        return []
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


PACKET_OBJ = os.path.join(BUILD, "packet.hip.o")


@pytest.mark.skipif(not os.path.exists(PACKET_OBJ) or not os.path.exists(os.path.join(LLVM, "llvm-objdump")),
                    reason="packet object or ROCm LLVM tools not present")
def test_packet_accesses_are_agent_scope(tmp_path):
    """Every 64-bit packet load and store of the polling kernels carries the
    sc1 bit (agent scope): the 8 XCDs have separate L2 caches, and a plain
    cached access could keep reading a stale line of a peer's packets."""
    co = code_object(PACKET_OBJ, tmp_path)
    asm = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", str(co)],
                         check=True, capture_output=True, text=True).stdout
    kernels = re.split(r"\n(?=[0-9a-f]+ <_ZN3mrr)", asm)
    checked = 0
    for k in kernels:
        m = re.match(r"[0-9a-f]+ <(_ZN3mrr\S+)>:", k)
        if not m or not (re.search(r"packet_(allpair|rsag|reduce)_k", m.group(1))
                         or m.group(1).startswith("_ZN3mrr6pack_k")):
            continue
        pkt = [l.strip() for l in k.splitlines()
               if l.strip().startswith(("global_load_dwordx2", "global_store_dwordx2"))]
        assert pkt, "no 64-bit packet accesses in %s" % m.group(1)
        plain = [l for l in pkt if " sc1" not in l]
        assert not plain, "%s: packet accesses without agent scope: %s" % (m.group(1), plain[:3])
        checked += 1
    assert checked >= 40, checked
