"""The C ABI used from plain C: tests/c_abi_client.c (built by
__graft_entry__.build() with gcc against include/mrr.h, libmrr.so and the HIP
runtime's C API) runs RS/AG, the dispatcher and the packet path on raw device
pointers and checks exact sums itself."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_client")


@pytest.mark.skipif(not os.path.exists(CLIENT), reason="C client not built (__graft_entry__.build())")
def test_plain_c_client():
    print("[gpu case] c client", file=sys.stderr, flush=True)
    r = subprocess.run([CLIENT], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c client ok" in r.stdout, r.stdout + r.stderr
