"""Every HIP kernel of the library compiles without scratch (private) memory.

A kernel that spills registers or copies an indexed array to scratch runs, but
slowly; the kernels are written to avoid both (no fully unrolled loops over more
registers than a wave has, no lane-dependent indexing of arrays held in
registers). The compiler's resource report for every kernel is read here, from
the same flags the library is built with. CPU only: hipcc cross-compiles gfx950.
"""
import glob
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from verifier_block_forward_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")


def _report(src, out_dir):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    r = subprocess.run([B.HIPCC, *B.FLAGS, "-c", src, "-o", obj, "-Rpass-analysis=kernel-resource-usage"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", r.stderr)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert len(names) == len(scratch), f"{src}: unreadable resource report"  # host-only files: none
    return list(zip(names, scratch))


def test_no_kernel_uses_scratch():
    srcs = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))
    out_dir = tempfile.mkdtemp(prefix="dbf_res_")
    try:
        with ThreadPoolExecutor(min(8, len(srcs))) as ex:
            reports = list(ex.map(lambda s: _report(s, out_dir), srcs))
    finally:
        shutil.rmtree(out_dir, ignore_errors=True)
    kernels = [k for rep in reports for k in rep]
    assert len(kernels) > 40
    bad = [(n, b) for n, b in kernels if b != 0]
    assert not bad, f"kernels with scratch: {bad}"
