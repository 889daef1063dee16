"""A guard over the compiled device code (gfx950 assembly of this library's
own sources, produced here with hipcc).

12- and 16-byte buffer stores whose scalar offset is an SGPR: the compiler's
hazard model assumes their data registers may be overwritten right after the
store issues, and inserts no wait states; on gfx950 such a store then wrote
wrong values (seen as a silently wrong decode state in a variant that put the
row offset in the scalar offset). The library keeps every such store's scalar
offset at the constant 0, where the compiler does insert the waits; this test
fails if a change (or the compiler folding a uniform offset) brings the form
back.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from matrix_memory_rnn_amd import build as gdr_build

HAZARD = re.compile(r"buffer_store_dwordx[34]\s+v\[\d+:\d+\],\s*v\d+,\s*s\[\d+:\d+\],\s*s\d+")


def _device_asm(src, out):
    flags = [f for f in gdr_build.CFLAGS if f != "-fPIC"]
    cmd = [gdr_build.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


@pytest.mark.skipif(not os.path.exists(gdr_build.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not available")
def test_no_wide_buffer_store_with_sgpr_offset():
    srcs = sorted(os.path.join(gdr_build.CSRC, f) for f in os.listdir(gdr_build.CSRC) if f.endswith(".hip"))
    with tempfile.TemporaryDirectory() as tmp:
        outs = [os.path.join(tmp, os.path.basename(s) + ".s") for s in srcs]
        with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
            list(ex.map(_device_asm, srcs, outs))
        bad = []
        for s, o in zip(srcs, outs):
            with open(o) as f:
                for line in f:
                    if HAZARD.search(line):
                        bad.append(f"{os.path.basename(s)}: {line.strip()}")
    assert not bad, "wide buffer stores with an SGPR offset:\n" + "\n".join(bad[:20])


def test_pattern_matches_the_hazardous_form():
    assert HAZARD.search("buffer_store_dwordx4 v[2:5], v98, s[12:15], s2 offen")
    assert not HAZARD.search("buffer_store_dwordx4 v[2:5], v98, s[12:15], 0 offen")
    assert not HAZARD.search("buffer_store_dwordx2 v[2:3], v98, s[12:15], s2 offen")
