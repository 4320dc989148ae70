"""Register budget of the decode kernels, from the compiler's resource report.

The expert kernels hold their loaded code chunks, scales and x values in
VGPRs.  A change that makes the compiler spill them to scratch memory still
computes the right results, so no parity test notices, while every spilled
register adds memory round trips to the hot loop (a multi-input dot whose
decodes the compiler hoisted above a branch once spilled hundreds).  This
compiles the decode sources for gfx950 with the library's own flags (hipcc
cross-compiles without a GPU) and requires every kernel to fit its registers.
"""

import os
import re
import subprocess

import pytest

from bit_dequant_gemv_amd import build

SOURCES = ("moe.hip", "moe_down.hip")

# Known exceptions, by symbol pattern: the per-token down kernels for
# reductions past 6144 (64 lanes x 4 chunks of 32 per row, intermediate sizes
# 6145 .. 8192) hold four code chunks per lane and spill 2-58 VGPRs at some
# row counts.  None of the measured configurations (intermediate sizes 768
# and 2880) runs them; they are correct, only slower.
ALLOWED = {"moe_down.hip": re.compile(r"moe_down_kernelILi\dELi64ELi4E")}


def _parse(stderr):
    """{kernel symbol: VGPRs spilled} from hipcc's kernel-resource-usage remarks."""
    spills, name = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+VGPRs Spill: (\d+)", line)
        if m and name is not None:
            spills[name] = int(m.group(1))
    return spills


@pytest.fixture(scope="module")
def reports(tmp_path_factory):
    """Both sources compiled at once (each compile takes a minute or two)."""
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("resources")
    procs = {}
    for src in SOURCES:
        cmd = [hipcc, *build.HIPCC_FLAGS, *build.FILE_FLAGS.get(src, []), "-c", os.path.join(build.CSRC, src),
               "-o", str(out / (src + ".o")), "-Rpass-analysis=kernel-resource-usage"]
        procs[src] = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True)
    res = {}
    for src, pr in procs.items():
        _, err = pr.communicate(timeout=900)
        assert pr.returncode == 0, err[-3000:]
        res[src] = _parse(err)
    return res


@pytest.mark.parametrize("src", SOURCES)
def test_decode_kernels_do_not_spill(reports, src):
    spills = reports[src]
    assert spills, f"no kernels reported for {src}"
    allowed = ALLOWED.get(src)
    bad = {k: v for k, v in spills.items() if v and not (allowed and allowed.search(k))}
    assert not bad, f"{len(bad)} kernel(s) of {src} spill VGPRs: {sorted(bad.items())[:8]}"
