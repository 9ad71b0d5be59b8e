"""The quantizers divide by their scale through its reciprocal plus one
fused correction (div_by_scale in the kernels' common header) instead of an
IEEE division.  This CPU check builds tests/div_by_scale_check.c and runs that
operation sequence against IEEE fp32 division over ~40 million (value, scale)
pairs of the kinds the INT8, INT4 and E4M3 codecs produce, plus every code
boundary: the quotients must have the same bits, or both lie below 2^-60
with the same sign (where every code is zero)."""
import re
import shutil
import subprocess
from pathlib import Path

import pytest

HERE = Path(__file__).resolve().parent
CC = shutil.which("cc") or shutil.which("gcc")


def _build(tmp_path, *defs):
    exe = tmp_path / ("divchk" + "".join(d.lower() for d in defs))
    cmd = [CC, "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", *[f"-D{d}" for d in defs],
           str(HERE / "div_by_scale_check.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def _run(exe, seed, per):
    p = subprocess.run([str(exe), str(seed), str(per)], capture_output=True, text=True, timeout=300)
    m = re.search(r"pairs=(\d+) equal=(\d+) tiny=(\d+) bad=(\d+) max_tiny=(\S+)", p.stdout)
    assert m, p.stdout + p.stderr
    return p.returncode, [int(g) for g in m.groups()[:4]], float.fromhex(m.group(5))


@pytest.mark.skipif(CC is None, reason="no C compiler")
def test_reciprocal_quotient_equals_ieee_division(tmp_path):
    exe = _build(tmp_path)
    rc, (pairs, equal, tiny, bad), max_tiny = _run(exe, 20240611, 13_000_000)
    assert pairs > 39_000_000
    assert rc == 0 and bad == 0, f"{bad} pairs differ from the IEEE quotient above 2^-60"
    assert equal + tiny == pairs
    # the only differences are far below every code boundary (E4M3's first is 2^-10)
    assert max_tiny < 2.0 ** -60


@pytest.mark.skipif(CC is None, reason="no C compiler")
def test_check_rejects_the_uncorrected_product(tmp_path):
    # the same harness with the correction step left out must report mismatches
    exe = _build(tmp_path, "WITHOUT_CORRECTION")
    rc, (pairs, equal, tiny, bad), _ = _run(exe, 5, 200_000)
    assert rc == 1 and bad > 0
