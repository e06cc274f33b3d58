"""Host check of the element division the blockwise quantiser kernels use (fl32(v / s) from a per-tile
reciprocal and two FMAs, for tiles with amax >= 2^-59): the E4M3 codes equal those of IEEE division for
every bf16 element below a strided sample of bf16 amax values, with IEEE and with flushed denormals.
A planted mistake (the sign of -0 not restored) must be caught.  Compiled with the host gcc."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    out = str(tmp_path_factory.mktemp("div") / "division_check")
    subprocess.run([gcc, "-O2", "-mfma", "-o", out, os.path.join(HERE, "division_check.c"), "-lm"], check=True)
    return out


def _run(exe, emin, stride, emax=255, nosign=0):
    r = subprocess.run([exe, str(emin), str(stride), str(emax), str(nosign)], capture_output=True, text=True,
                       check=True)
    pairs, bad = map(int, r.stdout.split())
    return pairs, bad


def test_fma_division_matches_ieee_codes(checker):
    pairs, bad = _run(checker, 68, 211)          # every 211th amax from 2^-59 up, all elements below it
    assert pairs > 4_000_000
    assert bad == 0


def test_planted_sign_mistake_is_caught(checker):
    # without the sign restore, v = -0 quantises to +0 (0x00 instead of 0x80)
    pairs, bad = _run(checker, 68, 997, nosign=1)
    assert bad > 0


def test_tiny_amax_tiles_need_the_division(checker):
    # below the threshold the remainder underflows and codes differ: why those tiles divide per element
    pairs, bad = _run(checker, 1, 5, emax=68)
    assert bad > 0
