"""The GPU activation quantizers take x / s without a per-element division
(reciprocal, one FMA for the exact residual, one FMA to correct; divide for
scales below 2^-100).  This runs tests/quotient_identity.c, which walks every
bf16 amax and every bf16 x with |x| <= amax and requires the E4M3FN and
int8 codes of that quotient to equal the codes of the correctly rounded x / s
(the oracle's rule).  A planted mistake (the sign of zero dropped) must be
caught by the same comparison."""
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
    exe = str(tmp_path_factory.mktemp("qi") / "quotient_identity")
    subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "quotient_identity.c"), "-lm"], check=True)
    return exe


def _run(exe, *args):
    out = subprocess.run([exe, *args], check=True, capture_output=True, text=True,
                         timeout=300).stdout
    rows = {}
    for line in out.split("\n"):
        if line.strip():
            q, pairs, qdiff, cdiff = line.split()
            rows[float(q)] = (int(pairs), int(qdiff), int(cdiff))
    return rows


def test_codes_equal_over_whole_domain(checker):
    rows = _run(checker)
    assert set(rows) == {448.0, 127.0}
    for q, (pairs, qdiff, cdiff) in rows.items():
        assert pairs > 10 ** 9, q      # every (amax, x) pair with s >= 2^-100
        assert qdiff > 0, q            # the quotients do differ (subnormal x) ...
        assert cdiff == 0, q           # ... but never in their codes


def test_planted_sign_mistake_is_caught(checker):
    rows = _run(checker, "nosign")
    assert rows[448.0][2] > 0          # -0.0 must encode as 0x80, not 0x00
