"""The engine divides a scope's amax or range by a constant (448, 57344, 127
for the FP8 E4M3, E5M2 and INT8 scales; 6 for the NVFP4 block scale; 15 and 3
for INT4 and 2- and 4-bit KIVI) with c = RN(1/d) and one fused multiply-add
correction instead of a division.  This checks that correction against IEEE
division for every float in several binades (CPU, gcc, IEEE binary32); page
"量化部署实战", section 伪量化实现, forms every scale as amax / 448 (or the
format's largest value) with a true division."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "div_const_check.c")
# binades of the dividend: the 1e-12 floor's (2^-40), ordinary amax values,
# large ranges and the float32 maximum's
BINADES = ["-40", "-20", "-1", "0", "1", "20", "100", "127"]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("divc") / "div_const_check")
    base = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", SRC, "-o", exe, "-lm"]
    r = subprocess.run(base[:1] + ["-march=native"] + base[1:], capture_output=True, text=True)
    if r.returncode != 0:
        subprocess.run(base, check=True, capture_output=True, text=True)
    return exe


@pytest.mark.parametrize("d", ["448", "57344", "127", "6", "15", "3"])
def test_constant_division_is_correctly_rounded(checker, d):
    out = subprocess.run([checker, d, *BINADES], capture_output=True, text=True, check=True)
    checked, bad = map(int, out.stdout.split())
    assert checked == len(BINADES) * (1 << 23)
    assert bad == 0, out.stderr


def test_checker_catches_a_planted_error(checker, tmp_path):
    """The same program with the correction dropped (q = RN(a * c) alone) must
    report mismatches, so a silent pass above means something."""
    src = open(SRC).read().replace("const float res = fmaf(-r, c, q);", "const float res = q; (void)r;")
    p = tmp_path / "planted.c"
    p.write_text(src)
    exe = str(tmp_path / "planted")
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", str(p), "-o", exe, "-lm"],
                   check=True, capture_output=True)
    out = subprocess.run([exe, "448", "0"], capture_output=True, text=True, check=True)
    assert int(out.stdout.split()[1]) > 0
