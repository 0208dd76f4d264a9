"""Host checks of arithmetic identities the device code relies on (no GPU)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_divide_by_15_by_two_fmas_is_correctly_rounded(tmp_path):
    # mlx4g32 encoder: the scale range / 15 by a product and one fma correction equals
    # the correctly rounded fp32 quotient for every range a group of fp16 values can
    # have (0, and [2^-24, 131008] within the binades [2^-26, 2^18) swept here)
    exe = tmp_path / "div15"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-march=native", "-o", str(exe),
                    os.path.join(HERE, "csrc", "div15_check.c"), "-lm"], check=True)
    out = subprocess.run([str(exe), "-26", "18"], check=True, capture_output=True, text=True)
    n, bad = map(int, out.stdout.split())
    assert n == 44 * (1 << 23) + 1
    assert bad == 0
