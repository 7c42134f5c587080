"""Host check of the arithmetic behind the per-token INT8 writer's
division-free codes and scales (quant_write.hip): compiled from
tests/native/quant_formula.c with gcc and run over every FP16 and BF16
input against every 13th FP16 scale (all FP16 and BF16 maxima for the scale
step). The kernel's own results are compared with the oracle by the GPU
tests; this pins the argument that makes them equal for inputs the GPU
tests cannot enumerate."""

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
    exe = str(tmp_path_factory.mktemp("qf") / "quant_formula")
    subprocess.run([gcc, "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "native", "quant_formula.c"), "-lm"], check=True)
    return exe


@pytest.mark.parametrize("fmt,first", [("f16", 1), ("bf16", 7)])
def test_division_free_codes_and_scales(checker, fmt, first):
    r = subprocess.run([checker, fmt, "13", str(first)], capture_output=True, text=True,
                       timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "scale: 64384 values, 0 mismatches" in r.stdout
    assert ", 0 mismatches" in r.stdout.splitlines()[1]
