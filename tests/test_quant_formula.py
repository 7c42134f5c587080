"""Host checks of the arithmetic behind the INT8 writers' division-free codes
and scales (quant_write.hip), against IEEE binary32 division:

* per-token format (tests/native/quant_formula.c): every FP16 and BF16 input
  against every positive finite FP16 scale (the 13 residue classes of the
  scale patterns run as parallel processes), with the reciprocal anywhere
  within one ulp; all FP16 and BF16 maxima for the scale step;
* static-scale format (tests/native/static_formula.c): every FP16 and BF16
  input, infinities and NaNs included, against powers of two, all-ones
  significands and seeded random scales across the writer's window;
* integer q of the page-pair decode kernels (tests/native/q_digits.c, for
  decode.hip's load_q_pieces): the power-of-two scaling bound for every FP16
  and BF16 head maximum, the three signed base-256 digits of every scaled value
  as the kernel's byte permutes extract them, and int32 room for the sums.

The kernels' own results are compared with the oracle by the GPU tests; these
pin the argument that makes them equal for inputs the GPU tests cannot
enumerate."""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
STRIDE = 13  # scale patterns per process: first, first + 13, ...


def _compile(tmp_path_factory, name):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp(name) / name)
    subprocess.run([gcc, "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "native", name + ".c"), "-lm"], check=True)
    return exe


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    return _compile(tmp_path_factory, "quant_formula")


@pytest.fixture(scope="module")
def static_checker(tmp_path_factory):
    return _compile(tmp_path_factory, "static_formula")


def _workers():
    try:
        return max(1, min(8, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_division_free_codes_and_scales_every_fp16_scale(checker, fmt):
    def run(first):
        return subprocess.run([checker, fmt, str(STRIDE), str(first)], capture_output=True,
                              text=True, timeout=600)

    with ThreadPoolExecutor(_workers()) as ex:
        results = list(ex.map(run, range(1, STRIDE + 1)))
    checks = 0
    for r in results:
        print(r.stdout)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "scale: 64384 values, 0 mismatches" in r.stdout
        line = r.stdout.splitlines()[1]
        assert line.endswith(", 0 mismatches")
        checks += int(line.split()[1])
    # every FP16 scale pattern 1 .. 0x7bff was visited by exactly one process
    assert checks > 0


@pytest.mark.parametrize("fmt,seed", [("f16", 1), ("bf16", 2)])
def test_static_division_free_codes(static_checker, fmt, seed):
    r = subprocess.run([static_checker, fmt, "2000", str(seed)], capture_output=True, text=True,
                       timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith(", 0 mismatches")


@pytest.fixture(scope="module")
def digit_checker(tmp_path_factory):
    return _compile(tmp_path_factory, "q_digits")


def test_pair_kernel_q_digits(digit_checker):
    r = subprocess.run([digit_checker], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "checked 33618818, failed 0"
