"""Exhaustive proofs of the kernels' division shortcuts (CPU only).

The encode kernel replaces two IEEE divisions by shorter sequences: RN(a/N)
for the constants N = 7, 15, 127 (uniform scale, INT8 scale) and RN(1/h) for
an FP16-valued h (the uniform reciprocal).  `fast_division_check.c` runs the
same binary32 sequences over every input they can see and counts results
that differ from the correctly rounded quotient.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("fastdiv") / "check")
    subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                    os.path.join(HERE, "fast_division_check.c"), "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
    out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env, timeout=600).stdout
    return {ln.split()[0]: (int(ln.split()[1]), int(ln.split()[2])) for ln in out.splitlines()}


@pytest.mark.parametrize("n", [7, 15, 127])
def test_div_const_exact_for_all_nonnegative_floats(results, n):
    bad, cases = results[f"div_const_{n}"]
    assert cases == 0x7F800000 and bad == 0


def test_recip_newton_exact_for_all_fp16_values(results):
    bad, cases = results["recip_f16"]
    assert cases == 3 * (0x7C00 - 1) and bad == 0
