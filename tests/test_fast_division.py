"""Exhaustive proofs of the kernels' division and square-root shortcuts (CPU only).

The encode kernel replaces IEEE divisions by shorter sequences: RN(a/N) for
the constants N = 7, 15, 127 (uniform scale, INT8 scale), RN(1/h) for an
FP16-valued h (the uniform reciprocal), and the per-element quotient x / s
by a vector's scale s (INT8, INT8 record, FP8 dynamic) through RN(1/s) and
one FMA correction.  `fast_division_check.c` and
`fast_division_scaled_check.c` run the same binary32 sequences over every
input they can see and count results that differ from the correctly
rounded quotient, or, for the scaled quotients, the stored codes that differ.
`fast_division_fixed_check.c` checks the same shortcut for a caller's FP8
fixed scale, where the scales cannot all be enumerated: every source value
against 256 scales in each binade the kernels take it for.
`fast_norm_check.c` does the same for the TurboQuant norm and its
reciprocal in the encoder's common case.
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


@pytest.fixture(scope="module")
def scaled(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("fastdiv_scaled") / "check")
    subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                    os.path.join(HERE, "fast_division_scaled_check.c"), "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
    out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env, timeout=900).stdout
    return {ln.split()[0]: tuple(int(v) for v in ln.split()[1:]) for ln in out.splitlines()}


@pytest.mark.parametrize("src", ["bf16", "fp16"])
@pytest.mark.parametrize("codec", ["int8", "int8rows", "fp8dyn"])
def test_scaled_division_gives_identical_codes(scaled, codec, src):
    """The per-vector shortcut q0 + fma(-q0, s, x) * RN(1/s) against the IEEE
    quotient x / s, for every scale the codec forms and every |x| <= amax:
    the stored code is identical in every case.  FP16 sources give identical
    quotients; BF16 sources differ only for quotients below 2^-10 (deep in
    the subnormal range), which the INT8 and FP8 codes both map to zero."""
    badq, badc, badf, cases = scaled[f"{codec}_{src}"]
    assert cases == (532701120 if src == "bf16" else 503856640)
    assert (badc if codec != "fp8dyn" else badf) == 0
    if src == "fp16":
        assert badq == 0


@pytest.fixture(scope="module")
def fixed(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("fastdiv_fixed") / "check")
    subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                    os.path.join(HERE, "fast_division_fixed_check.c"), "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
    out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env, timeout=600).stdout
    return {ln.split()[0]: tuple(int(v) for v in ln.split()[1:]) for ln in out.splitlines()}


@pytest.mark.parametrize("src", ["bf16", "fp16"])
def test_fixed_scale_division_gives_identical_codes(fixed, src):
    """The FP8 fixed-scale shortcut (the same sequence as above, with the
    caller's scale in [2^-60, 2^60]) against the IEEE quotient: every source
    value 0 <= x <= 448 against 256 scales per binade.  Markstein's theorem
    makes it exact wherever no step underflows, which covers every quotient
    that is not mapped to FP8 zero; no counted case differs."""
    bad, cases = fixed[f"fixed_{src}"]
    assert cases == (0x43E0 + 1 if src == "bf16" else 0x5F00 + 1) * (120 * 256 + 1)
    assert bad == 0


def test_rans_reciprocal_division_exact():
    """The rANS encoder's state update x + bias + q * (4096 - f), q = floor(x
    / f) through a 32-bit reciprocal (f = 1 through 2^32 - 1 and a bias of
    cum + 4095), equals floor(x / f) * 4096 + x mod f + cum for every
    frequency f of a 12-bit model (checked over small x, the top of the
    encoder's state range and random x; the division is exact for all
    x < 2^31 by Granlund-Montgomery)."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "check")
        subprocess.run([gcc, "-O2", "-o", exe, os.path.join(HERE, "ans_division_check.c")], check=True)
        bad, cases = (int(v) for v in subprocess.run([exe], check=True, capture_output=True, text=True,
                                                     timeout=300).stdout.split())
    assert cases > 4096 * 65536 and bad == 0


def test_uniform_quotient_code_exact():
    """The uniform encoder's quotient RN(RN(x - m_h) / sigma_h) through
    RN(1/sigma_h) and one FMA correction, then rounded to the nearest integer
    through the bits of RN(q + 1.5 * 2^23) and clamped: identical to the
    correctly rounded quotient over every pair of significands (which, by
    scaling, covers every positive finite FP16 sigma_h and every d >= s/4),
    and the full code identical to the definition for every FP16 sigma_h
    around every half-integer tie point and the clamp, and zero below s/4."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "check")
        subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                        os.path.join(HERE, "uniform_quotient_check.c"), "-lm"], check=True)
        env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
        out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env, timeout=600).stdout
    res = {ln.split()[0]: (int(ln.split()[1]), int(ln.split()[2])) for ln in out.splitlines()}
    assert res["pairs"] == (0, 1 << 33)
    assert res["ties_7"][0] == 0 and res["ties_7"][1] == (0x7C00 - 1) * 8 * 2050
    assert res["ties_15"][0] == 0 and res["ties_15"][1] == (0x7C00 - 1) * 16 * 2050
    assert res["small"] == (0, 3 * ((1 << 23) + (1 << 20)))


def test_norm_sqrt_and_reciprocal_exact():
    """TurboQuant encode, common case: RN(sqrt(S)) from the hardware estimate
    and one neighbour test each way, for every binary32 S in [2^-96, 2^31)
    and every start within one ulp; RN(1/n) from one Newton step for every
    binary32 n in [2^-48, 2^16) and every start within one ulp but the one
    fixed point per binade (n = (2 - 2^-23) 2^k from 2^-(k+1)), which
    tests/test_gpu_norm_sweep.py rules out for the device's own estimate."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "check")
        subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                        os.path.join(HERE, "fast_norm_check.c"), "-lm"], check=True)
        env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
        out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env, timeout=600).stdout
    res = {ln.split()[0]: (int(ln.split()[1]), int(ln.split()[2])) for ln in out.splitlines()}
    lo, hi = 0x0F800000, 0x4F000000          # bits of 2^-96 and 2^31
    assert res["sqrt_normal"] == (0, 3 * (hi - lo))
    bad, cases = res["recip_normal"]
    assert bad == 0 and cases >= 2 * (0x47800000 - 0x27800000)   # at least two starts per n
    assert res["recip_fixed_point"] == (64, 64)
