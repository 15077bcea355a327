"""The fast quantiser of the HIP append and tier kernels reaches the codes
of correctly rounded division (the readings of the quantisation: fp32,
correctly rounded r / qmax and x / s, ties to even).  tests/native/
quant_exact.c repeats its operation sequence on the CPU in IEEE single
precision: the scale formula over every finite fp32 range at 4 and 6 bits
(2^31 values each), and the guarded quotient on 2 * 10^8 reciprocal and
quotient combinations, half of them placed at half-integers.  Two planted
mistakes (the scale without its correction step, the quotient without
its correction step) must be caught.  CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "quant_exact.c")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    out = str(tmp_path_factory.mktemp("qe") / "quant_exact")
    flags = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp"]
    if " fma " in open("/proc/cpuinfo").read():
        flags.append("-mfma")  # hardware fused multiply-add (correctly rounded, as is libm's fmaf)
    subprocess.run(["gcc", *flags, "-o", out, SRC, "-lm"], check=True)
    return out


def _run(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout.strip()


@pytest.mark.parametrize("qmax", [15, 63])
def test_scale_equals_correctly_rounded_division_for_every_finite_range(exe, qmax):
    rc, out = _run(exe, "scale", qmax, 0, 1 << 31)
    assert rc == 0 and out == f"ok {1 << 31}", out


def test_guarded_quotient_rounds_as_correctly_rounded_division(exe):
    rc, out = _run(exe, "quotient", 2026, 40_000_000)  # x 5 reciprocals
    assert rc == 0 and out == "ok 200000000", out


def test_the_checks_catch_a_planted_mistake(exe):
    rc, out = _run(exe, "scale", 63, 0x3F000000, 1 << 20, "plain")
    assert rc == 1 and "mismatch" in out
    rc, out = _run(exe, "quotient", 7, 2_000_000, -1)  # no correction step, no lane deferred
    assert rc == 1 and "wrong" in out
